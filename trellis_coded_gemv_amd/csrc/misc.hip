// Stand-alone kernels: full-layer decode, the code table, and the randomized
// Hadamard transform on 128-blocks.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

// One thread per weight, in row-major output order (coalesced 16-bit stores).
// The state is read by random access: the 16 bits starting at stream bit K*t
// of the tile (2K*(t/2) for the pair code), taken cyclically ("Trellis
// Quantization" lecture, Part eight).
__global__ __launch_bounds__(256) void decode_kernel(const uint32_t* __restrict__ codes, uint16_t* __restrict__ out,
                                                     int m, int n, int K, int code_id) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)m * (size_t)n) return;
  const int o = (int)(idx / (size_t)n), i = (int)(idx - (size_t)o * n);
  const int wpt = 8 * K;
  const uint32_t* tile = codes + ((size_t)(o >> 4) * (size_t)(n >> 4) + (size_t)(i >> 4)) * (size_t)wpt;
  const int t = 16 * (o & 15) + (i & 15);
  const int p = code_id == 1 ? 2 * K * (t >> 1) : K * t;
  const int j = p >> 5, q = p & 31;
  const uint64_t v = ((uint64_t)tile[j] << 32) | (uint64_t)tile[(j + 1) % wpt];
  const uint32_t state = (uint32_t)(v >> (48 - q)) & 0xFFFFu;
  const CodeRegs cr;
  const uint32_t u = code_halves(state, cr);
  // the rounded GEMV forms' half add (halves_sum_word), so the bit-exact table and decode checks cover it
  if (code_id == 0) out[idx] = (uint16_t)halves_sum_word(u);
  else if (code_id == kCodeMcg) out[idx] = (uint16_t)halves_sum_word(mcg_halves(state, cr));
  else if (code_id == 2) out[idx] = mul1_weight_bits(state);
  else out[idx] = (uint16_t)(pair_weights_rne(u) >> (16 * (t & 1)));
}

// code_id 0, 2 and 3: out[S] = weight of state S; code_id 1: out[2S], out[2S+1] = the state's weight pair.
__global__ __launch_bounds__(256) void code_table_kernel(uint16_t* __restrict__ out, int code_id) {
  const uint32_t s = blockIdx.x * 256 + threadIdx.x;
  const CodeRegs cr;
  const uint32_t u = code_halves(s, cr);
  if (code_id == 0) {
    out[s] = (uint16_t)halves_sum_word(u);
  } else if (code_id == kCodeMcg) {
    out[s] = (uint16_t)halves_sum_word(mcg_halves(s, cr));
  } else if (code_id == 2) {
    out[s] = mul1_weight_bits(s);
  } else {
    const uint32_t w = pair_weights_rne(u);
    out[2 * s] = (uint16_t)w;
    out[2 * s + 1] = (uint16_t)(w >> 16);
  }
}

// One wave per (row, 128-block). inverse == 0: H diag(s) x; inverse == 1: diag(s) H x.
// fp32 butterflies on exact fp16 inputs, then the 1/sqrt(128) normalisation.
__global__ __launch_bounds__(64) void rht_kernel(const uint16_t* __restrict__ in, float* __restrict__ out,
                                                 const uint32_t* __restrict__ signs, int n, int inverse) {
  const int lane = threadIdx.x;
  const size_t base = (size_t)blockIdx.y * n + (size_t)blockIdx.x * kBlock;
  const int col = blockIdx.x * kBlock + lane;
  float v0 = half_bits_to_float(in[base + lane]);
  float v1 = half_bits_to_float(in[base + lane + 64]);
  const bool f0 = sign_bit(signs, col) != 0, f1 = sign_bit(signs, col + 64) != 0;
  if (!inverse) {
    if (f0) v0 = -v0;
    if (f1) v1 = -v1;
  }
  fwht128_wave(v0, v1, lane);
  v0 *= kRsqrt128;
  v1 *= kRsqrt128;
  if (inverse) {
    if (f0) v0 = -v0;
    if (f1) v1 = -v1;
  }
  out[base + lane] = v0;
  out[base + lane + 64] = v1;
}

hipError_t launch_decode(const uint32_t* codes, uint16_t* out, int m, int n, int k_bits, int code_id, hipStream_t s) {
  const size_t total = (size_t)m * (size_t)n;
  const size_t blocks = (total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, out, m, n, k_bits, code_id);
  return hipGetLastError();
}

hipError_t launch_code_table(int code_id, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(code_table_kernel, dim3(256), dim3(256), 0, s, out, code_id);
  return hipGetLastError();
}

hipError_t launch_rht(int n, int rows, const uint16_t* in, float* out, const uint32_t* signs, bool inverse,
                      hipStream_t s) {
  hipLaunchKernelGGL(rht_kernel, dim3(n / kBlock, rows), dim3(64), 0, s, in, out, signs, n, inverse ? 1 : 0);
  return hipGetLastError();
}

}  // namespace tg
