// Prefill / large-batch path: decode the layer once to fp16, then one dense
// GEMM on the matrix cores.
//
// With many activation rows the decode of the small-batch path, repeated for
// every block of 16 rows, dominates; here every weight is decoded exactly once
// per call ("Trellis Quantization" lecture, Part eleven: decoding amortised over
// the rows of a prefill batch), written as fp16 rows to the workspace, and the
// contraction Y~ = X~ W^T (fp16 in, fp32 accumulate) runs as a plain library
// GEMM (rocBLAS). The transforms on both sides stay in this library's kernels:
//   rows_rht_kernel     X~ = H diag(s_in) X / sqrt(128), fp16 rows
//   decode_rows_kernel  W^ as fp16 rows (16 tiles per wave, coalesced stores)
//   rows_out_kernel     Y = diag(s_out) H (g * Y~) / sqrt(128), in place
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

// Four waves per workgroup, one per (input row, 128-block): the input-side
// transform as fp16. A wave past the row's last block leaves (no barriers).
__global__ __launch_bounds__(256) void rows_rht_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                       const uint32_t* __restrict__ sign_in,
                                                       uint16_t* __restrict__ Xt, int n) {
  const int lane = threadIdx.x & 63, row = blockIdx.y, blk = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= (n >> 7)) return;
  const int base = blk * kBlock;
  const XBlock xb = load_x_block(X + (size_t)row * ldx, sign_in, base, lane);
  const uint16_t b0 = xb.b0 ^ (uint16_t)(((xb.s0 >> ((base + lane) & 31)) & 1u) << 15);
  const uint16_t b1 = xb.b1 ^ (uint16_t)(((xb.s1 >> ((base + lane + 64) & 31)) & 1u) << 15);
  float v0 = half_bits_to_float(b0), v1 = half_bits_to_float(b1);
  fwht128_wave(v0, v1, lane);
  uint16_t* out = Xt + (size_t)row * n + base;
  out[lane] = __builtin_bit_cast(uint16_t, (_Float16)(v0 * kRsqrt128));
  out[lane + 64] = __builtin_bit_cast(uint16_t, (_Float16)(v1 * kRsqrt128));
}

// One wave per (tile row, 16 consecutive tiles). Lane l decodes rows
// 4(l%4)..+3 of tile l/4 of the step -- 64 consecutive sequence steps, the
// same lane layout as the batch-1 kernel (the overlap bits past the lane's
// last window come from the next lane of its quad, which wraps to the tile's
// first word) -- and stores each of its 4 rows as 16 fp16 values (32 bytes);
// the 16 tiles of a step make every output row segment 512 contiguous bytes.
template <int K, int CODE>
__global__ __launch_bounds__(256) void decode_rows_kernel(const uint32_t* __restrict__ codes, uint16_t* __restrict__ W,
                                                          int m, int n) {
  constexpr int NW = 2 * K;
  const int lane = threadIdx.x & 63;
  const int n16 = n >> 4;
  const int steps = (n16 + 15) >> 4;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (m >> 4) * steps) return;   // whole waves only: no shuffles below cross waves
  const int R = wid / steps, st = wid - R * steps;
  const int jslot = lane >> 2, q = lane & 3;
  const int C = st * 16 + jslot;
  const bool ok = C < n16;
  const uint32_t* __restrict__ p = codes + ((size_t)R * n16 + (ok ? C : n16 - 1)) * (8 * K) + q * NW;
  uint32_t w[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = __builtin_nontemporal_load(p + i);
  const uint32_t nb = quad_rotate_next(w[0]);
  auto word = [&](int j) -> uint32_t { return j < NW ? w[j] : nb; };
  auto window = [&](int bitpos) -> uint32_t {
    const int j = bitpos >> 5, qq = bitpos & 31;
    return qq <= 16 ? ubfe(word(j), 16 - qq, 16) : ubfe(alignbit(word(j), word(j + 1), 16), 32 - qq, 16);
  };
  const CodeRegs cr;
  uint32_t out[4][8];   // 4 rows x 16 fp16
  if constexpr (CODE == 0) {
#pragma unroll
    for (int tl = 0; tl < 64; tl += 2) {
      const uint16_t a = __builtin_bit_cast(uint16_t, halves_sum_rne(code_halves(window(K * tl), cr)));
      const uint16_t b = __builtin_bit_cast(uint16_t, halves_sum_rne(code_halves(window(K * (tl + 1)), cr)));
      out[tl >> 4][(tl & 15) >> 1] = (uint32_t)a | ((uint32_t)b << 16);
    }
  } else if constexpr (CODE == 2) {
#pragma unroll
    for (int tl = 0; tl < 64; tl += 2) {
      const uint16_t a = mul1_weight_bits(window(K * tl));
      const uint16_t b = mul1_weight_bits(window(K * (tl + 1)));
      out[tl >> 4][(tl & 15) >> 1] = (uint32_t)a | ((uint32_t)b << 16);
    }
  } else {
#pragma unroll
    for (int sl = 0; sl < 32; ++sl) out[sl >> 3][sl & 7] = pair_weights_rne(code_halves(window(2 * K * sl), cr));
  }
  if (!ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4* dst = reinterpret_cast<u32x4*>(W + (size_t)(16 * R + 4 * q + i) * n + 16 * C);
    dst[0] = u32x4{out[i][0], out[i][1], out[i][2], out[i][3]};
    dst[1] = u32x4{out[i][4], out[i][5], out[i][6], out[i][7]};
  }
}

// Four waves per workgroup, one per (output row, 128-block): scale, output
// transform and signs in place.
__global__ __launch_bounds__(256) void rows_out_kernel(float* __restrict__ Y, int64_t ldy,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint32_t* __restrict__ sign_out, int m) {
  const int lane = threadIdx.x & 63, blk = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= (m >> 7)) return;
  const int base = blk * kBlock;
  float* y = Y + (size_t)blockIdx.y * ldy;
  rht_out_block(y[base + lane], y[base + lane + 64], scales, sign_out, y, base, lane);
}

hipError_t launch_prefill_rht(const uint16_t* X, int64_t ldx, const uint32_t* sign_in, uint16_t* Xt, int n, int M,
                              hipStream_t s) {
  hipLaunchKernelGGL(rows_rht_kernel, dim3((n / kBlock + 3) / 4, M), dim3(256), 0, s, X, ldx, sign_in, Xt, n);
  return hipGetLastError();
}

template <int CODE>
static hipError_t launch_dec(const uint32_t* codes, uint16_t* W, int m, int n, int k_bits, hipStream_t s) {
  const int waves = (m >> 4) * (((n >> 4) + 15) >> 4);
  const dim3 grid((waves + 3) / 4);
#define TG_CASE(K) \
  case K: hipLaunchKernelGGL((decode_rows_kernel<K, CODE>), grid, dim3(256), 0, s, codes, W, m, n); break;
  switch (k_bits) {
    TG_CASE(1) TG_CASE(2) TG_CASE(3) TG_CASE(4) TG_CASE(5) TG_CASE(6) TG_CASE(7) TG_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
  return hipGetLastError();
}

hipError_t launch_prefill_decode(const uint32_t* codes, uint16_t* W, int m, int n, int k_bits, int code_id,
                                 hipStream_t s) {
  if (code_id == 2) return launch_dec<2>(codes, W, m, n, k_bits, s);
  return code_id == 0 ? launch_dec<0>(codes, W, m, n, k_bits, s) : launch_dec<1>(codes, W, m, n, k_bits, s);
}

hipError_t launch_prefill_out(float* Y, int64_t ldy, const uint16_t* scales, const uint32_t* sign_out, int m, int M,
                              hipStream_t s) {
  hipLaunchKernelGGL(rows_out_kernel, dim3((m / kBlock + 3) / 4, M), dim3(256), 0, s, Y, ldy, scales, sign_out, m);
  return hipGetLastError();
}

}  // namespace tg
