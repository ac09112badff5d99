// Prefill / large-batch path: many activation rows through one layer.
//
// With many rows, the small-batch path's decode -- repeated for every block of
// 16 rows -- would dominate; here every weight is decoded once per 512 rows
// ("Trellis Quantization" lecture, Part eleven: decoding amortised over the
// rows of a prefill batch; Part fourteen) straight into matrix-core operands,
// and never stored. Two launches:
//   rows_rht_kernel      X~ = H diag(s_in) X / sqrt(128), fp16, in 32-column slabs
//   prefill_mfma_kernel  Y = diag(s_out) H (g * (X~ W^T)) / sqrt(128): decode into
//                        LDS, v_mfma_f32_16x16x32_f16, output transform in the epilogue
#include <type_traits>

#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

// Four waves per workgroup, one per (input row, 128-block): the input-side
// transform as fp16, stored in slabs of 32 columns, [n/32][M rows][32], so that
// the 32 columns of 16 consecutive rows the matrix-core loop reads at once are
// 1 KB of contiguous memory. A wave past the row's last block leaves (no
// barriers).
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
  const size_t M = gridDim.y;
  const int c0 = base + lane, c1 = c0 + 64;
  Xt[((size_t)(c0 >> 5) * M + row) * 32 + (c0 & 31)] = __builtin_bit_cast(uint16_t, (_Float16)(v0 * kRsqrt128));
  Xt[((size_t)(c1 >> 5) * M + row) * 32 + (c1 & 31)] = __builtin_bit_cast(uint16_t, (_Float16)(v1 * kRsqrt128));
}

// ---------------------------------------------------------------------------
// Decode-into-MFMA prefill: Y~ = X~ W^T with W^ decoded in registers, never
// stored ("Trellis Quantization" lecture, Part fourteen: decoding amortised over
// the rows of a prefill batch; Part eight: the 16x16 tile as the matrix tile).
//
// A workgroup of 8 waves owns one 128-output block (8 tile rows) and up to 512
// activation rows (64 per wave). The input runs in chunks of 32 columns (two
// tile columns). Per chunk, wave w decodes the B operand of tile row w -- lane
// l holds output row l%16 of the tile row and the 8 input columns 8g..8g+7 of
// the chunk, g = l/16, as fp16 -- into LDS (double-buffered, one barrier per
// chunk); every wave multiplies its 4 row blocks of X~ (32-column slabs of the
// transformed rows, L2-resident) with the 8 B operands: 32
// v_mfma_f32_16x16x32_f16 per chunk, interleaved with the decode of the next
// chunk so the two overlap. Each weight is decoded once per 512 rows, rounded
// to fp16 like the other batched paths (code 0: fp16(lo + hi); pair code:
// (fp16(a + b), fp16(b - a)); mul1: exact).
// A lane's 8 weights (4 states for the pair code) lie in one stream segment
// starting at bit K * (16 * (l%16) + 8 * (g%2)) of its tile; it loads the words
// of that segment (cyclically: the tail-biting wrap), aligns them once with
// v_alignbit and extracts the windows at fixed offsets.
// ---------------------------------------------------------------------------
constexpr int kPfWaves = 8;
constexpr int kPfWaveRows = 64;
constexpr int kPfRows = kPfWaveRows * kPfWaves;   // activation rows per workgroup

template <int K, int CODE>
struct PfGeom {
  static constexpr int V = CODE == 1 ? 2 : 1;        // weights per state
  static constexpr int NWIN = 8 / V;                 // windows per lane and chunk
  static constexpr int STEP = V * K;                 // stream bits between the lane's windows
  static constexpr int NA = ((STEP * (NWIN - 1) + 15) >> 5) + 1;   // aligned words the windows span
  static constexpr int NRAW = NA + 1;                // loaded words (one more for the alignment)
  static constexpr int WPT = 8 * K;
};

template <int K, int CODE>
__device__ __forceinline__ u32x4 pf_decode(const uint32_t (&w)[PfGeom<K, CODE>::NRAW], uint32_t shift,
                                           const CodeRegs& cr) {
  using G = PfGeom<K, CODE>;
  uint32_t al[G::NA];
#pragma unroll
  for (int i = 0; i < G::NA; ++i) al[i] = alignbit(w[i], w[i + 1], shift);   // stream bits from the segment start
  uint32_t st[G::NWIN];
#pragma unroll
  for (int i = 0; i < G::NWIN; ++i) {
    const int p = G::STEP * i, wi = p >> 5, q = p & 31;
    st[i] = q <= 16 ? ubfe(al[wi], 16 - q, 16) : ubfe(alignbit(al[wi], al[wi + 1], 16), 32 - q, 16);
  }
  u32x4 out;
  if constexpr (CODE == 1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = pair_weights_rne(code_halves(st[d], cr));
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if constexpr (CODE == 2) {
        out[d] = mul1_weight_pair(st[2 * d], st[2 * d + 1]);
      } else {
        const uint16_t lo = __builtin_bit_cast(uint16_t, halves_sum_rne(halves_of<CODE>(st[2 * d], cr)));
        const uint16_t hi = __builtin_bit_cast(uint16_t, halves_sum_rne(halves_of<CODE>(st[2 * d + 1], cr)));
        out[d] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
    }
  }
  return out;
}

template <int K, int CODE>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_mfma_kernel(const uint32_t* __restrict__ codes,
                                                                   const uint16_t* __restrict__ scales,
                                                                   const uint32_t* __restrict__ sign_out,
                                                                   const uint16_t* __restrict__ Xt,
                                                                   float* __restrict__ Y, int64_t ldy, int n, int M) {
  using G = PfGeom<K, CODE>;
  constexpr int NRAW = G::NRAW, WPT = G::WPT;
  __shared__ u32x4 bsh[2][kPfWaves][64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int nblk = gridDim.x;
  const int ob = (nblk & 7) == 0 ? (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int j = lane & 15, g = lane >> 4;
  const int n16 = n >> 4, nchunks = n >> 5;
  const int row0 = blockIdx.y * kPfRows + wave * kPfWaveRows;
  const bool rows = row0 < M;   // wave-uniform: this wave has activation rows

  // This lane's code segment: tile (8 ob + wave, 2c + g/2), first window at bit b0.
  const int b0 = K * (16 * j + 8 * (g & 1));
  const int q0 = b0 & 31;
  // A window that starts on a word boundary takes shift 0, where v_alignbit
  // returns its second operand: load from the word before it instead.
  const int jw0 = (b0 >> 5) - (q0 == 0 ? 1 : 0);
  const uint32_t shift = q0 == 0 ? 0u : 32u - (uint32_t)q0;
  int widx[NRAW];
#pragma unroll
  for (int i = 0; i < NRAW; ++i) widx[i] = (jw0 + i + WPT) % WPT;
  const uint32_t* __restrict__ tp = codes + ((size_t)(ob * 8 + wave) * n16 + (g >> 1)) * WPT;
  // A operands: rows row0 + 16a + j (past M: row M-1, never stored), columns 32c + 8g of slab c
  // (offsets in halves, below 2^32: M < 2^16 rows, n/32 < 2^12 slabs).
  uint32_t aoff[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int r = row0 + 16 * a + j;
    r = r < M ? r : M - 1;
    aoff[a] = (uint32_t)r * 32u + 8u * (uint32_t)g;
  }
  const uint32_t slab = (uint32_t)M * 32u;   // halves per 32-column slab

  auto load_codes = [&](int c, uint32_t(&wd)[NRAW]) {
    const uint32_t* t = tp + (size_t)c * 2 * WPT;
#pragma unroll
    for (int i = 0; i < NRAW; ++i) wd[i] = t[widx[i]];
  };
  auto load_a = [&](int c, u32x4(&xa)[4]) {
#pragma unroll
    for (int a = 0; a < 4; ++a) xa[a] = *reinterpret_cast<const u32x4*>(Xt + (aoff[a] + (uint32_t)c * slab));
  };

  float4_t acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[a][t] = float4_t{0.f, 0.f, 0.f, 0.f};

  const CodeRegs cr;
  // Operands in flight in two register sets used alternately: the A operands of chunk c in
  // set c % 2 (loaded two chunks ahead), the code words of chunk c in set c % 2 (loaded three
  // chunks ahead, decoded one chunk ahead into LDS). The loop runs two chunks per trip, so the
  // sets never rotate through copies. (Rotating a single pair, av = next, compiled to register
  // copies after the next loads, and so to a wait, once per chunk, for loads just issued.)
  const int last = nchunks - 1;
  uint32_t cw0[NRAW], cw1[NRAW];
  u32x4 av0[4], av1[4];
  load_codes(0, cw0);
  load_a(0, av0);
  load_codes(last < 1 ? last : 1, cw1);
  load_a(last < 1 ? last : 1, av1);
  bsh[0][wave][lane] = pf_decode<K, CODE>(cw0, shift, cr);
  load_codes(last < 2 ? last : 2, cw0);
  __syncthreads();
  // One chunk: B operands of chunk c from LDS, the next chunk's B decoded from its code words
  // while the matrix cores run (waves with activation rows; the others only decode), then the
  // loads of chunk c + 3's code words and chunk c + 2's A operands into the sets just used. No
  // branch inside: the chunk count is even (n is a multiple of 128) and the store of a B past
  // the last chunk goes to the buffer no wave reads any more.
  auto chunk = [&](int c, u32x4(&av)[4], uint32_t(&cwn)[NRAW], auto mm) {
    u32x4 bo[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) bo[t] = bsh[c & 1][t][lane];
    const u32x4 nb = pf_decode<K, CODE>(cwn, shift, cr);
    if constexpr (decltype(mm)::value) {
      // The next chunk's B operand is decoded in the same block as this chunk's
      // MFMAs, interleaved with them (one MFMA, then two VALU instructions), so
      // the decode runs while the matrix core works.
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av[a]),
                                                             __builtin_bit_cast(half8_t, bo[t]), acc[a][t], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // two VALU
      }
    }
    bsh[(c + 1) & 1][wave][lane] = nb;
    load_codes(c + 3 < last ? c + 3 : last, cwn);
    load_a(c + 2 < last ? c + 2 : last, av);
    __syncthreads();
  };
  if (rows) {
    for (int c = 0; c < nchunks; c += 2) {
      chunk(c, av0, cw1, std::true_type{});
      chunk(c + 1, av1, cw0, std::true_type{});
    }
  } else {
    for (int c = 0; c < nchunks; c += 2) {
      chunk(c, av0, cw1, std::false_type{});
      chunk(c + 1, av1, cw0, std::false_type{});
    }
  }

  // acc[a][t][v] = Y~[row0 + 16a + 4g + v][128 ob + 16t + j]. The output side
  // runs here: y = diag(s_out) H (g * y~) / sqrt(128) over the block's 128
  // outputs o = 16t + j of each row -- butterflies over t in registers, over j
  // across the 16 lanes of the row (lane bits 0..3).
  if (!rows) return;
  float gs[8];
  bool neg[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int o = ob * kBlock + 16 * t + j;
    gs[t] = half_bits_to_float(scales[o]);
    neg[t] = sign_bit(sign_out, o) != 0;
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) x[t] = acc[a][t][v] * gs[t];
#pragma unroll
      for (int hb = 1; hb < 8; hb <<= 1)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if ((t & hb) == 0) {
            const float p = x[t], q = x[t + hb];
            x[t] = p + q;
            x[t + hb] = p - q;
          }
#pragma unroll
      for (int hb = 1; hb < 16; hb <<= 1) {
        const bool upper = (j & hb) != 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float p = shfl_xor(x[t], hb);
          x[t] = upper ? p - x[t] : x[t] + p;
        }
      }
      const int r = row0 + 16 * a + 4 * g + v;
      if (r < M) {
        float* yr = Y + (size_t)r * ldy + (size_t)ob * kBlock + j;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float y = x[t] * kRsqrt128;
          yr[16 * t] = neg[t] ? -y : y;
        }
      }
    }
}

hipError_t launch_prefill_rht(const uint16_t* X, int64_t ldx, const uint32_t* sign_in, uint16_t* Xt, int n, int M,
                              hipStream_t s) {
  hipLaunchKernelGGL(rows_rht_kernel, dim3((n / kBlock + 3) / 4, M), dim3(256), 0, s, X, ldx, sign_in, Xt, n);
  return hipGetLastError();
}

template <int CODE>
static hipError_t launch_pf_mfma(const uint32_t* codes, const uint16_t* scales, const uint32_t* sign_out,
                                 const uint16_t* Xt, float* Y, int64_t ldy, int m, int n, int M, int k_bits,
                                 hipStream_t s) {
  const dim3 grid((unsigned)(m / kBlock), (unsigned)((M + kPfRows - 1) / kPfRows));
#define TG_CASE(K)                                                                                            \
  case K:                                                                                                   \
    hipLaunchKernelGGL((prefill_mfma_kernel<K, CODE>), grid, dim3(64 * kPfWaves), 0, s, codes, scales, sign_out, \
                       Xt, Y, ldy, n, M);                                                                   \
    break;
  switch (k_bits) {
    TG_CASE(1) TG_CASE(2) TG_CASE(3) TG_CASE(4) TG_CASE(5) TG_CASE(6) TG_CASE(7) TG_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const uint32_t* codes, const uint16_t* scales, const uint32_t* sign_out,
                               const uint16_t* Xt, float* Y, int64_t ldy, int m, int n, int M, int k_bits, int code_id,
                               hipStream_t s) {
  if (code_id == 1) return launch_pf_mfma<1>(codes, scales, sign_out, Xt, Y, ldy, m, n, M, k_bits, s);
  if (code_id == 2) return launch_pf_mfma<2>(codes, scales, sign_out, Xt, Y, ldy, m, n, M, k_bits, s);
  if (code_id == kCodeMcg) return launch_pf_mfma<kCodeMcg>(codes, scales, sign_out, Xt, Y, ldy, m, n, M, k_bits, s);
  return launch_pf_mfma<0>(codes, scales, sign_out, Xt, Y, ldy, m, n, M, k_bits, s);
}

}  // namespace tg
