// Small-batch trellis-coded GEMM on the gfx950 matrix cores: Y[r] = W X[r], r < M <= 64.
//
// The 16x16 trellis tile is the matrix-core tile ("Trellis Quantization"
// lecture, Part eight); decoding happens in registers and feeds the matrix
// units directly (lecture, Part eleven). One v_mfma_f32_16x16x32_f16 consumes
// exactly one decoded tile for 16 activation rows:
//   B (32 x 16): column j = output row j of the tile; k = 2c + {0: lo, 1: hi}
//                for input column c. Lane l supplies B[8g..8g+7][l%16],
//                g = l/16, i.e. the two fp16 halves of W^[l%16][4g..4g+3] --
//                exactly the four words the code's mask/XOR step produces.
//   A (16 x 32): row i = activation row; A[i][2c + b] = x~[i][c] for both b.
//                Lane l supplies A[l%16][8g..8g+7] = 4 pairs (x~, x~).
// The MFMA therefore forms sum_c (lo + hi) x~ in fp32 with the weight's two
// halves added exactly; TG_FLAG_ROUND_WEIGHTS puts fp16_rne(lo+hi) in the lo
// slot and 0 in the hi slot instead.
//
// Each lane decodes 4 weights per tile from one 32-bit register holding
// stream bits [K(16j+4g), K(16j+4g)+32) -- one v_alignbit with a per-lane,
// loop-invariant shift over two (three for K >= 6) loaded words -- then
// v_bfe + v_mad_u32_u24 + v_and_or_b32 per weight.
//
// Decomposition: a workgroup of 8 waves owns one 128-output block (a wave per
// tile row) and a chunk of the input; x~ rows (prepared once per call by
// xt_prep_kernel, already transformed) are staged through double-buffered LDS
// a sub-chunk at a time and shared by the 8 waves. Split-K partials and the
// last-arriving-workgroup epilogue are as in the batch-1 kernel.
#include "tg_device.hpp"
#include "tg_internal.hpp"

namespace tg {

// x~ = H diag(s_in) x / sqrt(128) for every row (rows >= M are zero), stored as fp16 pairs.
__global__ __launch_bounds__(64) void xt_prep_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                      const uint32_t* __restrict__ sign_in, uint32_t* __restrict__ xt,
                                                      int n, int M) {
  const int lane = threadIdx.x, row = blockIdx.y;
  const size_t ob = (size_t)row * n + (size_t)blockIdx.x * kBlock;
  uint32_t d0 = 0u, d1 = 0u;
  if (row < M) rht_in_block_dup(X + (size_t)row * ldx, sign_in, blockIdx.x * kBlock, lane, d0, d1);
  xt[ob + lane] = d0;
  xt[ob + lane + 64] = d1;
}

template <int SUB>   // tiles per LDS sub-chunk
struct GemmLds {
  static constexpr int kCols = SUB * 16;       // inputs per sub-chunk
  static constexpr int kStride = kCols + 4;    // padded row stride in words (bank spread)
};

template <int K, bool ROUND, int MB, int SUB>
__global__ __launch_bounds__(kGemvThreads) void gemm_small_kernel(GemmArgs a) {
  extern __shared__ uint32_t lds[];
  constexpr int NLW = K >= 6 ? 3 : 2;            // code words loaded per lane per tile
  constexpr int MPAD = 16 * MB;
  constexpr int STRIDE = GemmLds<SUB>::kStride;
  constexpr int COLS = GemmLds<SUB>::kCols;
  constexpr int WPT = 8 * K;                      // words per tile

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int ob = bid / a.splits, split = bid - ob * a.splits;

  const int nsub_total = a.n / COLS;
  const int sub0 = (int)((int64_t)split * nsub_total / a.splits);
  const int sub1 = (int)((int64_t)(split + 1) * nsub_total / a.splits);
  const int nsub = sub1 - sub0;

  // Per-lane decode geometry (identical for every tile).
  const int jrow = lane & 15, g = lane >> 4;
  const int b0 = K * (16 * jrow + 4 * g);
  const int q0 = b0 & 31, j0 = b0 >> 5;
  int widx[NLW];
  uint32_t shift;
  if (q0 == 0) {
    widx[0] = (j0 + WPT - 1) % WPT;
    shift = 0u;
#pragma unroll
    for (int i = 1; i < NLW; ++i) widx[i] = (j0 + i - 1) % WPT;
  } else {
    shift = 32u - (uint32_t)q0;
#pragma unroll
    for (int i = 0; i < NLW; ++i) widx[i] = (j0 + i) % WPT;
  }

  const int R = ob * 8 + wave;
  const uint32_t* __restrict__ rowp = a.codes + ((size_t)R * (size_t)(a.n >> 4) + (size_t)sub0 * SUB) * WPT;

  auto xb = [&](int b) -> uint32_t* { return lds + b * (MPAD * STRIDE); };

  // Stage x~ of sub-chunk `s` (rows 0..MPAD-1, COLS inputs) into LDS buffer `b`.
  constexpr int kStageVec = MPAD * COLS / 4;                       // u32x4 per sub-chunk
  constexpr int kStagePer = (kStageVec + kGemvThreads - 1) / kGemvThreads;
  u32x4 stage[kStagePer];
  auto stage_load = [&](int s) {
#pragma unroll
    for (int v = 0; v < kStagePer; ++v) {
      const int idx = threadIdx.x + v * kGemvThreads;
      if (idx < kStageVec) {
        const int row = idx / (COLS / 4), c4 = idx - row * (COLS / 4);
        const int sc = s < nsub ? sub0 + s : sub0;    // out of range: re-read a valid line
        stage[v] = *reinterpret_cast<const u32x4*>(a.xt + (size_t)row * a.n + (size_t)sc * COLS + c4 * 4);
      }
    }
  };
  auto stage_store = [&](int b) {
#pragma unroll
    for (int v = 0; v < kStagePer; ++v) {
      const int idx = threadIdx.x + v * kGemvThreads;
      if (idx < kStageVec) {
        const int row = idx / (COLS / 4), c4 = idx - row * (COLS / 4);
        *reinterpret_cast<u32x4*>(xb(b) + row * STRIDE + c4 * 4) = stage[v];
      }
    }
  };

  uint32_t cw[SUB][NLW];
  auto code_load = [&](int s) {
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
#pragma unroll
      for (int i = 0; i < NLW; ++i)
        cw[t][i] = __builtin_nontemporal_load((s < nsub ? rowp + ((size_t)s * SUB + t) * WPT : a.codes) + widx[i]);
    }
  };

  float4_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
  const CodeRegs cr;

  if (nsub > 0) {
    stage_load(0);
    code_load(0);
    stage_store(0);
    __syncthreads();
  }
  for (int s = 0; s < nsub; ++s) {
    const int cur = s & 1;
    uint32_t cc[SUB][NLW];
#pragma unroll
    for (int t = 0; t < SUB; ++t)
#pragma unroll
      for (int i = 0; i < NLW; ++i) cc[t][i] = cw[t][i];
    stage_load(s + 1);
    code_load(s + 1);
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      const uint32_t r1 = alignbit(cc[t][0], cc[t][1], shift);
      uint32_t r2 = 0u;
      if constexpr (NLW == 3) r2 = alignbit(cc[t][1], cc[t][2], shift);
      uint32_t bw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int P = K * e;
        uint32_t st;
        if (P <= 16) st = ubfe(r1, 16 - P, 16);
        else st = ubfe(alignbit(r1, r2, 48 - P), 0, 16);
        const uint32_t u = code_halves(st, cr);
        if constexpr (ROUND) bw[e] = (uint32_t)__builtin_bit_cast(uint16_t, halves_sum_rne(u));
        else bw[e] = u;
      }
      const half8_t bop = __builtin_bit_cast(half8_t, u32x4{bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(xb(cur) + (16 * mb + jrow) * STRIDE + t * 16 + 4 * g);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), bop, acc[mb], 0, 0, 0);
      }
    }
    if (s + 1 < nsub) stage_store(cur ^ 1);
    __syncthreads();
  }

  // acc[mb][v] = partial Y[16mb + 4g + v][16R + jrow]
  float* ybuf = reinterpret_cast<float*>(lds);   // [MPAD][128], reuses the staging buffers
  uint32_t* flag = lds + MPAD * 128;
  const int ocol = wave * 16 + jrow;
  if (a.splits == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int v = 0; v < 4; ++v) ybuf[(16 * mb + 4 * g + v) * 128 + ocol] = acc[mb][v];
    __syncthreads();
    for (int r = wave; r < a.M; r += kGemvWaves)
      rht_out_block(ybuf[r * 128 + lane], ybuf[r * 128 + lane + 64], a.scales, a.sign_out, a.y + (size_t)r * a.ldy,
                    ob * kBlock, lane);
    return;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * mb + 4 * g + v;
      if (r < a.M) store_partial(a.partials + ((size_t)split * a.M + r) * a.m + ob * kBlock + ocol, acc[mb][v]);
    }
  if (!arrive_is_last(&a.counters[ob], (uint32_t)a.splits, flag)) return;
  for (int r = wave; r < a.M; r += kGemvWaves) {
    float v0 = 0.f, v1 = 0.f;
#pragma unroll 8
    for (int t = 0; t < a.splits; ++t) {   // unrolled so the loads are in flight together
      const float* pp = a.partials + ((size_t)t * a.M + r) * a.m + ob * kBlock;
      v0 += load_partial(pp + lane);
      v1 += load_partial(pp + lane + 64);
    }
    rht_out_block(v0, v1, a.scales, a.sign_out, a.y + (size_t)r * a.ldy, ob * kBlock, lane);
  }
  if (threadIdx.x == 0) reset_counter(&a.counters[ob]);
}

template <int MB>
constexpr int gemm_sub() { return MB <= 2 ? 8 : 4; }

template <int MB>
size_t gemm_lds_bytes() {
  constexpr int SUB = gemm_sub<MB>();
  const size_t staging = 2ull * 16 * MB * GemmLds<SUB>::kStride * 4;
  const size_t ybuf = 16ull * MB * 128 * 4 + 16;
  return staging > ybuf ? staging : ybuf;
}

template <int K, bool ROUND, int MB>
static void launch_main(const GemmArgs& a, hipStream_t s) {
  const int grid = (a.m >> 7) * a.splits;
  hipLaunchKernelGGL((gemm_small_kernel<K, ROUND, MB, gemm_sub<MB>()>), dim3(grid), dim3(kGemvThreads),
                     gemm_lds_bytes<MB>(), s, a);
}

template <int K, bool ROUND>
static void launch_mb(const GemmArgs& a, hipStream_t s) {
  switch (a.mpad / 16) {
    case 1: launch_main<K, ROUND, 1>(a, s); break;
    case 2: launch_main<K, ROUND, 2>(a, s); break;
    case 3: launch_main<K, ROUND, 3>(a, s); break;
    default: launch_main<K, ROUND, 4>(a, s); break;
  }
}

int gemm_sub_tiles(int mpad) { return mpad <= 32 ? 8 : 4; }

hipError_t launch_gemm_small(const GemmArgs& a, const uint16_t* X, int64_t ldx, const uint32_t* sign_in, int k_bits,
                             bool round_weights, hipStream_t s) {
  hipLaunchKernelGGL(xt_prep_kernel, dim3(a.n / kBlock, a.mpad), dim3(64), 0, s, X, ldx, sign_in,
                     const_cast<uint32_t*>(a.xt), a.n, a.M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define TG_CASE(K) \
  case K: round_weights ? launch_mb<K, true>(a, s) : launch_mb<K, false>(a, s); break;
  switch (k_bits) {
    TG_CASE(1) TG_CASE(2) TG_CASE(3) TG_CASE(4) TG_CASE(5) TG_CASE(6) TG_CASE(7) TG_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
  return hipGetLastError();
}

}  // namespace tg
