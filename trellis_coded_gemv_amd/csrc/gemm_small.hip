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
// Decomposition: a workgroup of MW waves (16 for up to 16 activation rows,
// else 8) owns one 128-output block and a chunk of the input's tile columns;
// every wave covers all 8 tile rows of the block for every MW-th column of
// the chunk, so the MFMA accumulators of a wave stay put for the whole loop
// and the x~ operand of a column (prepared once per call by xt_prep_kernel,
// read from L2) is loaded once for 8 tiles. The waves are summed through LDS
// at the end. With split K, every workgroup stores its fp32 partials to the
// workspace with device-scope stores and bumps the block's arrival counter;
// the last to arrive sums the splits in a fixed order, applies scale, output
// FWHT and signs, and resets the counter to zero.
//
// Pair code (code_id 1): a state covers two input columns, so one tile row of
// 16 weights needs only 8 code words (k = 16) and one MFMA spans two adjacent
// tiles of a tile row (tile columns 2C, 2C+1 -- contiguous in memory):
// lane l decodes states 4(g%2)..+3 of row l%16 of tile 2C + g/2, and A holds
// the rotated input pairs (x~0 - x~1, x~0 + x~1) of the same column pairs, so
// the MFMA forms a (x~0 - x~1) + b (x~0 + x~1) = (a + b) x~0 + (b - a) x~1.
// TG_FLAG_ROUND_WEIGHTS pairs the rounded weights (RNE(a+b), RNE(b-a)) with
// the plain input pairs (x~0, x~1).
//
// mul1 (code_id 2): the geometry of code 0, with the exact fp16 weight in the
// lo slot of each B word and 0 in the hi slot, as code 0's rounded form.
// MCG (code_id 3): code 0 with v_mul_u32_u24 in place of v_mad_u32_u24.
// For both at K = 2, 4, 8 a lane's four columns are two pairs 16/K apart
// (MfmaGeom::PAIRED): per tile and lane three v_alignbit give two 32-bit
// spans, each holding two windows, and every window feeds its multiply through
// an SDWA word select, with no extract (11 VALU per 4 weights against 13); the
// x~ operand holds the same columns in the same order (xt_prep_kernel's
// paired order), and the B and A k-orders agree, so the product is unchanged.
#include "tg_device.hpp"
#include "tg_internal.hpp"

// Tiles whose B operands are decoded before their MFMAs are issued.
#ifndef TG_MFMA_GROUP
#define TG_MFMA_GROUP 4
#endif
// Steps of code words and x~ in flight per wave.
#ifndef TG_MFMA_PF
#define TG_MFMA_PF 2
#endif
// A workgroup has 16 waves when the activations fit one 16-row MFMA block and
// every wave still gets at least this many steps (more waves hide more
// latency; short loops do not amortise the start-up and the deeper reduction,
// and wider batches need the registers), else 8.
#ifndef TG_MFMA_MIN_STEPS16
#define TG_MFMA_MIN_STEPS16 24
#endif

namespace tg {

// Paired layout: lane group g of a tile row holds input columns lead, lead + 1, lead + D,
// lead + D + 1 with D = 16/K and lead = the (2g)-th column c of the tile with c mod 2D < D (the
// windows 16 stream bits after those of lead and lead + 1 are those of lead + D and lead + D + 1).
// For K = 8 that is 4g .. 4g+3, the plain order.
__host__ __device__ constexpr int paired_lead(int K, int g) {
  const int D = 16 / K, nl = 2 * g;
  return (nl / D) * 2 * D + nl % D;
}
// Position of tile column c in the paired order (the inverse of the layout above).
__host__ __device__ constexpr int paired_pos(int K, int c) {
  const int D = 16 / K, r = c % (2 * D);
  const int nl = (c / (2 * D)) * D + r % D;
  return 4 * (nl >> 1) + (r >= D ? 2 : 0) + (nl & 1);
}

// x~ = H diag(s_in) x / sqrt(128) for every row (rows >= M are zero). Mode 0:
// plain fp16 in tile-column order, [n/16][mpad rows][16 columns], so that the
// 16 rows x 16 columns one MFMA step reads are 512 contiguous bytes; with
// paired_k > 0 the 16 columns of a tile column are in the paired order of that
// K (paired_pos). Modes 1
// and 2: fp16 pairs, the rotated column pairs (x~0 - x~1, x~0 + x~1) or the
// plain pairs (x~0, x~1), row stride n/2 words.
__global__ __launch_bounds__(64) void xt_prep_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                      const uint32_t* __restrict__ sign_in, uint32_t* __restrict__ xt,
                                                      int n, int M, int mode, int paired_k) {
  const int lane = threadIdx.x, row = blockIdx.y;
  if (mode == 0) {
    uint32_t d0 = 0u, d1 = 0u;
    if (row < M) rht_in_block_dup(X + (size_t)row * ldx, sign_in, blockIdx.x * kBlock, lane, d0, d1);
    uint16_t* xh = reinterpret_cast<uint16_t*>(xt);
    const size_t mpad = gridDim.y;
    const int c0 = blockIdx.x * kBlock + lane, c1 = c0 + 64;
    const int p0 = paired_k ? paired_pos(paired_k, c0 & 15) : c0 & 15;
    const int p1 = paired_k ? paired_pos(paired_k, c1 & 15) : c1 & 15;
    xh[((size_t)(c0 >> 4) * mpad + row) * 16 + p0] = (uint16_t)d0;
    xh[((size_t)(c1 >> 4) * mpad + row) * 16 + p1] = (uint16_t)d1;
  } else {
    uint32_t d = 0u;
    if (row < M)
      d = rht_in_block_pair(load_x_block(X + (size_t)row * ldx, sign_in, blockIdx.x * kBlock, lane), lane, mode == 1);
    xt[(size_t)row * (n >> 1) + (size_t)blockIdx.x * 64 + pair_index(lane)] = d;
  }
}

// Geometry of one MFMA step per code.
template <int K, int CODE>
struct MfmaGeom {
  static constexpr int SPAN = CODE != 1 ? 1 : 2;          // tile columns per MFMA step
  static constexpr int STEP = CODE != 1 ? K : 2 * K;      // stream bits between a lane's 4 windows
  static constexpr int WPT = 8 * K;                       // code words per tile
  static constexpr int LW = SPAN * K;                     // code words a lane loads per step
  // Multiply-only codes with K dividing 16 (and K > 1): the lane's four columns are two pairs 16/K
  // apart, each pair's windows in one 32-bit span (paired_columns).
  static constexpr bool PAIRED = (CODE == kCodeMcg || CODE == kCodeMul1) && (K == 2 || K == 4 || K == 8);
  static constexpr int NLW = PAIRED || 3 * STEP > 16 ? 3 : 2;   // staged words a lane reads per tile
};

// Per-lane code words of one tile column step: lane l holds K words of tile
// l/8 of the column (tile rows R0..R0+7), starting at word (l%8)*K.
template <int K>
__device__ __forceinline__ void load_column(const uint32_t* __restrict__ p, uint32_t (&w)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) w[i] = __builtin_nontemporal_load(p + i);
}

// Store a lane's K staged words with the widest aligned LDS stores (contiguous
// across lanes, so conflict-free).
template <int K>
__device__ __forceinline__ void stage_words(uint32_t* dst, const uint32_t (&w)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int i = 0; i < K / 4; ++i)
      reinterpret_cast<u32x4*>(dst)[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  } else if constexpr (K % 2 == 0) {
#pragma unroll
    for (int i = 0; i < K / 2; ++i) reinterpret_cast<u32x2*>(dst)[i] = u32x2{w[2 * i], w[2 * i + 1]};
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) dst[i] = w[i];
  }
}

// One wave: 8 tile rows (a 128-output block) x the steps col0, col0+step, ...
// (a step is SPAN tile columns). For each step the wave loads the 8 x SPAN
// tiles (one contiguous 32*K*SPAN-byte run per tile row, 8 lanes per run),
// restages them through its private LDS slice so that each lane can pick the
// two (three) words its four windows need, decodes one B operand per tile row
// and issues MB MFMAs per tile row against the step's x~ rows.
template <int K, int CODE, bool ROUND, int MB, int PF>
__device__ __forceinline__ void gemm_wave(const GemmArgs& a, int ob, int col0, int ncol, int cstep, uint32_t* slice,
                                          float4_t (&acc)[8][MB]) {
  using G = MfmaGeom<K, CODE>;
  constexpr int NLW = G::NLW, WPT = G::WPT, LW = G::LW, SPAN = G::SPAN, STEP = G::STEP;
  const int lane = threadIdx.x & 63;
  const int jrow = lane & 15, g = lane >> 4;
  // first stream bit of the lane's four windows (paired: of its first span), and the tile of the
  // step they lie in
  const int b0 = G::PAIRED ? K * (16 * jrow + paired_lead(K, g))
                           : CODE != 1 ? K * (16 * jrow + 4 * g) : 2 * K * (8 * jrow + 4 * (g & 1));
  const int toff = CODE != 1 ? 0 : (g >> 1) * WPT;
  const int q0 = b0 & 31, j0 = b0 >> 5;
  int widx[NLW];
  uint32_t shift;
  if (q0 == 0) {        // window starts on a word: alignbit with shift 0 returns its second operand
    widx[0] = (j0 + WPT - 1) % WPT;
    shift = 0u;
#pragma unroll
    for (int i = 1; i < NLW; ++i) widx[i] = (j0 + i - 1) % WPT;
  } else {
    shift = 32u - (uint32_t)q0;
#pragma unroll
    for (int i = 0; i < NLW; ++i) widx[i] = (j0 + i) % WPT;
  }
#pragma unroll
  for (int i = 0; i < NLW; ++i) widx[i] += toff;
  const size_t n16 = (size_t)(a.n >> 4);
  const size_t xrow = (size_t)(a.n / SPAN);                  // words per x~ row
  const int tl = lane >> 3;                                  // tile row this lane loads
  const uint32_t* __restrict__ cptr =
      a.codes + ((size_t)(ob * 8 + tl) * n16 + (size_t)col0 * SPAN) * WPT + (lane & 7) * LW;
  // x~ of this lane: row jrow (+16 per row block), input columns 4g..4g+3 of the step
  const uint32_t* __restrict__ xptr = CODE != 1 ? a.xt + ((size_t)col0 * a.mpad + jrow) * 8 + 2 * g
                                                : a.xt + (size_t)jrow * xrow + 4 * g + (size_t)col0 * 16;
  const size_t xmb = CODE != 1 ? 128 : 16 * xrow;   // words between 16-row blocks
  const uint32_t* __restrict__ cfirst = cptr;
  const uint32_t* __restrict__ xfirst = xptr;
  const size_t cadv = (size_t)cstep * SPAN * WPT;
  const size_t xadv = CODE != 1 ? (size_t)cstep * a.mpad * 8 : (size_t)cstep * 16;

  // Prefetch ring; out-of-range steps re-read the first step (valid addresses,
  // and every path issues the same loads so the waits stay exact).
  uint32_t cw[PF][LW];
  u32x4 xa[PF][MB];
  int issued = 0;
  auto issue = [&](uint32_t(&dst)[LW], u32x4(&xd)[MB]) {
    const bool ok = issued < ncol;
    load_column<LW>(ok ? cptr : cfirst, dst);
    const uint32_t* xq = ok ? xptr : xfirst;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (CODE != 1) {   // four fp16 values; paired up at use
        const u32x2 v = *reinterpret_cast<const u32x2*>(xq + (size_t)mb * xmb);
        xd[mb] = u32x4{v.x, v.y, 0u, 0u};
      } else {
        xd[mb] = *reinterpret_cast<const u32x4*>(xq + (size_t)mb * xmb);
      }
    }
    cptr += cadv;
    xptr += xadv;
    ++issued;
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(cw[p], xa[p]);

  const CodeRegs cr;
  const MulReg mr;
  for (int i0 = 0; i0 < ncol; i0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (i0 + p < ncol) {
        // A operands: code 0 pairs each x~ with itself, (x~, x~) per column
        u32x4 av[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if constexpr (CODE != 1) {
            const uint32_t d0 = xa[p][mb].x, d1 = xa[p][mb].y;
            av[mb] = u32x4{__builtin_amdgcn_perm(d0, d0, 0x01000100u), __builtin_amdgcn_perm(d0, d0, 0x03020302u),
                           __builtin_amdgcn_perm(d1, d1, 0x01000100u), __builtin_amdgcn_perm(d1, d1, 0x03020302u)};
          } else {
            av[mb] = xa[p][mb];
          }
        }
        // stage the step's words, read back the words of all 8 tile rows,
        // decode all 8 B operands, then issue the MFMAs back to back
        stage_words<LW>(slice + lane * LW, cw[p]);   // lane l's LW words sit at word l*LW
        uint32_t wv[8][NLW];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int k = 0; k < NLW; ++k) wv[t][k] = slice[t * SPAN * WPT + widx[k]];
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += TG_MFMA_GROUP) {
        uint32_t bw[TG_MFMA_GROUP][4];
#pragma unroll
        for (int tt = 0; tt < TG_MFMA_GROUP; ++tt) {
          const int t = t0 + tt;
          const uint32_t r1 = alignbit(wv[t][0], wv[t][1], shift);
          uint32_t r2 = 0u;
          if constexpr (NLW == 3) r2 = alignbit(wv[t][1], wv[t][2], shift);
          if constexpr (G::PAIRED) {
            // spans at the lane's first two columns; each holds the window 16/K columns on in its
            // low half. B word order: lead, lead + 1, lead + D, lead + D + 1.
            const uint32_t sp[2] = {r1, alignbit(r1, r2, 32 - K)};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t ph = (sp[i] >> 16) * mr.m, pl = (sp[i] & 0xFFFFu) * mr.m;
              if constexpr (CODE == kCodeMul1) {
                bw[tt][i] = mul1_weight_word(ph & kByteMask);
                bw[tt][2 + i] = mul1_weight_word(pl & kByteMask);
              } else {
                const uint32_t uh = (ph & cr.mask) | cr.xr, ul = (pl & cr.mask) | cr.xr;
                bw[tt][i] = ROUND ? (uint32_t)__builtin_bit_cast(uint16_t, halves_sum_rne(uh)) : uh;
                bw[tt][2 + i] = ROUND ? (uint32_t)__builtin_bit_cast(uint16_t, halves_sum_rne(ul)) : ul;
              }
            }
            continue;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int P = STEP * e;
            const uint32_t st = P <= 16 ? ubfe(r1, 16 - P, 16) : ubfe(alignbit(r1, r2, 48 - P), 0, 16);
            const uint32_t u = halves_of<CODE>(st, cr);
            if constexpr (CODE == 2) bw[tt][e] = (uint32_t)mul1_weight_bits(st);   // (w, 0) against (x~, x~)
            else if constexpr (!ROUND) bw[tt][e] = u;
            else if constexpr (halves_form(CODE)) bw[tt][e] = (uint32_t)__builtin_bit_cast(uint16_t, halves_sum_rne(u));
            else bw[tt][e] = pair_weights_rne(u);
          }
        }
#pragma unroll
        for (int tt = 0; tt < TG_MFMA_GROUP; ++tt) {
          const half8_t bop = __builtin_bit_cast(half8_t, u32x4{bw[tt][0], bw[tt][1], bw[tt][2], bw[tt][3]});
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[t0 + tt][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av[mb]), bop,
                                                                      acc[t0 + tt][mb], 0, 0, 0);
        }
        }
      }
      issue(cw[p], xa[p]);
    }
  }
}

template <int K, int CODE, bool ROUND, int MB, int MW>
__global__ __launch_bounds__(64 * MW) void gemm_small_kernel(GemmArgs a) {
  extern __shared__ uint32_t lds[];
  constexpr int PF = TG_MFMA_PF;
  using G = MfmaGeom<K, CODE>;
  constexpr int SLICE = 8 * G::SPAN * G::WPT;   // staged words per wave
  const int lane = threadIdx.x & 63, wave = wave_id();
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int ob = bid / a.splits, split = bid - ob * a.splits;
  const int ncols = (a.n >> 4) / G::SPAN;   // MFMA steps along the input
  const int c0 = (int)((int64_t)split * ncols / a.splits);
  const int c1 = (int)((int64_t)(split + 1) * ncols / a.splits);
  // wave w takes steps c0+w, c0+w+8, ... of the chunk
  const int nmine = c1 - c0 > wave ? (c1 - c0 - wave + MW - 1) / MW : 0;

  float4_t acc[8][MB];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = float4_t{0.f, 0.f, 0.f, 0.f};
  if (nmine > 0) gemm_wave<K, CODE, ROUND, MB, PF>(a, ob, c0 + wave, nmine, MW, lds + wave * SLICE, acc);

  // Sum the waves' accumulators: a fixed tree through LDS (MW -> MW/2 -> ... -> 1
  // waves; wave w + half adds into wave w), at most four writer waves per round
  // and one 16-row group at a time to bound the LDS footprint.
  float* red = reinterpret_cast<float*>(lds + MW * SLICE);   // [4][8*4][64]
  constexpr int NV = 8 * 4;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int half = MW / 2; half >= 1; half >>= 1) {
#pragma unroll
      for (int base = 0; base < half; base += 4) {
        const int lo = base, hi = base + 4 < half ? base + 4 : half;   // this round's receivers [lo, hi)
        __syncthreads();
        if (wave >= half + lo && wave < half + hi) {
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(((wave - half - lo) * NV) + t * 4 + v) * 64 + lane] = acc[t][mb][v];
        }
        __syncthreads();
        if (wave >= lo && wave < hi) {
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][mb][v] += red[(((wave - lo) * NV) + t * 4 + v) * 64 + lane];
        }
      }
    }
  }

  // Wave 0 now holds the block: acc[t][mb][v] = Y[16mb + 4g + v][ob*128 + 16t + (lane&15)].
  float* ybuf = reinterpret_cast<float*>(lds);   // [16*MB][128]
  uint32_t* flag = lds + 16 * MB * 128;
  const int g = lane >> 4, jrow = lane & 15;
  __syncthreads();
  if (a.splits == 1) {
    if (wave == 0) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) ybuf[(16 * mb + 4 * g + v) * 128 + 16 * t + jrow] = acc[t][mb][v];
    }
    __syncthreads();
    for (int r = wave; r < a.M; r += MW)
      rht_out_block(ybuf[r * 128 + lane], ybuf[r * 128 + lane + 64], a.scales, a.sign_out, a.y + (size_t)r * a.ldy,
                    ob * kBlock, lane);
    return;
  }
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 16 * mb + 4 * g + v;
          if (r < a.M)
            store_partial(a.partials + ((size_t)split * a.M + r) * a.m + ob * kBlock + 16 * t + jrow, acc[t][mb][v]);
        }
  }
  if (!arrive_is_last(&a.counters[ob], (uint32_t)a.splits, flag)) return;
  for (int r = wave; r < a.M; r += MW) {
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

template <int K, int CODE, int MB, int MW>
size_t gemm_lds_bytes() {
  const size_t slices = (size_t)MW * 8 * MfmaGeom<K, CODE>::SPAN * 8 * K * 4;   // per-wave code staging
  const size_t red = 4ull * 8 * 4 * 64 * 4;                     // tree reduction buffer (one row group)
  const size_t ybuf = 16ull * MB * 128 * 4 + 16;
  const size_t a = slices + red;
  return a > ybuf ? a : ybuf;
}

template <int K, int CODE, bool ROUND, int MB, int MW>
static void launch_main(const GemmArgs& a, hipStream_t s) {
  const int grid = (a.m >> 7) * a.splits;
  const size_t lds = gemm_lds_bytes<K, CODE, MB, MW>();
  // raise the dynamic LDS limit (up to 96 KB here); if that fails the launch fails and reports it
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_small_kernel<K, CODE, ROUND, MB, MW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((gemm_small_kernel<K, CODE, ROUND, MB, MW>), dim3(grid), dim3(64 * MW), lds, s, a);
}

template <int K, int CODE, bool ROUND>
static void launch_mb(const GemmArgs& a, hipStream_t s) {
  const int steps = (a.n >> 4) / MfmaGeom<K, CODE>::SPAN / a.splits;   // MFMA steps per workgroup
  switch (a.mpad / 16) {
    case 1:
      if (steps >= 16 * TG_MFMA_MIN_STEPS16) launch_main<K, CODE, ROUND, 1, 16>(a, s);
      else launch_main<K, CODE, ROUND, 1, 8>(a, s);
      break;
    case 2: launch_main<K, CODE, ROUND, 2, 8>(a, s); break;
    case 3: launch_main<K, CODE, ROUND, 3, 8>(a, s); break;
    default: launch_main<K, CODE, ROUND, 4, 8>(a, s); break;
  }
}

template <int CODE>
static hipError_t launch_code(const GemmArgs& a, int k_bits, bool round_weights, hipStream_t s) {
#define TG_CASE(K) \
  case K:                                                                                                  \
    round_weights && rounded_form(CODE) ? launch_mb<K, CODE, rounded_form(CODE)>(a, s) : launch_mb<K, CODE, false>(a, s); \
    break;
  switch (k_bits) {
    TG_CASE(1) TG_CASE(2) TG_CASE(3) TG_CASE(4) TG_CASE(5) TG_CASE(6) TG_CASE(7) TG_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
  return hipGetLastError();
}

hipError_t launch_gemm_small(const GemmArgs& a, const uint16_t* X, int64_t ldx, const uint32_t* sign_in, int k_bits,
                             int code_id, bool round_weights, hipStream_t s) {
  const int mode = code_id == 1 ? (round_weights ? 2 : 1) : 0;
  // the paired column order of the multiply-only codes (identity at K = 8)
  const int paired_k = (code_id == kCodeMul1 || code_id == kCodeMcg) && (k_bits == 2 || k_bits == 4) ? k_bits : 0;
  hipLaunchKernelGGL(xt_prep_kernel, dim3(a.n / kBlock, a.mpad), dim3(64), 0, s, X, ldx, sign_in,
                     const_cast<uint32_t*>(a.xt), a.n, a.M, mode, paired_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (code_id == 2) return launch_code<2>(a, k_bits, false, s);
  if (code_id == kCodeMcg) return launch_code<kCodeMcg>(a, k_bits, round_weights, s);
  return code_id == 0 ? launch_code<0>(a, k_bits, round_weights, s) : launch_code<1>(a, k_bits, round_weights, s);
}

}  // namespace tg
