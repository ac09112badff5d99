// Per-step pieces of the batch-1 decode shared by the batch-1, grouped and
// fused kernels: a lane's code words of one 16-tile step, the decode and fused
// dot product of its 64 weights, the cross-lane reduction and the x~ reads.
// Window extraction follows the bitshift trellis of the "Trellis Quantization"
// lecture, Part eight; the code its Part nine.
#pragma once

#include "tg_device.hpp"

namespace tg {

// Load this lane's 2K words (8K bytes) of the current step.
template <int K>
__device__ __forceinline__ void load_lane_words(const uint32_t* __restrict__ p, uint32_t (&w)[2 * K]) {
  if constexpr (K % 2 == 0) {
#pragma unroll
    for (int i = 0; i < K / 2; ++i) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
      w[4 * i + 0] = v[0];
      w[4 * i + 1] = v[1];
      w[4 * i + 2] = v[2];
      w[4 * i + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p) + i);
      w[2 * i + 0] = v[0];
      w[2 * i + 1] = v[1];
    }
  }
}

#ifndef TG_DECODE_ILP
#define TG_DECODE_ILP 4
#endif

// Window (16-bit state) of the lane's sequence step tl: stream bits K*tl ..
// K*tl+15 of the lane's run (a compile-time position), the overlap past the
// lane's last word coming from the next lane's first word.
template <int K, int STEP>
__device__ __forceinline__ uint32_t lane_window(const uint32_t (&w)[2 * K], uint32_t nb, int tl) {
  constexpr int NW = 2 * K;
  const int p = STEP * tl;         // window start, bits from the lane's first stream bit
  const int j = p >> 5, q = p & 31;
  const uint32_t wj = j < NW ? w[j] : nb;
  if (q <= 16) return ubfe(wj, 16 - q, 16);
  const uint32_t wj1 = j + 1 < NW ? w[j + 1] : nb;
  return ubfe(alignbit(wj, wj1, 16), 32 - q, 16);
}

// Multiply-only codes (MCG, mul1): with K dividing 16, the window 16 stream
// bits after window tl is window tl + 16/K, so one 32-bit span holds two
// windows (tl in its high half, tl + 16/K in its low half) and one v_alignbit
// serves both. The multiplier sits in an SGPR (MulReg), so each half feeds
// v_mul_u32_u24 through an SDWA word select and needs no extract of its own.

// The 32 stream bits starting at window tl's first bit.
template <int K>
__device__ __forceinline__ uint32_t lane_span(const uint32_t (&w)[2 * K], uint32_t nb, int tl) {
  constexpr int NW = 2 * K;
  const int p = K * tl;
  const int j = p >> 5, q = p & 31;
  const uint32_t wj = j < NW ? w[j] : nb;
  if (q == 0) return wj;
  const uint32_t wj1 = j + 1 < NW ? w[j + 1] : nb;
  return alignbit(wj, wj1, 32 - q);
}

// The lane's 32 leading windows, in an order that gives consecutive leads
// different rows: lead n (0..31) -> window index. Its partner is lead + 16/K.
template <int K>
__device__ __forceinline__ constexpr int span_lead(int n) {
  constexpr int D = 16 / K;
  const int g = n >> 2, i = n & 3;
  if constexpr (K == 1) return 16 * (2 * (i & 1)) + 2 * g + (i >> 1);   // rows 0, 2 lead rows 1, 3
  else return 16 * i + (g / D) * 2 * D + g % D;                        // row i, columns paired D apart
}

// Decode the lane's 64 weights (4 rows x 16 columns of one tile) and
// accumulate their dot products with x~ of that tile column.
//   w   : the lane's 2K stream words (stream bits 0 .. 64K-1 of the lane, MSB first)
//   nb  : first word of the next lane in the tile (wrapping at the tile's end)
//   xx  : 16 pairs (x~_c, x~_c) for the tile's 16 input columns
// The weights are taken a column at a time for all 4 rows (and TG_DECODE_ILP / 4
// columns at once), each stage of the decode issued for the whole group before
// the next, into one accumulator per row and column parity: independent chains
// that a wave can issue back to back, instead of one chain through a register
// whose every instruction waits for the previous one.
// CODE: 0 or kCodeMcg (the two codes in halves_form).
template <int K, bool ROUND, int CODE = 0>
__device__ __forceinline__ void decode_dot_64(const uint32_t (&w)[2 * K], uint32_t nb, const uint32_t (&xx)[16],
                                              float (&acc)[4], const CodeRegs& cr) {
  constexpr int CW = TG_DECODE_ILP >= 8 ? 2 : 1;    // columns per group
  float a2[4][CW];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    a2[r][0] = acc[r];
    if constexpr (CW == 2) a2[r][1] = 0.f;
  }
#pragma unroll
  for (int c0 = 0; c0 < 16; c0 += CW) {
    uint32_t st[4][CW], u[4][CW];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[r][cc] = lane_window<K, K>(w, nb, 16 * r + c0 + cc);
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r][cc] = halves_of<CODE>(st[r][cc], cr);
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (ROUND) {
          const uint32_t wr = halves_sum_word(u[r][cc]);
          a2[r][cc] = dot2(wr, xx[c0 + cc], a2[r][cc]);
        } else {
          a2[r][cc] = dot2(u[r][cc], xx[c0 + cc], a2[r][cc]);
        }
      }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = CW == 2 ? a2[r][0] + a2[r][1] : a2[r][0];
}

// MCG (code_id 3) with the windows paired as for mul1 when K divides 16: per
// two weights one v_alignbit, then per weight an SDWA-selected v_mul_u32_u24,
// v_and_or_b32 and v_dot2c_f32_f16 against (x~, x~). Other K: decode_dot_64.
template <int K, bool ROUND>
__device__ __forceinline__ void decode_dot_mcg_64(const uint32_t (&w)[2 * K], uint32_t nb, const uint32_t (&xx)[16],
                                                  float (&acc)[4], const CodeRegs& cr) {
  if constexpr (16 % K == 0) {
    constexpr int D = 16 / K;
    const MulReg mr;
#pragma unroll
    for (int n0 = 0; n0 < 32; n0 += 4) {
      uint32_t u[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t t = lane_span<K>(w, nb, span_lead<K>(n0 + i));
        u[i][0] = (((t >> 16) * mr.m) & cr.mask) | cr.xr;
        u[i][1] = (((t & 0xFFFFu) * mr.m) & cr.mask) | cr.xr;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tl = span_lead<K>(n0 + i) + h * D;
          if constexpr (ROUND) {
            const uint32_t wr = halves_sum_word(u[i][h]);
            acc[tl >> 4] = dot2(wr, xx[tl & 15], acc[tl >> 4]);
          } else {
            acc[tl >> 4] = dot2(u[i][h], xx[tl & 15], acc[tl >> 4]);
          }
        }
    }
  } else {
    decode_dot_64<K, ROUND, kCodeMcg>(w, nb, xx, acc, cr);
  }
}

// Pair code (code_id 1): the lane's 64 weights are 32 states, state s at
// stream bit 2K*s (two weights per trellis step), weights 2s and 2s+1 of the
// lane's run = columns 2(s%8), 2(s%8)+1 of row s/8. Per state: one window
// extract, v_mad_u32_u24, v_and_or_b32 and one v_dot2c_f32_f16 against the
// rotated input pair (x~0 - x~1, x~0 + x~1) -- two weights per dot. States are
// grouped across the 4 rows as for code 0.
// ROUND: the rounded pair (RNE(a+b), RNE(b-a)) against the plain pair (x~0, x~1).
//   xp : 8 pair words for the tile's 8 column pairs
template <int K, bool ROUND>
__device__ __forceinline__ void decode_dot_pair_64(const uint32_t (&w)[2 * K], uint32_t nb, const uint32_t (&xp)[8],
                                                   float (&acc)[4], const CodeRegs& cr) {
  constexpr int CW = TG_DECODE_ILP >= 8 ? 2 : 1;    // column pairs per group
  float a2[4][CW];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    a2[r][0] = acc[r];
    if constexpr (CW == 2) a2[r][1] = 0.f;
  }
#pragma unroll
  for (int c0 = 0; c0 < 8; c0 += CW) {
    uint32_t st[4][CW], u[4][CW];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[r][cc] = lane_window<K, 2 * K>(w, nb, 8 * r + c0 + cc);
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r][cc] = code_halves(st[r][cc], cr);
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (ROUND) a2[r][cc] = dot2(pair_weights_rne(u[r][cc]), xp[c0 + cc], a2[r][cc]);
        else a2[r][cc] = dot2(u[r][cc], xp[c0 + cc], a2[r][cc]);
      }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = CW == 2 ? a2[r][0] + a2[r][1] : a2[r][0];
}

// mul1 (code_id 2) against x~ / 32 in fp32 (xf: 16 fp32 bit patterns, one
// per tile column). Per weight: one window extract, v_mul_u32_u24, v_and_b32,
// v_dot4_u32_u8 (the level as an exact integer), v_cvt_f32_i32 and one
// v_fmac_f32; with K dividing 16 two windows share one v_alignbit and need no
// extract (SDWA word selects). The weights are exact, so there is no rounded
// form.
template <int K>
__device__ __forceinline__ void decode_dot_mul1_64(const uint32_t (&w)[2 * K], uint32_t nb, const uint32_t (&xf)[16],
                                                   float (&acc)[4]) {
  if constexpr (16 % K == 0) {
    constexpr int D = 16 / K;
    const MulReg mr;
#pragma unroll
    for (int n0 = 0; n0 < 32; n0 += 4) {
      uint32_t b[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t t = lane_span<K>(w, nb, span_lead<K>(n0 + i));
        b[i][0] = ((t >> 16) * mr.m) & kByteMask;
        b[i][1] = ((t & 0xFFFFu) * mr.m) & kByteMask;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tl = span_lead<K>(n0 + i) + h * D;
          acc[tl >> 4] = __builtin_fmaf((float)mul1_level(b[i][h]), __builtin_bit_cast(float, xf[tl & 15]), acc[tl >> 4]);
        }
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    uint32_t b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = mul1_bytes(lane_window<K, K>(w, nb, 16 * r + c));
    const float xc = __builtin_bit_cast(float, xf[c]);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf((float)mul1_level(b[r]), xc, acc[r]);
  }
}

// mul1 with int8 activations: decode and multiply are one v_dot4_i32_i8 of the
// four masked code bytes against the activation's int8 in all four bytes
// (xq), which adds level_byte_sum * q; the integer accumulators start from the
// bias -126 sum(q) of the 16 columns, so they end at sum(level * q) exactly.
// One fp32 multiply-add per row then applies the block factor. With K dividing
// 16 the windows go by pairs as in decode_dot_mul1_64.
template <int K>
__device__ __forceinline__ void decode_dot_mul1_i8_64(const uint32_t (&w)[2 * K], uint32_t nb, const uint32_t (&xq)[16],
                                                      int32_t bias, float factor, float (&acc)[4]) {
  int32_t ai[4] = {bias, bias, bias, bias};
  if constexpr (16 % K == 0) {
    constexpr int D = 16 / K;
    const MulReg mr;
#pragma unroll
    for (int n0 = 0; n0 < 32; n0 += 4) {
      uint32_t b[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t t = lane_span<K>(w, nb, span_lead<K>(n0 + i));
        b[i][0] = ((t >> 16) * mr.m) & kByteMask;
        b[i][1] = ((t & 0xFFFFu) * mr.m) & kByteMask;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tl = span_lead<K>(n0 + i) + h * D;
          ai[tl >> 4] = __builtin_amdgcn_sdot4((int32_t)b[i][h], (int32_t)xq[tl & 15], ai[tl >> 4], false);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(factor, (float)ai[r], acc[r]);
    return;
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    uint32_t b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = mul1_bytes(lane_window<K, K>(w, nb, 16 * r + c));
#pragma unroll
    for (int r = 0; r < 4; ++r) ai[r] = __builtin_amdgcn_sdot4((int32_t)b[r], (int32_t)xq[c], ai[r], false);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(factor, (float)ai[r], acc[r]);
}

// Sum acc[g] over the 16 tile slots of the wave (lane bits 2..5) with a
// transposing reduction: the exchanges over bits 2 and 3 each halve the number
// of values a lane carries, so 5 shuffles replace 16. On return lanes 0..15
// hold the total of tile row 4*(l&3) + 2*((l>>2)&1) + ((l>>3)&1).
__device__ __forceinline__ float reduce_slots(const float (&acc)[4], int lane) {
  const bool b0 = (lane & 4) != 0, b1 = (lane & 8) != 0;
  const float s0 = b0 ? acc[0] : acc[2], s1 = b0 ? acc[1] : acc[3];
  const float c0 = (b0 ? acc[2] : acc[0]) + shfl_xor(s0, 4);
  const float c1 = (b0 ? acc[3] : acc[1]) + shfl_xor(s1, 4);
  float d = (b1 ? c1 : c0) + shfl_xor(b1 ? c0 : c1, 8);
  d += shfl_xor(d, 16);
  d += shfl_xor(d, 32);
  return d;
}

__device__ __forceinline__ int reduced_row(int lane) {
  return 4 * (lane & 3) + 2 * ((lane >> 2) & 1) + ((lane >> 3) & 1);
}

// The NX input words of one tile column (NX = 16 fp16 pairs (x~, x~) for
// code 0, 8 column-pair words for code 1).
template <int NX>
__device__ __forceinline__ void read_xx(const uint32_t* xx_lds, int tile, uint32_t (&xv)[NX]) {
  const u32x4* xs = reinterpret_cast<const u32x4*>(xx_lds + tile * NX);
#pragma unroll
  for (int v = 0; v < NX / 4; ++v) {
    const u32x4 t = xs[v];
    xv[4 * v + 0] = t[0];
    xv[4 * v + 1] = t[1];
    xv[4 * v + 2] = t[2];
    xv[4 * v + 3] = t[3];
  }
}

}  // namespace tg
