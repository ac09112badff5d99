// Device-side building blocks shared by the trellis-coded GEMV kernels (gfx950).
//
// Window extraction follows the bitshift trellis of the "Trellis Quantization"
// lecture, Part eight (weight t's 16-bit state starts at stream bit K*t, the
// stream of a 16x16 tile is a circle) and the code follows its Part nine
// (three-instruction code). Storage conventions are those of trellis_gemv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_internal.hpp"

namespace tg {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Code constants (shared by code_id 0, the pair code (code_id 1) and MCG (code_id 3);
// mul1 uses the multiplier).
constexpr uint32_t kMul = 0x009E3779u;   // 24-bit LCG multiplier: one full-rate v_mad_u32_u24
constexpr uint32_t kAdd = 0x7F4A7C15u;
constexpr uint32_t kMask = 0x8FFF8FFFu;  // sign, 2 low exponent bits, 10 fraction bits per half
constexpr uint32_t kXor = 0x30003000u;   // exponent field 0b011xx: |half| in [1/8, 2)

constexpr float kRsqrt128 = 0.088388347648318440550f;  // 1/sqrt(128), correctly rounded

// The mask/XOR constants are laundered through empty asm so the compiler keeps
// them in registers and emits the bit insert as one v_and_or_b32 (the constant
// bus allows one SGPR operand, the other constant lives in a VGPR). Since the
// XOR constant only touches masked-off bits, AND-then-OR equals AND-then-XOR.
struct CodeRegs {
  uint32_t mask, xr;
  __device__ __forceinline__ CodeRegs() : mask(kMask), xr(kXor) {
    asm volatile("" : "+s"(mask));
    asm volatile("" : "+v"(xr));
  }
};

// 16-bit state -> 32-bit word holding the two fp16 halves of the weight.
__device__ __forceinline__ uint32_t code_halves(uint32_t state, const CodeRegs& c) {
  const uint32_t h = state * kMul + kAdd;  // state < 2^16: v_mad_u32_u24
  return (h & c.mask) | c.xr;
}

// The multiplier in an SGPR, known to fit 24 bits: a multiply-only code's v_mul_u32_u24 can then
// take its state through an SDWA word select (SDWA operands take no literal).
struct MulReg {
  uint32_t m;
  __device__ __forceinline__ MulReg() : m(kMul) {
    asm volatile("" : "+s"(m));
    m &= 0xFFFFFFu;
  }
};

// MCG (code_id 3; "Trellis Quantization" lecture, Part eleven): the same
// halves from the generator with its additive constant dropped (multiply only).
__device__ __forceinline__ uint32_t mcg_halves(uint32_t state, const CodeRegs& c) {
  return ((state * kMul) & c.mask) | c.xr;   // v_mul_u32_u24, v_and_or_b32
}

// The halves word of a state for either code in halves_form.
template <int CODE>
__device__ __forceinline__ uint32_t halves_of(uint32_t state, const CodeRegs& c) {
  if constexpr (CODE == kCodeMcg) return mcg_halves(state, c);
  else return code_halves(state, c);
}

// fp16 weight = round-to-nearest-even(lo + hi), as a 16-bit pattern.
__device__ __forceinline__ _Float16 halves_sum_rne(uint32_t u) {
  const half2_t p = __builtin_bit_cast(half2_t, u);
  return p[0] + p[1];
}

// The same weight as the word (w, 0): one v_add_f16 whose SDWA selects take the two halves
// and whose unused destination bits are written as zeros (the compiler adds a v_pack for the
// zero half otherwise). The VALU dot products of the rounded forms take it against (x~, x~).
// Not for matrix-core operands: the compiler's wait states between a VALU write and an MFMA
// read do not see inside inline asm, so the MFMA path keeps halves_sum_rne.
__device__ __forceinline__ uint32_t halves_sum_word(uint32_t u) {
  uint32_t w;
  asm("v_add_f16_sdwa %0, %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:WORD_1"
      : "=v"(w)
      : "v"(u));
  return w;
}

__device__ __forceinline__ uint32_t ubfe(uint32_t v, uint32_t off, uint32_t width) {
  return __builtin_amdgcn_ubfe(v, off, width);
}

// 32 bits of the stream starting "shift" bits before the end of hi:  ({hi, lo} >> shift)[31:0].
__device__ __forceinline__ uint32_t alignbit(uint32_t hi, uint32_t lo, uint32_t shift) {
  return __builtin_amdgcn_alignbit(hi, lo, shift);
}

// fp32 accumulate of (a.lo*b.lo + a.hi*b.hi).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), acc, false);
}

// Value of lane (lane+1) mod 4 within each quad (DPP quad_perm [1,2,3,0]).
__device__ __forceinline__ uint32_t quad_rotate_next(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, 0x39, 0xF, 0xF, false);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value:
// the compiler cannot tell on its own that threadIdx.x / 64 is the same for all
// lanes, and would otherwise keep everything derived from it (step counts, row
// pointers, loop tests) in vector registers with exec-mask branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ uint32_t sign_bit(const uint32_t* __restrict__ words, int i) {
  return (words[i >> 5] >> (i & 31)) & 1u;
}

// Unnormalised 128-point Sylvester-order Walsh-Hadamard transform held by one
// wave: lane l owns elements l (v0) and l+64 (v1). Seven butterfly stages
// (a, b) -> (a+b, a-b); the stride-64 stage is in-lane, the others pair lanes
// l and l^h.
__device__ __forceinline__ void fwht128_wave(float& v0, float& v1, int lane) {
  const float a = v0 + v1, b = v0 - v1;
  v0 = a;
  v1 = b;
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const float p0 = shfl_xor(v0, h), p1 = shfl_xor(v1, h);
    const bool upper = (lane & h) != 0;
    v0 = upper ? (p0 - v0) : (v0 + p0);
    v1 = upper ? (p1 - v1) : (v1 + p1);
  }
}

// Raw inputs of one 128-block for the input-side transform: the fp16 patterns
// of elements lane and lane+64 and the sign words that hold their bits. No
// arithmetic happens at load time, so the loads can be issued early.
struct XBlock {
  uint16_t b0, b1;
  uint32_t s0, s1;
  int base;
};

__device__ __forceinline__ XBlock load_x_block(const uint16_t* __restrict__ x, const uint32_t* __restrict__ sign_in,
                                               int base, int lane) {
  XBlock r;
  r.b0 = x[base + lane];
  r.b1 = x[base + lane + 64];
  r.s0 = sign_in[(base + lane) >> 5];
  r.s1 = sign_in[(base + lane + 64) >> 5];
  r.base = base;
  return r;
}

// Input-side transform of one 128-block held by a wave: x~ = H diag(s) x / sqrt(128),
// returned as fp16 in both halves of a 32-bit word (the fused dot consumes pairs (x~, x~)).
__device__ __forceinline__ void rht_in_block_dup(XBlock xb, int lane, uint32_t& d0, uint32_t& d1) {
  const uint16_t b0 = xb.b0 ^ (uint16_t)(((xb.s0 >> ((xb.base + lane) & 31)) & 1u) << 15);
  const uint16_t b1 = xb.b1 ^ (uint16_t)(((xb.s1 >> ((xb.base + lane + 64) & 31)) & 1u) << 15);
  float v0 = half_bits_to_float(b0), v1 = half_bits_to_float(b1);
  fwht128_wave(v0, v1, lane);
  const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)(v0 * kRsqrt128));
  const uint16_t h1 = __builtin_bit_cast(uint16_t, (_Float16)(v1 * kRsqrt128));
  d0 = (uint32_t)h0 | ((uint32_t)h0 << 16);
  d1 = (uint32_t)h1 | ((uint32_t)h1 << 16);
}

__device__ __forceinline__ void rht_in_block_dup(const uint16_t* __restrict__ x, const uint32_t* __restrict__ sign_in,
                                                 int base, int lane, uint32_t& d0, uint32_t& d1) {
  rht_in_block_dup(load_x_block(x, sign_in, base, lane), lane, d0, d1);
}

// Pair code (code_id 1): a state carries the weights of input columns 2j and
// 2j+1, and w0 x0 + w1 x1 = a (x0 - x1) + b (x0 + x1) for the halves a, b of
// the state's code word (w0 = a + b, w1 = b - a). The input side is therefore
// kept as one fp16 pair per column pair. Lane 2i returns pair i (elements 2i,
// 2i+1 of the block), lane 2i+1 returns pair 32+i (elements 64+2i, 64+2i+1).
__device__ __forceinline__ int pair_index(int lane) { return (lane & 1) ? 32 + (lane >> 1) : (lane >> 1); }

// rotate: (x~0 - x~1, x~0 + x~1); otherwise the plain pair (x~0, x~1). Low half first.
__device__ __forceinline__ uint32_t rht_in_block_pair(XBlock xb, int lane, bool rotate) {
  const uint16_t b0 = xb.b0 ^ (uint16_t)(((xb.s0 >> ((xb.base + lane) & 31)) & 1u) << 15);
  const uint16_t b1 = xb.b1 ^ (uint16_t)(((xb.s1 >> ((xb.base + lane + 64) & 31)) & 1u) << 15);
  float v0 = half_bits_to_float(b0), v1 = half_bits_to_float(b1);
  fwht128_wave(v0, v1, lane);
  v0 *= kRsqrt128;
  v1 *= kRsqrt128;
  const float p0 = shfl_xor(v0, 1), p1 = shfl_xor(v1, 1);
  const bool odd = (lane & 1) != 0;
  const float e = odd ? p1 : v0;   // even element of the pair
  const float o = odd ? v1 : p0;   // odd element
  const float lo = rotate ? e - o : e;
  const float hi = rotate ? e + o : o;
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// Pair code weights rounded to fp16: (RNE(a + b), RNE(b - a)) from the code word's halves.
__device__ __forceinline__ uint32_t pair_weights_rne(uint32_t u) {
  const half2_t p = __builtin_bit_cast(half2_t, u);
  const _Float16 w0 = p[0] + p[1], w1 = p[1] - p[0];
  return (uint32_t)__builtin_bit_cast(uint16_t, w0) | ((uint32_t)__builtin_bit_cast(uint16_t, w1) << 16);
}

// ---------------------------------------------------------------------------
// mul1 (code_id 2; "Trellis Quantization" lecture, Parts eleven and twelve):
// the state times the multiplier with no additive term, each product byte
// masked to six bits, the four bytes summed and 126 subtracted; the weight is
// that level / 32, exact in binary16.
constexpr uint32_t kByteMask = 0x3F3F3F3Fu;
constexpr uint32_t kByteOnes = 0x01010101u;
constexpr int kMul1Offset = 126;
constexpr float kMul1Step = 0.03125f;   // 1/32

// Masked product bytes of a 16-bit state: v_mul_u32_u24 and v_and_b32.
__device__ __forceinline__ uint32_t mul1_bytes(uint32_t state) { return (state * kMul) & kByteMask; }

// Level = byte sum - 126 as an int32: one v_dot4_u32_u8 whose accumulator is
// -126 (the unsigned sum wraps modulo 2^32 to the signed level).
__device__ __forceinline__ int32_t mul1_level(uint32_t bytes) {
  return (int32_t)__builtin_amdgcn_udot4(bytes, kByteOnes, (uint32_t)-kMul1Offset, false);
}

// The weight as binary16 without a conversion: fp16 48.0 is 0x5200, and the
// binade [32, 64) steps by exactly 1/32, so 0x5200 + level (|level| <= 126 keeps
// the exponent) is the pattern of 48 + level/32. One v_dot4_u32_u8 with
// accumulator 0x5200 - 126 forms it; subtracting 48 in binary16 is exact.
constexpr uint32_t kMul1Magic = 0x5200u;   // binary16 48.0

__device__ __forceinline__ uint32_t mul1_biased_half(uint32_t state) {
  return __builtin_amdgcn_udot4(mul1_bytes(state), kByteOnes, kMul1Magic - (uint32_t)kMul1Offset, false);
}

__device__ __forceinline__ uint16_t mul1_weight_bits(uint32_t state) {
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)mul1_biased_half(state));
  return __builtin_bit_cast(uint16_t, (_Float16)(h - (_Float16)48.0f));
}

// The same from the masked product bytes (state * multiplier & 0x3F3F3F3F), as the word (w, 0).
__device__ __forceinline__ uint32_t mul1_weight_word(uint32_t bytes) {
  const uint32_t biased = __builtin_amdgcn_udot4(bytes, kByteOnes, kMul1Magic - (uint32_t)kMul1Offset, false);
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)biased);
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(h - (_Float16)48.0f));
}

// Two weights as one packed word (a in the low half): one packed binary16 subtract.
__device__ __forceinline__ uint32_t mul1_weight_pair(uint32_t sa, uint32_t sb) {
  const uint32_t biased = mul1_biased_half(sa) | (mul1_biased_half(sb) << 16);
  const half2_t w = __builtin_bit_cast(half2_t, biased) - half2_t{(_Float16)48.0f, (_Float16)48.0f};
  return __builtin_bit_cast(uint32_t, w);
}

// ---------------------------------------------------------------------------
// Input-side transform of many 128-blocks at once, 8 lanes per block.
//
// Lane s (= lane % 8 of its block) first holds elements 16s..16s+15 (one
// 32-byte load), applies their signs and the 1/sqrt(128) scale, and runs the
// four butterfly stages over index bits 0..3 in registers (x16_phase1). One
// exchange through LDS then gives it elements 16j + 2s and 16j + 2s + 1 for
// j = 0..7, and the stages over index bits 4..6 finish in registers
// (x16_phase2): the lane ends with x~ of column pairs q = 8j + s. The
// Sylvester matrix is the tensor product of its 2x2 factors, so the stages
// may run in any order. No cross-lane shuffles are needed.
// ---------------------------------------------------------------------------
struct X16 {
  u32x4 lo, hi;   // fp16 patterns of elements first .. first+15
  uint32_t sw;    // the sign word holding their 16 sign bits
};

// `first` is the element index of the lane's 16 elements (a multiple of 16).
__device__ __forceinline__ X16 load_x16(const uint16_t* __restrict__ x, const uint32_t* __restrict__ sign_in,
                                        int first) {
  X16 r;
  const u32x4* p = reinterpret_cast<const u32x4*>(x + first);
  r.lo = p[0];
  r.hi = p[1];
  r.sw = sign_in[first >> 5];
  return r;
}

// Gated-MLP input of one lane: 16 fp32 gate and up values and the sign word.
// The vector loads are copied out component by component (.x .. .w): this
// compiler turned a bit_cast of a subscripted vector element into a read of
// component 0.
struct XGated16 {
  float g[16], u[16];
  uint32_t sw;
};

__device__ __forceinline__ XGated16 load_gated16(const float* __restrict__ hg, const float* __restrict__ hu,
                                                 const uint32_t* __restrict__ sign_in, int first) {
  XGated16 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4_t vg = reinterpret_cast<const float4_t*>(hg + first)[i];
    const float4_t vu = reinterpret_cast<const float4_t*>(hu + first)[i];
    r.g[4 * i] = vg.x, r.g[4 * i + 1] = vg.y, r.g[4 * i + 2] = vg.z, r.g[4 * i + 3] = vg.w;
    r.u[4 * i] = vu.x, r.u[4 * i + 1] = vu.y, r.u[4 * i + 2] = vu.z, r.u[4 * i + 3] = vu.w;
  }
  r.sw = sign_in[first >> 5];
  return r;
}

// x = fp16(silu(g) * u), silu(v) = v / (1 + exp(-v)), packed as the fp16 input
// words. exp(-v) = 2^(-v log2 e) and the reciprocal use the hardware's
// v_exp_f32 and v_rcp_f32 (relative error ~2^-22, far below the 2^-11 of the
// fp16 rounding that follows); exp overflows to +inf for v < -88, and
// v * rcp(inf) = -0 as silu's limit demands.
__device__ __forceinline__ float silu_fast(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

__device__ __forceinline__ X16 gated_to_x16(const XGated16& r) {
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const float h0 = silu_fast(r.g[j]) * r.u[j];
    const float h1 = silu_fast(r.g[j + 1]) * r.u[j + 1];
    w[j >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)h0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)h1) << 16);
  }
  X16 x;
  x.lo = u32x4{w[0], w[1], w[2], w[3]};
  x.hi = u32x4{w[4], w[5], w[6], w[7]};
  x.sw = r.sw;
  return x;
}

// v[j] = s[first+j] * x[first+j] * c, then the 16-point transform over j.
// c = 1/sqrt(128), or (mul1) 1/(32 sqrt(128)), which carries the weight step:
// a power-of-two multiple of the same constant, so the sums scale exactly.
template <bool MUL1 = false>
__device__ __forceinline__ void x16_phase1(const X16& r, int first, float (&v)[16]) {
  const uint32_t sb = r.sw >> (first & 16);   // bit j: sign of element first + j
  const uint32_t w[8] = {r.lo[0], r.lo[1], r.lo[2], r.lo[3], r.hi[0], r.hi[1], r.hi[2], r.hi[3]};
  const uint32_t cbits = __builtin_bit_cast(uint32_t, MUL1 ? kRsqrt128 * kMul1Step : kRsqrt128);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint16_t h = (uint16_t)((j & 1) ? (w[j >> 1] >> 16) : w[j >> 1]);
    const float cs = __builtin_bit_cast(float, cbits | ((sb << (31 - j)) & 0x80000000u));
    v[j] = half_bits_to_float(h) * cs;
  }
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((j & h) == 0) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

// The 8-point transform over j for the even (e) and odd (o) elements 16j + 2s (+1).
__device__ __forceinline__ void x16_phase2(float (&e)[8], float (&o)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & h) == 0) {
        const float a = e[j], b = e[j + h];
        e[j] = a + b;
        e[j + h] = a - b;
        const float c = o[j], d = o[j + h];
        o[j] = c + d;
        o[j + h] = c - d;
      }
}

// int8 form of x~ for mul1 with int8 activations ("Trellis Quantization"
// lecture, Part eleven), in float64:
//   u = (+-1 Hadamard) diag(s_in) x -- every partial sum of binary16 values is
//       a multiple of 2^-24 below 2^23, so each butterfly is exact and u does
//       not depend on their order;
//   e = the smallest integer with max|u| 2^-e <= 127 over the block (0 if the
//       block is zero);
//   q = round-half-even(u 2^-e), an exact power-of-two scaling.
// The layout follows the fp32 transform: x16_int8_phase1 takes the lane's 16
// elements 16s..16s+15 through the butterflies over index bits 0..3; one
// exchange through LDS (two rounds of 32-bit halves) gives the lane elements
// 16j + 2s and 16j + 2s + 1 (e[j], o[j]); x16_int8_phase2 runs the bits 4..6.
__device__ __forceinline__ void x16_int8_phase1(const X16& r, int first, double (&v)[16]) {
  const uint32_t sb = r.sw >> (first & 16);
  const uint32_t w[8] = {r.lo[0], r.lo[1], r.lo[2], r.lo[3], r.hi[0], r.hi[1], r.hi[2], r.hi[3]};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint16_t h = (uint16_t)((j & 1) ? (w[j >> 1] >> 16) : w[j >> 1]);
    const double x = (double)half_bits_to_float(h);
    v[j] = ((sb >> j) & 1u) ? -x : x;
  }
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((j & h) == 0) {
        const double a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

__device__ __forceinline__ void x16_int8_phase2(double (&e)[8], double (&o)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & h) == 0) {
        const double a = e[j], b = e[j + h];
        e[j] = a + b;
        e[j + h] = a - b;
        const double c = o[j], d = o[j + h];
        o[j] = c + d;
        o[j + h] = c - d;
      }
}

// Exchange of the 16 float64 values of each lane of a block's 8 lanes through
// the block's 128-word LDS area `sc` (write: the lane's 16 values; read: the
// values of elements 16j + 2s, 16j + 2s + 1), one 32-bit half at a time. Only
// lanes of one wave share a block's area, so wave barriers order it; the area
// is free again once the caller's next workgroup barrier has passed.
__device__ __forceinline__ void int8_exchange(uint32_t* sc, int xs, bool active, bool live, const double (&v)[16],
                                              double (&e)[8], double (&o)[8]) {
  uint32_t el[8], ol[8];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 t;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint64_t b = __builtin_bit_cast(uint64_t, v[4 * i + c]);
          t[c] = (uint32_t)(half ? (b >> 32) : b);
        }
        reinterpret_cast<u32x4*>(sc + 16 * xs)[i] = t;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x2 t = active ? *reinterpret_cast<const u32x2*>(sc + 16 * j + 2 * xs) : u32x2{0u, 0u};
      if (half == 0) {
        el[j] = t[0];
        ol[j] = t[1];
      } else {
        e[j] = live ? __builtin_bit_cast(double, ((uint64_t)t[0] << 32) | el[j]) : 0.0;
        o[j] = live ? __builtin_bit_cast(double, ((uint64_t)t[1] << 32) | ol[j]) : 0.0;
      }
    }
    __builtin_amdgcn_wave_barrier();   // every lane has read this half before the next one is written
  }
}

// Block exponent and int8 values of the lane's 16 transformed elements (the
// maximum is taken over the block's 8 lanes).
__device__ __forceinline__ void int8_quantize(const double (&e)[8], const double (&o)[8], int32_t (&qe)[8],
                                              int32_t (&qo)[8], int& ex) {
  double amax = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = __builtin_fmax(amax, __builtin_fmax(__builtin_fabs(e[j]), __builtin_fabs(o[j])));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) amax = __builtin_fmax(amax, __shfl_xor(amax, h, 64));
  ex = 0;
  if (amax > 0.0) {
    int E;
    const double f = __builtin_frexp(amax, &E);   // amax = f 2^E, f in [1/2, 1)
    ex = f * 128.0 <= 127.0 ? E - 7 : E - 6;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    qe[j] = (int32_t)__builtin_rint(__builtin_ldexp(e[j], -ex));
    qo[j] = (int32_t)__builtin_rint(__builtin_ldexp(o[j], -ex));
  }
}

// -126 times the sum of q over tile column group s (elements 16s..16s+15) of
// the block, for lane s of the block's 8 lanes: each lane holds two elements
// of every group; a transposing reduction over the lane bits 2, 1, 0 leaves
// lane s with group s (7 shuffles).
__device__ __forceinline__ int32_t int8_group_bias(const int32_t (&qe)[8], const int32_t (&qo)[8], int lane) {
  int32_t a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = qe[j] + qo[j];
#pragma unroll
  for (int h = 4, n = 4; h >= 1; h >>= 1, n >>= 1) {
    const bool upper = (lane & h) != 0;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int32_t send = upper ? a[i] : a[i + n];
      const int32_t keep = upper ? a[i + n] : a[i];
      a[i] = keep + __shfl_xor(send, h, 64);
    }
  }
  return -kMul1Offset * a[0];
}

// An int8 value repeated in all four bytes of a word (for v_dot4_i32_i8
// against the four masked code bytes of one weight), and the block's fp32
// factor 2^e / (32 sqrt(128)) that turns the integer dot product into y~.
__device__ __forceinline__ uint32_t int8_word(int32_t q) { return ((uint32_t)q & 0xFFu) * kByteOnes; }

__device__ __forceinline__ float int8_factor(int e) { return __builtin_ldexpf(kRsqrt128 * kMul1Step, e); }

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// Output-side epilogue of one 128-block held by a wave:
// y = diag(s_out) H (g * y~) / sqrt(128), written as fp32.
__device__ __forceinline__ void rht_out_block(float v0, float v1, const uint16_t* __restrict__ scales,
                                              const uint32_t* __restrict__ sign_out, float* __restrict__ y,
                                              int base, int lane) {
  v0 *= half_bits_to_float(scales[base + lane]);
  v1 *= half_bits_to_float(scales[base + lane + 64]);
  fwht128_wave(v0, v1, lane);
  v0 *= kRsqrt128;
  v1 *= kRsqrt128;
  if (sign_bit(sign_out, base + lane)) v0 = -v0;
  if (sign_bit(sign_out, base + lane + 64)) v1 = -v1;
  y[base + lane] = v0;
  y[base + lane + 64] = v1;
}

// ---------------------------------------------------------------------------
// Split-K handoff between workgroups without cache writebacks.
//
// Partial sums are written and read with device-scope relaxed atomic stores /
// loads, which this target performs coherently at device scope (write-through
// stores and L2-coherent loads), so no L2 writeback or invalidate is needed.
// Each workgroup waits for its own partial stores to complete before it
// increments the arrival counter; the workgroup that sees the count reach
// `total - 1` reads all partials (issued after it observed the counter) and
// resets the counter to zero for the next call. No workgroup ever waits for
// another one.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in every thread of the last-arriving workgroup. `flag` is a word of LDS.
__device__ __forceinline__ bool arrive_is_last(uint32_t* counter, uint32_t total, uint32_t* flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = (__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1u) ? 1u : 0u;
  __syncthreads();
  return *flag != 0u;
}

__device__ __forceinline__ void reset_counter(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-K by ticket and slots (batch-1 and grouped paths). Every workgroup of
// an output block takes a ticket once its input has arrived; the holder of the
// last ticket of the call reduces. The others have all started by then and
// finish without waiting on anything, so the reducer's wait for their
// partials ends. The ticket counter advances by kTicketCall per call (the
// reducer tops it up), so a ticket's low 16 bits rank the workgroups of the
// call and its high 16 bits number the call. A slot is one 64-bit word per
// partial: the fp32 bits, and above them a tag, the call number and the split
// count (slot_tag). Slot (counter c, split s, lane i) sits at (c*S + s)*128 + i
// for S splits, so the same address under another split count belongs to
// another block and counter, and is never taken for this call's: its tag has
// another split count. Under the same split count the address belongs to this
// counter, whose earlier calls carry earlier call numbers (equal only after
// 2^16 calls of other split counts on the block in between). Every workgroup
// of the block, the reducer included, writes its slots in every call, so
// nothing is cleared, and one atomic store publishes value and tag together:
// a writer never waits for its store to land. A zeroed workspace starts at
// call 0 with no slot tagged (a tag's split count is at least 2).
constexpr uint32_t kSlotPolls = 1u << 20;     // bound of one wait: re-reads, about a second in all
constexpr uint32_t kTicketCall = 1u << 16;    // tickets per call (splits < 2^16)

__device__ __forceinline__ uint32_t take_ticket(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The reducer, holder of the call's last ticket: move the counter to the next call.
__device__ __forceinline__ void finish_call(uint32_t* counter, uint32_t splits) {
  __hip_atomic_fetch_add(counter, kTicketCall - splits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t slot_tag(uint32_t ticket, uint32_t splits) {
  return (ticket & ~(kTicketCall - 1u)) | splits;
}

__device__ __forceinline__ void put_slot(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, (uint64_t)__builtin_bit_cast(uint32_t, v) | ((uint64_t)tag << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t peek_slot(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool slot_ready(uint64_t s, uint32_t tag) { return (uint32_t)(s >> 32) == tag; }

// Set sticky error bits in a workspace's status word (device scope, any lane may call).
__device__ __forceinline__ void report_status(uint32_t* status, uint32_t bits) {
  __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Value of a slot read; NaN if it does not hold this call's partial (a wait that ran out).
__device__ __forceinline__ float slot_value(uint64_t s, uint32_t tag) {
  return slot_ready(s, tag) ? __builtin_bit_cast(float, (uint32_t)s) : __builtin_nanf("");
}

}  // namespace tg
