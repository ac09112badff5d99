// Several batch-1 GEMVs that read the same input vector (a decoder layer's
// q/k/v, or gate/up), in one launch with work split evenly over the GPU.
//
// Same computation per layer as gemv.hip ("ExLlamaV3 & EXL3 Deep Dive",
// Section 2; "Trellis Quantization" lecture, Parts eight, nine and eleven).
// The work of all layers is cut into units of one 16-tile step (two 128-blocks
// of the input) of one 128-output block: layer-major, then output block, then
// step. Workgroup w takes the contiguous run of units
// [w * upw, (w + 1) * upw), so every workgroup has the same decode work
// whatever the layers' shapes, and the launch needs no more workgroups than
// the GPU has compute units (no partly filled last round, no idle units).
//
// A workgroup's run crosses output blocks (and at most one layer boundary).
// It transforms the input vector once per layer it touches (each layer has its
// own input signs) into LDS, then streams its run: the code prefetch ring runs
// over the global unit index, so it flows across block boundaries without a
// bubble. At the end of each block segment the 8 waves reduce their sums; a
// block covered by one workgroup is finished there (scale, output transform,
// signs); otherwise each contributor takes a ticket of the block when its
// segment's decode is done and publishes its partial sums in call-tagged
// slots, and the holder of the last ticket sums the partials in contributor
// order and finishes the block. Every other contributor has finished its
// decode by then and publishes without waiting, so no workgroup ever waits
// for one that has not run yet.
#include "tg_decode.hpp"
#include "tg_internal.hpp"

namespace tg {

#ifndef TG_FUSED_PF
#define TG_FUSED_PF 2
#endif

// Input transform of the run's x~ into LDS: for each layer the run touches (one or
// two, each with its own input signs and LDS area), the nn blocks fb, fb + 1, ...
// (modulo nbp) that the run's units of that layer read -- two per 16-tile step --
// of the nbp blocks (the padding block of an odd block count is zero). Both
// layers' blocks are taken in one sequence, 8 lanes per block, 64 blocks per pass
// of the workgroup's 512 threads: a run that crosses a layer boundary transforms
// both in the time of one. `raw` holds this lane's raw inputs of the first pass
// (loaded early by the caller); later passes load their own. Transforming only
// the blocks read leaves the other waves idle and the SIMDs to the ones that work
// (a short run reads 20 of 64 blocks).
// The int8 form (mul1 with int8 activations) also writes each tile column's
// bias (xbias) and each block's factor (xfac).
struct TransformPart {
  const uint32_t* sign_in;
  uint32_t* xx;
  int32_t* xbias;
  float* xfac;
  int fb, nn;
};

// Block of the idx-th of the nn needed ones: fb + idx modulo nbp (fb < nbp, nn <= nbp); a
// thread past them (idx >= nn, it writes nothing) takes block fb, so every address it forms
// stays inside the layer's area.
__device__ __forceinline__ int fused_block(int fb, int idx, int nn, int nbp) {
  const int b = fb + (idx < nn ? idx : 0);
  return b >= nbp ? b - nbp : b;
}

// The layer part and block of sequence position idx (parts p0 then p1), and the first
// input element of this lane's 16 (clamped to the last block for the padding block).
__device__ __forceinline__ void fused_slot(const TransformPart& p0, const TransformPart& p1, int idx, int nb,
                                           int nbp, bool& second, int& xb, int& first) {
  second = idx >= p0.nn;
  xb = second ? fused_block(p1.fb, idx - p0.nn, p1.nn, nbp) : fused_block(p0.fb, idx, p0.nn, nbp);
  first = (xb < nb ? xb : nb - 1) * kBlock + 16 * (threadIdx.x & 7);
}

template <int CODE, bool ROUND>
__device__ __forceinline__ void fused_transform(const uint16_t* __restrict__ x, int nb, int nbp,
                                                const TransformPart& p0, const TransformPart& p1, int total, X16 raw) {
  constexpr int XB = (CODE == 1 ? 8 : 16) * 8;   // input words per 128-block
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int xs = lane & 7;
  for (int pass = 0; pass * 64 < total; ++pass) {
    const int idx = pass * 64 + 8 * wave + (lane >> 3);
    bool second;
    int xb, first;
    fused_slot(p0, p1, idx, nb, nbp, second, xb, first);
    uint32_t* xx = second ? p1.xx : p0.xx;
    int32_t* xbias = second ? p1.xbias : p0.xbias;
    float* xfac = second ? p1.xfac : p0.xfac;
    if (pass > 0) raw = load_x16(x, second ? p1.sign_in : p0.sign_in, first);
    const bool active = idx < total, live = xb < nb;
    if constexpr (CODE == kCodeMul1I8) {
      int32_t qe[8], qo[8];
      int e;
      {
        double v[16], de[8], dof[8];
        x16_int8_phase1(raw, first, v);
        int8_exchange(xx + xb * kBlock, xs, active, live, v, de, dof);
        x16_int8_phase2(de, dof);
        int8_quantize(de, dof, qe, qo, e);
      }
      const int32_t bias = int8_group_bias(qe, qo, lane);
      __syncthreads();   // every wave has read its exchange values before the area is overwritten
      if (active) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<u32x2*>(xx + xb * XB + 16 * j + 2 * xs) = u32x2{int8_word(qe[j]), int8_word(qo[j])};
        xbias[xb * 8 + xs] = bias;
        if (xs == 0) xfac[xb] = live ? int8_factor(e) : 0.f;
      }
      __syncthreads();
      continue;
    }
    float* sc = reinterpret_cast<float*>(xx) + xb * kBlock;
    float e[8], o[8];
    {
      float v[16];
      x16_phase1<CODE == kCodeMul1>(raw, first, v);
      if (active) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          reinterpret_cast<float4_t*>(sc + 16 * xs)[i] = float4_t{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 t = active ? *reinterpret_cast<const float2*>(sc + 16 * j + 2 * xs) : float2{0.f, 0.f};
        e[j] = live ? t.x : 0.f;
        o[j] = live ? t.y : 0.f;
      }
      x16_phase2(e, o);
    }
    __syncthreads();   // every wave has read its exchange values before the area is overwritten
    if (active) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (halves_form(CODE)) {
          const uint32_t he = pack_half2(e[j], e[j]), ho = pack_half2(o[j], o[j]);
          *reinterpret_cast<u32x2*>(xx + xb * XB + 16 * j + 2 * xs) = u32x2{he, ho};
        } else if constexpr (CODE == kCodeMul1) {
          *reinterpret_cast<u32x2*>(xx + xb * XB + 16 * j + 2 * xs) =
              u32x2{__builtin_bit_cast(uint32_t, e[j]), __builtin_bit_cast(uint32_t, o[j])};
        } else if constexpr (ROUND) {
          xx[xb * XB + 8 * j + xs] = pack_half2(e[j], o[j]);
        } else {
          xx[xb * XB + 8 * j + xs] = pack_half2(e[j] - o[j], e[j] + o[j]);
        }
      }
    }
    __syncthreads();
  }
}

// Layer of unit u: unit0 increases along the table and unused entries hold
// INT32_MAX, so the layer is the number of later entries starting at or before
// u (u0 of the table's unit0 column, read beforehand).
__device__ __forceinline__ int fused_layer_of(const int (&uz)[kFusedMaxLayers], int u) {
  int l = 0;
#pragma unroll
  for (int i = 1; i < kFusedMaxLayers; ++i) l += u >= uz[i] ? 1 : 0;
  return l;
}

template <int K, int CODE, bool ROUND>
__global__ __launch_bounds__(512) void fused_kernel(FusedArgs a) {
  constexpr int NW = 2 * K;
  constexpr int NX = CODE == 1 ? 8 : 16;
  constexpr int PF = TG_FUSED_PF;
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63, wave = wave_id();   // wave = tile row within the block
  const int jslot = lane >> 2;
  // The kernel arguments the start needs, the layer table's unit0 column included, are read in
  // one batch of scalar loads (the empty asm wants them all at once): a search of the table
  // indexed by the running layer was a chain of dependent loads ahead of the first input load.
  // The batch also brings every table entry into the scalar cache for the reads below.
  int uz[kFusedMaxLayers];
#pragma unroll
  for (int i = 0; i < kFusedMaxLayers; ++i) uz[i] = a.L[i].unit0;
  const int upw = a.upw, total_units = a.total_units, n = a.n;
  const uint16_t* __restrict__ xin = a.x;
  asm volatile("" ::"s"(upw), "s"(total_units), "s"(n), "s"(xin), "s"(uz[1]), "s"(uz[2]), "s"(uz[3]), "s"(uz[4]),
               "s"(uz[5]), "s"(uz[6]), "s"(uz[7]));
  static_assert(kFusedMaxLayers == 8, "the batch above names every entry");
  const int w = blockIdx.x;
  const int u0 = w * upw;
  const int u1 = u0 + upw < total_units ? u0 + upw : total_units;
  if (u0 >= u1) return;
  const int nb = n >> 7, nbp = (nb + 1) & ~1, n16 = n >> 4, spr = nbp >> 1;
  const int lay0 = fused_layer_of(uz, u0), lay1 = fused_layer_of(uz, u1 - 1);
  const int unit0_0 = a.L[lay0].unit0, unit0_1 = a.L[lay1].unit0;
  const size_t buf_words = (size_t)nbp * kBlock;                   // one layer's x~ area (fp32 exchange size)
  uint32_t* xx0 = lds;
  uint32_t* xx1 = lds + buf_words;
  float* ybuf = reinterpret_cast<float*>(lds + 2 * buf_words);    // [128]
  uint32_t* flag = lds + 2 * buf_words + kBlock;                   // [2]
  int32_t* xbias0 = reinterpret_cast<int32_t*>(flag + 4);          // int8 form: [nbp * 8] per layer
  int32_t* xbias1 = xbias0 + nbp * 8;
  float* xfac0 = reinterpret_cast<float*>(xbias1 + nbp * 8);       // int8 form: [nbp] per layer
  float* xfac1 = xfac0 + nbp;

  // The input blocks the run reads: in lay0 from the step of its first unit on, one step per
  // unit (wrapping into the next output block), in lay1 from step 0 on.
  const int end0 = lay1 != lay0 ? unit0_1 : u1;
  const int step0 = (u0 - unit0_0) % spr;
  const int fb0 = 2 * step0, nn0 = 2 * (end0 - u0) < nbp ? 2 * (end0 - u0) : nbp;
  const int nn1 = 2 * (u1 - unit0_1) < nbp ? 2 * (u1 - unit0_1) : nbp;
  const TransformPart tp0{a.L[lay0].sign_in, xx0, xbias0, xfac0, fb0, nn0};
  const TransformPart tp1{a.L[lay1].sign_in, xx1, xbias1, xfac1, 0, nn1};
  const int ttotal = nn0 + (lay1 != lay0 ? nn1 : 0);
  // Raw inputs of the first transform pass, before the code prefetch (loads complete in order).
  X16 raw;
  {
    bool second;
    int xb, first;
    fused_slot(tp0, tp1, 8 * wave + (lane >> 3), nb, nbp, second, xb, first);
    raw = load_x16(xin, second ? tp1.sign_in : tp0.sign_in, first);
  }
  __builtin_amdgcn_sched_barrier(0);

  // Code prefetch ring over the run's units; units past the run read a dummy line. Units are
  // issued in order, so the issue position (layer il, output block iob, step ist) advances by one
  // per issue in registers: no division and no search of the layer table per unit (each was a
  // chain of scalar loads and a division sequence in front of every prefetch).
  // A run touches lay0 and at most lay1, so both layers' code pointers are read here, once; the
  // issue pointer itself moves by one step (16 tiles) per issue and is recomputed only at a block
  // boundary. Issues past the run read the dummy line whatever the position says.
  uint32_t buf[PF][NW];
  const uint32_t* __restrict__ dummy = a.L[lay0].codes;
  const uint32_t* __restrict__ codes1 = a.L[lay1].codes;
  int inext = lay1 != lay0 ? unit0_1 : INT32_MAX;   // where the run enters lay1
  int iu = u0, iob, ist;
  const uint32_t* __restrict__ icodes = a.L[lay0].codes;
  {
    const int rel = u0 - unit0_0;
    iob = rel / spr;
    ist = rel - iob * spr;
  }
  constexpr size_t kStepWords = (size_t)16 * 8 * K;         // code words of one 16-tile step of a tile row
  const uint32_t* __restrict__ ibase = icodes + ((size_t)(iob * 8 + wave) * n16 + (size_t)ist * 16) * (8 * K);
  const uint32_t lane_bytes = (uint32_t)lane * NW * 4u;
  auto issue = [&](uint32_t(&dst)[NW]) {
    // past the run: the dummy line (a uniform choice); a lane past the last tile of a ragged step
    // reads the step's first tile (its x~ is the zero padding block)
    const char* base = reinterpret_cast<const char*>(iu < u1 ? ibase : dummy);
    const uint32_t off = ist * 16 + jslot < n16 ? lane_bytes : 0u;
    load_lane_words<K>(reinterpret_cast<const uint32_t*>(base + off), dst);
    ++iu;
    ibase += kStepWords;
    if (++ist == spr) {   // next output block, or the first of lay1
      ist = 0;
      ++iob;
      if (iu == inext) {
        iob = 0;
        icodes = codes1;
        inext = INT32_MAX;
      }
      ibase = icodes + (size_t)(iob * 8 + wave) * n16 * (8 * K);
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(buf[p]);

  fused_transform<CODE, ROUND>(xin, nb, nbp, tp0, tp1, ttotal, raw);

  const CodeRegs cr;
  // The current block segment: layer l, output block ob, units [seg_u0, seg_end).
  int l = lay0, ob = 0, seg_u0 = u0, seg_end = u0, count = 1;
  const uint32_t* xx = xx0;
  const int32_t* xbias = xbias0;
  const float* xfac = xfac0;
  auto start_segment = [&](int u) {
    l = u >= unit0_1 ? lay1 : lay0;   // the run enters lay1 at its first unit
    const int lu0 = l == lay0 ? unit0_0 : unit0_1;
    ob = (u - lu0) / spr;
    seg_u0 = lu0 + ob * spr;
    const int e = seg_u0 + spr;
    seg_end = e < u1 ? e : u1;
    xx = l == lay0 ? xx0 : xx1;
    xbias = l == lay0 ? xbias0 : xbias1;
    xfac = l == lay0 ? xfac0 : xfac1;
    count = (seg_u0 + spr - 1) / upw - seg_u0 / upw + 1;       // workgroups contributing to the block
  };
  start_segment(u0);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  // Segment epilogue (uniform): reduce the waves' sums of the block, then finish the block here
  // (one contributor) or publish this workgroup's partial sums and hand over by ticket.
  auto finish_segment = [&]() {
    const FusedLayer& Ld = a.L[l];
    const float d = reduce_slots(acc, lane);
    const int orow = wave * 16 + reduced_row(lane);
    const int first_wg = seg_u0 / upw;
    __syncthreads();                                                   // ybuf is free (previous segment done)
    if (lane < 16) ybuf[orow] = d;
    if (count == 1) {
      __syncthreads();
      if (wave == 0) rht_out_block(ybuf[lane], ybuf[lane + 64], Ld.scales, Ld.sign_out, Ld.y, ob * kBlock, lane);
      return;
    }
    const int me = w - first_wg;
    const int bglob = Ld.block0 + ob;
    uint32_t* counter = a.counters + bglob;
    uint64_t* slots = a.slots + (size_t)bglob * a.max_contrib * kBlock;
    // The ticket is taken once this segment's decode is done (one round trip; its high bits give
    // the call number of the slot tag), so the holder of the block's last ticket finds every
    // other contributor done with its decode: they publish at once and never wait on it.
    if (threadIdx.x == 0) {
      const uint32_t ticket = take_ticket(counter);
      flag[0] = (ticket & (kTicketCall - 1u)) == (uint32_t)count - 1u ? 1u : 0u;
      flag[1] = slot_tag(ticket, (uint32_t)count);                     // the call number and the count
    }
    __syncthreads();
    const uint32_t tag = flag[1];
    if (lane < 16) put_slot(slots + (size_t)me * kBlock + orow, d, tag);
    if (flag[0] == 0u || wave != 0) return;
    // The last contributor: every other one has published. Up to J contributors' slots are read
    // together (one memory round trip, not one per contributor), the ones not yet holding this
    // call's partial re-read together until all do (bounded), and the partials summed in
    // contributor order.
    constexpr int J = 4;
    float v0 = 0.f, v1 = 0.f;
    bool late = false;
    for (int i0 = 0; i0 < count; i0 += J) {
      uint64_t s0[J], s1[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int i = i0 + j;
        s0[j] = s1[j] = (uint64_t)tag << 32;   // contributors past the count, and this one, count as ready
        if (i < count && i != me) {
          s0[j] = peek_slot(slots + (size_t)i * kBlock + lane);
          s1[j] = peek_slot(slots + (size_t)i * kBlock + lane + 64);
        }
      }
      bool empty = true;
      for (uint32_t it = 0; it < kSlotPolls; ++it) {
        empty = false;
#pragma unroll
        for (int j = 0; j < J; ++j) empty |= !slot_ready(s0[j], tag) || !slot_ready(s1[j], tag);
        if (!empty) break;
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int i = i0 + j;
          if (!slot_ready(s0[j], tag)) s0[j] = peek_slot(slots + (size_t)i * kBlock + lane);
          if (!slot_ready(s1[j], tag)) s1[j] = peek_slot(slots + (size_t)i * kBlock + lane + 64);
        }
      }
      late |= empty;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int i = i0 + j;
        if (i >= count) break;
        v0 += i == me ? ybuf[lane] : slot_value(s0[j], tag);
        v1 += i == me ? ybuf[lane + 64] : slot_value(s1[j], tag);
      }
    }
    if (late) report_status(a.status, kStatusSplitkTimeout);
    rht_out_block(v0, v1, Ld.scales, Ld.sign_out, Ld.y, ob * kBlock, lane);
    if (lane == 0) finish_call(counter, (uint32_t)count);
  };

  // Main loop in groups of PF units with the ring slot fixed per position, so every load is issued
  // unconditionally in program order and the compiler's waits for the ring stay exact.
  for (int ub = u0; ub < u1; ub += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int u = ub + p;
      const bool live = u < u1;
      if (live) {
        uint32_t xv[NX];
        const int tile = (u - seg_u0) * 16 + jslot;
        read_xx(xx, tile, xv);
        const uint32_t nbw = quad_rotate_next(buf[p][0]);
        if constexpr (CODE == 0) decode_dot_64<K, ROUND>(buf[p], nbw, xv, acc, cr);
        else if constexpr (CODE == kCodeMcg) decode_dot_mcg_64<K, ROUND>(buf[p], nbw, xv, acc, cr);
        else if constexpr (CODE == 1) decode_dot_pair_64<K, ROUND>(buf[p], nbw, xv, acc, cr);
        else if constexpr (CODE == kCodeMul1) decode_dot_mul1_64<K>(buf[p], nbw, xv, acc);
        else decode_dot_mul1_i8_64<K>(buf[p], nbw, xv, xbias[tile], xfac[tile >> 3], acc);
      }
      issue(buf[p]);     // refill after use with unit u + PF; past the run: the dummy line
      if (live && u + 1 == seg_end) {
        finish_segment();
        if (u + 1 < u1) {
          start_segment(u + 1);
          acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
        }
      }
    }
  }
}

size_t fused_lds_bytes(int n, bool int8) {
  const int nbp = ((n >> 7) + 1) & ~1;
  return (size_t)2 * nbp * kBlock * 4 + kBlock * 4 + 16 + (int8 ? (size_t)2 * nbp * 9 * 4 : 0);
}

template <int K, int CODE, bool ROUND>
static hipError_t launch_fused_t(const FusedArgs& a, int grid, hipStream_t s) {
  const size_t lds = fused_lds_bytes(a.n, CODE == kCodeMul1I8);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_kernel<K, CODE, ROUND>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((fused_kernel<K, CODE, ROUND>), dim3(grid), dim3(512), lds, s, a);
  return hipGetLastError();
}

template <int CODE, bool ROUND>
static hipError_t launch_fused_k(const FusedArgs& a, int k_bits, int grid, hipStream_t s) {
  switch (k_bits) {
    case 1: return launch_fused_t<1, CODE, ROUND>(a, grid, s);
    case 2: return launch_fused_t<2, CODE, ROUND>(a, grid, s);
    case 3: return launch_fused_t<3, CODE, ROUND>(a, grid, s);
    case 4: return launch_fused_t<4, CODE, ROUND>(a, grid, s);
    case 5: return launch_fused_t<5, CODE, ROUND>(a, grid, s);
    case 6: return launch_fused_t<6, CODE, ROUND>(a, grid, s);
    case 7: return launch_fused_t<7, CODE, ROUND>(a, grid, s);
    case 8: return launch_fused_t<8, CODE, ROUND>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fused(const FusedArgs& a, int k_bits, int variant, bool round_weights, int grid, hipStream_t s) {
  switch (variant) {
    case 0:
      return round_weights ? launch_fused_k<0, true>(a, k_bits, grid, s) : launch_fused_k<0, false>(a, k_bits, grid, s);
    case 1:
      return round_weights ? launch_fused_k<1, true>(a, k_bits, grid, s) : launch_fused_k<1, false>(a, k_bits, grid, s);
    case kCodeMcg:
      return round_weights ? launch_fused_k<kCodeMcg, true>(a, k_bits, grid, s)
                           : launch_fused_k<kCodeMcg, false>(a, k_bits, grid, s);
    case kCodeMul1: return launch_fused_k<kCodeMul1, false>(a, k_bits, grid, s);
    case kCodeMul1I8: return launch_fused_k<kCodeMul1I8, false>(a, k_bits, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tg
