// Batch-1 trellis-coded GEMV for gfx950 (VALU decode + v_dot2 accumulate).
//
// Computes y = diag(s_out) H (g * (W^ (H diag(s_in) x))) for one activation
// vector ("ExLlamaV3 & EXL3 Deep Dive", Section 2; "Trellis Quantization"
// lecture, Parts eight, nine and eleven).
//
// Work decomposition. A workgroup of 8 waves owns one 128-output block (8
// tile rows, one wave per tile row) and one contiguous chunk of 128-blocks of
// the input ("split"). In one step a wave covers 16 tiles of its tile row:
// lane l takes tile slot l/4 and rows 4*(l%4)..+3 of that tile, i.e. 64
// consecutive sequence steps = 2K consecutive code words. Lanes therefore load
// 8K contiguous bytes each and the wave one contiguous 1024K-byte run of the
// tile row: fully coalesced 64/128-bit streaming loads. The 16-K bits of
// overlap past a lane's last window come from the first word of the next lane
// of the quad; the last lane of a quad takes the quad's first word, which is
// exactly the tail-biting wrap of the tile (DPP quad_perm [1,2,3,0]).
//
// Per weight the VALU work is: one v_bfe_u32 window extract (plus one
// v_alignbit per 32 stream bits for windows that straddle words), one
// v_mad_u32_u24, one v_and_or_b32, one v_dot2c_f32_f16. The two fp16 halves
// of the code enter the dot product against the pair (x~, x~), so the weight
// lo+hi is used exactly inside the fp32 product; TG_FLAG_ROUND_WEIGHTS
// instead rounds lo+hi to fp16 first (one v_add_f16 more per weight).
//
// Pair code (code_id 1): one state per two weights, so a lane's 64 weights
// take 32 windows, and the fused product a (x~0 - x~1) + b (x~0 + x~1) needs
// one v_dot2c per state: about half the decode work per weight of code 0.
//
// Prologue: each workgroup transforms its input chunk (signs, 128-point
// Walsh-Hadamard transform, 1/sqrt(128)) into LDS as fp16 pairs, eight lanes
// per block with one fp32 exchange through LDS and no lane shuffles. Epilogue: lane -> wave reduction by lane shuffles,
// then either a direct output transform (1 split) or fp32 split-K partials in
// call-tagged workspace slots. The workgroup that took the block's last ticket
// of the call (tickets are taken once the input has arrived, so every other
// workgroup of the block is already running and finishes without waiting)
// waits for those slots, sums them in a fixed order and applies scale, output
// FWHT and signs. No other workgroup waits on anything.
#include "tg_decode.hpp"
#include "tg_internal.hpp"

namespace tg {

// Prefetch depth in steps (each step is 8K bytes per lane). Kept even so the
// x~ double buffer alternates statically inside the unrolled loop.
#ifndef TG_GEMV_PF_SMALL_K
#define TG_GEMV_PF_SMALL_K 2
#endif
#ifndef TG_GEMV_XDB
#define TG_GEMV_XDB 0   // double-buffer x~ across steps
#endif
template <int K>
constexpr int gemv_pf() { return K <= 4 ? TG_GEMV_PF_SMALL_K : 2; }

// One workgroup = 8 tile rows (a 128-output block) x one input chunk, with P
// waves per tile row that take interleaved 16-tile steps of the chunk.
// GATED: the input is fp16(silu(a.hg) * a.hu) (the down projection of a gated
// expert MLP) instead of the fp16 vector a.x.
// Split-K handoff: the reducer is chosen by a ticket taken once the input has
// arrived, and the partials travel in call-tagged slots (tg_device.hpp).
template <int K, int CODE, bool ROUND, int PF, int P, bool GATED = false>
__device__ __forceinline__ void gemv_workgroup(const GemvArgs& a, int ob, int split, uint32_t* lds) {
  static_assert(!(GATED && CODE == kCodeMul1I8), "the gated input has no int8 form");
  constexpr int NW = 2 * K;
  constexpr int NX = CODE == 1 ? 8 : 16;   // input words per tile column
  constexpr int XB = NX * 8;               // input words per 128-block
  constexpr int WAVES = 8 * P;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int rw = wave & 7, kp = wave >> 3;     // tile row within the block, step phase
  const int nb128 = a.n >> 7;
  // n <= 2^22, so split * nb128 <= 2^30 and 32-bit division suffices
  const int blk0 = split * nb128 / a.splits;
  const int blk1 = (split + 1) * nb128 / a.splits;
  const int cb = blk1 - blk0;             // 128-blocks in this chunk
  const int ntiles = cb * 8;              // tiles of the chunk in one tile row
  const int nsteps = (cb + 1) >> 1;       // 16 tiles per step
  const int nls = nsteps > kp ? (nsteps - kp + P - 1) / P : 0;   // this wave's steps: kp, kp+P, ...
  const int jslot = lane >> 2;
  const int R = ob * 8 + rw;
  const uint32_t* __restrict__ rowp =
      a.codes + ((size_t)R * (size_t)(a.n >> 4) + (size_t)blk0 * 8) * (size_t)(8 * K) + (size_t)lane * NW;

  uint32_t* xx_lds = lds;                                        // [2*nsteps blocks][XB] words
  float* ybuf = reinterpret_cast<float*>(lds + nsteps * 256);    // [128]
  float* red = ybuf + 128;                                       // [P-1][128]
  uint32_t* flag = lds + nsteps * 256 + 128 * P;
  int32_t* xbias = reinterpret_cast<int32_t*>(flag + 4);          // int8 form: [2*nsteps*8] per tile column
  float* xfac = reinterpret_cast<float*>(xbias + nsteps * 16);    // int8 form: [2*nsteps] per block

  uint64_t* slots = a.slots + (size_t)ob * a.splits * kBlock;   // split-K by ticket: [split][128]

  // This lane's part of the input chunk (8 lanes per 128-block, 16 elements
  // per lane) is fetched before the code prefetch: loads complete in order,
  // so fetching it later would make the transform below wait for every
  // prefetched code word as well. Blocks past the chunk read its last block
  // (valid addresses) and are zeroed below.
  static_assert(kMaxChunkBlocks <= 8 * WAVES, "one prologue pass covers the largest chunk");
  const int nbp = 2 * nsteps;                       // blocks incl. the zero padding to whole steps
  const int xb = 8 * wave + (lane >> 3), xs = lane & 7;
  const int xfirst = (blk0 + (xb < cb ? xb : cb - 1)) * kBlock + 16 * xs;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wunused-variable"
  X16 xraw;
  XGated16 graw;
#pragma clang diagnostic pop
  // Waves whose lanes all lie past the chunk's blocks (uniform) skip the
  // transform below but still issue these loads, so that every path keeps
  // the same loads in flight and the waits on the prefetch stay exact.
  const bool xwave = 8 * wave < nbp;
  if constexpr (GATED) graw = load_gated16(a.hg, a.hu, a.sign_in, xfirst);
  else xraw = load_x16(a.x, a.sign_in, xfirst);
  __builtin_amdgcn_sched_barrier(0);   // keep these loads ahead of the prefetch below

  // Prefetch ring. Every issue is unconditional (out-of-range steps and tiles
  // read a dummy line at the start of the code array instead), so each path
  // through the loop issues the same loads and the waits stay exact.
  uint32_t buf[PF][NW];
  const uint32_t* __restrict__ dummy = a.codes;
  auto issue = [&](int ls, uint32_t(&dst)[NW]) {
    const int st = kp + ls * P;
    const bool ok = ls < nls && st * 16 + jslot < ntiles;
    load_lane_words<K>(ok ? rowp + (size_t)st * (128 * K) : dummy, dst);
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, buf[p]);

  // Prologue: x~ of the chunk into LDS (zeros for the padding blocks), in the
  // word layout the decode loop reads. The fp32 exchange uses the x~ area
  // itself; the words are written only after every wave has read its part.
  uint32_t ticket = 0;
  if constexpr (CODE == kCodeMul1I8) {
    // int8 form: exact float64 transform, exchanged through the block's x~ area in two halves.
    const bool active = xb < nbp, live = xb < cb;
    int32_t qe[8], qo[8], bias = 0;
    int e = 0;
    if (xwave) {
      double v[16], de[8], dof[8];
      x16_int8_phase1(xraw, xfirst, v);
      int8_exchange(xx_lds + xb * kBlock, xs, active, live, v, de, dof);
      x16_int8_phase2(de, dof);
      int8_quantize(de, dof, qe, qo, e);
      bias = int8_group_bias(qe, qo, lane);
    }
    __syncthreads();   // every wave has read its exchange values
    if (a.splits > 1 && threadIdx.x == 0) ticket = take_ticket(&a.counters[ob]);
    if (active) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<u32x2*>(xx_lds + xb * XB + 16 * j + 2 * xs) = u32x2{int8_word(qe[j]), int8_word(qo[j])};
      xbias[xb * 8 + xs] = bias;
      if (xs == 0) xfac[xb] = live ? int8_factor(e) : 0.f;
    }
  } else {
    const bool active = xb < nbp, live = xb < cb;
    float* sc = reinterpret_cast<float*>(xx_lds) + xb * kBlock;
    float e[8], o[8];
    if (xwave) {
      float v[16];
      if constexpr (GATED) xraw = gated_to_x16(graw);
      x16_phase1<CODE == kCodeMul1>(xraw, xfirst, v);
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
    __syncthreads();   // every wave has read its exchange values
    // Split-K ticket: taken once the input has arrived (issued earlier, the
    // atomic would hold back the loads queued behind it); the answer is
    // needed only at the end.
    if (a.splits > 1 && threadIdx.x == 0) ticket = take_ticket(&a.counters[ob]);
    if (active) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (halves_form(CODE)) {
          const uint32_t he = pack_half2(e[j], e[j]), ho = pack_half2(o[j], o[j]);
          *reinterpret_cast<u32x2*>(xx_lds + xb * XB + 16 * j + 2 * xs) = u32x2{he, ho};
        } else if constexpr (CODE == kCodeMul1) {
          *reinterpret_cast<u32x2*>(xx_lds + xb * XB + 16 * j + 2 * xs) =
              u32x2{__builtin_bit_cast(uint32_t, e[j]), __builtin_bit_cast(uint32_t, o[j])};
        } else if constexpr (ROUND) {
          xx_lds[xb * XB + 8 * j + xs] = pack_half2(e[j], o[j]);
        } else {
          xx_lds[xb * XB + 8 * j + xs] = pack_half2(e[j] - o[j], e[j] + o[j]);
        }
      }
    }
  }
  __syncthreads();

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const CodeRegs cr;
  // x~ of the current and the next step (double buffer, alternating with p).
  uint32_t xv[1 + TG_GEMV_XDB][NX];
  if (TG_GEMV_XDB && nls > 0) read_xx(xx_lds, kp * 16 + jslot, xv[0]);
  for (int ls0 = 0; ls0 < nls; ls0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int ls = ls0 + p;
      if (ls < nls) {
        if constexpr (TG_GEMV_XDB) {
          const int nxt = ls + 1 < nls ? kp + (ls + 1) * P : kp + ls * P;
          read_xx(xx_lds, nxt * 16 + jslot, xv[(p + 1) & TG_GEMV_XDB]);   // in flight during this step
        } else {
          read_xx(xx_lds, (kp + ls * P) * 16 + jslot, xv[0]);
        }
        const uint32_t nbw = quad_rotate_next(buf[p][0]);
        if constexpr (CODE == 0) {
          decode_dot_64<K, ROUND>(buf[p], nbw, xv[p & TG_GEMV_XDB], acc, cr);
        } else if constexpr (CODE == kCodeMcg) {
          decode_dot_mcg_64<K, ROUND>(buf[p], nbw, xv[p & TG_GEMV_XDB], acc, cr);
        } else if constexpr (CODE == 1) {
          decode_dot_pair_64<K, ROUND>(buf[p], nbw, xv[p & TG_GEMV_XDB], acc, cr);
        } else if constexpr (CODE == kCodeMul1) {
          decode_dot_mul1_64<K>(buf[p], nbw, xv[p & TG_GEMV_XDB], acc);
        } else {
          const int tile = (kp + ls * P) * 16 + jslot;
          decode_dot_mul1_i8_64<K>(buf[p], nbw, xv[p & TG_GEMV_XDB], xbias[tile], xfac[tile >> 3], acc);
        }
      }
      issue(ls + PF, buf[p]);   // refill after use: the ring needs no register copies
    }
  }

  float d = reduce_slots(acc, lane);
  const int orow = rw * 16 + reduced_row(lane);   // output within the 128-block (lanes 0..15)
  if constexpr (P > 1) {
    if (kp > 0 && lane < 16) red[(kp - 1) * kBlock + orow] = d;
    __syncthreads();
    if (kp == 0) {
#pragma unroll
      for (int t = 1; t < P; ++t) d += red[(t - 1) * kBlock + orow];
    }
  }

  if (a.splits == 1) {
    if (kp == 0 && lane < 16) ybuf[orow] = d;
    __syncthreads();
    if (wave == 0) rht_out_block(ybuf[lane], ybuf[lane + 64], a.scales, a.sign_out, a.y, ob * kBlock, lane);
    return;
  }

  // Split-K. The reducer sums the splits in a fixed order (wave w takes
  // splits w, w+WAVES, ..., then wave 0 adds the per-wave sums), so the
  // result does not depend on which workgroup reduced.
  float v0 = 0.f, v1 = 0.f;
  // The call's last ticket holder reduces, with its own partial from LDS;
  // every workgroup publishes its 128 partials (the reducer too, so that no
  // slot is ever more than one call old), and all but the reducer leave.
  if (threadIdx.x == 0) {
    flag[0] = (ticket & (kTicketCall - 1u)) == (uint32_t)a.splits - 1u ? 1u : 0u;
    flag[1] = slot_tag(ticket, (uint32_t)a.splits);
  }
  if (kp == 0 && lane < 16) ybuf[orow] = d;
  __syncthreads();
  const uint32_t tag = flag[1];
  if (kp == 0 && lane < 16) put_slot(slots + (size_t)split * kBlock + orow, d, tag);
  if (flag[0] == 0u) return;
  constexpr int J = 4;   // splits per wave whose slots are read together
  for (int t0 = 0; t0 < a.splits; t0 += WAVES * J) {
    // Read this wave's slots of up to J splits at once; re-read the ones that
    // do not hold this call's partial yet, together, until all do (bounded),
    // then add in split order.
    uint64_t s0[J], s1[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int t = t0 + wave + j * WAVES;
      s0[j] = s1[j] = (uint64_t)tag << 32;   // splits outside the range, and this one's own, count as ready
      if (t < a.splits && t != split) {
        s0[j] = peek_slot(slots + (size_t)t * kBlock + lane);
        s1[j] = peek_slot(slots + (size_t)t * kBlock + lane + 64);
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
        const int t = t0 + wave + j * WAVES;
        if (!slot_ready(s0[j], tag)) s0[j] = peek_slot(slots + (size_t)t * kBlock + lane);
        if (!slot_ready(s1[j], tag)) s1[j] = peek_slot(slots + (size_t)t * kBlock + lane + 64);
      }
    }
    // A wait that ran out: its outputs become NaN (slot_value) and the
    // workspace's status word records it for the host.
    if (empty) report_status(a.status, kStatusSplitkTimeout);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int t = t0 + wave + j * WAVES;
      if (t >= a.splits) break;
      v0 += t == split ? ybuf[lane] : slot_value(s0[j], tag);
      v1 += t == split ? ybuf[lane + 64] : slot_value(s1[j], tag);
    }
  }
  {
    float* wsum = reinterpret_cast<float*>(xx_lds);   // reuse x~ storage: [WAVES][128]; may overlap ybuf
    __syncthreads();
    wsum[wave * kBlock + lane] = v0;
    wsum[wave * kBlock + lane + 64] = v1;
    __syncthreads();
    if (wave == 0) {
      v0 = 0.f;
      v1 = 0.f;
      const int nw = a.splits < WAVES ? a.splits : WAVES;
      for (int w = 0; w < nw; ++w) {
        v0 += wsum[w * kBlock + lane];
        v1 += wsum[w * kBlock + lane + 64];
      }
      rht_out_block(v0, v1, a.scales, a.sign_out, a.y, ob * kBlock, lane);
      if (lane == 0) finish_call(&a.counters[ob], (uint32_t)a.splits);
    }
  }
}

// Blocks are issued round-robin over the 8 XCDs; remap so that the splits of
// one output block, and the blocks reading the same input chunk, share an XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  return (nblk & 7) == 0 ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
}

template <int K, int CODE, bool ROUND, int PF, int P>
__global__ __launch_bounds__(64 * 8 * P) void gemv_kernel(GemvArgs a) {
  extern __shared__ uint32_t lds[];
  // Every argument the kernel reads goes out in one batch of scalar loads (the empty asm wants
  // them all here); loaded where first used, the pointers came a round trip after the sizes,
  // ahead of the input load.
  asm volatile("" ::"s"(a.codes), "s"(a.scales), "s"(a.sign_in), "s"(a.sign_out), "s"(a.x), "s"(a.y), "s"(a.slots),
               "s"(a.counters), "s"(a.status), "s"(a.m), "s"(a.n), "s"(a.splits));
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int ob = bid / a.splits;
  gemv_workgroup<K, CODE, ROUND, PF, P>(a, ob, bid - ob * a.splits, lds);
}

template <int CODE, bool ROUND, bool GATED>
__device__ __forceinline__ void grouped_dispatch(const GemvArgs& a, int k_bits, int ob, int split, uint32_t* lds) {
  switch (k_bits) {
    case 1: gemv_workgroup<1, CODE, ROUND, gemv_pf<1>(), kGemvP, GATED>(a, ob, split, lds); break;
    case 2: gemv_workgroup<2, CODE, ROUND, gemv_pf<2>(), kGemvP, GATED>(a, ob, split, lds); break;
    case 3: gemv_workgroup<3, CODE, ROUND, gemv_pf<3>(), kGemvP, GATED>(a, ob, split, lds); break;
    case 4: gemv_workgroup<4, CODE, ROUND, gemv_pf<4>(), kGemvP, GATED>(a, ob, split, lds); break;
    case 5: gemv_workgroup<5, CODE, ROUND, gemv_pf<5>(), kGemvP, GATED>(a, ob, split, lds); break;
    case 6: gemv_workgroup<6, CODE, ROUND, gemv_pf<6>(), kGemvP, GATED>(a, ob, split, lds); break;
    case 7: gemv_workgroup<7, CODE, ROUND, gemv_pf<7>(), kGemvP, GATED>(a, ob, split, lds); break;
    default: gemv_workgroup<8, CODE, ROUND, gemv_pf<8>(), kGemvP, GATED>(a, ob, split, lds); break;
  }
}

// Selection e of the launch runs layer sel[e] (or, with sel_pairs, layer
// 2*sel[e/2] + e%2: the gate and up of the selected experts, from one id each).
template <bool ROUND, bool GATED>
__global__ __launch_bounds__(64 * 8 * kGemvP) void grouped_kernel(GroupedArgs g, int max_ob) {
  extern __shared__ uint32_t lds[];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_sel = max_ob * g.splits;
  const int e = bid / per_sel;
  const int rem = bid - e * per_sel;
  const int ob = rem / g.splits, split = rem - ob * g.splits;
  const int sv = g.sel[g.sel_pairs ? (e >> 1) : e];
  if (sv < 0 || sv >= (g.sel_pairs ? (g.n_layers >> 1) : g.n_layers)) return;
  const int li = g.sel_pairs ? 2 * sv + (e & 1) : sv;
  const LayerDev L = g.layers[li];
  if (ob >= (L.m >> 7)) return;
  // The launch's split count comes from the table's widest layer; a layer with
  // fewer 128-blocks runs one chunk per block, so no chunk is ever empty.
  const int splits = g.splits < (L.n >> 7) ? g.splits : (L.n >> 7);
  if (split >= splits) return;
  GemvArgs a;
  a.codes = L.codes;
  a.scales = L.scales;
  a.sign_in = L.sign_in;
  a.sign_out = L.sign_out;
  a.x = g.x + (size_t)e * g.x_stride;
  a.y = g.y + (size_t)e * g.y_stride;
  a.slots = g.slots + (size_t)e * g.splits * g.max_m;
  a.counters = g.counters + (size_t)e * (g.max_m >> 7);
  a.status = g.status;
  a.m = L.m;
  a.n = L.n;
  a.splits = splits;
  a.hg = GATED ? g.hin + (size_t)(2 * e) * g.hin_stride : nullptr;
  a.hu = GATED ? g.hin + (size_t)(2 * e + 1) * g.hin_stride : nullptr;
  if (L.code_id == 0) grouped_dispatch<0, ROUND, GATED>(a, L.k_bits, ob, split, lds);
  else if (L.code_id == 1) grouped_dispatch<1, ROUND, GATED>(a, L.k_bits, ob, split, lds);
  else if (L.code_id == kCodeMcg) grouped_dispatch<kCodeMcg, ROUND, GATED>(a, L.k_bits, ob, split, lds);
  else grouped_dispatch<kCodeMul1, false, GATED>(a, L.k_bits, ob, split, lds);
}

// Router-weighted sum of the selected experts' outputs, in selection order;
// selections outside [0, n_experts) contribute nothing. Every row of Y2 is a
// valid address (one per selection), so each thread loads eight experts' rows
// together with their selection and weight (uniform, scalar loads) in one
// round of memory latency, and an invalid selection's row -- never written,
// so possibly not a number -- is dropped by a select, not multiplied by zero.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ Y2, int64_t y2_stride,
                                                          const int32_t* __restrict__ sel, const float* __restrict__ w,
                                                          int top_k, int n_experts, int hidden, float* __restrict__ y) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= hidden) return;
  float acc = 0.f;
  for (int e0 = 0; e0 < top_k; e0 += 8) {
    float v[8], wt[8];
    int32_t sv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + j < top_k ? e0 + j : top_k - 1;   // past the end: re-read the last, unused
      sv[j] = sel[e];
      wt[j] = w[e];
      v[j] = Y2[(size_t)e * y2_stride + o];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = e0 + j < top_k && sv[j] >= 0 && sv[j] < n_experts;
      const float t = wt[j] * v[j];
      acc = ok ? acc + t : acc;
    }
  }
  y[o] = acc;
}

template <int K, int CODE, bool ROUND>
static hipError_t launch_k(const GemvArgs& a, hipStream_t s) {
  constexpr int PF = gemv_pf<K>();
  const int nb128 = a.n >> 7;
  const int max_chunk = (nb128 + a.splits - 1) / a.splits;
  const int grid = (a.m >> 7) * a.splits;
  hipLaunchKernelGGL((gemv_kernel<K, CODE, ROUND, PF, kGemvP>), dim3(grid), dim3(64 * 8 * kGemvP),
                     gemv_lds_bytes(max_chunk, CODE == kCodeMul1I8), s, a);
  return hipGetLastError();
}

// The mul1 forms have exact weights: rounding them changes nothing, so they
// are built once, without the rounded form.
template <int CODE>
static hipError_t launch_code(const GemvArgs& a, int k_bits, bool round_weights, hipStream_t s) {
#define TG_CASE(K)                                                                                \
  case K:                                                                                         \
    return round_weights && rounded_form(CODE) ? launch_k<K, CODE, rounded_form(CODE)>(a, s)      \
                                               : launch_k<K, CODE, false>(a, s);
  switch (k_bits) {
    TG_CASE(1) TG_CASE(2) TG_CASE(3) TG_CASE(4) TG_CASE(5) TG_CASE(6) TG_CASE(7) TG_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
}

hipError_t launch_gemv(const GemvArgs& a, int k_bits, int variant, bool round_weights, hipStream_t s) {
  switch (variant) {
    case 0: return launch_code<0>(a, k_bits, round_weights, s);
    case 1: return launch_code<1>(a, k_bits, round_weights, s);
    case kCodeMul1: return launch_code<kCodeMul1>(a, k_bits, false, s);
    case kCodeMcg: return launch_code<kCodeMcg>(a, k_bits, round_weights, s);
    case kCodeMul1I8: return launch_code<kCodeMul1I8>(a, k_bits, false, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool ROUND, bool GATED>
static void launch_grouped_t(const GroupedArgs& g, int max_ob, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((grouped_kernel<ROUND, GATED>), dim3(grid), dim3(64 * 8 * kGemvP), lds, s, g, max_ob);
}

hipError_t launch_grouped(const GroupedArgs& g, int max_ob, int max_n, hipStream_t s) {
  const int grid = g.n_sel * max_ob * g.splits;
  if (grid == 0) return hipSuccess;
  const int max_chunk = ((max_n >> 7) + g.splits - 1) / g.splits;
  const size_t lds = gemv_lds_bytes(max_chunk);
  const bool gated = g.hin != nullptr;
  if (g.round_weights) {
    if (gated) launch_grouped_t<true, true>(g, max_ob, grid, lds, s);
    else launch_grouped_t<true, false>(g, max_ob, grid, lds, s);
  } else {
    if (gated) launch_grouped_t<false, true>(g, max_ob, grid, lds, s);
    else launch_grouped_t<false, false>(g, max_ob, grid, lds, s);
  }
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* Y2, int64_t y2_stride, const int32_t* sel, const float* w, int top_k,
                              int n_experts, int hidden, float* y, hipStream_t s) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3((hidden + 255) / 256), dim3(256), 0, s, Y2, y2_stride, sel, w, top_k,
                     n_experts, hidden, y);
  return hipGetLastError();
}

// Decode-only rate of the batch-1 loop (the VALU ceiling of the path): each
// wave runs the same per-step work as gemv_workgroup -- the x~ words of its
// tile column from LDS, the quad rotate for the overlap bits, the window
// extraction, code and dot product of its 64 weights per lane -- but reads
// its code words from LDS instead of HBM (on odd steps those of the lane 64
// threads on, so nothing can be hoisted out of the loop). The per-lane sums
// are written out so that no work is dead.
template <int K, int CODE>
__global__ __launch_bounds__(512) void decode_ceiling_kernel(float* __restrict__ out, int steps, uint32_t seed) {
  constexpr int NW = 2 * K;
  constexpr int NX = CODE == 1 ? 8 : 16;
  __shared__ uint32_t xx_lds[16 * NX];
  __shared__ uint32_t words[512 * NW];
  const int tid = threadIdx.x, lane = tid & 63, jslot = lane >> 2;
  for (int i = tid; i < 16 * NX; i += 512) xx_lds[i] = 0x3C003C00u ^ ((uint32_t)i * 0x00010001u);
  for (int i = tid; i < 512 * NW; i += 512) {
    uint32_t h = (uint32_t)i * 0x9E3779B1u + seed + blockIdx.x * 0x85EBCA6Bu;
    h ^= h >> 15;
    words[i] = h * 0x2C1B3C6Du;
  }
  __syncthreads();
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const CodeRegs cr;
  for (int st = 0; st < steps; ++st) {
    uint32_t w[NW], xv[NX];
    const uint32_t* src = &words[((tid + (st & 1) * 64) & 511) * NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = src[i];
    read_xx(xx_lds, jslot, xv);
    const uint32_t nbw = quad_rotate_next(w[0]);
    if constexpr (CODE == 0) decode_dot_64<K, false>(w, nbw, xv, acc, cr);
    else if constexpr (CODE == kCodeMcg) decode_dot_mcg_64<K, false>(w, nbw, xv, acc, cr);
    else if constexpr (CODE == 1) decode_dot_pair_64<K, false>(w, nbw, xv, acc, cr);
    else if constexpr (CODE == kCodeMul1) decode_dot_mul1_64<K>(w, nbw, xv, acc);
    else decode_dot_mul1_i8_64<K>(w, nbw, xv, (int32_t)xx_lds[jslot] >> 8, 1.0f, acc);
  }
  out[(size_t)blockIdx.x * 512 + tid] = acc[0] + acc[1] + acc[2] + acc[3];
}

hipError_t launch_decode_ceiling(int k_bits, int variant, int workgroups, int steps, float* out, hipStream_t s) {
#define TG_LAUNCH(K, C) hipLaunchKernelGGL((decode_ceiling_kernel<K, C>), dim3(workgroups), dim3(512), 0, s, out, steps, 1u)
#define TG_CASE(K)                                       \
  case K:                                                \
    switch (variant) {                                   \
      case 0: TG_LAUNCH(K, 0); break;                    \
      case 1: TG_LAUNCH(K, 1); break;                    \
      case kCodeMul1: TG_LAUNCH(K, kCodeMul1); break;     \
      case kCodeMcg: TG_LAUNCH(K, kCodeMcg); break;       \
      default: TG_LAUNCH(K, kCodeMul1I8); break;          \
    }                                                    \
    break;
  switch (k_bits) {
    TG_CASE(1) TG_CASE(2) TG_CASE(3) TG_CASE(4) TG_CASE(5) TG_CASE(6) TG_CASE(7) TG_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
#undef TG_LAUNCH
  return hipGetLastError();
}

}  // namespace tg
