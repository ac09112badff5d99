// Tail-biting Viterbi encoder for gfx950: the bitstream of each 16x16 tile
// that minimises sum_t (alpha * w(S_t) - v_t)^2.
//
// The search is the one of the "Trellis Quantization" lecture, Part seven
// (per state the best path ending there; every state looks back at the few
// states that lead into it; trace back from the best final state), made
// tail-biting by its Part eight two-pass approximation (rotate the sequence by
// half, run Viterbi, take the state in the middle as the start window, run
// again constrained to start and end on it). Part eight notes the search has
// 65,536 states per tile and parallelises well on a GPU.
//
// Formulation. A step shifts B = V*K bits into the 16-bit window, so the
// states that lead into s are p = (s >> B) | (a << (16 - B)), a < 2^B: they
// depend on s only through u = s >> B. With
//     M_t(u) = min_a cost_t(u | a << (16-B)),   A_t(u) = the first such a,
// every step is cost_t(s) = d_t(s) + M_{t-1}(s >> B) followed by the new
// minima M_t over the top bits. Only M (2^(16-B) floats, 128 KB at B = 1)
// lives in LDS; A_t is packed B bits per entry into the workspace, and one
// lane traces the path back through it.
//
// Work split: 1024 threads, 64 state evaluations each per step. Thread i owns
// NE consecutive entries u and the predecessor range a in [a0, a0 + NA)
// (entries with more than 64 candidates are split over TPE lanes and combined
// by shuffles). Each step: stage the M values the thread needs, barrier,
// evaluate, write M and the packed A word, barrier.
//
// Arithmetic follows the oracle exactly (float32, no contraction):
// p = alpha*w, e = p - v, d = e*e (pair code: d = e0*e0 + e1*e1), c = d + M;
// minima keep the first candidate, the open end takes the smallest state.
#include "tg_device.hpp"
#include "tg_internal.hpp"

#pragma clang fp contract(off)

namespace tg {

constexpr int kEncThreads = 1024;

template <int B>
struct EncGeom {
  static constexpr int NU = 1 << (16 - B);                        // entries of M
  static constexpr int TPE = NU >= kEncThreads ? 1 : kEncThreads / NU;   // lanes per entry
  static constexpr int NE = NU >= kEncThreads ? NU / kEncThreads : 1;    // entries per thread
  static constexpr int NA = (1 << B) / TPE;                       // predecessor top bits per thread
  static constexpr int NJ = (NE >> B) > 0 ? (NE >> B) : 1;        // distinct u >> B per thread
  static constexpr int NS = NJ * NA;                              // staged M values
  static constexpr int NW = NU / NE;                              // packed A words per step
  static_assert(NE * NA == 64, "64 state evaluations per thread and step");
  static_assert(NE * B <= 32, "one packed word per thread");
};

// Squared error of state s against the step's target(s).
template <int CODE>
__device__ __forceinline__ float state_error(uint32_t s, float alpha, float v0, float v1, const CodeRegs& cr) {
  const uint32_t u = CODE == kCodeMcg ? mcg_halves(s, cr) : code_halves(s, cr);
  if constexpr (CODE == 2) {
    const float w = (float)mul1_level(mul1_bytes(s)) * kMul1Step;   // exact
    const float e = alpha * w - v0;
    return e * e;
  } else if constexpr (CODE == 0 || CODE == kCodeMcg) {
    const float w = (float)halves_sum_rne(u);
    const float e = alpha * w - v0;
    return e * e;
  } else {
    const uint32_t wp = pair_weights_rne(u);
    const float w0 = half_bits_to_float((uint16_t)wp), w1 = half_bits_to_float((uint16_t)(wp >> 16));
    const float e0 = alpha * w0 - v0;
    const float e1 = alpha * w1 - v1;
    return e0 * e0 + e1 * e1;
  }
}

// One Viterbi pass over the tile's T steps. rot: the sequence is read from
// step rot on (cyclically). start < 0: free start; otherwise the forced first
// state. The packed minima arguments of every step go to bp [T][NW].
//
// M is double-buffered in LDS (Mb[0], Mb[1]; one barrier per step) when two
// copies fit; at B = 1 (2 x 128 KB) it is updated in place instead: each
// thread first copies the 32 values it reads into registers, and a second
// barrier separates those reads from the writes. Returns the index of the
// buffer that holds the last step's minima.
template <int B, int CODE>
__device__ int viterbi_pass(const float* tgt, float alpha, int rot, int start, float* const (&Mb)[2],
                            uint32_t* __restrict__ bp, float& end_cost, uint32_t& end_state) {
  using G = EncGeom<B>;
  constexpr int V = CODE == 1 ? 2 : 1;
  constexpr int T = 256 / V;
  constexpr bool INPLACE = B == 1;
  constexpr int EPJ = G::NE / G::NJ;          // entries sharing one u >> B
  const int tid = threadIdx.x;
  const int e0 = (tid / G::TPE) * G::NE;      // first entry u of this thread
  const int a0 = (tid % G::TPE) * G::NA;      // first predecessor top-bit value
  const int j0 = e0 >> B;
  const bool leader = tid % G::TPE == 0;
  const CodeRegs cr;
  int cur = 0;                                // buffer holding M_{t-1}
  for (int t = 0; t < T; ++t) {
    const int ts = (t + rot) % T;
    const float v0 = tgt[V * ts], v1 = V == 2 ? tgt[V * ts + 1] : 0.f;
    const float* Msrc = Mb[cur];
    float* Mdst = INPLACE ? Mb[0] : Mb[cur ^ 1];
    float ms[INPLACE ? G::NS : 1];
    if constexpr (INPLACE) {
      if (t > 0) {
#pragma unroll
        for (int jj = 0; jj < G::NJ; ++jj)
#pragma unroll
          for (int ai = 0; ai < G::NA; ++ai) ms[jj * G::NA + ai] = Msrc[(j0 + jj) | ((a0 + ai) << (16 - 2 * B))];
      }
      __syncthreads();   // every thread has its M values before any is overwritten
    }
    uint32_t word = 0u;
    float lc = __builtin_inff();
    uint32_t lk = 0xFFFFFFFFu;
#pragma unroll 4
    for (int e = 0; e < G::NE; ++e) {
      const uint32_t u = (uint32_t)(e0 + e);
      const int jj = e / EPJ;
      float bc = __builtin_inff();
      uint32_t ba = (uint32_t)a0;
#pragma unroll 8
      for (int ai = 0; ai < G::NA; ++ai) {
        const uint32_t a = (uint32_t)(a0 + ai);
        const uint32_t s = u | (a << (16 - B));
        const float d = state_error<CODE>(s, alpha, v0, v1, cr);
        float c;
        if (t > 0) {
          float m;
          if constexpr (INPLACE) m = ms[jj * G::NA + ai];
          else m = Msrc[(uint32_t)(j0 + jj) | (a << (16 - 2 * B))];
          c = d + m;
        } else {
          c = (start < 0 || s == (uint32_t)start) ? d : __builtin_inff();
        }
        if (c < bc) {
          bc = c;
          ba = a;
        }
      }
      if constexpr (G::TPE > 1) {   // combine the entry's lanes; lower lanes hold smaller a
#pragma unroll
        for (int m = 1; m < G::TPE; m <<= 1) {
          const float oc = __shfl_xor(bc, m, 64);
          const uint32_t oa = (uint32_t)__shfl_xor((int)ba, m, 64);
          if (oc < bc || (oc == bc && oa < ba)) {
            bc = oc;
            ba = oa;
          }
        }
      }
      if (leader) Mdst[u] = bc;
      word |= ba << (e * B);
      if (t == T - 1) {               // the smallest final state of least cost among this thread's entries
        const uint32_t key = u | (ba << (16 - B));
        if (bc < lc || (bc == lc && key < lk)) {
          lc = bc;
          lk = key;
        }
      }
    }
    if (leader) bp[(size_t)t * G::NW + tid / G::TPE] = word;
    end_cost = leader ? lc : __builtin_inff();
    end_state = leader ? lk : 0xFFFFFFFFu;
    __syncthreads();
    if constexpr (!INPLACE) cur ^= 1;
  }
  return cur;
}

// A_t(u) from the packed words (written by other waves of this workgroup).
template <int B>
__device__ __forceinline__ uint32_t read_arg(const uint32_t* bp, int t, uint32_t u) {
  using G = EncGeom<B>;
  const uint32_t w = __hip_atomic_load(const_cast<uint32_t*>(bp + (size_t)t * G::NW + u / G::NE), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return (w >> ((u % G::NE) * B)) & ((1u << B) - 1u);
}

template <int K, int CODE>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(const float* __restrict__ targets, float alpha,
                                                             int n_tiles, uint32_t* __restrict__ codes,
                                                             float* __restrict__ sq_err, uint32_t* __restrict__ ws) {
  constexpr int V = CODE == 1 ? 2 : 1;
  constexpr int B = V * K;
  constexpr int T = 256 / V;
  constexpr int WPT = 8 * K;
  using G = EncGeom<B>;
  extern __shared__ uint32_t lds[];
  constexpr int NBUF = B == 1 ? 1 : 2;                         // copies of M (see viterbi_pass)
  float* M0 = reinterpret_cast<float*>(lds);                   // [NBUF][NU]
  float* const Mb[2] = {M0, M0 + (NBUF - 1) * G::NU};
  float* tgt = M0 + NBUF * G::NU;                              // [256]
  float* rc = tgt + 256;                                       // [16] per-wave best cost
  uint32_t* rk = reinterpret_cast<uint32_t*>(rc + 16);         // [16] per-wave best state
  uint32_t* words = rk + 16;                                   // [WPT] the tile's stream
  uint32_t* bcast = words + WPT;                               // [2]
  uint32_t* bp = ws + (size_t)blockIdx.x * T * G::NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    if (tid < 256) tgt[tid] = targets[(size_t)tile * 256 + tid];
    __syncthreads();
    float bc;
    uint32_t bk;

    // Pass 1: the rotated sequence, free start and end; keep the state at its middle.
    viterbi_pass<B, CODE>(tgt, alpha, T / 2, -1, Mb, bp, bc, bk);
    __builtin_amdgcn_s_waitcnt(0);   // this thread's argument words have reached memory
    {
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float oc = __shfl_xor(bc, m, 64);
        const uint32_t ok = (uint32_t)__shfl_xor((int)bk, m, 64);
        if (oc < bc || (oc == bc && ok < bk)) {
          bc = oc;
          bk = ok;
        }
      }
      if (lane == 0) {
        rc[wave] = bc;
        rk[wave] = bk;
      }
      __syncthreads();
      if (tid == 0) {
        float c = rc[0];
        uint32_t s = rk[0];
        for (int w = 1; w < kEncThreads / 64; ++w)
          if (rc[w] < c || (rc[w] == c && rk[w] < s)) {
            c = rc[w];
            s = rk[w];
          }
        for (int t = T - 1; t > T / 2; --t) s = (s >> B) | (read_arg<B>(bp, t - 1, s >> B) << (16 - B));
        bcast[0] = s;
      }
      __syncthreads();
    }
    const int s0 = (int)bcast[0];

    // Pass 2: the original sequence from s0, ending where the circle closes.
    const int last = viterbi_pass<B, CODE>(tgt, alpha, 0, s0, Mb, bp, bc, bk);
    __builtin_amdgcn_s_waitcnt(0);
    if (tid < WPT) words[tid] = 0u;
    __syncthreads();
    if (tid == 0) {
      const uint32_t u = (uint32_t)s0 >> B;
      uint32_t s = u | (read_arg<B>(bp, T - 1, u) << (16 - B));
      const float cost = Mb[last][u];
      for (int t = T - 1; t >= 0; --t) {
#pragma unroll
        for (int i = 0; i < B; ++i) {   // stream bits [B t, B t + B) = the top B bits of S_t
          const int p = B * t + i;
          words[p >> 5] |= ((s >> (15 - i)) & 1u) << (31 - (p & 31));
        }
        if (t > 0) s = (s >> B) | (read_arg<B>(bp, t - 1, s >> B) << (16 - B));
      }
      if (sq_err) sq_err[tile] = cost;
    }
    __syncthreads();
    if (tid < WPT) codes[(size_t)tile * WPT + tid] = words[tid];
    __syncthreads();
  }
}

template <int K, int CODE>
size_t encode_lds_bytes() {
  constexpr int B = (CODE == 1 ? 2 : 1) * K;
  return (size_t)EncGeom<B>::NU * 4 * (B == 1 ? 1 : 2) + 256 * 4 + 32 * 4 + 8 * K * 4 + 8;
}

template <int K, int CODE>
static hipError_t launch_enc(const float* targets, float alpha, int n_tiles, uint32_t* codes, float* sq_err,
                             uint32_t* ws, int slots, hipStream_t s) {
  const size_t lds = encode_lds_bytes<K, CODE>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&encode_kernel<K, CODE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((encode_kernel<K, CODE>), dim3(slots), dim3(kEncThreads), lds, s, targets, alpha, n_tiles, codes,
                     sq_err, ws);
  return hipGetLastError();
}

size_t encode_ws_words_per_slot(int k_bits, int code_id) {
  const int B = (code_id == 1 ? 2 : 1) * k_bits;
  const int T = code_id == 1 ? 128 : 256;
  const int NU = 1 << (16 - B);
  const int NE = NU >= kEncThreads ? NU / kEncThreads : 1;
  return (size_t)T * (NU / NE);
}

hipError_t launch_encode(const float* targets, float alpha, int n_tiles, int k_bits, int code_id, uint32_t* codes,
                         float* sq_err, uint32_t* ws, int slots, hipStream_t s) {
#define TG_CASE(K, C) \
  case K: return launch_enc<K, C>(targets, alpha, n_tiles, codes, sq_err, ws, slots, s);
  if (code_id == 0) {
    switch (k_bits) {
      TG_CASE(1, 0) TG_CASE(2, 0) TG_CASE(3, 0) TG_CASE(4, 0) TG_CASE(5, 0) TG_CASE(6, 0) TG_CASE(7, 0) TG_CASE(8, 0)
      default: return hipErrorInvalidValue;
    }
  }
  if (code_id == 2) {
    switch (k_bits) {
      TG_CASE(1, 2) TG_CASE(2, 2) TG_CASE(3, 2) TG_CASE(4, 2) TG_CASE(5, 2) TG_CASE(6, 2) TG_CASE(7, 2) TG_CASE(8, 2)
      default: return hipErrorInvalidValue;
    }
  }
  if (code_id == kCodeMcg) {
    switch (k_bits) {
      TG_CASE(1, 3) TG_CASE(2, 3) TG_CASE(3, 3) TG_CASE(4, 3) TG_CASE(5, 3) TG_CASE(6, 3) TG_CASE(7, 3) TG_CASE(8, 3)
      default: return hipErrorInvalidValue;
    }
  }
  switch (k_bits) {
    TG_CASE(1, 1) TG_CASE(2, 1) TG_CASE(3, 1) TG_CASE(4, 1)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
}

}  // namespace tg
