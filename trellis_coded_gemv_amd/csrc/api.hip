// C ABI of the trellis-coded GEMV library: argument validation, workspace
// sizing, split selection and kernel launches. Nothing here touches the GPU
// before every argument has been checked.
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <map>
#include <mutex>

#include "trellis_gemv.h"
#include "tg_internal.hpp"

#define TG_API extern "C" __attribute__((visibility("default")))

#ifndef TG_BUILD_ID
#define TG_BUILD_ID "unversioned"
#endif

namespace {

using namespace tg;

constexpr size_t kAlign = 256;

static_assert(sizeof(tg_layer) == sizeof(LayerDev), "device layer table mirrors tg_layer");
static_assert(offsetof(tg_layer, codes) == offsetof(LayerDev, codes), "device layer table mirrors tg_layer");
static_assert(offsetof(tg_layer, sign_out) == offsetof(LayerDev, sign_out), "device layer table mirrors tg_layer");

// Entry points that write a dense fp16 copy of the weights (decode, prefill)
// take at most 2^38 of them: 512 GiB, more than any device holds, and the
// bound keeps their grids within 32 bits.
constexpr int64_t kMaxDenseWeights = (int64_t)1 << 38;

// Batch-1 split-K slots in a layer workspace: room for kSlotPairs (output
// block, split) pairs of 128 64-bit slots, 2 MiB at a fixed offset. The split
// choice below uses about 256 pairs; only a layer that needs many input chunks
// to fit the LDS (some 2^31 weights and more) needs more, and is refused.
constexpr int kSlotPairs = 2048;
constexpr size_t kSlotArea = (size_t)kSlotPairs * kBlock * 8;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p % a) != 0; }

// Kernel form of a layer: its code_id, or mul1 against the int8 form of x~.
int kernel_form(const tg_layer* L) { return (L->flags & TG_FLAG_INT8_ACT) != 0 ? kCodeMul1I8 : L->code_id; }

int32_t check_layer(const tg_layer* L) {
  if (!L) return TG_ERR_NULL;
  if (L->code_id < 0 || L->code_id > 3) return TG_ERR_CODE_ID;
  if (L->k_bits < 1 || L->k_bits > 8) return TG_ERR_KBITS;
  if (L->m <= 0 || L->n <= 0 || (L->m % kBlock) != 0 || (L->n % kBlock) != 0) return TG_ERR_SHAPE;
  if (L->m > (1 << 22) || L->n > (1 << 22)) return TG_ERR_SHAPE;
  if ((L->flags & ~(TG_FLAG_ROUND_WEIGHTS | TG_FLAG_INT8_ACT)) != 0 || L->splits < 0 || L->splits > 65535)
    return TG_ERR_ARG;
  if ((L->flags & TG_FLAG_INT8_ACT) != 0 && L->code_id != 2) return TG_ERR_ARG;   // the int8 form is mul1's
  if (!L->codes || !L->scales || !L->sign_in || !L->sign_out) return TG_ERR_NULL;
  if (misaligned(L->codes, 16) || misaligned(L->scales, 2) || misaligned(L->sign_in, 4) ||
      misaligned(L->sign_out, 4))
    return TG_ERR_ALIGN;
  return TG_OK;
}

// Number of input chunks (split-K) for a batch-1 GEMV. About 256 workgroups
// (one 128-output block x one chunk each) measured best on 256 CUs for most
// shapes, 1024 for long inputs (below); chunks are kept equal and a whole number of 16-tile steps
// (two 128-blocks), since a half step costs the decode work of a full one.
// The chunk also has to fit the LDS budget. A layer's `splits` field, when
// positive, forces the count (a tuning aid; still clamped to what fits).
int split_for_target(int nb, int target) {
  const int steps = nb / 2;                      // whole steps along the input
  if (steps < 1) return 1;
  int best = 1;
  for (int s = 1; s <= steps; ++s) {
    if (steps % s) continue;
    const int d = abs(s - target), bd = abs(best - target);
    if (d < bd || (d == bd && s > best)) best = s;
  }
  return best;
}

int gemv_splits(int m, int n, int forced) {
  const int ob = m / kBlock, nb = n / kBlock;
  int s = forced;
  if (s <= 0) {
    // chunks of a single step lose to two-step chunks: the split-K handoff
    // costs more than the extra parallelism gains (1024 x 8192: 8.9 vs 7.3 us).
    // A long input (192 blocks or more) aims at 1024 workgroups instead: four
    // per compute unit hide the code loads better than one, and its chunks
    // stay long (8192 x 28672: 16 chunks of 7 steps, 0.5 us faster per call)
    const int max_s = nb / 4 > 1 ? nb / 4 : 1;
    const int wgs = nb >= 192 ? 1024 : 256;
    const int target = (wgs + ob / 2) / ob;
    s = split_for_target(nb, target < max_s ? target : max_s);
  }
  const int cap = kSlotPairs / ob;               // (block, split) pairs the slot area holds
  if (s > cap) s = cap;
  const int min_s = (nb + kMaxChunkBlocks - 1) / kMaxChunkBlocks;
  if (s < min_s) s = min_s;
  if (s > nb) s = nb;
  if (s < 1) s = 1;
  return s;
}

// Splits of the small-batch path: about 256 workgroups, but the fp32 partials
// cost 8*S*M*m bytes of traffic against m*n*K/8 code bytes, so they are kept
// to 1/8 of the code bytes; a chunk keeps at least 8 MFMA steps (one per
// wave): 8 tile columns for code 0, 16 for the pair code, whose MFMA spans two
// tiles.
int gemm_splits(int m, int n, int M, int k_bits, int code_id, int forced) {
  const int ob = m / kBlock;
  const int nsub = n / (code_id == 1 ? 2 * kBlock : kBlock);
  int s = forced;
  if (s <= 0) {
    s = (256 + ob / 2) / ob;                                     // about 256 workgroups
    const int cap = (int)((int64_t)n * k_bits / (512 * M));    // partial traffic <= 1/8 of the code bytes
    if (s > cap) s = cap;
  }
  if (s > nsub) s = nsub;
  if (s < 1) s = 1;
  return s;
}

// A layer's workspace, at fixed offsets for every layer: the header (its first
// word is the status word, see tg_workspace_status), the batch-1 ticket
// counters and the small-batch arrival counters, each in an area sized for the
// largest layer; the batch-1 split-K slots, in an area of kSlotPairs (block,
// split) pairs; then the small-batch scratch (input transform, partials). A
// batch-1 call leaves its ticket counters on a call boundary (a multiple of
// 2^16) and a small-batch call leaves its arrival counters at zero. The slots
// carry their call's number and split count, and the small-batch scratch never
// reaches the slot area, so no stale word is ever taken for a partial. One
// buffer can therefore serve any sequence of layers and paths.
constexpr size_t kCounterArea = (size_t)((1 << 22) / kBlock) * 4;

struct GemvWs {
  size_t counters, slots, total;
};

GemvWs gemv_ws(int m, int splits) {
  GemvWs w;
  w.counters = kWsHeader;
  w.slots = kWsHeader + 2 * kCounterArea;
  w.total = w.slots + (splits > 1 ? round_up((size_t)splits * m * 8, kAlign) : 0);
  return w;
}

// A batch-1 split that the slot area cannot hold (layers of more than about
// 2^31 weights, whose chunks must be many to fit the LDS).
bool gemv_slots_overflow(int m, int splits) { return splits > 1 && (int64_t)splits * (m / kBlock) > kSlotPairs; }

struct GemmWs {
  size_t counters, xt, partials, total;
};

GemmWs gemm_ws(int m, int n, int M, int splits) {
  GemmWs w;
  const int mpad = (M + 15) / 16 * 16;
  w.counters = kWsHeader + kCounterArea;
  w.xt = kWsHeader + 2 * kCounterArea + kSlotArea;
  w.partials = w.xt + round_up((size_t)mpad * n * 4, kAlign);
  w.total = w.partials + (splits > 1 ? round_up((size_t)splits * M * m * 4, kAlign) : 0);
  return w;
}

struct GroupedWs {
  int max_m, max_n, splits;
  size_t counters, slots, total;
};

int32_t grouped_geometry(const tg_layer* layers, int32_t n_layers, int32_t n_sel, GroupedWs* g) {
  if (!layers) return TG_ERR_NULL;
  if (n_layers <= 0 || n_sel <= 0 || n_sel > 65536) return TG_ERR_ARG;
  int max_m = 0, max_n = 0, flags = layers[0].flags;
  for (int i = 0; i < n_layers; ++i) {
    const int32_t st = check_layer(&layers[i]);
    if (st != TG_OK) return st;
    if (layers[i].flags != flags || layers[i].splits != layers[0].splits) return TG_ERR_ARG;
    if ((layers[i].flags & TG_FLAG_INT8_ACT) != 0) return TG_ERR_ARG;   // batch-1 and fused paths only
    if (layers[i].m > max_m) max_m = layers[i].m;
    if (layers[i].n > max_n) max_n = layers[i].n;
  }
  const int max_ob = max_m / kBlock, max_nb = max_n / kBlock;
  if ((int64_t)n_sel * max_ob * max_nb > INT32_MAX) return TG_ERR_SHAPE;   // the grid (splits <= max_nb) fits 31 bits
  int s = layers[0].splits;
  if (s <= 0) {
    // at most one workgroup per CU: a second round of a few workgroups costs a whole chunk's time
    const int per = n_sel * max_ob;
    s = split_for_target(max_nb, per >= 256 ? 1 : 256 / per);
    while (s > 1 && (int64_t)s * per > 256) --s;
  }
  const int min_s = (max_nb + kMaxChunkBlocks - 1) / kMaxChunkBlocks;
  if (s < min_s) s = min_s;
  if (s > max_nb) s = max_nb;
  if (s < 1) s = 1;
  g->max_m = max_m;
  g->max_n = max_n;
  g->splits = s;
  g->counters = kWsHeader;
  g->slots = kWsHeader + round_up((size_t)n_sel * max_ob * 4, kAlign);
  g->total = g->slots + round_up((size_t)n_sel * s * max_m * 8, kAlign);
  return TG_OK;
}

int32_t launch_status(hipError_t e) { return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH; }

}  // namespace

TG_API int32_t tg_abi_version(void) { return TG_ABI_VERSION; }

TG_API const char* tg_build_id(void) { return TG_BUILD_ID; }

TG_API int32_t tg_workspace_status(void* ws, int32_t clear, uint32_t* status, void* stream) {
  if (!ws || !status) return TG_ERR_NULL;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess) return TG_ERR_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return TG_ERR_LAUNCH;
  *status = word;
  if (clear && word != 0u && hipMemsetAsync(ws, 0, sizeof(word), s) != hipSuccess) return TG_ERR_LAUNCH;
  return TG_OK;
}

TG_API const char* tg_status_str(int32_t status) {
  switch (status) {
    case TG_OK: return "TG_OK";
    case TG_ERR_NULL: return "TG_ERR_NULL: a required pointer is NULL";
    case TG_ERR_SHAPE: return "TG_ERR_SHAPE: shape or row count out of range";
    case TG_ERR_KBITS: return "TG_ERR_KBITS: k_bits must be 1..8";
    case TG_ERR_ALIGN: return "TG_ERR_ALIGN: pointer misaligned";
    case TG_ERR_WORKSPACE: return "TG_ERR_WORKSPACE: workspace missing or too small";
    case TG_ERR_CODE_ID: return "TG_ERR_CODE_ID: unsupported code_id";
    case TG_ERR_LAUNCH: return "TG_ERR_LAUNCH: kernel launch failed";
    case TG_ERR_ARG: return "TG_ERR_ARG: invalid argument";
    default: return "unknown tg_status";
  }
}

TG_API size_t tg_workspace_size(const tg_layer* L, int32_t M) {
  if (check_layer(L) != TG_OK || M < 1 || M > 64) return 0;
  const size_t g = gemm_ws(L->m, L->n, M, gemm_splits(L->m, L->n, M, L->k_bits, L->code_id, L->splits)).total;
  const size_t v = gemv_ws(L->m, gemv_splits(L->m, L->n, L->splits)).total;
  return v > g ? v : g;
}

TG_API int32_t trellis_gemv(const tg_layer* L, const uint16_t* x, float* y, void* ws, size_t ws_bytes,
                            void* stream) {
  int32_t st = check_layer(L);
  if (st != TG_OK) return st;
  if (!x || !y) return TG_ERR_NULL;
  if (misaligned(x, 2) || misaligned(y, 4)) return TG_ERR_ALIGN;
  const int splits = gemv_splits(L->m, L->n, L->splits);
  if (gemv_slots_overflow(L->m, splits)) return TG_ERR_SHAPE;
  const GemvWs w = gemv_ws(L->m, splits);
  if (!ws || ws_bytes < w.total) return TG_ERR_WORKSPACE;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  GemvArgs a;
  a.codes = L->codes;
  a.scales = L->scales;
  a.sign_in = L->sign_in;
  a.sign_out = L->sign_out;
  a.x = x;
  a.y = y;
  a.counters = reinterpret_cast<uint32_t*>((char*)ws + w.counters);
  a.slots = reinterpret_cast<uint64_t*>((char*)ws + w.slots);
  a.status = reinterpret_cast<uint32_t*>(ws);
  a.m = L->m;
  a.n = L->n;
  a.splits = splits;
  a.hg = nullptr;
  a.hu = nullptr;
  return launch_status(
      launch_gemv(a, L->k_bits, kernel_form(L), (L->flags & TG_FLAG_ROUND_WEIGHTS) != 0, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Batch-1 GEMV without a caller workspace (for callers that cannot allocate).
// Its split-K state lives in `scratch`, one file-scope device array per GPU:
// [header 256 B][ticket counters kNoAllocCounterBytes][slots kNoAllocSlotBytes].
// The kernels are the batch-1 ones; they get the array's device address, taken
// once per device with hipGetSymbolAddress (host code never uses the symbol
// itself). The array keeps its contents between calls; like a shared caller
// workspace, the tickets and call-tagged slots need no clearing between calls,
// only a zero start, which the set-up provides.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocCounterBytes = 64 * 1024;                 // 16384 output blocks: m <= 2^21
constexpr int kNoAllocSlotPairs = 1024;                            // (output block, split) pairs
constexpr size_t kNoAllocSlotBytes = (size_t)kNoAllocSlotPairs * kBlock * 8;   // 1 MiB
constexpr size_t kNoAllocScratchBytes = kWsHeader + kNoAllocCounterBytes + kNoAllocSlotBytes;

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;   // device -> device address of that device's `scratch`

// Device address of the current device's array; on the first call on a device
// (not allowed during stream capture) it is looked up and zero-filled.
int32_t scratch_address(hipStream_t s, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    *out = it->second;
    return TG_OK;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return TG_ERR_LAUNCH;
  if (cap != hipStreamCaptureStatusNone) return TG_ERR_ARG;   // set-up must run outside capture
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TG_ERR_LAUNCH;
  if (hipMemset(p, 0, kNoAllocScratchBytes) != hipSuccess) return TG_ERR_LAUNCH;
  if (hipDeviceSynchronize() != hipSuccess) return TG_ERR_LAUNCH;
  g_scratch[dev] = p;
  *out = p;
  return TG_OK;
}

}  // namespace

TG_API size_t tg_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

TG_API int32_t trellis_gemv_noalloc(const tg_layer* L, const uint16_t* x, float* y, void* stream) {
  int32_t st = check_layer(L);
  if (st != TG_OK) return st;
  if (!x || !y) return TG_ERR_NULL;
  if (misaligned(x, 2) || misaligned(y, 4)) return TG_ERR_ALIGN;
  const int splits = gemv_splits(L->m, L->n, L->splits);
  if (gemv_slots_overflow(L->m, splits)) return TG_ERR_SHAPE;
  if ((size_t)(L->m / kBlock) * 4 > kNoAllocCounterBytes) return TG_ERR_WORKSPACE;
  if (splits > 1 && (int64_t)splits * (L->m / kBlock) > kNoAllocSlotPairs) return TG_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void* p = nullptr;
  st = scratch_address(s, &p);
  if (st != TG_OK) return st;
  char* base = (char*)p;
  GemvArgs a;
  a.codes = L->codes;
  a.scales = L->scales;
  a.sign_in = L->sign_in;
  a.sign_out = L->sign_out;
  a.x = x;
  a.y = y;
  a.status = reinterpret_cast<uint32_t*>(base);
  a.counters = reinterpret_cast<uint32_t*>(base + kWsHeader);
  a.slots = reinterpret_cast<uint64_t*>(base + kWsHeader + kNoAllocCounterBytes);
  a.m = L->m;
  a.n = L->n;
  a.splits = splits;
  a.hg = nullptr;
  a.hu = nullptr;
  return launch_status(launch_gemv(a, L->k_bits, kernel_form(L), (L->flags & TG_FLAG_ROUND_WEIGHTS) != 0, s));
}

// ---------------------------------------------------------------------------
// Fused batch-1 GEMVs of layers that read one input vector (q/k/v, gate/up).
// ---------------------------------------------------------------------------
namespace {

constexpr int kFusedMaxN = 16384;   // two layers' x~ in LDS: 2 x n x 4 bytes

struct FusedGeom {
  int upw, grid, total_units, total_blocks, max_contrib;
  int unit0[kFusedMaxLayers], block0[kFusedMaxLayers];
  size_t counters, slots, total;
};

int32_t fused_geometry(const tg_layer* layers, int32_t n_layers, FusedGeom* g) {
  if (!layers) return TG_ERR_NULL;
  if (n_layers < 1 || n_layers > kFusedMaxLayers) return TG_ERR_ARG;
  for (int i = 0; i < n_layers; ++i) {
    const int32_t st = check_layer(&layers[i]);
    if (st != TG_OK) return st;
    if (layers[i].n != layers[0].n) return TG_ERR_SHAPE;
    if (layers[i].k_bits != layers[0].k_bits || layers[i].code_id != layers[0].code_id ||
        layers[i].flags != layers[0].flags || layers[i].splits != layers[0].splits)
      return TG_ERR_ARG;
  }
  if (layers[0].n > kFusedMaxN) return TG_ERR_SHAPE;
  const int nb = layers[0].n / kBlock, spr = (nb + 1) / 2;
  int64_t units = 0, blocks = 0, min_units = INT64_MAX;
  for (int i = 0; i < n_layers; ++i) {
    g->unit0[i] = (int)units;
    g->block0[i] = (int)blocks;
    const int64_t u = (int64_t)(layers[i].m / kBlock) * spr;
    units += u;
    blocks += layers[i].m / kBlock;
    if (u < min_units) min_units = u;
  }
  if (units > INT32_MAX / 2) return TG_ERR_SHAPE;
  // One workgroup per compute unit by default, two where each still gets at least 16 units
  // and two fit a compute unit's 160 KB of LDS: more waves per SIMD hide more of the decode's
  // dependent latency (2 x 28672 x 8192 gate/up: 70.8 against 75.0 us; the 10-unit runs of a
  // decoder layer's q/k/v lose instead: 22.9 against 21.9). The layer's splits field forces
  // another count. A run is never longer than the smallest layer, so it crosses at most one
  // layer boundary.
  const bool int8 = (layers[0].flags & TG_FLAG_INT8_ACT) != 0;
  int target = units >= (int64_t)512 * 16 && 2 * fused_lds_bytes(layers[0].n, int8) <= (size_t)160 * 1024 ? 512 : 256;
  if (layers[0].splits > 0) target = layers[0].splits;
  int upw = (int)((units + target - 1) / target);
  if (upw > min_units) upw = (int)min_units;
  if (upw < 1) upw = 1;
  g->upw = upw;
  g->total_units = (int)units;
  g->grid = (int)((units + upw - 1) / upw);
  if (g->grid > 65535 * 16) return TG_ERR_SHAPE;
  g->total_blocks = (int)blocks;
  int maxc = 1;
  for (int i = 0; i < n_layers; ++i)
    for (int ob = 0; ob < layers[i].m / kBlock; ++ob) {
      const int64_t b0 = g->unit0[i] + (int64_t)ob * spr;
      const int c = (int)((b0 + spr - 1) / upw - b0 / upw + 1);
      if (c > maxc) maxc = c;
    }
  g->max_contrib = maxc;
  g->counters = kWsHeader;
  g->slots = kWsHeader + round_up((size_t)blocks * 4, kAlign);
  g->total = g->slots + (maxc > 1 ? round_up((size_t)blocks * maxc * kBlock * 8, kAlign) : 0);
  return TG_OK;
}

}  // namespace

TG_API size_t tg_fused_workspace_size(const tg_layer* layers, int32_t n_layers) {
  FusedGeom g;
  if (fused_geometry(layers, n_layers, &g) != TG_OK) return 0;
  return g.total;
}

TG_API int32_t trellis_gemv_fused(const tg_layer* layers, int32_t n_layers, const uint16_t* x, float* const* ys,
                                  void* ws, size_t ws_bytes, void* stream) {
  FusedGeom g;
  int32_t st = fused_geometry(layers, n_layers, &g);
  if (st != TG_OK) return st;
  if (!x || !ys) return TG_ERR_NULL;
  if (misaligned(x, 2)) return TG_ERR_ALIGN;
  for (int i = 0; i < n_layers; ++i) {
    if (!ys[i]) return TG_ERR_NULL;
    if (misaligned(ys[i], 4)) return TG_ERR_ALIGN;
  }
  if (!ws || ws_bytes < g.total) return TG_ERR_WORKSPACE;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  FusedArgs a;
  for (int i = 0; i < kFusedMaxLayers; ++i) {
    const tg_layer& L = layers[i < n_layers ? i : 0];
    a.L[i].codes = L.codes;
    a.L[i].scales = L.scales;
    a.L[i].sign_in = L.sign_in;
    a.L[i].sign_out = L.sign_out;
    a.L[i].y = ys[i < n_layers ? i : 0];
    a.L[i].unit0 = i < n_layers ? g.unit0[i] : INT32_MAX;
    a.L[i].block0 = i < n_layers ? g.block0[i] : 0;
  }
  a.x = x;
  a.counters = reinterpret_cast<uint32_t*>((char*)ws + g.counters);
  a.slots = reinterpret_cast<uint64_t*>((char*)ws + g.slots);
  a.status = reinterpret_cast<uint32_t*>(ws);
  a.n_layers = n_layers;
  a.n = layers[0].n;
  a.upw = g.upw;
  a.total_units = g.total_units;
  a.max_contrib = g.max_contrib;
  return launch_status(launch_fused(a, layers[0].k_bits, kernel_form(&layers[0]),
                                    (layers[0].flags & TG_FLAG_ROUND_WEIGHTS) != 0, g.grid, (hipStream_t)stream));
}

TG_API int32_t trellis_gemm_small(const tg_layer* L, int32_t M, const uint16_t* X, int64_t ldx, float* Y,
                                  int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_layer(L);
  if (st != TG_OK) return st;
  if ((L->flags & TG_FLAG_INT8_ACT) != 0) return TG_ERR_ARG;   // batch-1 and fused paths only
  if (M < 1 || M > 64) return TG_ERR_SHAPE;
  if (!X || !Y) return TG_ERR_NULL;
  if (ldx < L->n || ldy < L->m) return TG_ERR_ARG;
  if (misaligned(X, 2) || misaligned(Y, 4)) return TG_ERR_ALIGN;
  const int splits = gemm_splits(L->m, L->n, M, L->k_bits, L->code_id, L->splits);
  const GemmWs w = gemm_ws(L->m, L->n, M, splits);
  if (!ws || ws_bytes < w.total) return TG_ERR_WORKSPACE;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  GemmArgs a;
  a.codes = L->codes;
  a.scales = L->scales;
  a.sign_out = L->sign_out;
  a.xt = reinterpret_cast<const uint32_t*>((char*)ws + w.xt);
  a.y = Y;
  a.ldy = ldy;
  a.counters = reinterpret_cast<uint32_t*>((char*)ws + w.counters);
  a.partials = reinterpret_cast<float*>((char*)ws + w.partials);
  a.m = L->m;
  a.n = L->n;
  a.M = M;
  a.mpad = (M + 15) / 16 * 16;
  a.splits = splits;
  return launch_status(launch_gemm_small(a, X, ldx, L->sign_in, L->k_bits, L->code_id,
                                         (L->flags & TG_FLAG_ROUND_WEIGHTS) != 0, (hipStream_t)stream));
}

TG_API int32_t rht_apply(int32_t n, int32_t rows, const uint16_t* in, float* out, const uint32_t* signs,
                         int32_t inverse, void* stream) {
  if (n <= 0 || n % kBlock != 0 || n > (1 << 22) || rows < 1 || rows > 65535) return TG_ERR_SHAPE;
  if (!in || !out || !signs) return TG_ERR_NULL;
  if (misaligned(in, 2) || misaligned(out, 4) || misaligned(signs, 4)) return TG_ERR_ALIGN;
  return launch_status(launch_rht(n, rows, in, out, signs, inverse != 0, (hipStream_t)stream));
}

TG_API size_t tg_grouped_workspace_size(const tg_layer* layers, int32_t n_layers, int32_t n_sel) {
  GroupedWs g;
  if (grouped_geometry(layers, n_layers, n_sel, &g) != TG_OK) return 0;
  return g.total;
}

TG_API int32_t trellis_gemv_grouped(const tg_layer* layers, const tg_layer* d_layers, int32_t n_layers,
                                    const int32_t* d_sel, int32_t n_sel, const uint16_t* X, int64_t x_stride,
                                    float* Y, int64_t y_stride, void* ws, size_t ws_bytes, void* stream) {
  GroupedWs g;
  int32_t st = grouped_geometry(layers, n_layers, n_sel, &g);
  if (st != TG_OK) return st;
  if (!d_layers || !d_sel || !X || !Y) return TG_ERR_NULL;
  if (misaligned(d_layers, 8) || misaligned(d_sel, 4) || misaligned(X, 2) || misaligned(Y, 4)) return TG_ERR_ALIGN;
  if (x_stride < 0 || (x_stride != 0 && x_stride < g.max_n) || y_stride < g.max_m) return TG_ERR_ARG;
  if (!ws || ws_bytes < g.total) return TG_ERR_WORKSPACE;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  GroupedArgs a;
  a.layers = reinterpret_cast<const LayerDev*>(d_layers);
  a.sel = d_sel;
  a.n_layers = n_layers;
  a.n_sel = n_sel;
  a.x = X;
  a.x_stride = x_stride;
  a.y = Y;
  a.y_stride = y_stride;
  a.counters = reinterpret_cast<uint32_t*>((char*)ws + g.counters);
  a.slots = reinterpret_cast<uint64_t*>((char*)ws + g.slots);
  a.status = reinterpret_cast<uint32_t*>(ws);
  a.max_m = g.max_m;
  a.splits = g.splits;
  a.round_weights = (layers[0].flags & TG_FLAG_ROUND_WEIGHTS) != 0;
  a.sel_pairs = 0;
  a.hin = nullptr;
  a.hin_stride = 0;
  return launch_status(launch_grouped(a, g.max_m / kBlock, g.max_n, (hipStream_t)stream));
}

TG_API int32_t trellis_decode(const tg_layer* L, uint16_t* w_out, void* stream) {
  if (!L) return TG_ERR_NULL;
  if (L->code_id < 0 || L->code_id > 3) return TG_ERR_CODE_ID;
  if (L->k_bits < 1 || L->k_bits > 8) return TG_ERR_KBITS;
  if (L->m <= 0 || L->n <= 0 || L->m % kTile != 0 || L->n % kTile != 0 || L->m > (1 << 22) || L->n > (1 << 22))
    return TG_ERR_SHAPE;
  if ((int64_t)L->m * L->n > kMaxDenseWeights) return TG_ERR_SHAPE;
  if (!L->codes || !w_out) return TG_ERR_NULL;
  if (misaligned(L->codes, 4) || misaligned(w_out, 2)) return TG_ERR_ALIGN;
  return launch_status(launch_decode(L->codes, w_out, L->m, L->n, L->k_bits, L->code_id, (hipStream_t)stream));
}

TG_API int32_t tg_decode_ceiling(int32_t k_bits, int32_t code_id, int32_t flags, int32_t workgroups, int32_t steps,
                                 float* out, void* stream) {
  if (code_id < 0 || code_id > 3) return TG_ERR_CODE_ID;
  if ((flags & ~TG_FLAG_INT8_ACT) != 0 || ((flags & TG_FLAG_INT8_ACT) != 0 && code_id != 2)) return TG_ERR_ARG;
  if (k_bits < 1 || k_bits > 8) return TG_ERR_KBITS;
  if (workgroups < 1 || workgroups > 65535 || steps < 1 || steps > (1 << 20)) return TG_ERR_ARG;
  if (!out) return TG_ERR_NULL;
  if (misaligned(out, 4)) return TG_ERR_ALIGN;
  const int form = (flags & TG_FLAG_INT8_ACT) != 0 ? kCodeMul1I8 : code_id;
  return launch_status(launch_decode_ceiling(k_bits, form, workgroups, steps, out, (hipStream_t)stream));
}

TG_API int32_t tg_code_table(int32_t code_id, uint16_t* out, void* stream) {
  if (code_id < 0 || code_id > 3) return TG_ERR_CODE_ID;
  if (!out) return TG_ERR_NULL;
  if (misaligned(out, 2)) return TG_ERR_ALIGN;
  return launch_status(launch_code_table(code_id, out, (hipStream_t)stream));
}

namespace {

int32_t check_encode(int32_t n_tiles, int32_t k_bits, int32_t code_id, float scale) {
  if (code_id < 0 || code_id > 3) return TG_ERR_CODE_ID;
  if (k_bits < 1 || k_bits > 8 || (code_id == 1 && k_bits > 4)) return TG_ERR_KBITS;
  if (n_tiles < 1 || n_tiles > (1 << 24)) return TG_ERR_SHAPE;
  if (!(scale > 0.f) || !(scale < 3.0e38f)) return TG_ERR_ARG;
  return TG_OK;
}

int encode_slots(int32_t n_tiles) { return n_tiles < kEncMaxSlots ? n_tiles : kEncMaxSlots; }

}  // namespace

TG_API size_t tg_encode_workspace_size(int32_t n_tiles, int32_t k_bits, int32_t code_id) {
  if (check_encode(n_tiles, k_bits, code_id, 1.f) != TG_OK) return 0;
  return round_up((size_t)encode_slots(n_tiles) * encode_ws_words_per_slot(k_bits, code_id) * 4, kAlign);
}

TG_API int32_t trellis_encode(int32_t n_tiles, int32_t k_bits, int32_t code_id, float scale, const float* targets,
                              uint32_t* codes, float* sq_err, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_encode(n_tiles, k_bits, code_id, scale);
  if (st != TG_OK) return st;
  if (!targets || !codes) return TG_ERR_NULL;
  if (misaligned(targets, 4) || misaligned(codes, 4) || misaligned(sq_err, 4)) return TG_ERR_ALIGN;
  const size_t need = tg_encode_workspace_size(n_tiles, k_bits, code_id);
  if (!ws || ws_bytes < need) return TG_ERR_WORKSPACE;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  return launch_status(launch_encode(targets, scale, n_tiles, k_bits, code_id, codes, sq_err,
                                     reinterpret_cast<uint32_t*>(ws), encode_slots(n_tiles), (hipStream_t)stream));
}

namespace {

// The prefill workspace holds the transformed input rows in 32-column slabs.
size_t prefill_ws_bytes(int n, int M) { return round_up((size_t)M * n * 2, kAlign); }

}  // namespace

TG_API size_t tg_prefill_workspace_size(const tg_layer* L, int32_t M) {
  if (check_layer(L) != TG_OK || (L->flags & TG_FLAG_INT8_ACT) != 0 || M < 1 || M > 65535) return 0;
  return prefill_ws_bytes(L->n, M);
}

TG_API int32_t trellis_gemm_prefill(const tg_layer* L, int32_t M, const uint16_t* X, int64_t ldx, float* Y,
                                    int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_layer(L);
  if (st != TG_OK) return st;
  if ((L->flags & TG_FLAG_INT8_ACT) != 0) return TG_ERR_ARG;   // batch-1 and fused paths only
  if (M < 1 || M > 65535) return TG_ERR_SHAPE;
  if (!X || !Y) return TG_ERR_NULL;
  if (ldx < L->n || ldy < L->m) return TG_ERR_ARG;
  if (misaligned(X, 2) || misaligned(Y, 4)) return TG_ERR_ALIGN;
  if (!ws || ws_bytes < prefill_ws_bytes(L->n, M)) return TG_ERR_WORKSPACE;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint16_t* Xt = reinterpret_cast<uint16_t*>(ws);
  if (launch_prefill_rht(X, ldx, L->sign_in, Xt, L->n, M, s) != hipSuccess) return TG_ERR_LAUNCH;
  return launch_status(launch_prefill_mfma(L->codes, L->scales, L->sign_out, Xt, Y, ldy, L->m, L->n, M, L->k_bits,
                                           L->code_id, s));
}

namespace {

struct MoeWs {
  GroupedWs gu, dn;
  int inter, hidden;
  size_t gu_off, dn_off, y1, y2, total;
};

// Gate/up table: entry 2e = gate of expert e, 2e+1 = up (inter x hidden); down table:
// entry e (hidden x inter). All experts share inter and hidden and the flags.
int32_t moe_geometry(const tg_layer* gu, int32_t n_gu, const tg_layer* dn, int32_t n_dn, int32_t top_k, MoeWs* w) {
  if (!gu || !dn) return TG_ERR_NULL;
  if (n_dn < 1 || n_gu != 2 * n_dn || top_k < 1 || top_k > n_dn || top_k > 256) return TG_ERR_ARG;
  int32_t st = grouped_geometry(gu, n_gu, 2 * top_k, &w->gu);
  if (st != TG_OK) return st;
  st = grouped_geometry(dn, n_dn, top_k, &w->dn);
  if (st != TG_OK) return st;
  w->inter = gu[0].m;
  w->hidden = gu[0].n;
  for (int i = 0; i < n_gu; ++i)
    if (gu[i].m != w->inter || gu[i].n != w->hidden) return TG_ERR_SHAPE;
  for (int i = 0; i < n_dn; ++i)
    if (dn[i].m != w->hidden || dn[i].n != w->inter) return TG_ERR_SHAPE;
  if (gu[0].flags != dn[0].flags || gu[0].splits != dn[0].splits) return TG_ERR_ARG;
  w->gu_off = 0;
  w->dn_off = round_up(w->gu.total, kAlign);
  w->y1 = w->dn_off + round_up(w->dn.total, kAlign);
  w->y2 = w->y1 + round_up((size_t)2 * top_k * w->inter * 4, kAlign);
  w->total = w->y2 + round_up((size_t)top_k * w->hidden * 4, kAlign);
  return TG_OK;
}

GroupedArgs grouped_args(const tg_layer* d_layers, int32_t n_layers, const int32_t* d_sel, int32_t n_sel,
                         const GroupedWs& g, char* ws, float* y, int64_t y_stride, bool round, uint32_t* status) {
  GroupedArgs a;
  a.layers = reinterpret_cast<const LayerDev*>(d_layers);
  a.sel = d_sel;
  a.n_layers = n_layers;
  a.n_sel = n_sel;
  a.x = nullptr;
  a.x_stride = 0;
  a.y = y;
  a.y_stride = y_stride;
  a.counters = reinterpret_cast<uint32_t*>(ws + g.counters);
  a.slots = reinterpret_cast<uint64_t*>(ws + g.slots);
  a.status = status;
  a.max_m = g.max_m;
  a.splits = g.splits;
  a.round_weights = round ? 1 : 0;
  a.sel_pairs = 0;
  a.hin = nullptr;
  a.hin_stride = 0;
  return a;
}

}  // namespace

TG_API size_t tg_moe_workspace_size(const tg_layer* gate_up, int32_t n_gate_up, const tg_layer* down, int32_t n_down,
                                    int32_t top_k) {
  MoeWs w;
  if (moe_geometry(gate_up, n_gate_up, down, n_down, top_k, &w) != TG_OK) return 0;
  return w.total;
}

TG_API int32_t trellis_moe_block(const tg_layer* gate_up, const tg_layer* d_gate_up, int32_t n_gate_up,
                                 const tg_layer* down, const tg_layer* d_down, int32_t n_down, const int32_t* d_sel,
                                 const float* d_weights, int32_t top_k, const uint16_t* x, float* y, void* ws,
                                 size_t ws_bytes, void* stream) {
  MoeWs w;
  int32_t st = moe_geometry(gate_up, n_gate_up, down, n_down, top_k, &w);
  if (st != TG_OK) return st;
  if (!d_gate_up || !d_down || !d_sel || !d_weights || !x || !y) return TG_ERR_NULL;
  if (misaligned(d_gate_up, 8) || misaligned(d_down, 8) || misaligned(d_sel, 4) || misaligned(d_weights, 4) ||
      misaligned(x, 2) || misaligned(y, 4))
    return TG_ERR_ALIGN;
  if (!ws || ws_bytes < w.total) return TG_ERR_WORKSPACE;
  if (misaligned(ws, kAlign)) return TG_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  float* Y1 = reinterpret_cast<float*>(base + w.y1);   // [2 top_k][inter]: gate, up rows per selection
  float* Y2 = reinterpret_cast<float*>(base + w.y2);   // [top_k][hidden]
  const bool round = (gate_up[0].flags & TG_FLAG_ROUND_WEIGHTS) != 0;
  uint32_t* status = reinterpret_cast<uint32_t*>(base);   // the first region's header
  GroupedArgs g1 = grouped_args(d_gate_up, n_gate_up, d_sel, 2 * top_k, w.gu, base + w.gu_off, Y1, w.inter, round,
                                status);
  g1.x = x;
  g1.sel_pairs = 1;
  if (launch_grouped(g1, w.gu.max_m / kBlock, w.gu.max_n, s) != hipSuccess) return TG_ERR_LAUNCH;
  GroupedArgs g2 = grouped_args(d_down, n_down, d_sel, top_k, w.dn, base + w.dn_off, Y2, w.hidden, round, status);
  g2.hin = Y1;
  g2.hin_stride = w.inter;
  if (launch_grouped(g2, w.dn.max_m / kBlock, w.dn.max_n, s) != hipSuccess) return TG_ERR_LAUNCH;
  return launch_status(launch_moe_combine(Y2, w.hidden, d_sel, d_weights, top_k, n_down, w.hidden, y, s));
}
