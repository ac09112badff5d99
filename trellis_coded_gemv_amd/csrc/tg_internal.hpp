// Host-side declarations shared by the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tg {

constexpr int kTile = 16;
constexpr int kBlock = 128;              // Hadamard block; 8 tile rows / 8 tile columns
constexpr int kGemvWaves = 8;            // one wave per tile row of a 128-output block (MFMA path)
constexpr int kGemvThreads = 64 * kGemvWaves;
#ifndef TG_GEMV_P
#define TG_GEMV_P 1
#endif
constexpr int kGemvP = TG_GEMV_P;        // batch-1 path: waves per tile row (interleaved steps)
// Kernel forms of the codes: code_id 0, 1 and 3 (MCG) as they are; code_id 2
// (mul1) against fp32 x~, and against the int8 form of x~ (TG_FLAG_INT8_ACT).
constexpr int kCodeMul1 = 2;
constexpr int kCodeMcg = 3;
constexpr int kCodeMul1I8 = 4;
// Codes whose weight is the sum of two binary16 halves, dotted against (x~, x~) pairs.
constexpr bool halves_form(int code) { return code == 0 || code == kCodeMcg; }
// Codes whose weights involve a rounding (mul1's are exact): they also have the TG_FLAG_ROUND_WEIGHTS form.
constexpr bool rounded_form(int code) { return code == 0 || code == 1 || code == kCodeMcg; }
constexpr int kMaxChunkBlocks = 64;      // 128-blocks of x~ held in LDS by one GEMV workgroup
constexpr size_t kWsHeader = 256;        // every workspace starts with this header; word 0 = status
constexpr uint32_t kStatusSplitkTimeout = 1u;   // a split-K wait ran out (its outputs were written as NaN)

// One batch-1 GEMV as a workgroup sees it.
struct GemvArgs {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* sign_in;
  const uint32_t* sign_out;
  const uint16_t* x;
  float* y;
  uint64_t* slots;      // [m/128][splits][128] call-tagged split-K slots (unused when splits == 1)
  uint32_t* counters;   // [m/128] ticket counters, on a call boundary (multiple of 2^16) between calls
  uint32_t* status;     // the workspace's status word (sticky error bits)
  int32_t m, n, splits;
  const float* hg;      // gated-MLP input mode: x = fp16(silu(hg) * hu), fp32 rows of n values
  const float* hu;
};

// Grouped batch-1 GEMVs: the layer table lives in device memory.
struct LayerDev {          // mirrors tg_layer
  int32_t m, n, k_bits, code_id, flags, splits;
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* sign_in;
  const uint32_t* sign_out;
};

struct GroupedArgs {
  const LayerDev* layers;
  const int32_t* sel;
  int32_t n_layers, n_sel;
  const uint16_t* x;
  int64_t x_stride;
  float* y;
  int64_t y_stride;
  uint64_t* slots;      // per selection [max_m/128][splits][128] call-tagged split-K slots
  uint32_t* counters;   // [n_sel][max_m/128] ticket counters
  uint32_t* status;     // the workspace's status word
  int32_t max_m, splits, round_weights;
  int32_t sel_pairs;    // 1: selection e uses layer 2*sel[e/2] + e%2 (gate and up of the selected experts)
  const float* hin;     // non-null: selection e's input is fp16(silu(hin row 2e) * hin row 2e+1)
  int64_t hin_stride;   // floats between hin rows
};

// Fused batch-1 GEMVs of several layers that read one input vector (fused.hip).
constexpr int kFusedMaxLayers = 8;
struct FusedLayer {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* sign_in;
  const uint32_t* sign_out;
  float* y;
  int32_t unit0;        // first unit of this layer in the launch's unit order
  int32_t block0;       // first output block of this layer among all layers' blocks
};

struct FusedArgs {
  FusedLayer L[kFusedMaxLayers];
  const uint16_t* x;
  uint32_t* counters;   // [all layers' output blocks] ticket counters
  uint64_t* slots;      // [all blocks][max_contrib][128] call-tagged partials
  uint32_t* status;
  int32_t n_layers, n, upw, total_units, max_contrib;
};

// Small-batch MFMA path.
struct GemmArgs {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* sign_out;
  const uint32_t* xt;   // [mpad][n] (code 0) or [mpad][n/2] (code 1) fp16 pair words from the input transform
  float* y;
  int64_t ldy;
  float* partials;      // [splits][M][m]
  uint32_t* counters;   // [m/128]
  int32_t m, n, M, mpad, splits;
};

hipError_t launch_gemv(const GemvArgs& a, int k_bits, int code_id, bool round_weights, hipStream_t s);
hipError_t launch_grouped(const GroupedArgs& a, int max_ob, int max_n, hipStream_t s);
hipError_t launch_fused(const FusedArgs& a, int k_bits, int code_id, bool round_weights, int grid, hipStream_t s);
size_t fused_lds_bytes(int n, bool int8);
hipError_t launch_decode_ceiling(int k_bits, int code_id, int workgroups, int steps, float* out, hipStream_t s);
hipError_t launch_moe_combine(const float* Y2, int64_t y2_stride, const int32_t* sel, const float* w, int top_k,
                              int n_experts, int hidden, float* y, hipStream_t s);
hipError_t launch_gemm_small(const GemmArgs& a, const uint16_t* X, int64_t ldx, const uint32_t* sign_in,
                             int k_bits, int code_id, bool round_weights, hipStream_t s);
hipError_t launch_rht(int n, int rows, const uint16_t* in, float* out, const uint32_t* signs, bool inverse,
                      hipStream_t s);
hipError_t launch_decode(const uint32_t* codes, uint16_t* out, int m, int n, int k_bits, int code_id, hipStream_t s);
hipError_t launch_code_table(int code_id, uint16_t* out, hipStream_t s);
hipError_t launch_encode(const float* targets, float alpha, int n_tiles, int k_bits, int code_id, uint32_t* codes,
                         float* sq_err, uint32_t* ws, int slots, hipStream_t s);
size_t encode_ws_words_per_slot(int k_bits, int code_id);
hipError_t launch_prefill_rht(const uint16_t* X, int64_t ldx, const uint32_t* sign_in, uint16_t* Xt, int n, int M,
                              hipStream_t s);
hipError_t launch_prefill_mfma(const uint32_t* codes, const uint16_t* scales, const uint32_t* sign_out,
                               const uint16_t* Xt, float* Y, int64_t ldy, int m, int n, int M, int k_bits, int code_id,
                               hipStream_t s);
constexpr int kEncMaxSlots = 256;        // encoder workgroups in flight (one tile each at a time)

// LDS bytes a GEMV workgroup needs for a chunk of `chunk_blocks` 128-blocks.
// The x~ region doubles as [8P][128] fp32 per-wave sums in the final reduction.
// int8: the int8 form's bias (8 words) and factor (1 word) per block follow.
inline size_t gemv_lds_bytes(int chunk_blocks, bool int8 = false) {
  int padded_blocks = (chunk_blocks + 1) & ~1;   // steps cover 2 blocks
  if (padded_blocks < 8 * kGemvP) padded_blocks = 8 * kGemvP;
  return (size_t)padded_blocks * kBlock * 4 + (size_t)kBlock * 4 * kGemvP + 16 +
         (int8 ? (size_t)padded_blocks * 9 * 4 : 0);
}

}  // namespace tg
