/*
 * trellis_gemv.h -- C ABI of the MI355X (gfx950) trellis-coded GEMV library.
 *
 * A linear layer y = W x is stored the QTIP / EXL3 way:
 *   - W is rotated on both sides by randomized 128-point Hadamard blocks
 *     ("ExLlamaV3 & EXL3 Deep Dive", Section 2, the two incoherence
 *     equations; "Trellis Quantization" lecture, Part eleven: EXL3 rotates
 *     blocks of 128 along each axis);
 *   - the rotated matrix is cut into 16x16 tiles, each one tail-biting
 *     bitshift-trellis sequence of 256 weights at K bits per weight, a 16-bit
 *     state window sliding K bits per weight (lecture, Part eight; Deep Dive,
 *     Section 3, transition equation);
 *   - each weight is rebuilt from its state by a computed code: a 32-bit
 *     multiply-add, a mask/XOR to two fp16 halves, their fp16 sum (lecture,
 *     Part nine, three-instruction code);
 *   - a per-output fp16 scale ("out_scales", LLM Cal EXL3 field guide).
 *
 * At run time the library computes
 *     x~ = blockdiag(H) diag(s_in) x,   y~ = diag(g) W^ x~,   y = diag(s_out) blockdiag(H) y~
 * with H the normalised 128x128 Sylvester-Hadamard matrix, entirely in HIP
 * kernels on the caller's stream.
 *
 * Storage format (code_id 0):
 *   codes   : uint32, (m/16)*(n/16) tiles in tile-row-major order (tile (R,C) is
 *             tile R*(n/16)+C), 8*K words per tile. Stream bit p of a tile is bit
 *             31-(p%32) of word p/32. Weight (16R+r, 16C+c) is sequence step
 *             t = 16r+c; its state is the 16 stream bits starting at bit K*t,
 *             taken cyclically (tail-biting), first bit most significant.
 *   code    : h = (0x9E3779*S + 0x7F4A7C15) mod 2^32; u = (h & 0x8FFF8FFF) ^ 0x30003000;
 *             w = fp16_rne(half(u[15:0]) + half(u[31:16])).
 *
 * Storage format (code_id 1, the pair code): as code_id 0, except that one
 *   trellis step carries two weights (Deep Dive, Section 3: b*V bits per
 *   V-dimensional step, here V = 2): weights t = 2*tau and 2*tau+1 of a tile
 *   (the same row, columns 2j and 2j+1) share the state whose 16-bit window
 *   starts at stream bit 2*K*tau, taken cyclically. With a = half(u[15:0]),
 *   b = half(u[31:16]) of the same u as above, w_{2 tau} = fp16_rne(a + b) and
 *   w_{2 tau + 1} = fp16_rne(b - a). Each weight is again a sum of two bounded
 *   halves (lecture, Part nine); the pair costs one code evaluation, so the
 *   decode work per weight is about half that of code_id 0.
 *
 * Storage format (code_id 2, "mul1", the EXL3 converter's default codebook;
 *   lecture, Part eleven: the MCG generator drops the additive constant, mul1
 *   sums the product's bytes with one four-byte dot product; Part twelve: each
 *   byte masked to six bits, the sum offset to about -126..126; LLM Cal field
 *   guide, "What the EXL3 converter actually sets"): stream layout as code_id 0,
 *   one state per weight, and
 *     h = 0x9E3779*S mod 2^32;  m = h & 0x3F3F3F3F;
 *     level = (sum of the four bytes of m) - 126;  w = level / 32 (exact in fp16).
 *   The pages fix none of these constants; these are this library's.
 *   With TG_FLAG_INT8_ACT the batch-1 and fused paths multiply by an int8 form
 *   of x~ instead (lecture, Part eleven: with int8 activations the decode and
 *   the multiply are one four-byte dot product), defined per 128-block b as
 *     u = blockdiag(+-1 Hadamard) diag(s_in) x  (exact: computed in float64),
 *     e_b = the smallest integer with max_b |u| * 2^-e_b <= 127 (0 if all zero),
 *     q = round-half-even(u * 2^-e_b),   x~ replaced by q * 2^e_b / sqrt(128).
 *   The integer products are exact; only the per-block fp32 scaling rounds.
 *
 * Storage format (code_id 3, "MCG", one of the EXL3 converter's codebooks;
 *   lecture, Part eleven: the three-instruction code's generator with the
 *   additive constant dropped; LLM Cal field guide, "What the EXL3 converter
 *   actually sets"): as code_id 0 with
 *     h = 0x9E3779*S mod 2^32;  u = (h & 0x8FFF8FFF) ^ 0x30003000;
 *     w = fp16_rne(half(u[15:0]) + half(u[31:16])).
 *   The pages print no multiplier for it; this is code_id 0's.
 *
 *   scales  : m fp16 bit patterns (g).
 *   sign_in : ceil(n/32) uint32 words; bit i%32 of word i/32 set means s_in[i] = -1.
 *   sign_out: ceil(m/32) uint32 words, same convention.
 *
 * Conventions for every entry point:
 *   - Pointers named d_* or documented "device" are device pointers (hipMalloc
 *     or any allocator of device memory); the tg_layer struct itself is read on
 *     the host. The caller owns every buffer; the library never allocates,
 *     frees, or keeps a pointer after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; the library never synchronises (except
 *     tg_workspace_status, which has to wait for the word it reads).
 *   - Every argument is validated on the host before anything is enqueued; on
 *     error a negative tg_status is returned and nothing is enqueued. A failed
 *     launch returns TG_ERR_LAUNCH. No exception crosses the ABI.
 *   - Outputs must not alias inputs or the workspace.
 *   - Results are bitwise deterministic for identical inputs and launch
 *     configuration.
 *   - Calls that share a workspace must not run concurrently.
 *   - The workspaces of trellis_gemv, trellis_gemv_fused, trellis_gemm_small,
 *     trellis_gemv_grouped and trellis_moe_block start with a 256-byte header whose first 32-bit
 *     word is the status word: sticky TG_STATUS_* bits the kernels set and
 *     tg_workspace_status() reads (zero-filling a workspace clears it).
 *   - The library reads no environment variables; the only tuning input is a
 *     layer's `splits` field, which the workspace-size queries see as well.
 */
#ifndef TRELLIS_GEMV_H
#define TRELLIS_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_ABI_VERSION 4

typedef enum tg_status {
  TG_OK = 0,
  TG_ERR_NULL = -1,       /* a required pointer is NULL                               */
  TG_ERR_SHAPE = -2,      /* m, n not positive multiples of 128, or M / rows out of range */
  TG_ERR_KBITS = -3,      /* k_bits outside 1..8                                      */
  TG_ERR_ALIGN = -4,      /* a pointer is not aligned as documented                   */
  TG_ERR_WORKSPACE = -5,  /* workspace missing or smaller than tg_workspace_size()     */
  TG_ERR_CODE_ID = -6,    /* code_id other than 0, 1, 2 or 3                          */
  TG_ERR_LAUNCH = -7,     /* the HIP runtime rejected a kernel launch                 */
  TG_ERR_ARG = -8         /* any other invalid argument (stride, flags, index range)   */
} tg_status;

/* Status word bits (sticky; see tg_workspace_status). */
#define TG_STATUS_SPLITK_TIMEOUT 1u  /* a split-K reducer's bounded wait (about a second) ran out;
                                        the outputs of that block were written as NaN */

/* Layer flags. */
#define TG_FLAG_ROUND_WEIGHTS 1  /* GEMV paths round each weight to fp16 before the product
                                    (the default adds the two fp16 halves inside the fp32
                                    product, which is exact up to fp32 rounding). No effect
                                    with code_id 2, whose weights are exact. */
#define TG_FLAG_INT8_ACT 2       /* code_id 2 only (else TG_ERR_ARG): trellis_gemv,
                                    trellis_gemv_noalloc and trellis_gemv_fused multiply by
                                    the int8 form of x~ defined above; the small-batch,
                                    prefill, grouped and mixture-of-experts paths refuse it
                                    (TG_ERR_ARG). */

/* One trellis-coded linear layer: out_features m, in_features n. Read on the host. */
typedef struct tg_layer {
  int32_t m;                 /* out_features, multiple of 128                              */
  int32_t n;                 /* in_features, multiple of 128                               */
  int32_t k_bits;            /* bits per weight K, 1..8 (lecture, Part eleven)              */
  int32_t code_id;           /* 0 = three-instruction code; 1 = pair code; 2 = mul1; 3 = MCG */
  int32_t flags;             /* TG_FLAG_*                                                  */
  int32_t splits;            /* input chunks (split-K) of the batch-1, grouped and          *
                              * small-batch paths: 0 = the library's choice; S > 0 forces  *
                              * S (a tuning aid; clamped to what the path supports); at   *
                              * most 65535. Layers of one grouped table share it.          */
  const uint32_t *codes;     /* device, (m/16)*(n/16)*8*K words, 16-byte aligned            */
  const uint16_t *scales;    /* device, m fp16 patterns, 2-byte aligned                     */
  const uint32_t *sign_in;   /* device, ceil(n/32) words                                   */
  const uint32_t *sign_out;  /* device, ceil(m/32) words                                   */
} tg_layer;

/* ABI version of the loaded library (TG_ABI_VERSION it was built with). */
int32_t tg_abi_version(void);

/* Identifier of the sources the library was built from (a hash of its HIP sources and this
 * header, set at build time), so a binding can refuse a library older than its sources. */
const char *tg_build_id(void);

/*
 * Read a workspace's status word (TG_STATUS_* bits set by kernels that used it since it
 * was last cleared): enqueues a 4-byte device-to-host copy on `stream` and waits for the
 * stream, so every call enqueued before it has finished. clear != 0 then enqueues a reset
 * of the word to zero (only when it was non-zero). Not for use inside graph capture.
 *   ws     : device workspace of trellis_gemv, trellis_gemv_fused, trellis_gemm_small,
 *            trellis_gemv_grouped or trellis_moe_block, 256-byte aligned.
 *   status : host, receives the word.
 * Returns TG_OK, or TG_ERR_LAUNCH if the runtime reports an error.
 */
int32_t tg_workspace_status(void *ws, int32_t clear, uint32_t *status, void *stream);

/* Human-readable name of a status code. Never NULL. */
const char *tg_status_str(int32_t status);

/*
 * Workspace bytes needed by trellis_gemv (M == 1) or trellis_gemm_small
 * (1 <= M <= 64) for this layer, or 0 if the layer / M is invalid.
 * Layout, at the same offsets for every layer: the 256-byte header, two counter areas (256 KiB in
 * all: the batch-1 tickets and the small-batch arrival counters, each sized
 * for the largest layer), the batch-1 split-K slots (2 MiB), then the
 * small-batch scratch (input transform, split-K partials). It must be
 * zero-filled before its first use. Every completed call leaves the
 * small-batch counters at zero and each batch-1 ticket counter on a call
 * boundary (a multiple of 65536: the counter advances by 65536 per call).
 * A batch-1 slot carries the number of its call on its output block and the
 * layer's split count, so slots are never cleared: a slot left by another
 * layer or an earlier call is never taken for this call's partial, unless
 * 65535 or more calls with other split counts ran on that output block since
 * the last call with this split count. The small-batch scratch may hold
 * anything between calls. One buffer, as large as each layer needs, can
 * therefore serve any sequence of layers and of both entry points on one
 * stream. 256-byte alignment is required.
 */
size_t tg_workspace_size(const tg_layer *layer, int32_t M);

/*
 * Batch-1 trellis-coded GEMV: y = W x (the hot path; lecture, Parts eight,
 * nine and eleven; Deep Dive, Section 2).
 *   x  : device, n fp16 patterns.
 *   y  : device, m fp32 outputs, 4-byte aligned.
 *   ws : device workspace of ws_bytes >= tg_workspace_size(layer, 1).
 * With split-K, the workgroups of an output block hand their partial sums to
 * one of them through the workspace; its wait for them is bounded (about a
 * second) and, should the device ever stall a workgroup that long, the
 * affected outputs are written as NaN (the workspace stays usable: a late
 * partial carries its own call's tag). A layer whose input must be cut into
 * more chunks than the slot area holds ((m/128) * chunks > 2048; some 2^31
 * weights and more, since a chunk spans at most 8192 inputs) returns
 * TG_ERR_SHAPE.
 */
int32_t trellis_gemv(const tg_layer *layer, const uint16_t *x, float *y,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * trellis_gemv for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation
 * and kernels, with the split-K state (ticket counters and slots) in a
 * file-scope device array of the library instead of a caller workspace. No
 * memory is allocated or freed by this call.
 *   x, y  : as for trellis_gemv.
 * Limits: the array holds tg_noalloc_scratch_bytes() bytes (about 1.1 MiB): at
 * most 16384 output blocks (m <= 2^21) and at most 1024 (output block, input
 * chunk) pairs (m/128 times the layer's split count); a layer beyond either
 * returns TG_ERR_WORKSPACE with nothing enqueued.
 * Each GPU holds its own copy of the array until the process ends; every call
 * on that GPU shares it, and it keeps the last call's state (which, as in a
 * shared caller workspace, needs no clearing between calls). Calls that overlap
 * on one GPU (concurrent streams or threads) race on it and must not happen.
 * The first call on a device looks the array up and zero-fills it, waiting
 * for the device; it must not be made while a stream is being captured
 * (TG_ERR_ARG then). Later calls enqueue one kernel launch and may be captured.
 * The status word (TG_STATUS_*) is the array's first word; it is not readable
 * through tg_workspace_status.
 */
int32_t trellis_gemv_noalloc(const tg_layer *layer, const uint16_t *x, float *y, void *stream);

/* Size in bytes of trellis_gemv_noalloc's per-device array. */
size_t tg_noalloc_scratch_bytes(void);

/*
 * Several batch-1 GEMVs that read the same input vector x -- a decoder layer's
 * q, k and v projections, or its gate and up projections -- in one launch:
 * y_l = W_l x for l < n_layers (the same computation as trellis_gemv, per
 * layer; lecture, Parts eight, nine and eleven; Deep Dive, Section 2). The
 * layers' work is cut into units of 16 tiles of one 128-output block and split
 * evenly over the launch's workgroups (about one per compute unit), so small
 * layers cost no launch of their own and no compute unit idles; blocks shared
 * by several workgroups are summed in a fixed order, so results are bitwise
 * deterministic.
 *   layers   : host array of 1..8 layer descriptors with equal n (<= 16384),
 *              k_bits, code_id, flags and splits (each layer keeps its own
 *              codes, scales and sign vectors); splits > 0 forces the number
 *              of workgroups (a tuning aid).
 *   x        : device, n fp16 patterns, shared by all layers.
 *   ys       : host array of n_layers device pointers; ys[l] receives m_l fp32.
 *   ws       : device workspace, ws_bytes >= tg_fused_workspace_size(layers,
 *              n_layers), 256-byte aligned, zero-filled before its first use;
 *              every call leaves its ticket counters on a call boundary. Calls
 *              that share it must be ordered (one stream), and a workspace used
 *              before with other layer shapes or another count must be
 *              zero-filled again.
 */
int32_t trellis_gemv_fused(const tg_layer *layers, int32_t n_layers, const uint16_t *x, float *const *ys,
                           void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for trellis_gemv_fused over these layers (0 if invalid). */
size_t tg_fused_workspace_size(const tg_layer *layers, int32_t n_layers);

/*
 * Small-batch trellis-coded GEMM on the matrix cores: Y[r] = W X[r] for
 * r < M, 1 <= M <= 64. Each decoded 16x16 tile feeds an fp32-accumulating
 * MFMA (lecture, Part eight: the 16x16 tile matches the matrix-multiply tile;
 * Part eleven: decoding happens in registers feeding the matrix units).
 *   X   : device, M rows of n fp16 patterns, row stride ldx >= n elements.
 *   Y   : device, M rows of m fp32, row stride ldy >= m elements.
 *   ws  : device workspace of ws_bytes >= tg_workspace_size(layer, M).
 */
int32_t trellis_gemm_small(const tg_layer *layer, int32_t M,
                           const uint16_t *X, int64_t ldx, float *Y, int64_t ldy,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Prefill / large batch: Y[r] = W X[r] for r < M, 1 <= M <= 65535, on the
 * matrix cores. Every weight is decoded once per 512 rows (lecture, Part
 * eleven: the prefill side of the bill, decoding amortised over the batch;
 * Part fourteen), straight into the MFMA operands in registers and LDS -- the
 * decoded weights never reach memory -- and multiplied with fp16 x~ rows, fp32
 * accumulation; the output transform runs in the same kernel. This path always
 * multiplies the fp16-rounded weights (TG_FLAG_ROUND_WEIGHTS has no further
 * effect here); TG_FLAG_INT8_ACT is refused (TG_ERR_ARG).
 *   X, ldx, Y, ldy : as for trellis_gemm_small.
 *   ws : device workspace of ws_bytes >= tg_prefill_workspace_size(layer, M):
 *        M*n*2 bytes of transformed inputs (no zero-fill needed).
 * Each output is summed by one wave in a fixed order: results are bitwise
 * deterministic.
 */
int32_t trellis_gemm_prefill(const tg_layer *layer, int32_t M,
                             const uint16_t *X, int64_t ldx, float *Y, int64_t ldy,
                             void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for trellis_gemm_prefill (0 if the layer / M is invalid). */
size_t tg_prefill_workspace_size(const tg_layer *layer, int32_t M);

/*
 * Randomized Hadamard transform on 128-blocks of `rows` rows of n values
 * (Deep Dive, Section 2; lecture, Part eleven):
 *   inverse == 0: out = blockdiag(H) diag(s) in      (input side)
 *   inverse != 0: out = diag(s) blockdiag(H) in      (output side)
 *   in    : device, rows*n fp16 patterns, contiguous rows.
 *   out   : device, rows*n fp32, contiguous rows.
 *   signs : device, ceil(n/32) words.
 * n must be a positive multiple of 128; 1 <= rows <= 65535.
 */
int32_t rht_apply(int32_t n, int32_t rows, const uint16_t *in, float *out,
                  const uint32_t *signs, int32_t inverse, void *stream);

/*
 * Grouped batch-1 GEMVs over layers selected at run time on the device (the
 * mixture-of-experts case: per token a few experts out of many, each tensor
 * with its own K; Deep Dive, Section 4 and lecture, Part eleven on per-tensor
 * bit widths).
 *   layers    : host array of n_layers descriptors (validated on the host).
 *   d_layers  : device array holding the same n_layers descriptors.
 *   d_sel     : device, n_sel int32 indices into the layer array (each < n_layers).
 *   X         : device fp16 inputs; selection e reads X + e*x_stride
 *               (x_stride == 0: all selections share one input vector).
 *   Y         : device fp32 outputs; selection e writes Y + e*y_stride.
 *   ws        : device workspace, ws_bytes >= tg_grouped_workspace_size(...),
 *               zero-filled before its first use; every call leaves its ticket
 *               counters on a call boundary (as for trellis_gemv), and calls
 *               that share it must be ordered (one stream). After the 256-byte
 *               header, n_sel * (largest m / 128) words are ticket counters and
 *               the split-K slots follow, so a workspace used before with another
 *               n_sel or largest m must be zero-filled again (one geometry's slots
 *               lie where another keeps its counters).
 * Every layer's n must fit the input stride (n <= x_stride when x_stride != 0)
 * and m <= y_stride. Indices in d_sel outside [0, n_layers) make the affected
 * selection write nothing. n_sel * (max m / 128) * (max n / 128) must stay
 * below 2^31 (TG_ERR_SHAPE otherwise). The launch's split count S comes from
 * the widest layer of the table (or the layers' common `splits` field); a
 * selected layer with fewer than S 128-blocks of input runs one chunk per block.
 */
int32_t trellis_gemv_grouped(const tg_layer *layers, const tg_layer *d_layers, int32_t n_layers,
                             const int32_t *d_sel, int32_t n_sel,
                             const uint16_t *X, int64_t x_stride, float *Y, int64_t y_stride,
                             void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for trellis_gemv_grouped over these layers and n_sel selections (0 if invalid). */
size_t tg_grouped_workspace_size(const tg_layer *layers, int32_t n_layers, int32_t n_sel);

/*
 * Mixture-of-experts block for one token over trellis-coded experts (Deep Dive,
 * Section 4 and lecture, Part eleven: expert models, per-tensor bit widths):
 *     y = sum_i w_i * down_{e_i}( fp16( silu(gate_{e_i}(x)) * up_{e_i}(x) ) ),
 * silu(v) = v / (1 + exp(-v)), over the top_k selected experts e_i. Three
 * launches: the 2*top_k gate/up GEMVs (one grouped launch, shared x), the
 * top_k down GEMVs whose input transform forms fp16(silu(g)*u) from the first
 * launch's fp32 rows, and the router-weighted sum in selection order.
 *   gate_up / d_gate_up : host / device tables of n_gate_up = 2*n_down layers;
 *                         entry 2e = gate and 2e+1 = up of expert e, each
 *                         inter x hidden (out x in); all of one shape.
 *   down / d_down       : host / device tables of n_down layers, hidden x inter.
 *   d_sel               : device, top_k int32 expert ids (1 <= top_k <= min(n_down, 256));
 *                         ids outside [0, n_down) contribute nothing.
 *   d_weights           : device, top_k fp32 router weights.
 *   x                   : device, hidden fp16; y : device, hidden fp32.
 *   ws                  : device workspace, ws_bytes >= tg_moe_workspace_size(...),
 *                         256-byte aligned and zero-filled before its first use. Every
 *                         call leaves its ticket counters on a call boundary; the rest holds
 *                         the call's intermediate rows. Calls that share a workspace
 *                         must be ordered (one stream); a workspace used before with
 *                         other table shapes or another top_k must be zero-filled again
 *                         (the intermediate rows sit where another shape keeps its
 *                         split-K slots).
 * All layers must share TG_FLAG_* flags. Errors: a negative tg_status (shape, table,
 * top_k, alignment or workspace checks) with nothing launched.
 */
int32_t trellis_moe_block(const tg_layer *gate_up, const tg_layer *d_gate_up, int32_t n_gate_up,
                          const tg_layer *down, const tg_layer *d_down, int32_t n_down,
                          const int32_t *d_sel, const float *d_weights, int32_t top_k,
                          const uint16_t *x, float *y, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for trellis_moe_block (0 if the tables / top_k are invalid). */
size_t tg_moe_workspace_size(const tg_layer *gate_up, int32_t n_gate_up,
                             const tg_layer *down, int32_t n_down, int32_t top_k);

/*
 * Decode the whole layer to fp16 weights (test / export hook): w_out[o*n + i]
 * = W^[o, i] as fp16 patterns, bit-exact with the code's definition: every
 * weight's state is the 16-bit window of its tile's circular stream at bit K*t
 * (lecture, Part eight: random access into the bitshift trellis, 16x16 tiles,
 * tail-biting), put through the computed code (lecture, Part nine; code_id 1:
 * Deep Dive, Section 3, a V = 2 step per state). Only
 * codes, k_bits, code_id and shape are used; m, n need only be positive
 * multiples of 16, and m*n <= 2^38 (TG_ERR_SHAPE beyond: 512 GiB of output).
 *   w_out : device, m*n uint16.
 */
int32_t trellis_decode(const tg_layer *layer, uint16_t *w_out, void *stream);

/*
 * The whole computed code as a table (test / export hook; lecture, Part nine:
 * each state's weight is a function of the 16-bit state alone, so the code has
 * exactly 2^16 entries), for every state S < 65536:
 *   code_id 0, 2, 3: out[S] = fp16 pattern of the weight for state S  (65536 entries);
 *   code_id 1:    out[2S], out[2S+1] = the state's weight pair      (131072 entries).
 *   out : device, 2-byte aligned.
 */
int32_t tg_code_table(int32_t code_id, uint16_t *out, void *stream);

/*
 * Decode-only rate probe (measurement hook): runs the batch-1 kernel's per-step
 * loop -- x~ words from LDS, the quad rotate, window extraction, computed code
 * and fused dot product of 64 weights per lane -- on code words held in LDS, so
 * no HBM traffic is involved. Its rate is the VALU ceiling of trellis_gemv for
 * this K and code (lecture, Part three: the decode's integer-instruction budget
 * per weight; Part eleven: the same decode is compute-bound on data-centre
 * cards). workgroups of 512 threads (8 waves) each run `steps` steps, i.e.
 * decode workgroups * 512 * 64 * steps weights.
 *   k_bits     : 1..8;  code_id : 0, 1, 2 or 3.
 *   flags      : 0, or TG_FLAG_INT8_ACT with code_id 2 (the int8-activation loop).
 *   workgroups : 1..65535;  steps : 1..2^20.
 *   out        : device, workgroups * 512 fp32 (one per thread, keeps the work live).
 */
int32_t tg_decode_ceiling(int32_t k_bits, int32_t code_id, int32_t flags, int32_t workgroups, int32_t steps,
                          float *out, void *stream);

/*
 * Tail-biting Viterbi encoder (offline conversion; lecture, Part seven: the
 * Viterbi search keeps per state the best path ending there; Part eight: the
 * tail-biting circle is approximated in two passes -- rotate the sequence by
 * half, search, take the middle state as the start window, search again
 * constrained to start and end on it). For every tile it stores the stream
 * whose decoded weights w minimise sum_t (scale * w_t - target_t)^2.
 *   n_tiles  : 1 .. 2^24 tiles.
 *   k_bits   : 1..8 for code_id 0, 2 and 3; 1..4 for the pair code (2K bits per step).
 *   scale    : reconstruction scale, finite and > 0.
 *   targets  : device, n_tiles * 256 fp32, each tile in sequence order
 *              t = 16r + c, 4-byte aligned.
 *   codes    : device, n_tiles * 8K words out (the storage format above).
 *   sq_err   : device, n_tiles fp32 out (the minimised sum of squared errors),
 *              or NULL.
 *   ws       : device workspace of ws_bytes >= tg_encode_workspace_size(...)
 *              (the search's backpointers; no zero-fill needed).
 * Errors are float32 with a fixed operation order (p = scale*w, e = p - v,
 * d = e*e, pair code d = e0*e0 + e1*e1; cost = d + best predecessor cost),
 * and ties keep the smallest predecessor top bits and, at the open end, the
 * smallest state, so the result is deterministic.
 */
int32_t trellis_encode(int32_t n_tiles, int32_t k_bits, int32_t code_id, float scale,
                       const float *targets, uint32_t *codes, float *sq_err,
                       void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for trellis_encode (0 if the arguments are invalid). */
size_t tg_encode_workspace_size(int32_t n_tiles, int32_t k_bits, int32_t code_id);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_GEMV_H */
