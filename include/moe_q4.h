/*
 * moe_q4.h -- C ABI of the MI355X (gfx950) mixture-of-experts layer with
 * 4-bit affine expert weights.
 *
 * The layer (Lily pages: lefilia.fr article body; mechatronicstore.cl
 * article, sections "Tres formas de carga" and "Prefill: pesos comprimidos y
 * enrutamiento en la GPU"; neuro-ai.ru article, "Пять приёмов"):
 *   router logits over E = 256 experts, top-8 per token, plus one shared
 *   expert that every token uses; GPU-resident routing (expert histogram,
 *   prefix scan, token scatter, block map) with no host synchronisation;
 *   a grouped SwiGLU expert GEMM that reads the 4-bit weights directly and
 *   accumulates in FP32; a routing-weighted combine.  Decode (1 to 8 tokens
 *   per call) is a separate weight-streaming path (mechatronicstore.cl,
 *   "Decode: mover menos bytes por token"; neuro-ai.ru, "Спекулятивное
 *   декодирование не взлетело"); long prompts can run in chunks with a
 *   bounded workspace (greatopti.com, "Les gains viennent surtout des
 *   mouvements de données").
 *
 * Conventions common to every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory)
 *     unless marked "host".  Every pointer must be 16-byte aligned.
 *   - bf16 values are passed as their uint16_t bit patterns.
 *   - A 4-bit projection W[N][K] is { q, scale, bias }: q holds uint32 words
 *     [N][K/8], code k of row n in word k/8 at bits 4*(k%8)..+3 (low nibble
 *     first); scale and bias are bf16 [N][K/64]; w[n][k] = q*scale + bias
 *     with group k/64.  Routed experts stack E projections: [E][N][...].
 *     gate and up have N = I, K = H; down has N = H, K = I.
 *     This row layout is the checkpoint format; moe_pack_weights turns it
 *     into the tile layout below, which is what the layer calls read.
 *   - Tile layout (the `packed` buffer, written by moe_pack_weights): the
 *     same data regrouped so that one 64-wide K step of one 256-column GEMM
 *     tile is one contiguous 9216-byte block, read by a few whole-line copies
 *     (the pages rebuild weights tile by tile inside the grouped GEMM and get
 *     their decode bandwidth from coalesced reads: mechatronicstore.cl,
 *     "Prefill: ..." and "Decode: ...").  A block is
 *       bytes [0, 8192):     codes of 256 columns, 32 bytes each: 16-byte
 *                            half hh of column c holds code words
 *                            4 * (hh ^ ((c >> 3) & 1)) .. +3 of the group,
 *                            each word with its codes reordered: code 2m in
 *                            nibble m, code 2m + 1 in nibble m + 4 (m = 0..3),
 *                            so that the kernels unpack the nibble pairs
 *                            (m, m + 4) as consecutive codes;
 *       bytes [8192, 8704):  bf16 scales of the 256 columns;
 *       bytes [8704, 9216):  bf16 biases of the 256 columns.
 *     Sections, in this order, each starting 256-byte aligned:
 *       routed gate/up  [E][I/128][H/64] blocks: block (e, j, g) column c is
 *                       row 128 j + 32 (c / 64) + c % 32 of gate (c % 64 < 32)
 *                       or of up (c % 64 >= 32), group g;
 *       shared gate/up  [I/128][H/64] blocks, the same columns;
 *       routed down     [E][H/256][I/64] blocks: column c is row 256 j + c;
 *       shared down     [H/256][I/64] blocks.
 *     moe_packed_bytes gives the size.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     only ENQUEUES work on `stream`; none synchronises or copies
 *     device->host.  The caller owns every buffer; the library never
 *     allocates, frees or caches device memory, so calls on different streams
 *     are independent as long as they use different workspaces (a workspace
 *     holds a call's scratch rows and the GEMMs' work-queue counters: two
 *     calls in flight on one workspace race).  The only global state is the
 *     per-GPU scratch array of moe_decode_static (see there) and the kernels'
 *     dynamic-LDS limits, raised once per device on first use (thread-safe).
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a call that returns an error has enqueued nothing.
 *     MOE_ERR_INVALID_ARG: NULL or misaligned pointer, T < 1, bad sizes.
 *     MOE_ERR_UNSUPPORTED: bits != 4, group != 64, E != 256, top_k != 8,
 *       H not a multiple of 256 or above 2048, I not a multiple of 128 or
 *       above 2048, T > 65536 (moe_layer_chunked: T > 2^24), the
 *       checkpoint-format validation that refuses every other format.
 *     MOE_ERR_WORKSPACE: workspace NULL, not 256-byte aligned, or smaller
 *       than moe_query reports.
 *     MOE_ERR_HIP: a launch failed (hipGetLastError after the launch).
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,
    MOE_ERR_UNSUPPORTED = -2,
    MOE_ERR_WORKSPACE = -3,
    MOE_ERR_HIP = -4
} moe_status;

/* host struct; group must be 64 and bits 4 */
typedef struct {
    int32_t T, H, I, E, top_k, group, bits;
} moe_shape;

/* one 4-bit projection (device pointers) */
typedef struct {
    const uint32_t *q;
    const uint16_t *scale;
    const uint16_t *bias;
} moe_q4;

/* the layer's weights (host struct holding device pointers) */
typedef struct {
    moe_q4 gate, up, down;          /* routed experts, stacked [E][...]      */
    moe_q4 sh_gate, sh_up, sh_down; /* the shared expert                     */
    const uint16_t *router_wt;      /* bf16 [E][H]: router weight, row/expert */
    const float *router_bias;       /* fp32 [E] additive logit bias, or NULL  */
    const void *packed;             /* the six projections in the tile layout
                                       (moe_pack_weights), 256-byte aligned;
                                       the expert GEMMs and decode read only
                                       this and the router fields            */
} moe_weights;

/* Routing outputs (host struct holding device pointers).  Row r of the
 * routed part of h is one (token, pick) pair; rows are ordered by expert,
 * then token.  row_w[r] is the routing weight of row r.  blocks[b] =
 * {expert, first row, row count} tiles the rows of each expert in blocks of
 * at most block_rows rows (moe_query); *num_blocks stays on the device. */
typedef struct {
    float *logits;      /* fp32 [T][E] router logits, or NULL (then kept in ws) */
    int32_t *topk_ids;  /* [T][top_k], by logit descending, index ascending    */
    float *topk_w;      /* [T][top_k], softmax restricted to the picks          */
    int32_t *counts;    /* [E]                                                   */
    int32_t *offsets;   /* [E+1], exclusive scan of counts, offsets[E] = T*top_k */
    int32_t *row_token; /* [T*top_k]                                             */
    int32_t *tok_row;   /* [T][top_k]                                            */
    float *row_w;       /* [T*top_k]                                             */
    int32_t *blocks;    /* [max_blocks][3]                                        */
    int32_t *num_blocks;/* [1]                                                    */
} moe_routing;

/* Host only.  Workspace bytes needed by every call below for `shape`, the
 * capacity max_blocks of routing.blocks, and the rows per block (BM). */
moe_status moe_query(const moe_shape *shape, size_t *workspace_bytes, int32_t *max_blocks,
                     int32_t *block_rows);

/* Host only.  Bytes of the tile-layout buffer for `shape`. */
moe_status moe_packed_bytes(const moe_shape *shape, size_t *packed_bytes);

/* Load the six row-layout projections of w into the tile layout, once, when the
 * weights are loaded; the pages' engine validates the checkpoint format at load and
 * refuses every other (greatopti.com, "Une spécialisation assumée").
 * The codes move with the in-word reordering above.  Each projection row's scales and biases are stored times
 * a power of two 2^k that puts the row's largest |scale| in [2^10, 2^11), with 2^-k
 * kept per row in a meta section after the blocks; the kernels undo it exactly.  The
 * meta section also holds per expert a bound on the L2 norm of its gate and up rows
 * (used to keep the hidden activations in range) and a status word of validation
 * flags, copied to *status (device int32, may be NULL) when the pack completes:
 *   0  supported: the layer calls compute on these weights as documented;
 *   1  a scale or bias is NaN or infinite;
 *   2  a row's nonzero |scales| span more than 2^23 (its rebuilt fp16 weights would
 *      not be exact);
 *   4  a bias times the row's 2^k leaves the bf16 range.
 * A nonzero status means the weights are refused: the layer calls must not be used
 * with this buffer (their results would not be those documented).  The caller reads
 * *status once the stream has reached it.
 * packed: device buffer of at least moe_packed_bytes bytes, 256-byte aligned, not
 * overlapping the sources; w->packed is not read.  MOE_ERR_INVALID_ARG for a NULL or
 * misaligned pointer or a short buffer. */
moe_status moe_pack_weights(const moe_shape *shape, const moe_weights *w, void *packed,
                            size_t packed_bytes, int32_t *status, void *stream);

/* Router and routing (the pages' "histogram, prefix scan, scatter and block
 * map in one GPU command buffer", mechatronicstore.cl "Prefill: ...").
 * x: bf16 [T][H], finite.  Logits are float32 in a fixed order (within each chunk
 * of 64 inputs a sequential sum from the chunk's first product, then a
 * sequential sum over chunks, then + bias), so routing is reproducible bit
 * for bit.  topk_w: the softmax over all experts renormalised over the picks,
 * from the picks' fixed-order logits, evaluated in fp64 and rounded once.
 * Also prepares x for moe_expert_gemm_q4 in the workspace: an fp16 copy of
 * each token's row times 2^-e (e = 0 while max |x| lies in [2^-6, 2^14),
 * otherwise the power of two that puts it in [2^13, 2^14): exact), its group
 * sums, 2^e and ||x||. */
moe_status moe_route(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                     const moe_routing *r, void *ws, size_t ws_bytes, void *stream);

/* Grouped gate/up GEMM over the routed rows and the shared expert, reading
 * 4-bit codes directly (mechatronicstore.cl "Prefill: ...": weights rebuilt
 * tile by tile inside the grouped GEMM, FP32 accumulation), with the SwiGLU
 * epilogue h = silu(W_gate x) * (W_up x).
 * x is not read: the GEMM reads the fp16 copy of x that moe_route prepared in
 * the workspace (the argument is kept for symmetry with the other calls).
 * h: fp16 [T*top_k + T][I] (bits as uint16_t), natural column order; rows
 * 0..T*top_k-1 follow routing order, row T*top_k + t is the shared expert of
 * token t.  A row is stored as h 2^-f with f = 0 unless the bound (L2 norm of the expert's rows x
 * ||x||)^2 on |h| leaves [2^-2, 2^15); the workspace keeps 2^f per row.  Needs
 * moe_route's outputs and workspace; leaves the group sums of h and the row
 * factors in the workspace for moe_down_combine.
 * Reads the expert weights from w->packed (tile layout).
 * Weights are rebuilt exactly as (q - 8) * scale * 2^k in fp16 plus an fp32-accurate
 * term for bias + 8 * scale; the activations enter the matrix cores in fp16 at the
 * token's power of two.  So for weights that moe_pack_weights accepted and finite
 * x, the only roundings are those of fp32 accumulation and of h to fp16 (as long as
 * the values stay in the fp32 range). */
moe_status moe_expert_gemm_q4(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                              const moe_routing *r, uint16_t *h, void *ws, size_t ws_bytes,
                              void *stream);

/* Down GEMM plus routing-weighted combine:
 * y[t] = sum_j topk_w[t][j] * W_down[ids[t][j]] h[tok_row[t][j]] + W_sh_down h[T*top_k + t].
 * y: fp32 [T][H] (overwritten).  Reads the expert weights from w->packed.
 * h must be the output of moe_expert_gemm_q4
 * with the same workspace (whose group sums of h it reads).  Each routed row's
 * weighted output is rounded to bf16 into a workspace staging row (fp32 range,
 * relative error at most 2^-9 per routed term) and every token then adds its
 * eight rows in pick order in fp32, so y is reproducible bit for bit. */
moe_status moe_down_combine(const moe_shape *shape, const uint16_t *h, const moe_weights *w,
                            const moe_routing *r, float *y, void *ws, size_t ws_bytes,
                            void *stream);

/* moe_expert_gemm_q4 followed by moe_down_combine, with both GEMMs in one persistent
 * launch (the same routing blocks, grouped GEMMs and combine as mechatronicstore.cl
 * "Prefill: ...", scheduled as one queue: every gate/up tile, then every down tile).
 * Workgroups freed by the last gate/up tiles start on down tiles while those finish; a down
 * tile waits, inside the launch, for the gate/up tiles of its routing block.  h and y are
 * bit for bit those of the two calls: every tile computes the same operations in the same
 * order.  Arguments, layouts and preconditions as for the two calls: x is not read (the GEMMs
 * read moe_route's prepared copy in the workspace); h fp16 [T*top_k + T][I] (written, as by
 * moe_expert_gemm_q4); y fp32 [T][H] (overwritten).  Needs moe_route's outputs and workspace.
 * combine != 0: each token then adds its top_k staged routed rows to y, as moe_down_combine
 * does.  combine == 0: on return y holds the shared expert's output only and the routed rows'
 * weighted outputs stay staged in the workspace, for moe_combine or moe_combine_residual.
 * Calls that share a workspace must not overlap (the launch keeps its queue and per-block
 * counters there and zeroes them again when it ends). */
moe_status moe_expert_ffn_q4(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                             const moe_routing *r, uint16_t *h, float *y, int32_t combine,
                             void *ws, size_t ws_bytes, void *stream);

/* The combine that completes moe_expert_ffn_q4(combine = 0) on the same routing and
 * workspace: y[t] += sum_j staged row tok_row[t][j], in pick order j = 0..top_k-1, in fp32
 * (the combine of moe_down_combine).  y: fp32 [T][H]. */
moe_status moe_combine(const moe_shape *shape, const moe_routing *r, float *y, void *ws,
                       size_t ws_bytes, void *stream);

/* The same combine fused with the residual add and RMSNorm of a stack of layers, after
 * moe_expert_ffn_q4(combine = 0): with y_layer = y + the staged rows (what moe_combine would
 * leave in y), res <- res + y_layer, u = bf16(res / sqrt(mean(res^2) + eps)), bit for bit
 * as the combine of moe_down_combine_residual.  y is only read.  res, y fp32 [T][H]; u bf16
 * [T][H].  MOE_ERR_INVALID_ARG if res, y and u overlap pairwise (by start address) or
 * eps < 0. */
moe_status moe_combine_residual(const moe_shape *shape, const moe_routing *r, float *y, float *res,
                                float eps, uint16_t *u, void *ws, size_t ws_bytes, void *stream);

/* moe_down_combine fused with the residual add and RMSNorm that follow it in a stack of
 * layers (moe_rmsnorm_residual): with y_layer the output moe_down_combine would write,
 *   res <- res + y_layer,   u = bf16(res / sqrt(mean(res^2) + eps))   (unit weight),
 * bit for bit as moe_down_combine followed by moe_rmsnorm_residual (the same operations in
 * the same order: the eight routed rows are added to the shared expert's row in pick
 * order, in fp32, while the residual row is read).  y_layer is never stored, which saves
 * writing and re-reading T*H*4 bytes: y is scratch and holds only the shared expert's part
 * on return.  res, y: fp32 [T][H]; u: bf16 [T][H]; h, weights, routing and workspace as
 * for moe_down_combine.  MOE_ERR_INVALID_ARG if res, y and u overlap pairwise (by start
 * address) or eps < 0. */
moe_status moe_down_combine_residual(const moe_shape *shape, const uint16_t *h,
                                     const moe_weights *w, const moe_routing *r, float *y,
                                     float *res, float eps, uint16_t *u, void *ws,
                                     size_t ws_bytes, void *stream);

/* The whole layer: moe_route, then moe_expert_ffn_q4 (the same h and y as moe_route,
 * moe_expert_gemm_q4, moe_down_combine). */
moe_status moe_layer(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                     const moe_routing *r, uint16_t *h, float *y, void *ws, size_t ws_bytes,
                     void *stream);

/* Chunked prefill for long prompts (greatopti.com, "Les gains viennent surtout
 * des mouvements de données": long prompts are processed in fragments so that
 * the temporary activations stay bounded).  The layer runs on consecutive
 * chunks of at most `chunk` tokens, each a complete moe_layer over its tokens
 * (every token's routing and output depend on that token alone, so the result
 * equals the unchunked layer's).  The routing arrays and h of one chunk live in
 * the workspace, which is sized by moe_query_chunked for (shape, chunk) and so
 * bounded by the chunk, not by T.  All chunks are enqueued on `stream` with no
 * host synchronisation between them.
 * x: bf16 [T][H]; y: fp32 [T][H] (overwritten).  1 <= T <= 2^24
 * (MOE_ERR_UNSUPPORTED above); chunk >= 1 (MOE_ERR_INVALID_ARG otherwise) and
 * min(chunk, T) must be a token count that moe_query admits.  Weights as for
 * moe_layer (router + tile-layout buffer).  MOE_ERR_WORKSPACE if ws is not
 * 256-byte aligned or smaller than moe_query_chunked's size.  Validation
 * happens before anything is enqueued. */
moe_status moe_query_chunked(const moe_shape *shape, int32_t chunk, size_t *workspace_bytes);
moe_status moe_layer_chunked(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                             float *y, int32_t chunk, void *ws, size_t ws_bytes, void *stream);

/* Decode of 1 <= T <= 8 tokens (MOE_ERR_INVALID_ARG above 8): per token the
 * router, top-8 and weights, then the eight routed experts and the shared
 * expert as weight-streaming GEMVs that read only the selected experts' packed
 * weights (mechatronicstore.cl "Decode: mover menos bytes por token";
 * neuro-ai.ru "Спекулятивное декодирование не взлетело": decode at batch 1 and
 * small verify batches is bound by weight bandwidth).  The tokens are
 * independent problems in the same launches; an expert picked by several
 * tokens is streamed once per token (the repeats come from the caches).
 * x: bf16 [T][H]; topk_ids int32 [T][top_k], topk_w fp32 [T][top_k] (picks in
 * rank order), y fp32 [T][H] (overwritten).  Reads the expert weights from
 * w->packed and the router from w->router_wt (+ router_bias).  The ids equal
 * those of the fixed-order logits; h is kept in fp16 between the two GEMVs.
 * The workspace comes from moe_query for the same shape. */
moe_status moe_decode(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                      int32_t *topk_ids, float *topk_w, float *y, void *ws, size_t ws_bytes,
                      void *stream);

/* moe_decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  It takes no
 * workspace; the decode scratch (each token's 256 router logits and its nine h rows,
 * at most 303616 bytes for 8 tokens at H = I = 2048) lives in a device array inside
 * the library, one per GPU, held until the process ends.  Arguments, layout and
 * results are those of moe_decode, bit for bit.  The call allocates nothing; its first
 * call on a device looks up that device's array address (hipGetSymbolAddress) once.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (several streams, or several host threads) race and must be serialised by the
 * caller.  MOE_ERR_INVALID_ARG for T > 8 (and as moe_decode otherwise); MOE_ERR_HIP
 * if the array's address cannot be obtained. */
moe_status moe_decode_static(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                             int32_t *topk_ids, float *topk_w, float *y, void *stream);

/* One layer of a decode stack after the first (the stacked-layer workload: a
 * residual add and RMSNorm with unit weight between MoE layers), with the add
 * and the norm folded into the layer's router pass instead of a kernel of
 * their own:
 *   r <- r + y_prev (fp32);  u = bf16(r / sqrt(mean(r^2) + eps));
 *   then exactly moe_decode on u (ids, weights, y).
 * r, y_prev: fp32 [T][H]; u: bf16 [T][H] (written: the layer input, for the
 * caller's use); y: fp32 [T][H] (overwritten).  y_prev may be the same buffer
 * as y (the previous layer's output); r, y_prev and u must not overlap each
 * other otherwise (MOE_ERR_INVALID_ARG if r == y_prev or u == r).  T <= 8,
 * eps >= 0.  The first layer of a stack is plain moe_decode on x with r = x. */
moe_status moe_decode_residual(const moe_shape *shape, float *r, const float *y_prev, float eps,
                               uint16_t *u, const moe_weights *w, int32_t *topk_ids, float *topk_w,
                               float *y, void *ws, size_t ws_bytes, void *stream);

/* Between stacked layers: r <- r + y (fp32), u = bf16(r / sqrt(mean(r^2) + eps))
 * (unit RMSNorm weight).  r, y: fp32 [T][H]; u: bf16 [T][H]. */
moe_status moe_rmsnorm_residual(int32_t T, int32_t H, float eps, float *r, const float *y,
                                uint16_t *u, void *stream);

/* Test hook: dequantise one projection to bf16, out[n][k] =
 * bf16_round_nearest_even(fp32 fma(code, scale, bias)).  out: bf16 [N][K]. */
moe_status moe_dequant_q4(const moe_q4 *p, int32_t N, int32_t K, uint16_t *out, void *stream);

/* Device index checks of a MOE_DEBUG build of the library (build.py debug=True).  Where a
 * kernel meets an index that valid routing structures never hold (an expert id, row, token
 * or block map entry out of range) it skips or clamps it in every build; the debug build
 * also records it.  This call waits for the device (hipDeviceSynchronize: it is the one
 * call that synchronises) and stores in *flags (host) the OR of what the kernels recorded
 * since the last clear: 1 scatter index, 2 block map entry, 4 row token, 8 combine row,
 * 16 decode expert id, 32 a moe_expert_ffn_q4 down tile that gave up waiting for its block's
 * gate/up tiles (about a second; never with the launch alone on the device); clear != 0
 * resets the record.  MOE_ERR_UNSUPPORTED (and *flags = 0)
 * in a regular build; MOE_ERR_HIP if the device or the record cannot be read. */
moe_status moe_debug_status(uint32_t *flags, int32_t clear);

/* Static string for a status code (any value: unknown codes get a generic string). */
const char *moe_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_Q4_H */
