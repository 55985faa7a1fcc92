// Host side of libmoeq4: argument validation, workspace layout and launch
// order.  Every check runs before the first launch, so an error return
// means nothing was enqueued.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int max_blocks_for(int T, int E, int k) {
    const int rows = T * k;
    return (rows + kBM - 1) / kBM + (rows < E ? rows : E);
}

int ffn_slots(int T, int E, int k) { return (T + kBM - 1) / kBM + max_blocks_for(T, E, k); }

size_t decode_scratch_bytes(int T, int H, int I, int k);

WsLayout ws_layout(int T, int H, int I, int E, int k) {
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t nTB = (size_t)(T + kTB - 1) / kTB;
    L.logits = take((size_t)T * E * 4);
    L.xsum = take((size_t)T * (H / 64) * 4);
    L.xp = take((size_t)T * H * 2);
    L.xsq = take((size_t)T * (H / 64) * 4);
    L.part = take((size_t)4 * T * E * 4);
    L.wn2 = take((size_t)4 * E * 4);
    L.hsum = take((size_t)(T * k + T) * (I / 64) * 4);
    L.stage = take((size_t)T * k * H * 2);
    L.blk_cnt = take(nTB * E * 4);
    L.lrank = take((size_t)T * k * 4);
    L.sup = take(nTB <= (size_t)kSupBlk * kSupMax ? (nTB + kSupBlk - 1) / kSupBlk * E * 4 : 0);
    L.sched = take((size_t)max_blocks_for(T, E, k) * 4);
    L.qctl = take((size_t)(QCTL_WORDS + ffn_slots(T, E, k)) * 4);
    L.xmx = take((size_t)T * (H / 64) * 4);
    L.tok = take((size_t)T * 2 * 4);
    L.hexp = take((size_t)(T * k + T) * 4);
    L.dec = take(T <= kDecodeMaxT ? decode_scratch_bytes(T, H, I, k) : 0);
    L.total = off;
    return L;
}

// Workspace of moe_layer_chunked for chunks of C tokens: the layer workspace of the
// largest chunk, then the chunk's routing arrays and h.
struct ChunkLayout {
    size_t ids, tw, counts, offsets, row_token, tok_row, row_w, blocks, num_blocks, h, total;
};

static ChunkLayout chunk_layout(int T, int C, int H, int I, int E, int k) {
    ChunkLayout L{};
    const int last = T % C;
    size_t off = ws_layout(C, H, I, E, k).total;
    if (last) off = std::max(off, ws_layout(last, H, I, E, k).total);
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    L.ids = take((size_t)C * k * 4);
    L.tw = take((size_t)C * k * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.row_token = take((size_t)C * k * 4);
    L.tok_row = take((size_t)C * k * 4);
    L.row_w = take((size_t)C * k * 4);
    L.blocks = take((size_t)max_blocks_for(C, E, k) * 3 * 4);
    L.num_blocks = take(4);
    L.h = take((size_t)(C * k + C) * I * 2);
    L.total = off;
    return L;
}

}  // namespace moe

using namespace moe;

namespace {

bool aligned(const void *p) { return p && (((uintptr_t)p) & 15u) == 0; }

moe_status check_shape(const moe_shape *s) {
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->T < 1 || s->H < 1 || s->I < 1 || s->E < 1 || s->top_k < 1) return MOE_ERR_INVALID_ARG;
    if (s->bits != 4 || s->group != 64) return MOE_ERR_UNSUPPORTED;
    if (s->E != 256 || s->top_k != 8) return MOE_ERR_UNSUPPORTED;
    if (s->H % 256 != 0 || s->H > 2048) return MOE_ERR_UNSUPPORTED;
    if (s->I % 128 != 0 || s->I > 2048) return MOE_ERR_UNSUPPORTED;
    if (s->T > 65536) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

bool q4_ok(const moe_q4 &p) { return aligned(p.q) && aligned(p.scale) && aligned(p.bias); }

moe_status check_weights(const moe_weights *w, bool need_router, bool need_gu, bool need_down) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (need_router) {
        if (!aligned(w->router_wt)) return MOE_ERR_INVALID_ARG;
        if (w->router_bias && !aligned(w->router_bias)) return MOE_ERR_INVALID_ARG;
    }
    // the expert GEMMs and decode read the tile-layout buffer only
    if ((need_gu || need_down) && (!w->packed || (((uintptr_t)w->packed) & 255u) != 0))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_routing(const moe_routing *r) {
    if (!r) return MOE_ERR_INVALID_ARG;
    if (r->logits && !aligned(r->logits)) return MOE_ERR_INVALID_ARG;
    if (!aligned(r->topk_ids) || !aligned(r->topk_w) || !aligned(r->counts) ||
        !aligned(r->offsets) || !aligned(r->row_token) || !aligned(r->tok_row) ||
        !aligned(r->row_w) || !aligned(r->blocks) || !aligned(r->num_blocks))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_ws(const moe_shape *s, void *ws, size_t ws_bytes) {
    const WsLayout L = ws_layout(s->T, s->H, s->I, s->E, s->top_k);
    if (!ws || (((uintptr_t)ws) & 255u) != 0 || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// moe_layer_chunked: any number of tokens up to kChunkedMaxT, chunks that a single layer
// call admits
constexpr long kChunkedMaxT = 1L << 24;
moe_status check_chunked(const moe_shape *s, int32_t chunk) {
    if (!s || chunk < 1 || s->T < 1) return MOE_ERR_INVALID_ARG;
    if (s->T > kChunkedMaxT) return MOE_ERR_UNSUPPORTED;
    moe_shape sc = *s;
    sc.T = std::min<int32_t>(chunk, s->T);
    return check_shape(&sc);
}

moe_status launched() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

GemmProj gp(const moe_q4 &p) { return GemmProj{p.q, p.scale, p.bias}; }

#define MOE_TRY(x)                      \
    do {                                \
        const moe_status st_ = (x);     \
        if (st_ != MOE_OK) return st_;  \
    } while (0)

moe_status enqueue_route(const moe_shape *s, const uint16_t *x, const moe_weights *w,
                         const moe_routing *r, char *ws, hipStream_t st) {
    const WsLayout L = ws_layout(s->T, s->H, s->I, s->E, s->top_k);
    int32_t *blk_cnt = (int32_t *)(ws + L.blk_cnt);
    int32_t *lrank = (int32_t *)(ws + L.lrank);
    float *xsq = (float *)(ws + L.xsq);
    // superblock counts of the single-pass routing structures (T <= 4096): zeroed by the
    // router pass, accumulated by the select kernel
    const int nTB = (s->T + kTB - 1) / kTB;
    const int nsup = nTB <= kSupBlk * kSupMax ? (nTB + kSupBlk - 1) / kSupBlk * s->E : 0;
    int32_t *sup = nsup ? (int32_t *)(ws + L.sup) : nullptr;
    if (r->logits) {
        launch_prep_act(x, s->T, s->H, (uint16_t *)(ws + L.xp), (float *)(ws + L.xsum), xsq,
                        (float *)(ws + L.xmx), st);
        if (sup) launch_zero_i32(sup, nsup, st);
        // every logit requested: compute them all in the fixed order, select on them directly
        launch_router_logits(x, w->router_wt, w->router_bias, s->T, s->H, s->E, r->logits, st);
        launch_route_select(nullptr, r->logits, xsq, nullptr, w->router_bias, x, w->router_wt,
                            s->T, s->H, s->E, s->top_k, r->topk_ids, r->topk_w, blk_cnt, lrank,
                            sup, (const float *)(ws + L.xmx), (uint16_t *)(ws + L.xp),
                            (float *)(ws + L.xsum), (float *)(ws + L.tok), st);
    } else {
        float *part = (float *)(ws + L.part), *wn2 = (float *)(ws + L.wn2);
        launch_router_fast(x, w->router_wt, s->T, s->H, s->E, part, wn2, (uint16_t *)(ws + L.xp),
                           (float *)(ws + L.xsum), xsq, (float *)(ws + L.xmx), sup, nsup, st);
        launch_route_select(part, nullptr, xsq, wn2, w->router_bias, x, w->router_wt, s->T, s->H,
                            s->E, s->top_k, r->topk_ids, r->topk_w, blk_cnt, lrank, sup,
                            (const float *)(ws + L.xmx), (uint16_t *)(ws + L.xp),
                            (float *)(ws + L.xsum), (float *)(ws + L.tok), st);
    }
    launch_scan_scatter(r->topk_ids, r->topk_w, blk_cnt, sup, lrank, s->T, s->E, s->top_k, kBM,
                        r->counts, r->offsets, r->row_token, r->tok_row, r->row_w, r->blocks,
                        r->num_blocks, (int32_t *)(ws + L.sched), (int32_t *)(ws + L.qctl),
                        ffn_slots(s->T, s->E, s->top_k), st);
    return launched();
}

moe_status enqueue_gateup(const moe_shape *s, const uint16_t *x, const moe_weights *w,
                          const moe_routing *r, uint16_t *h, char *ws, hipStream_t st) {
    const WsLayout L = ws_layout(s->T, s->H, s->I, s->E, s->top_k);
    (void)x;   // the GEMM reads moe_route's prepared copy of x in the workspace
    const GemmWeights gw = gemm_weights(w->packed, s->H, s->I, s->E, true);
    launch_gateup(*s, (const uint16_t *)(ws + L.xp), (const float *)(ws + L.xsum),
                  (const float *)(ws + L.tok), gw, r->blocks, r->num_blocks,
                  (const int32_t *)(ws + L.sched), (int32_t *)(ws + L.qctl),
                  max_blocks_for(s->T, s->E, s->top_k), r->row_token, h, (float *)(ws + L.hsum),
                  (float *)(ws + L.hexp), st);
    return launched();
}

moe_status enqueue_down(const moe_shape *s, const uint16_t *h, const moe_weights *w,
                        const moe_routing *r, float *y, char *ws, hipStream_t st,
                        bool combine = true) {
    const WsLayout L = ws_layout(s->T, s->H, s->I, s->E, s->top_k);
    // group sums of h: left in the workspace by the gate/up pass
    const float *hsum = (const float *)(ws + L.hsum);
    const GemmWeights gw = gemm_weights(w->packed, s->H, s->I, s->E, false);
    launch_down(*s, h, hsum, (const float *)(ws + L.hexp), gw, r->blocks, r->num_blocks,
                (const int32_t *)(ws + L.sched), (int32_t *)(ws + L.qctl),
                max_blocks_for(s->T, s->E, s->top_k), r->row_token, r->row_w, r->tok_row,
                (uint16_t *)(ws + L.stage), y, combine, st);
    return launched();
}

// gate/up and down in one launch, then (combine) the combine
moe_status enqueue_ffn(const moe_shape *s, const moe_weights *w, const moe_routing *r, uint16_t *h,
                       float *y, bool combine, char *ws, hipStream_t st) {
    const WsLayout L = ws_layout(s->T, s->H, s->I, s->E, s->top_k);
    launch_ffn(*s, (const uint16_t *)(ws + L.xp), (const float *)(ws + L.xsum),
               (const float *)(ws + L.tok), gemm_weights(w->packed, s->H, s->I, s->E, true),
               gemm_weights(w->packed, s->H, s->I, s->E, false), r->blocks, r->num_blocks,
               (const int32_t *)(ws + L.sched), (int32_t *)(ws + L.qctl),
               max_blocks_for(s->T, s->E, s->top_k), r->row_token, r->row_w, r->tok_row, h,
               (float *)(ws + L.hsum), (float *)(ws + L.hexp), (uint16_t *)(ws + L.stage), y,
               combine, st);
    return launched();
}

}  // namespace

extern "C" {

moe_status moe_query(const moe_shape *shape, size_t *workspace_bytes, int32_t *max_blocks,
                     int32_t *block_rows) {
    MOE_TRY(check_shape(shape));
    const WsLayout L = ws_layout(shape->T, shape->H, shape->I, shape->E, shape->top_k);
    if (workspace_bytes) *workspace_bytes = L.total;
    if (max_blocks) *max_blocks = max_blocks_for(shape->T, shape->E, shape->top_k);
    if (block_rows) *block_rows = kBM;
    return MOE_OK;
}

moe_status moe_packed_bytes(const moe_shape *shape, size_t *packed_bytes) {
    MOE_TRY(check_shape(shape));
    if (!packed_bytes) return MOE_ERR_INVALID_ARG;
    *packed_bytes = pack_layout(shape->H, shape->I, shape->E).total;
    return MOE_OK;
}

moe_status moe_pack_weights(const moe_shape *shape, const moe_weights *w, void *packed,
                            size_t packed_bytes, int32_t *status, void *stream) {
    MOE_TRY(check_shape(shape));
    if (!w || !(q4_ok(w->gate) && q4_ok(w->up) && q4_ok(w->down) && q4_ok(w->sh_gate) &&
                q4_ok(w->sh_up) && q4_ok(w->sh_down)))
        return MOE_ERR_INVALID_ARG;
    if (!packed || (((uintptr_t)packed) & 255u) != 0 ||
        packed_bytes < pack_layout(shape->H, shape->I, shape->E).total)
        return MOE_ERR_INVALID_ARG;
    if (status && (((uintptr_t)status) & 3u) != 0) return MOE_ERR_INVALID_ARG;
    launch_pack(*shape, *w, (uint8_t *)packed, status, (hipStream_t)stream);
    return launched();
}

moe_status moe_route(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                     const moe_routing *r, void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(x)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, true, false, false));
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    return enqueue_route(shape, x, w, r, (char *)ws, (hipStream_t)stream);
}

moe_status moe_expert_gemm_q4(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                              const moe_routing *r, uint16_t *h, void *ws, size_t ws_bytes,
                              void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(x) || !aligned(h)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, false, true, false));
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    return enqueue_gateup(shape, x, w, r, h, (char *)ws, (hipStream_t)stream);
}

moe_status moe_down_combine(const moe_shape *shape, const uint16_t *h, const moe_weights *w,
                            const moe_routing *r, float *y, void *ws, size_t ws_bytes,
                            void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(h) || !aligned(y)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, false, false, true));
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    return enqueue_down(shape, h, w, r, y, (char *)ws, (hipStream_t)stream);
}

moe_status moe_expert_ffn_q4(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                             const moe_routing *r, uint16_t *h, float *y, int32_t combine,
                             void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(x) || !aligned(h) || !aligned(y)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, false, true, true));
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    (void)x;   // the GEMMs read moe_route's prepared copy of x in the workspace
    return enqueue_ffn(shape, w, r, h, y, combine != 0, (char *)ws, (hipStream_t)stream);
}

moe_status moe_combine(const moe_shape *shape, const moe_routing *r, float *y, void *ws,
                       size_t ws_bytes, void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(y)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(shape->T, shape->H, shape->I, shape->E, shape->top_k);
    launch_combine(*shape, (const uint16_t *)((char *)ws + L.stage), r->tok_row, y,
                   (hipStream_t)stream);
    return launched();
}

moe_status moe_combine_residual(const moe_shape *shape, const moe_routing *r, float *y, float *res,
                                float eps, uint16_t *u, void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(y) || !aligned(res) || !aligned(u) || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if ((const void *)res == (const void *)y || (const void *)u == (const void *)res ||
        (const void *)u == (const void *)y)
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(shape->T, shape->H, shape->I, shape->E, shape->top_k);
    launch_combine_residual_norm(shape->T, shape->H, shape->top_k, eps, res, y,
                                 (const uint16_t *)((char *)ws + L.stage), r->tok_row, u,
                                 (hipStream_t)stream);
    return launched();
}

moe_status moe_down_combine_residual(const moe_shape *shape, const uint16_t *h,
                                     const moe_weights *w, const moe_routing *r, float *y,
                                     float *res, float eps, uint16_t *u, void *ws,
                                     size_t ws_bytes, void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(h) || !aligned(y) || !aligned(res) || !aligned(u) || !(eps >= 0.0f))
        return MOE_ERR_INVALID_ARG;
    if ((const void *)res == (const void *)y || (const void *)u == (const void *)res ||
        (const void *)u == (const void *)y)
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, false, false, true));
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    MOE_TRY(enqueue_down(shape, h, w, r, y, (char *)ws, st, false));
    const WsLayout L = ws_layout(shape->T, shape->H, shape->I, shape->E, shape->top_k);
    launch_combine_residual_norm(shape->T, shape->H, shape->top_k, eps, res, y,
                                 (const uint16_t *)((char *)ws + L.stage), r->tok_row, u, st);
    return launched();
}

moe_status moe_layer(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                     const moe_routing *r, uint16_t *h, float *y, void *ws, size_t ws_bytes,
                     void *stream) {
    MOE_TRY(check_shape(shape));
    if (!aligned(x) || !aligned(h) || !aligned(y)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, true, true, true));
    MOE_TRY(check_routing(r));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    MOE_TRY(enqueue_route(shape, x, w, r, (char *)ws, st));
    return enqueue_ffn(shape, w, r, h, y, true, (char *)ws, st);
}

moe_status moe_query_chunked(const moe_shape *shape, int32_t chunk, size_t *workspace_bytes) {
    MOE_TRY(check_chunked(shape, chunk));
    const int C = std::min<int>(chunk, shape->T);
    if (workspace_bytes)
        *workspace_bytes = chunk_layout(shape->T, C, shape->H, shape->I, shape->E, shape->top_k).total;
    return MOE_OK;
}

moe_status moe_layer_chunked(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                             float *y, int32_t chunk, void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_chunked(shape, chunk));
    if (!aligned(x) || !aligned(y)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, true, true, true));
    const int T = shape->T, H = shape->H, C = std::min<int>(chunk, T);
    const ChunkLayout CL = chunk_layout(T, C, H, shape->I, shape->E, shape->top_k);
    if (!ws || (((uintptr_t)ws) & 255u) != 0 || ws_bytes < CL.total) return MOE_ERR_WORKSPACE;
    char *base = (char *)ws;
    moe_routing r{};
    r.logits = nullptr;
    r.topk_ids = (int32_t *)(base + CL.ids);
    r.topk_w = (float *)(base + CL.tw);
    r.counts = (int32_t *)(base + CL.counts);
    r.offsets = (int32_t *)(base + CL.offsets);
    r.row_token = (int32_t *)(base + CL.row_token);
    r.tok_row = (int32_t *)(base + CL.tok_row);
    r.row_w = (float *)(base + CL.row_w);
    r.blocks = (int32_t *)(base + CL.blocks);
    r.num_blocks = (int32_t *)(base + CL.num_blocks);
    uint16_t *h = (uint16_t *)(base + CL.h);
    hipStream_t st = (hipStream_t)stream;
    // each chunk is a whole layer call on its tokens; nothing leaves the device between them
    for (long c0 = 0; c0 < T; c0 += C) {
        moe_shape sc = *shape;
        sc.T = (int32_t)std::min<long>(C, T - c0);
        const uint16_t *xc = x + (size_t)c0 * H;
        float *yc = y + (size_t)c0 * H;
        MOE_TRY(enqueue_route(&sc, xc, w, &r, base, st));
        MOE_TRY(enqueue_ffn(&sc, w, &r, h, yc, true, base, st));
    }
    return MOE_OK;
}

moe_status moe_decode(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                      int32_t *topk_ids, float *topk_w, float *y, void *ws, size_t ws_bytes,
                      void *stream) {
    MOE_TRY(check_shape(shape));
    if (shape->T > kDecodeMaxT) return MOE_ERR_INVALID_ARG;
    if (!aligned(x) || !aligned(topk_ids) || !aligned(topk_w) || !aligned(y))
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, true, true, true));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(shape->T, shape->H, shape->I, shape->E, shape->top_k);
    launch_decode(*shape, x, *w, topk_ids, topk_w, y, (char *)ws + L.dec, (hipStream_t)stream);
    return launched();
}

}  // extern "C"

// ---- decode without a caller workspace ----
// The decode kernels' scratch (each token's router logits and its nine h rows) in a
// file-scope device array, sized for the largest decode call the API admits (8 tokens,
// H = I = 2048).  Each GPU holds its own copy until the process ends.  Host code never
// passes the array's name to a kernel: it is a host-side stand-in for the symbol.  The
// device address is looked up once per device (with that device current) and cached.
namespace {
constexpr size_t kStaticScratchBytes = decode_scratch_size(kDecodeMaxT, 2048, 8);   // 303616
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

moe_status static_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_decode_static(const moe_shape *shape, const uint16_t *x, const moe_weights *w,
                             int32_t *topk_ids, float *topk_w, float *y, void *stream) {
    MOE_TRY(check_shape(shape));
    if (shape->T > kDecodeMaxT) return MOE_ERR_INVALID_ARG;
    if (!aligned(x) || !aligned(topk_ids) || !aligned(topk_w) || !aligned(y))
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, true, true, true));
    if (decode_scratch_bytes(shape->T, shape->H, shape->I, shape->top_k) > kStaticScratchBytes)
        return MOE_ERR_WORKSPACE;
    void *sp = nullptr;
    MOE_TRY(static_scratch(&sp));
    launch_decode(*shape, x, *w, topk_ids, topk_w, y, sp, (hipStream_t)stream);
    return launched();
}

moe_status moe_decode_residual(const moe_shape *shape, float *r, const float *y_prev, float eps,
                               uint16_t *u, const moe_weights *w, int32_t *topk_ids, float *topk_w,
                               float *y, void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_shape(shape));
    if (shape->T > kDecodeMaxT || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (!aligned(r) || !aligned(y_prev) || !aligned(u) || !aligned(topk_ids) || !aligned(topk_w) ||
        !aligned(y))
        return MOE_ERR_INVALID_ARG;
    if ((const void *)r == (const void *)y_prev || (const void *)u == (const void *)r)
        return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_weights(w, true, true, true));
    MOE_TRY(check_ws(shape, ws, ws_bytes));
    const WsLayout L = ws_layout(shape->T, shape->H, shape->I, shape->E, shape->top_k);
    launch_decode(*shape, nullptr, *w, topk_ids, topk_w, y, (char *)ws + L.dec, (hipStream_t)stream,
                  r, y_prev, eps, u);
    return launched();
}

moe_status moe_rmsnorm_residual(int32_t T, int32_t H, float eps, float *r, const float *y,
                                uint16_t *u, void *stream) {
    if (T < 1 || H < 4 || H % 4 != 0 || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (!aligned(r) || !aligned(y) || !aligned(u)) return MOE_ERR_INVALID_ARG;
    launch_rmsnorm_residual(T, H, eps, r, y, u, (hipStream_t)stream);
    return launched();
}

moe_status moe_dequant_q4(const moe_q4 *p, int32_t N, int32_t K, uint16_t *out, void *stream) {
    if (!p || N < 1 || K < 64 || K % 64 != 0) return MOE_ERR_INVALID_ARG;
    if (!q4_ok(*p) || !aligned(out)) return MOE_ERR_INVALID_ARG;
    launch_dequant(gp(*p), N, K, out, (hipStream_t)stream);
    return launched();
}

moe_status moe_debug_status(uint32_t *flags, int32_t clear) {
    if (!flags) return MOE_ERR_INVALID_ARG;
#ifdef MOE_DEBUG
    if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
    const uint32_t v = dbg_read_route(clear != 0) | dbg_read_gemm(clear != 0) |
                       dbg_read_decode(clear != 0) | dbg_read_misc(clear != 0);
    *flags = v;
    return (v & 0x80000000u) ? MOE_ERR_HIP : MOE_OK;
#else
    (void)clear;
    *flags = 0;
    return MOE_ERR_UNSUPPORTED;
#endif
}

const char *moe_status_str(int32_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer or bad size)";
        case MOE_ERR_UNSUPPORTED: return "unsupported format or shape";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

}  // extern "C"
