/*
 * CPU oracle for one 4-bit mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, and shares no code with the HIP library.
 *
 * It is the plain definition written out as a per-token loop: route, then
 * dequantize and evaluate each selected expert and the shared expert, then
 * sum with the routing weights.  Everything is float64 except the router
 * logits, whose float32 summation order is part of the definition (see
 * oracle_router_logits).  Sources, by page and section:
 *
 *  - Mixture structure: 256 routed experts scored by a router, 8 chosen per
 *    token, plus one shared expert that every token uses
 *    (lefilia.fr article, body; mechatronicstore.cl article, "Tres formas de
 *    carga"; neuro-ai.ru article, "Пять приёмов").
 *  - Weight format: 4-bit affine quantisation, groups of 64 weights sharing
 *    one bf16 scale and one bf16 bias (mechatronicstore.cl, "Prefill: pesos
 *    comprimidos y enrutamiento en la GPU"; greatopti.com, "Une
 *    spécialisation assumée").  Packing of 8 codes per uint32, low nibble
 *    first; router softmax / top-8 / renormalisation; SwiGLU form
 *    down(silu(gate x) * up x); distributions: the workload definitions.
 *  - Routing structures (histogram, prefix scan, scatter, block map):
 *    mechatronicstore.cl, "Prefill: ..." (they are named there only; their
 *    exact layout is this implementation's reading, stated per function).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no -ffast-math).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the OpenMP loops below (timing the CPU baseline at one thread and at all). */
void oracle_set_threads(int32_t n)
{
    if (n > 0) omp_set_num_threads(n);
}

typedef struct {
    const uint32_t *q;   /* codes [N][K/8], 8 per word, low nibble first   */
    const uint16_t *s;   /* bf16 scale [N][K/64]                           */
    const uint16_t *b;   /* bf16 bias  [N][K/64]                           */
} oq4;

typedef struct {
    int32_t T, H, I, E, top_k;
    const uint16_t *x;     /* bf16 [T][H]                                  */
    const uint16_t *wr_t;  /* bf16 [E][H]: router weight, one row/expert   */
    const float *rbias;    /* float32 [E] additive logit bias, or NULL     */
    oq4 gate, up, down;    /* routed experts, stacked [E][...]             */
    oq4 sh_gate, sh_up, sh_down;
} olayer;

static float bf16_f(uint16_t v)
{
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---- format ------------------------------------------------------------ */

/* Code k of row n of a [N][K] projection: word k/8, nibble k%8 (low first). */
int oracle_code(const uint32_t *q, int32_t K, int32_t n, int32_t k)
{
    uint32_t word = q[(size_t)n * (K / 8) + (size_t)(k / 8)];
    return (int)((word >> (4 * (k % 8))) & 0xFu);
}

/* Affine dequantisation w = code * scale + bias, group = k / 64.  Exact in
 * float64: a 4-bit integer times an 8-bit significand plus another bf16. */
double oracle_weight(const oq4 *p, int32_t K, int32_t n, int32_t k)
{
    size_t g = (size_t)n * (K / 64) + (size_t)(k / 64);
    return (double)oracle_code(p->q, K, n, k) * (double)bf16_f(p->s[g]) + (double)bf16_f(p->b[g]);
}

void oracle_dequant(const uint32_t *q, const uint16_t *s, const uint16_t *b,
                    int32_t N, int32_t K, double *w)
{
    oq4 p = {q, s, b};
    for (int32_t n = 0; n < N; ++n)
        for (int32_t k = 0; k < K; ++k)
            w[(size_t)n * K + k] = oracle_weight(&p, K, n, k);
}

/* ---- router ------------------------------------------------------------ */

/* Router logit l[t][e] = sum_k x[t][k] * Wr[k][e] (+ bias[e]).
 *
 * The pages fix no summation order, but routing must be reproducible bit for
 * bit, so the order is part of the definition: float32 throughout; within
 * each consecutive chunk of 64 inputs a sequential sum starting from the
 * chunk's first product; then a sequential sum of the chunk partials
 * starting from chunk 0; then one float32 addition of the bias.  Every
 * product of two bf16 values is exact in float32, so fusing a product into
 * an addition does not change any result. */
static float router_logit(const uint16_t *xr, const uint16_t *wr, int32_t H, const float *bias, int32_t e)
{
    float total = 0.0f;
    for (int32_t c = 0; c < H / 64; ++c) {
        const uint16_t *xc = xr + 64 * c, *wc = wr + 64 * c;
        float part = bf16_f(xc[0]) * bf16_f(wc[0]);
        for (int32_t k = 1; k < 64; ++k)
            part = part + bf16_f(xc[k]) * bf16_f(wc[k]);
        total = (c == 0) ? part : total + part;
    }
    if (bias)
        total = total + bias[e];
    return total;
}

void oracle_router_logits(const uint16_t *x, const uint16_t *wr_t, const float *bias,
                          int32_t T, int32_t H, int32_t E, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e)
            logits[(size_t)t * E + e] = router_logit(x + (size_t)t * H, wr_t + (size_t)e * H, H, bias, e);
}

/* Top-k of one token's logits by (logit descending, expert index ascending):
 * the k picks are returned in that order.  Selection uses the float32
 * logits themselves (softmax is monotone, so the ranking is the same), and a
 * strict ">" scan over ascending indices keeps the lower index on a tie.
 * Weights: softmax over all experts restricted to the k picks and
 * renormalised, i.e. w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the
 * picks, in float64. */
static void topk_one(const float *l, int32_t E, int32_t k, int32_t *ids, double *w)
{
    char taken[4096];
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || l[e] > l[best]))
                best = e;
        taken[best] = 1;
        ids[j] = best;
    }
    double m = (double)l[ids[0]], sum = 0.0, p[64];
    for (int32_t j = 0; j < k; ++j) {
        p[j] = exp((double)l[ids[j]] - m);
        sum += p[j];
    }
    for (int32_t j = 0; j < k; ++j)
        w[j] = p[j] / sum;
}

void oracle_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids, double *w)
{
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t)
        topk_one(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

/* ---- routing structures ---------------------------------------------- */

/* Expert histogram, exclusive prefix scan, stable scatter and block map.
 * Reading of the layouts: rows are ordered by (expert ascending, token
 * ascending); row r of expert e serves token row_token[r]; tok_row[t][j] is
 * the row of pick j of token t; offsets has E+1 entries, offsets[E] = T*k;
 * the block map lists, expert by expert, blocks of at most BM consecutive
 * rows as (expert, first row, row count).  Returns the number of blocks. */
int32_t oracle_routing(const int32_t *ids, int32_t T, int32_t E, int32_t k, int32_t BM,
                       int32_t *counts, int32_t *offsets, int32_t *row_token, int32_t *tok_row,
                       int32_t *blocks)
{
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j)
            counts[ids[(size_t)t * k + j]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    for (int32_t e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int32_t r = cursor[ids[(size_t)t * k + j]]++;
            row_token[r] = t;
            tok_row[(size_t)t * k + j] = r;
        }
    int32_t nb = 0;
    for (int32_t e = 0; e < E; ++e)
        for (int32_t r0 = 0; r0 < counts[e]; r0 += BM) {
            blocks[3 * nb + 0] = e;
            blocks[3 * nb + 1] = offsets[e] + r0;
            blocks[3 * nb + 2] = (counts[e] - r0 < BM) ? counts[e] - r0 : BM;
            ++nb;
        }
    free(cursor);
    return nb;
}

/* ---- experts ----------------------------------------------------------- */

static oq4 slice(const oq4 *p, int32_t e, int32_t N, int32_t K)
{
    oq4 r = {p->q + (size_t)e * N * (K / 8), p->s + (size_t)e * N * (K / 64), p->b + (size_t)e * N * (K / 64)};
    return r;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU activation of one expert for one input row: a[i] = silu(g_i) * u_i
 * with g = W_gate x, u = W_up x (no bias terms).  e == E selects the shared
 * expert. */
void oracle_expert_act(const olayer *L, int32_t e, const uint16_t *xrow, double *a)
{
    int32_t H = L->H, I = L->I;
    oq4 g = (e == L->E) ? L->sh_gate : slice(&L->gate, e, I, H);
    oq4 u = (e == L->E) ? L->sh_up : slice(&L->up, e, I, H);
    for (int32_t i = 0; i < I; ++i) {
        double gs = 0.0, us = 0.0;
        for (int32_t k = 0; k < H; ++k) {
            double xv = (double)bf16_f(xrow[k]);
            gs += xv * oracle_weight(&g, H, i, k);
            us += xv * oracle_weight(&u, H, i, k);
        }
        a[i] = silu(gs) * us;
    }
}

/* Down projection of one expert: o[n] = sum_i W_down[n][i] * a[i]. */
void oracle_expert_down(const olayer *L, int32_t e, const double *a, double *o)
{
    int32_t H = L->H, I = L->I;
    oq4 d = (e == L->E) ? L->sh_down : slice(&L->down, e, H, I);
    for (int32_t n = 0; n < H; ++n) {
        double s = 0.0;
        for (int32_t i = 0; i < I; ++i)
            s += oracle_weight(&d, I, n, i) * a[i];
        o[n] = s;
    }
}

/* The layer for selected tokens: for each token, route it (logits, top-k,
 * weights), evaluate its k experts and the shared expert, and sum
 *   y = sum_j w_j * expert_{ids_j}(x) + shared(x)      (shared weight 1).
 * Writes y [n_tok][H] (float64), ids [n_tok][k], w [n_tok][k]. */
void oracle_moe_tokens(const olayer *L, const int32_t *tokens, int32_t n_tok,
                       double *y, int32_t *ids_out, double *w_out)
{
    int32_t H = L->H, I = L->I, E = L->E, k = L->top_k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t n = 0; n < n_tok; ++n) {
        int32_t t = tokens[n];
        const uint16_t *xr = L->x + (size_t)t * H;
        float *l = (float *)malloc(sizeof(float) * (size_t)E);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        int32_t ids[64];
        double w[64];
        for (int32_t e = 0; e < E; ++e)
            l[e] = router_logit(xr, L->wr_t + (size_t)e * H, H, L->rbias, e);
        topk_one(l, E, k, ids, w);
        double *yr = y + (size_t)n * H;
        for (int32_t h = 0; h < H; ++h)
            yr[h] = 0.0;
        for (int32_t j = 0; j <= k; ++j) {
            int32_t e = (j < k) ? ids[j] : E;
            double wt = (j < k) ? w[j] : 1.0;
            oracle_expert_act(L, e, xr, a);
            oracle_expert_down(L, e, a, o);
            for (int32_t h = 0; h < H; ++h)
                yr[h] += wt * o[h];
        }
        for (int32_t j = 0; j < k; ++j) {
            ids_out[(size_t)n * k + j] = ids[j];
            w_out[(size_t)n * k + j] = w[j];
        }
        free(l);
        free(a);
        free(o);
    }
}

/* ---- between layers of a stack ---------------------------------------- */

static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Residual add then RMSNorm with unit weight (the workload's stack reading):
 * r_out = r + y;  u = bf16( r_out / sqrt(mean(r_out^2) + eps) ), float64
 * except the final rounding to bf16 (via float32, round to nearest even). */
void oracle_rmsnorm_residual(int32_t T, int32_t H, double eps, const double *r, const double *y,
                             double *r_out, uint16_t *u)
{
    for (int32_t t = 0; t < T; ++t) {
        double ms = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            double v = r[(size_t)t * H + h] + y[(size_t)t * H + h];
            r_out[(size_t)t * H + h] = v;
            ms += v * v;
        }
        ms /= (double)H;
        double inv = 1.0 / sqrt(ms + eps);
        for (int32_t h = 0; h < H; ++h)
            u[(size_t)t * H + h] = f32_to_bf16_rne((float)(r_out[(size_t)t * H + h] * inv));
    }
}
