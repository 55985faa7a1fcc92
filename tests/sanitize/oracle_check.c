/* The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every entry point on a
 * small seeded layer (T = 40, H = 512, I = 128, 256 experts, top-8 plus the shared expert,
 * the Zipf router bias), with the invariants that need no second implementation: picks
 * distinct and in range, weights summing to 1, counts summing to 8 T, blocks tiling every
 * row once.  Exits nonzero on a violated invariant; the sanitizers abort on any error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { const uint32_t *q; const uint16_t *s; const uint16_t *b; } oq4;
typedef struct {
    int32_t T, H, I, E, top_k;
    const uint16_t *x, *wr_t;
    const float *rbias;
    oq4 gate, up, down, sh_gate, sh_up, sh_down;
} olayer;

void oracle_set_threads(int32_t n);
int oracle_code(const uint32_t *q, int32_t K, int32_t n, int32_t k);
void oracle_dequant(const uint32_t *q, const uint16_t *s, const uint16_t *b, int32_t N, int32_t K,
                    double *w);
void oracle_router_logits(const uint16_t *x, const uint16_t *wr_t, const float *bias, int32_t T,
                          int32_t H, int32_t E, float *out);
void oracle_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids, double *w);
int32_t oracle_routing(const int32_t *ids, int32_t T, int32_t E, int32_t k, int32_t BM,
                       int32_t *counts, int32_t *offsets, int32_t *row_token, int32_t *tok_row,
                       int32_t *blocks);
void oracle_expert_act(const olayer *L, int32_t e, const uint16_t *xrow, double *a);
void oracle_expert_down(const olayer *L, int32_t e, const double *a, double *o);
void oracle_moe_tokens(const olayer *L, const int32_t *tokens, int32_t n_tok, double *y,
                       int32_t *ids, double *w);
void oracle_rmsnorm_residual(int32_t T, int32_t H, double eps, const double *r, const double *y,
                             double *r_out, uint16_t *u);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 32);
}
static uint16_t bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float unif(void) { return (rnd() + 0.5f) * (1.0f / 4294967296.0f); }
static float normal(void) { return sqrtf(-2.0f * logf(unif())) * cosf(6.2831853f * unif()); }

static oq4 proj(int n_exp, int N, int K)
{
    const size_t words = (size_t)n_exp * N * K / 8, groups = (size_t)n_exp * N * K / 64;
    uint32_t *q = malloc(words * 4);
    uint16_t *s = malloc(groups * 2), *b = malloc(groups * 2);
    for (size_t i = 0; i < words; ++i) q[i] = rnd();
    for (size_t i = 0; i < groups; ++i) {
        const float sc = 0.002f + 0.018f * unif();
        s[i] = bf16(sc);
        b[i] = bf16(-8.0f * sc + (i % 2 ? 0.5f * sc : 0.0f));
    }
    oq4 p = {q, s, b};
    return p;
}

int main(void)
{
    const int T = 40, H = 512, I = 128, E = 256, k = 8, BM = 128;
    oracle_set_threads(2);
    uint16_t *x = malloc((size_t)T * H * 2), *wr = malloc((size_t)E * H * 2);
    float *bias = malloc(E * 4);
    for (int i = 0; i < T * H; ++i) x[i] = bf16(normal());
    for (int i = 0; i < E * H; ++i) wr[i] = bf16(normal() / sqrtf((float)H));
    for (int e = 0; e < E; ++e) bias[e] = -1.1f * logf((float)(e + 1));
    olayer L = {T, H, I, E, k, x, wr, bias, proj(E, I, H), proj(E, I, H), proj(E, H, I),
                proj(1, I, H), proj(1, I, H), proj(1, H, I)};
    int bad = 0;
    if (oracle_code(L.gate.q, H, 3, 17) != (int)((L.gate.q[3 * (H / 8) + 2] >> 4) & 15)) ++bad;
    double *wd = malloc((size_t)I * H * 8);
    oracle_dequant(L.gate.q, L.gate.s, L.gate.b, I, H, wd);
    float *lg = malloc((size_t)T * E * 4);
    oracle_router_logits(x, wr, bias, T, H, E, lg);
    int32_t *ids = malloc(T * k * 4);
    double *w = malloc(T * k * 8);
    oracle_topk(lg, T, E, k, ids, w);
    for (int t = 0; t < T; ++t) {
        double sw = 0.0;
        for (int j = 0; j < k; ++j) {
            sw += w[t * k + j];
            if (ids[t * k + j] < 0 || ids[t * k + j] >= E) ++bad;
            for (int i = 0; i < j; ++i) bad += ids[t * k + i] == ids[t * k + j];
        }
        if (fabs(sw - 1.0) > 1e-12) ++bad;
    }
    int32_t counts[256], offsets[257], *row_token = malloc(T * k * 4), *tok_row = malloc(T * k * 4);
    const int max_blocks = (T * k + BM - 1) / BM + E;
    int32_t *blocks = calloc((size_t)max_blocks * 3, 4);
    const int nb = oracle_routing(ids, T, E, k, BM, counts, offsets, row_token, tok_row, blocks);
    int csum = 0, covered = 0;
    for (int e = 0; e < E; ++e) csum += counts[e];
    for (int b = 0; b < nb; ++b) covered += blocks[3 * b + 2];
    if (csum != T * k || covered != T * k || offsets[E] != T * k || nb > max_blocks) ++bad;
    double *a = malloc(I * 8), *o = malloc(H * 8);
    oracle_expert_act(&L, 5, x, a);
    oracle_expert_down(&L, 5, a, o);
    oracle_expert_act(&L, E, x + H, a);                   /* the shared expert */
    int32_t tok[T];
    for (int t = 0; t < T; ++t) tok[t] = T - 1 - t;
    double *y = malloc((size_t)T * H * 8);
    int32_t *ids2 = malloc(T * k * 4);
    double *w2 = malloc(T * k * 8);
    oracle_moe_tokens(&L, tok, T, y, ids2, w2);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) bad += ids2[t * k + j] != ids[(T - 1 - t) * k + j];
    for (int i = 0; i < T * H; ++i) bad += !isfinite(y[i]);
    double *r = malloc((size_t)T * H * 8), *rout = malloc((size_t)T * H * 8);
    uint16_t *u = malloc((size_t)T * H * 2);
    for (int i = 0; i < T * H; ++i) r[i] = normal();
    oracle_rmsnorm_residual(T, H, 1e-6, r, y, rout, u);
    if (bad) {
        fprintf(stderr, "oracle_check: %d violated invariants\n", bad);
        return 1;
    }
    printf("oracle_check ok\n");
    return 0;
}
