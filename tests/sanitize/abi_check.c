/* Host-side checks of libmoeq4 under AddressSanitizer and UndefinedBehaviorSanitizer:
 * the size queries for every admitted shape class and the argument validation of every
 * entry point (each call fails before it would launch anything, so no GPU is needed).
 * Exits nonzero on the first unexpected status; the sanitizers abort on any error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/moe_q4.h"

static int fails = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const moe_status st_ = (call);                                                  \
        if (st_ != (want)) {                                                            \
            fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, st_, want); \
            ++fails;                                                                    \
        }                                                                               \
    } while (0)

static moe_shape shape(int T, int H, int I)
{
    moe_shape s = {T, H, I, 256, 8, 64, 4};
    return s;
}

int main(void)
{
    /* aligned, never dereferenced: validation fails before anything is enqueued */
    void *fake = (void *)(uintptr_t)0x10000;
    moe_q4 q = {(const uint32_t *)fake, (const uint16_t *)fake, (const uint16_t *)fake};
    moe_weights w = {q, q, q, q, q, q, (const uint16_t *)fake, NULL, fake};
    moe_routing r = {NULL, fake, fake, fake, fake, fake, fake, fake, fake, fake};
    const int Ts[] = {1, 7, 8, 9, 129, 2048, 65536};
    const int HIs[][2] = {{256, 128}, {512, 128}, {768, 384}, {2048, 512}, {2048, 2048}};
    for (size_t a = 0; a < sizeof Ts / sizeof Ts[0]; ++a)
        for (size_t b = 0; b < sizeof HIs / sizeof HIs[0]; ++b) {
            moe_shape s = shape(Ts[a], HIs[b][0], HIs[b][1]);
            size_t ws = 0, pk = 0, cws = 0;
            int32_t mb = 0, br = 0;
            EXPECT(moe_query(&s, &ws, &mb, &br), MOE_OK);
            EXPECT(moe_packed_bytes(&s, &pk), MOE_OK);
            EXPECT(moe_query_chunked(&s, 64, &cws), MOE_OK);
            if (ws == 0 || pk == 0 || mb < 1 || br != 128) ++fails;
            /* every entry point: a workspace one byte short */
            EXPECT(moe_route(&s, fake, &w, &r, fake, ws - 1, NULL), MOE_ERR_WORKSPACE);
            EXPECT(moe_expert_gemm_q4(&s, fake, &w, &r, fake, fake, ws - 1, NULL), MOE_ERR_WORKSPACE);
            EXPECT(moe_down_combine(&s, fake, &w, &r, fake, fake, ws - 1, NULL), MOE_ERR_WORKSPACE);
            EXPECT(moe_expert_ffn_q4(&s, fake, &w, &r, fake, fake, 1, fake, ws - 1, NULL), MOE_ERR_WORKSPACE);
            EXPECT(moe_combine(&s, &r, fake, fake, ws - 1, NULL), MOE_ERR_WORKSPACE);
            EXPECT(moe_combine_residual(&s, &r, (float *)fake, (float *)fake + 64, 1e-6f,
                                        (uint16_t *)fake + 4096, fake, ws - 1, NULL),
                   MOE_ERR_WORKSPACE);
            EXPECT(moe_down_combine_residual(&s, fake, &w, &r, (float *)fake, (float *)fake + 64,
                                             1e-6f, (uint16_t *)fake + 4096, fake, ws - 1, NULL),
                   MOE_ERR_WORKSPACE);
            EXPECT(moe_layer(&s, fake, &w, &r, fake, fake, fake, ws - 1, NULL), MOE_ERR_WORKSPACE);
            EXPECT(moe_layer_chunked(&s, fake, &w, fake, 64, fake, cws - 1, NULL), MOE_ERR_WORKSPACE);
            if (s.T <= 8) {
                EXPECT(moe_decode(&s, fake, &w, fake, fake, fake, fake, ws - 1, NULL), MOE_ERR_WORKSPACE);
                EXPECT(moe_decode_residual(&s, fake, (float *)fake + 64, 1e-6f, (uint16_t *)fake + 4096,
                                           &w, fake, fake, fake, fake, ws - 1, NULL),
                       MOE_ERR_WORKSPACE);
            } else {
                EXPECT(moe_decode(&s, fake, &w, fake, fake, fake, fake, ws, NULL), MOE_ERR_INVALID_ARG);
                EXPECT(moe_decode_static(&s, fake, &w, fake, fake, fake, NULL), MOE_ERR_INVALID_ARG);
            }
            EXPECT(moe_pack_weights(&s, &w, fake, pk - 1, NULL, NULL), MOE_ERR_INVALID_ARG);
        }
    /* unsupported formats and bad arguments */
    moe_shape s = shape(64, 2048, 512);
    s.bits = 8;
    EXPECT(moe_query(&s, NULL, NULL, NULL), MOE_ERR_UNSUPPORTED);
    s = shape(64, 2048 + 64, 512);
    EXPECT(moe_query(&s, NULL, NULL, NULL), MOE_ERR_UNSUPPORTED);
    s = shape(0, 2048, 512);
    EXPECT(moe_query(&s, NULL, NULL, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_query(NULL, NULL, NULL, NULL), MOE_ERR_INVALID_ARG);
    s = shape(64, 2048, 512);
    EXPECT(moe_route(&s, NULL, &w, &r, fake, 1u << 30, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_route(&s, fake, NULL, &r, fake, 1u << 30, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_route(&s, fake, &w, NULL, fake, 1u << 30, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_layer_chunked(&s, fake, &w, fake, 0, fake, 1u << 30, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_rmsnorm_residual(0, 2048, 1e-6f, fake, fake, fake, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_dequant_q4(NULL, 64, 64, fake, NULL), MOE_ERR_INVALID_ARG);
    for (int st = -5; st <= 0; ++st)
        if (!moe_status_str(st)) ++fails;
    if (fails) {
        fprintf(stderr, "%d unexpected results\n", fails);
        return 1;
    }
    printf("abi_check ok\n");
    return 0;
}
