// Batch-1 decode: one token through the router, top-8 and the nine selected
// experts (eight routed + the shared one).  At batch 1 there is no weight
// reuse, so the path is bound by how fast the selected experts' packed
// weights stream from HBM (mechatronicstore.cl, "Decode: mover menos bytes
// por token"; neuro-ai.ru, "Спекулятивное декодирование не взлетело").  Only
// the picked experts' rows are read; the expert ids never leave the device.
//
// Three short kernels over the tile layout (one 9216-byte block per 256
// columns x 64 inputs); no kernel combines results across workgroups:
//  1. router: one wave per expert computes its logit exactly in the fixed
//     order (sequential within each 64-chunk, then over chunks, then + bias),
//     so the ids need no certification step at batch 1;
//  2. gate/up: a workgroup takes one slot and 32 gate + the 32 matching up
//     columns (2 KB of each block, contiguous) over all of K.  Every wave
//     takes the top-8 itself (logit descending, index ascending; softmax
//     weights restricted to them) and then issues all of its loads at once.
//     Codes become 128+q in bf16 with one and-or per pair and meet x in packed
//     bf16 dot products:
//        sum_k x_k (q_k s + b) = s (sum x (128 + q) - 128 sum x) + b sum x;
//     the two halves of a column meet by DPP, the waves' groups through LDS
//     in order, and h = silu(gate) * up is written in fp16;
//  3. down: a workgroup takes 32 outputs (1 KB of each block) for all nine
//     slots and all groups, with h of every slot staged in LDS; codes become
//     1024+q in fp16.  Each lane adds its slots in pick order with their
//     routing weights, then the shared expert, group by group.
#include "common.h"

namespace moe {


__device__ __forceinline__ uint32_t dec_and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
    return r;
}

// 1. logits[e] = sum over chunks c (in order) of sum_{k in chunk c} x_k w_ek (in order), + bias
__global__ __launch_bounds__(256) void decode_router_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ wr,
                                                            const float *__restrict__ bias, int H,
                                                            int E, float *__restrict__ logits) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    const int G = H / 64;          // <= 32 chunks: lane c < G sums chunk c
    float P = 0.0f;
    if (lane < G) {
        const u32x4 *px = (const u32x4 *)(x + 64 * lane);
        const u32x4 *pw = (const u32x4 *)(wr + (size_t)e * H + 64 * lane);
        u32x4 xv[8], wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            xv[j] = px[j];
            wv[j] = pw[j];
        }
        // bf16 x bf16 products are exact in fp32, so each fma adds one product
        // with a single rounding, exactly as the sequential sum does
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                P = __builtin_fmaf(bf16_lo(xv[j][r]), bf16_lo(wv[j][r]), P);
                P = __builtin_fmaf(bf16_hi(xv[j][r]), bf16_hi(wv[j][r]), P);
            }
    }
    // chunk sums in chunk order (uniform lane index: read as scalars)
    float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), 0));
    for (int c = 1; c < G; ++c) l += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), c));
    if (bias) l += bias[e];
    if (lane == 0) logits[e] = l;
}

// Top-k (k <= 8) of E = 256 logits by (logit desc, index asc) and the weights
// exp(l - l_1) / sum, computed by one wave (all lanes end with the same picks).
// wl: 32 words of wave-local LDS.
__device__ void select_topk(const float *__restrict__ logits, int E, int k, int *pick_e,
                            float *pick_w, uint32_t *wl) {
    const int lane = threadIdx.x & 63;
    uint32_t key[4];
    bool taken[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        key[j] = e < E ? ordered_key(logits[e]) : 0u;
    }
    int pe;
    uint32_t pkey;
    wave_topk_radix(key, k, taken, pe, pkey, wl);
    float pick_l[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        pick_e[r] = r < k ? __builtin_amdgcn_readlane(pe, r) : 0;
        pick_l[r] = r < k ? key_to_float((uint32_t)__builtin_amdgcn_readlane((int)pkey, r)) : 0.0f;
    }
    const float m = pick_l[0];
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        pick_w[r] = r < k ? expf(pick_l[r] - m) : 0.0f;
        sum += pick_w[r];
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) pick_w[r] = pick_w[r] / sum;
}

constexpr int DW = 8;                  // waves per decode workgroup
constexpr int NSLOT = 9;               // top-8 routed experts + the shared one (top_k is 8)

// code pair p of word w as two 16-bit values q_p, q_{p+4} in a magic-number
// format (and-or with C = 128.0 bf16 pairs or 1024.0 fp16 pairs)
// x (or h) pairs in the same order: (v_p, v_{p+4}) of each 8-block
__device__ __forceinline__ void pair_order(const u32x4 v, uint32_t *o) {
    o[0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
}

// sum of lanes l and l ^ 1
__device__ __forceinline__ float pair_sum(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// 2. gate/up.  Workgroup (slot, tile j, slice q of 32 gate + 32 up columns);
// wave w takes groups w, w + DW, ...
__global__ __launch_bounds__(64 * DW) void decode_gateup_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ logits, int H, int I, int k, int E,
    const uint8_t *__restrict__ pk, const uint8_t *__restrict__ pk_sh, int32_t *__restrict__ ids_out,
    float *__restrict__ tw_out, uint16_t *__restrict__ hbuf) {
    __shared__ float red[DW][2][32];
    __shared__ uint32_t selw[DW][32];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int G = H / 64, JT = I / 128;
    const int b = blockIdx.x;
    const int slot = b / (JT * 4), j = (b >> 2) % JT, q = b & 3;
    int ex = 0;
    if (slot < k) {
        int pe[8];
        float pw[8];
        select_topk(logits, E, k, pe, pw, selw[wave]);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (r == slot) ex = pe[r];
        ex = (ex < 0 || ex >= E) ? 0 : ex;
        if (b == 0 && wave == 0 && lane < k) {
            int e = 0;
            float wv = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (r == lane) {
                    e = pe[r];
                    wv = pw[r];
                }
            ids_out[lane] = e;
            tw_out[lane] = wv;
        }
    }
    const uint8_t *tile = slot == k ? pk_sh + (size_t)j * G * PK_BLOCK
                                    : pk + ((size_t)ex * JT + j) * G * PK_BLOCK;
    const int hh = (lane & 1) ^ ((lane >> 4) & 1);      // logical half of my pieces
    const int cg = 64 * q + (lane >> 1);                 // my gate column; up is cg + 32
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t cM = 0x000F000Fu, cC = 0x43004300u;
    asm volatile("" : "+v"(cM), "+v"(cC));
    float ag = 0.0f, au = 0.0f;
    constexpr int GPW = 4;                               // groups per pass of a wave
    for (int g0 = wave; g0 < G; g0 += DW * GPW) {
        u32x4 cw[GPW][2];
        uint16_t sv[GPW][2], bv[GPW][2];
#pragma unroll
        for (int t = 0; t < GPW; ++t) {
            const int g = min(g0 + DW * t, G - 1);
            const uint8_t *blk = tile + (size_t)g * PK_BLOCK;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                cw[t][r] = *(const u32x4 *)(blk + 16 * (128 * q + 64 * r + lane));
                sv[t][r] = *(const uint16_t *)(blk + PK_CODES + 2 * (cg + 32 * r));
                bv[t][r] = *(const uint16_t *)(blk + PK_CODES + 512 + 2 * (cg + 32 * r));
            }
        }
#pragma unroll
        for (int t = 0; t < GPW; ++t) {
            const int g = g0 + DW * t;
            if (g >= G) break;
            const u32x4 *px = (const u32x4 *)(x + 64 * g + 32 * hh);
            uint32_t xp[16];
            float sx = 0.0f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const u32x4 v = px[qq];
                pair_order(v, xp + 4 * qq);
#pragma unroll
                for (int r = 0; r < 4; ++r) sx += bf16_lo(v[r]) + bf16_hi(v[r]);
            }
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                float d = 0.0f;
                const uint32_t ww[4] = {cw[t][r].x, cw[t][r].y, cw[t][r].z, cw[t][r].w};
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const uint32_t c = dec_and_or(ww[qq] >> (4 * p), cM, cC);
                        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c),
                                                            __builtin_bit_cast(bf16x2, xp[4 * qq + p]), d, false);
                    }
                const float v = bf16_to_f32(sv[t][r]) * (d - 128.0f * sx) + bf16_to_f32(bv[t][r]) * sx;
                if (r == 0) ag += v; else au += v;
            }
        }
    }
    ag = pair_sum(ag);
    au = pair_sum(au);
    if ((lane & 1) == 0) {
        red[wave][0][lane >> 1] = ag;
        red[wave][1][lane >> 1] = au;
    }
    __syncthreads();
    if (threadIdx.x < 32) {
        const int m = threadIdx.x;
        float gs = red[0][0][m], us = red[0][1][m];
#pragma unroll
        for (int w = 1; w < DW; ++w) {
            gs += red[w][0][m];
            us += red[w][1][m];
        }
        const int i = 128 * j + 32 * q + m;
        hbuf[(size_t)slot * I + i] = f32_to_f16(gs / (1.0f + expf(-gs)) * us);
    }
}

// 3. down.  Workgroup (tile j, slice q of 32 outputs); wave w takes groups
// w, w + DW, .. of every slot.
__global__ __launch_bounds__(64 * DW) void decode_down_kernel(
    const uint16_t *__restrict__ hbuf, int H, int I, const int32_t *__restrict__ ids,
    const float *__restrict__ tw, int k, int E, const uint8_t *__restrict__ pk,
    const uint8_t *__restrict__ pk_sh, float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    uint16_t *hs = (uint16_t *)dsm;                                  // fp16 [k+1][I]
    float *red = (float *)(dsm + (size_t)(k + 1) * I * 2);           // [DW][32]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
    const int G = I / 64, JD = H / 256;
    const int j = blockIdx.x >> 3, q = blockIdx.x & 7;
    const int hh = (lane & 1) ^ ((lane >> 4) & 1);
    const int col = 32 * q + (lane >> 1);
    int sid[8];
    float sw[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int e = r < k ? ids[r] : 0;
        sid[r] = (e < 0 || e >= E) ? 0 : e;
        sw[r] = r < k ? tw[r] : 0.0f;
    }
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    uint32_t cM = 0x000F000Fu, cC = 0x64006400u;
    asm volatile("" : "+v"(cM), "+v"(cC));
    float acc = 0.0f;
    bool staged = false;
    for (int g = wave; g < G || !staged; g += DW) {
        const int gg = min(g, G - 1);
        // this group's 1 KB slice of every slot's block
        u32x4 cw[NSLOT];
        uint16_t sv[NSLOT], bv[NSLOT];
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) {
            const uint8_t *blk = (s == k ? pk_sh + (size_t)j * G * PK_BLOCK
                                         : pk + ((size_t)sid[s] * JD + j) * G * PK_BLOCK) +
                                 (size_t)gg * PK_BLOCK;
            cw[s] = *(const u32x4 *)(blk + 16 * (64 * q + lane));
            sv[s] = *(const uint16_t *)(blk + PK_CODES + 2 * col);
            bv[s] = *(const uint16_t *)(blk + PK_CODES + 512 + 2 * col);
        }
        if (!staged) {                                  // h of every slot into LDS
            const int nh = (k + 1) * I / 8;
            for (int u = tid; u < nh; u += 64 * DW) ((u32x4 *)hs)[u] = ((const u32x4 *)hbuf)[u];
            __syncthreads();
            staged = true;
        }
        if (g >= G) break;
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) {
            uint32_t hp[16];
            float shs = 0.0f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const u32x4 v = *(const u32x4 *)(hs + (size_t)s * I + 64 * g + 32 * hh + 8 * qq);
                pair_order(v, hp + 4 * qq);
#pragma unroll
                for (int r = 0; r < 4; ++r) shs += f16_lo(v[r]) + f16_hi(v[r]);
            }
            float d = 0.0f;
            const uint32_t ww[4] = {cw[s].x, cw[s].y, cw[s].z, cw[s].w};
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t c = dec_and_or(ww[qq] >> (4 * p), cM, cC);
                    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, c), __builtin_bit_cast(h2, hp[4 * qq + p]),
                                               d, false);
                }
            const float v = bf16_to_f32(sv[s]) * (d - 1024.0f * shs) + bf16_to_f32(bv[s]) * shs;
            float wgt = 1.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (r == s) wgt = sw[r];
            acc = s < k ? __builtin_fmaf(wgt, v, acc) : acc + v;
        }
    }
    acc = pair_sum(acc);
    if ((lane & 1) == 0) red[wave * 32 + (lane >> 1)] = acc;
    __syncthreads();
    if (tid < 32) {
        float sum = red[tid];
#pragma unroll
        for (int w = 1; w < DW; ++w) sum += red[w * 32 + tid];
        y[256 * j + 32 * q + tid] = sum;
    }
}

void launch_decode(const moe_shape &sh, const uint16_t *x, const moe_weights &w, int32_t *ids,
                   float *tw, float *y, void *scratch, hipStream_t s) {
    const int H = sh.H, I = sh.I, E = sh.E, k = sh.top_k;
    char *p = (char *)scratch;
    float *logits = (float *)p;                 // [E]
    uint16_t *hbuf = (uint16_t *)(p + 4096);    // fp16 [k+1][I]
    if (k + 1 != NSLOT) return;                 // the API admits top_k = 8 only
    const PackLayout P = pack_layout(H, I, E);
    const uint8_t *pk = (const uint8_t *)w.packed;
    hipLaunchKernelGGL(decode_router_kernel, dim3((E + 3) / 4), dim3(256), 0, s, x, w.router_wt,
                       w.router_bias, H, E, logits);
    hipLaunchKernelGGL(decode_gateup_kernel, dim3((k + 1) * (I / 128) * 4), dim3(64 * DW), 0, s, x,
                       logits, H, I, k, E, pk + P.gu, pk + P.sh_gu, ids, tw, hbuf);
    const size_t lds = (size_t)(k + 1) * I * 2 + DW * 32 * 4;
    hipLaunchKernelGGL(decode_down_kernel, dim3((H / 256) * 8), dim3(64 * DW), lds, s, hbuf, H, I,
                       ids, tw, k, E, pk + P.down, pk + P.sh_down, y);
}

size_t decode_scratch_bytes(int H, int I, int k) {
    (void)H;
    return 4096 + (size_t)(k + 1) * I * 2;
}

}  // namespace moe
