// Batch-1 decode: one token through the router, top-8 and the nine selected
// experts (eight routed + the shared one).  At batch 1 there is no weight
// reuse, so the path is bound by how fast the selected experts' packed
// weights stream from HBM (mechatronicstore.cl, "Decode: mover menos bytes
// por token"; neuro-ai.ru, "Спекулятивное декодирование не взлетело").  Only
// the picked experts' rows are read; the expert ids never leave the device.
//
// Per weight row the dot product uses the same split as the prefill GEMM:
//   sum_k x_k (q_k s + b) = s * sum x_k q_k + b * sum x_k   (per 64-group),
// all in fp32 on the vector ALUs (no matrix cores at batch 1).
#include "common.h"

namespace moe {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// dot of one packed word (8 codes) with 8 fp32 activations: returns sum x*q, and sum x in *sx
__device__ __forceinline__ float word_dot(uint32_t w, const float *xv, float *sx) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    float d = xv[0] * (float)(lo & 0xffu);
    d = __builtin_fmaf(xv[2], (float)((lo >> 8) & 0xffu), d);
    d = __builtin_fmaf(xv[4], (float)((lo >> 16) & 0xffu), d);
    d = __builtin_fmaf(xv[6], (float)(lo >> 24), d);
    d = __builtin_fmaf(xv[1], (float)(hi & 0xffu), d);
    d = __builtin_fmaf(xv[3], (float)((hi >> 8) & 0xffu), d);
    d = __builtin_fmaf(xv[5], (float)((hi >> 16) & 0xffu), d);
    d = __builtin_fmaf(xv[7], (float)(hi >> 24), d);
    *sx = ((xv[0] + xv[1]) + (xv[2] + xv[3])) + ((xv[4] + xv[5]) + (xv[6] + xv[7]));
    return d;
}

// gate/up rows: wave = one intermediate index i of one of the nine slots
__global__ __launch_bounds__(256) void decode_gateup_kernel(
    const uint16_t *__restrict__ x, int H, int I, const int32_t *__restrict__ ids, int k,
    GemmProj gate, GemmProj up, GemmProj sgate, GemmProj sup, float *__restrict__ hbuf) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gi = blockIdx.x * 4 + wave;
    const int slot = gi / I, i = gi % I;
    if (slot > k) return;
    const bool sh = slot == k;
    const int ex = sh ? 0 : ids[slot];
    if (ex < 0 || ex >= 256) return;
    const size_t rr = sh ? (size_t)i : (size_t)ex * I + i;
    const GemmProj pg = sh ? sgate : gate, pu = sh ? sup : up;
    const int W = H / 8, G = H / 64;
    const uint32_t *qg = pg.q + rr * W, *qu = pu.q + rr * W;
    const uint16_t *sg = pg.s + rr * G, *bg = pg.b + rr * G;
    const uint16_t *su = pu.s + rr * G, *bu = pu.b + rr * G;
    float accg = 0.0f, accu = 0.0f;
    for (int wd = lane; wd < W; wd += 64) {
        const u32x4 xr = *(const u32x4 *)(x + 8 * wd);
        const float xv[8] = {bf16_lo(xr.x), bf16_hi(xr.x), bf16_lo(xr.y), bf16_hi(xr.y),
                             bf16_lo(xr.z), bf16_hi(xr.z), bf16_lo(xr.w), bf16_hi(xr.w)};
        const int g = wd >> 3;
        float sx;
        const float dg = word_dot(qg[wd], xv, &sx);
        const float du = word_dot(qu[wd], xv, &sx);
        accg += bf16_to_f32(sg[g]) * dg + bf16_to_f32(bg[g]) * sx;
        accu += bf16_to_f32(su[g]) * du + bf16_to_f32(bu[g]) * sx;
    }
    accg = wave_sum(accg);
    accu = wave_sum(accu);
    if (lane == 0) hbuf[(size_t)slot * I + i] = accg / (1.0f + expf(-accg)) * accu;
}

// down rows: wave = one output n; sums the nine slots with their routing weights
__global__ __launch_bounds__(256) void decode_down_kernel(const float *__restrict__ hbuf, int H,
                                                          int I, const int32_t *__restrict__ ids,
                                                          const float *__restrict__ tw, int k,
                                                          GemmProj down, GemmProj sdown,
                                                          float *__restrict__ y) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + wave;
    if (n >= H) return;
    const int W = I / 8, G = I / 64;
    float total = 0.0f;
    for (int slot = 0; slot <= k; ++slot) {
        const bool sh = slot == k;
        const int ex = sh ? 0 : ids[slot];
        if (ex < 0 || ex >= 256) continue;
        const size_t rr = sh ? (size_t)n : (size_t)ex * H + n;
        const GemmProj p = sh ? sdown : down;
        const float wt = sh ? 1.0f : tw[slot];
        const float *hv = hbuf + (size_t)slot * I;
        float acc = 0.0f;
        for (int wd = lane; wd < W; wd += 64) {
            const float4 h0 = *(const float4 *)(hv + 8 * wd);
            const float4 h1 = *(const float4 *)(hv + 8 * wd + 4);
            const float xv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            float sx;
            const float d = word_dot(p.q[rr * W + wd], xv, &sx);
            const int g = wd >> 3;
            acc += bf16_to_f32(p.s[rr * G + g]) * d + bf16_to_f32(p.b[rr * G + g]) * sx;
        }
        total = __builtin_fmaf(wt, acc, total);
    }
    total = wave_sum(total);
    if (lane == 0) y[n] = total;
}

void launch_decode(const moe_shape &sh, const uint16_t *x, const moe_weights &w, int32_t *ids,
                   float *tw, float *y, void *scratch, hipStream_t s) {
    const int H = sh.H, I = sh.I, E = sh.E, k = sh.top_k;
    char *p = (char *)scratch;
    float *part = (float *)p;           // [4][1][E]
    p += 4096;
    float *wn2 = (float *)p;            // [4][E]
    p += 4096;
    float *xsum = (float *)p;           // [H/64]
    p += 256;
    float *xsq = (float *)p;            // [H/64]
    p += 256;
    int32_t *blk_cnt = (int32_t *)p;    // [1][E]
    p += 1024;
    int32_t *lrank = (int32_t *)p;      // [k]
    p += 256;
    uint16_t *xp = (uint16_t *)p;       // [H]
    p += 2 * 2048;
    float *hbuf = (float *)p;           // [k+1][I]
    launch_router_fast(x, w.router_wt, 1, H, E, part, wn2, xp, xsum, xsq, s);
    launch_route_select(part, nullptr, xsq, wn2, w.router_bias, x, w.router_wt, 1, H, E, k, ids,
                        tw, blk_cnt, lrank, s);
    const GemmProj gate{w.gate.q, w.gate.scale, w.gate.bias}, up{w.up.q, w.up.scale, w.up.bias};
    const GemmProj sgate{w.sh_gate.q, w.sh_gate.scale, w.sh_gate.bias};
    const GemmProj sup{w.sh_up.q, w.sh_up.scale, w.sh_up.bias};
    const GemmProj down{w.down.q, w.down.scale, w.down.bias};
    const GemmProj sdown{w.sh_down.q, w.sh_down.scale, w.sh_down.bias};
    const int rows = (k + 1) * I;
    hipLaunchKernelGGL(decode_gateup_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, x, H, I, ids,
                       k, gate, up, sgate, sup, hbuf);
    hipLaunchKernelGGL(decode_down_kernel, dim3((H + 3) / 4), dim3(256), 0, s, hbuf, H, I, ids,
                       tw, k, down, sdown, y);
}

size_t decode_scratch_bytes(int I, int k) { return 20480 + (size_t)(k + 1) * I * 4; }

}  // namespace moe
