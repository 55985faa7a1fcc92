// Router logits, top-k, and GPU-resident routing structures (histogram,
// prefix scan, stable token scatter, block map) -- the routing work that the
// Lily pages keep inside one GPU command buffer with no CPU synchronisation
// (mechatronicstore.cl, "Prefill: pesos comprimidos y enrutamiento en la GPU";
// lefilia.fr body).  Here it is three kernels on one stream; the block count
// never leaves the device.
#include "common.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits in the fixed float32 order: inside each chunk of 64 inputs a
// sequential sum that starts from the chunk's first product, then a
// sequential sum of the chunk partials from chunk 0, then + bias.  Products of
// two bf16 values are exact in fp32, so each step is one fma.
//
// Tile: 32 tokens x 64 experts per workgroup.  A round stages 4 chunks (256
// inputs) of x and of the router rows in LDS as fp32; wave g computes the
// partials of chunk 4*round+g for the whole tile (each lane a 4x8 block, 32
// independent chains); the partials go through LDS and each thread adds its 8
// outputs' partials in chunk order.
// ---------------------------------------------------------------------------
constexpr int RT_T = 32, RT_E = 64, RT_CH = 4, RT_LD = 256 + 4;

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ wr,
                                                            const float *__restrict__ bias, int T,
                                                            int H, int E,
                                                            float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) float xs[RT_T][RT_LD];
    __shared__ __attribute__((aligned(16))) float wsm[RT_E][RT_LD];
    __shared__ __attribute__((aligned(16))) float ps[RT_CH][RT_T][RT_E];

    const int t0 = blockIdx.x * RT_T, e0 = blockIdx.y * RT_E;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tb = lane >> 3, eb = lane & 7;
    const int nchunks = H / 64;
    const int own_t = (tid * 8) / RT_E, own_e = (tid * 8) % RT_E;
    float total[8];

    for (int r = 0; r * RT_CH < nchunks; ++r) {
        const int kbase = r * 256;
        const int kn = min(256, H - kbase);
        const int segs = kn / 8;
        __syncthreads();
        for (int idx = tid; idx < RT_T * segs; idx += 256) {
            const int row = idx / segs, seg = idx % segs;
            const int t = t0 + row;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t < T) v = *(const u32x4 *)(x + (size_t)t * H + kbase + seg * 8);
            float4 *d = (float4 *)&xs[row][seg * 8];
            d[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
            d[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
        }
        for (int idx = tid; idx < RT_E * segs; idx += 256) {
            const int row = idx / segs, seg = idx % segs;
            u32x4 v = *(const u32x4 *)(wr + (size_t)(e0 + row) * H + kbase + seg * 8);
            float4 *d = (float4 *)&wsm[row][seg * 8];
            d[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
            d[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
        }
        __syncthreads();
        if (wave * 64 < kn) {
            float acc[4][8];
            const int kc = wave * 64;
#pragma unroll
            for (int k = 0; k < 64; k += 4) {
                float4 xv[4], wv[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = *(const float4 *)&xs[4 * tb + i][kc + k];
#pragma unroll
                for (int j = 0; j < 8; ++j) wv[j] = *(const float4 *)&wsm[eb + 8 * j][kc + k];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (k == 0)
                            acc[i][j] = xv[i].x * wv[j].x;
                        else
                            acc[i][j] = __builtin_fmaf(xv[i].x, wv[j].x, acc[i][j]);
                        acc[i][j] = __builtin_fmaf(xv[i].y, wv[j].y, acc[i][j]);
                        acc[i][j] = __builtin_fmaf(xv[i].z, wv[j].z, acc[i][j]);
                        acc[i][j] = __builtin_fmaf(xv[i].w, wv[j].w, acc[i][j]);
                    }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) ps[wave][4 * tb + i][eb + 8 * j] = acc[i][j];
        }
        __syncthreads();
        const int nc = min(RT_CH, nchunks - r * RT_CH);
        for (int c = 0; c < nc; ++c) {
            const float4 p0 = *(const float4 *)&ps[c][own_t][own_e];
            const float4 p1 = *(const float4 *)&ps[c][own_t][own_e + 4];
            const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int o = 0; o < 8; ++o) total[o] = (r == 0 && c == 0) ? pv[o] : total[o] + pv[o];
        }
    }
    const int t = t0 + own_t;
    if (t < T) {
        float v[8];
#pragma unroll
        for (int o = 0; o < 8; ++o) v[o] = bias ? total[o] + bias[e0 + own_e + o] : total[o];
        float4 *d = (float4 *)(out + (size_t)t * E + e0 + own_e);
        d[0] = make_float4(v[0], v[1], v[2], v[3]);
        d[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

void launch_router_logits(const uint16_t *x, const uint16_t *wr_t, const float *bias, int T, int H,
                          int E, float *logits, hipStream_t s) {
    dim3 grid((T + RT_T - 1) / RT_T, E / RT_E);
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, s, x, wr_t, bias, T, H, E, logits);
}

// ---------------------------------------------------------------------------
// Fast certified routing.
//
// 1. router_mfma: approximate logits on the matrix cores, split over K into S
//    partial sums (each 64-wide chunk is one 4-step MFMA chain from zero,
//    chunks added in fp32).  Whatever order or rounding the hardware uses
//    inside a chain, |approx - exact| <= (2*63 + 32) u (sum|x_k w_k| + |b|)
//    with u = 2^-24, and the fixed-order logit is within 95 u of the same
//    quantity, so every approximate logit lies within
//        delta = 2^-16 (||x|| ||w|| + |b|)  (+ a denormal guard)
//    of the fixed-order logit (Cauchy-Schwarz bounds sum|x_k w_k|).
// 2. route_select (one wave per token): the top-8 by approximate logits, and
//    every other expert whose interval reaches the lowest lower bound of those
//    8, are the only experts that can hold a top-8 fixed-order logit.  Their
//    fixed-order logits are recomputed exactly (same order as router_logits)
//    and the top-8 is taken from those, so the ids equal those of the
//    fixed-order logits bit for bit, and the routing weights are computed from
//    the exact logits of the picks.
// ---------------------------------------------------------------------------
constexpr int TB = kTB;           // tokens per routing block (one wave each)
constexpr int RS_SPLIT = 4;       // K splits of the approximate router

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// 8 bf16 values -> fp16, in order.  Exact for |x| in the fp16 normal range (bf16 has
// 8 significant bits, fp16 11).
__device__ __forceinline__ u32x4 to_f16x8(u32x4 v) {
    u32x4 o;
    o.x = pack_f16x2(bf16_lo(v.x), bf16_hi(v.x));
    o.y = pack_f16x2(bf16_lo(v.y), bf16_hi(v.y));
    o.z = pack_f16x2(bf16_lo(v.z), bf16_hi(v.z));
    o.w = pack_f16x2(bf16_lo(v.w), bf16_hi(v.w));
    return o;
}

// Approximate logits (no bias), partial over K range s: part[s][t][e].  A
// workgroup takes 32 tokens x one half of the 256 experts x one K range: per
// 64-wide chunk the x rows (4 KB) and the half's router rows (16 KB) are copied
// into a 4-stage LDS ring by whole-line DMA (16-byte slots XOR-swizzled by row,
// so that the MFMA operand reads are free of bank conflicts), three chunks
// ahead, and wave w computes experts 128 h + 32 w .. + 31.  The ring is 80 KB, so
// two workgroups share a CU.  The expert-half-0 workgroups also prepare x for
// the expert GEMM from the staged chunk (fp16, and per group of 64 the sum, the
// sum of squares and the largest magnitude), and the workgroups of token tile 0
// the squared norms of their router rows per K range.
constexpr int RT_TOK = 32;
constexpr int RT_EH = 128;                        // experts per workgroup (half of 256)
constexpr int RX_BYTES = RT_TOK * 128;            // x chunk [32 rows][8 x 16 B]
constexpr int RW_BYTES = RT_EH * 128;             // router chunk [128 rows][8 x 16 B]
constexpr int R_STAGE = RX_BYTES + RW_BYTES;
constexpr int R_NST = 4;
constexpr int R_PER = 1 + RT_EH / 32;             // copies per thread and chunk

// global->LDS copy of 16 B per lane (inline asm: the statement keeps the wait state that gfx9
// needs between the M0 write and the LDS DMA reading it)
__device__ __forceinline__ void rdma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}

__global__ __launch_bounds__(256, 2) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, int T, int H, int E, int S,
    float *__restrict__ part, uint16_t *__restrict__ xp, float *__restrict__ xsum,
    float *__restrict__ xsq, float *__restrict__ wn2part, float *__restrict__ xmx,
    int32_t *__restrict__ zbuf, int nzero) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t rsm[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)rsm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, gg = lane >> 5;
    const int t0 = blockIdx.x * RT_TOK, sp = blockIdx.y, e0 = blockIdx.z * RT_EH;
    const int klen = H / S, kbeg = sp * klen, nch = klen / 64, G = H / 64;
    const bool do_prep = blockIdx.z == 0;          // x preparation: one expert half only
    // DMA: thread tid copies slot tid&7 of row tid/8 (x) and of rows 32 i + tid/8
    // (router); the slot holds segment slot ^ (row & 7) of the row's 128 bytes
    const int seg = (tid & 7) ^ ((tid >> 3) & 7);
    const uint16_t *xsrc = x + (size_t)min(t0 + (tid >> 3), T - 1) * H + kbeg + 8 * seg;
    const uint16_t *wsrc = wr + (size_t)(e0 + (tid >> 3)) * H + kbeg + 8 * seg;
    auto issue = [&](int c) {
        const uint32_t base = lds0 + (uint32_t)((c % R_NST) * R_STAGE);
        rdma16(xsrc + 64 * c, base + (uint32_t)(wave * 1024));
#pragma unroll
        for (int i = 0; i < RT_EH / 32; ++i)
            rdma16(wsrc + (size_t)32 * i * H + 64 * c, base + (uint32_t)(RX_BYTES + 4096 * i + wave * 1024));
    };
#pragma unroll
    for (int c = 0; c < R_NST - 1; ++c)
        if (c < nch) issue(c);
    floatx16 tot;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot[i] = 0.0f;
    const floatx16 zero = {};
    float wsq = 0.0f;
    const bool do_norm = blockIdx.x == 0 && tid < RT_EH;
    // x preparation results, stored after the loop: a store issued inside it
    // would count against the DMA waits (one vmcnt for loads and stores)
    constexpr int MAXCH = 8;                       // H <= 2048, four K ranges
    u32x4 xpv[MAXCH];
    float s1v[MAXCH], s2v[MAXCH], mxv[MAXCH];
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
        if (c >= nch) break;
        // chunks issued after c: min(R_NST - 2, nch - 1 - c), R_PER copies each
        const int after = min(R_NST - 2, nch - 1 - c);
        if (after >= 2)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * R_PER) : "memory");
        else if (after == 1)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(R_PER) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();                           // chunk c in; chunk c-1 no longer read
        if (c + R_NST - 1 < nch) issue(c + R_NST - 1);
        const uint8_t *sx = rsm + (c % R_NST) * R_STAGE;
        const uint8_t *sw = sx + RX_BYTES;
        // 32 tokens x 32 experts per wave: per 16-wide k step j, segment 2 j + gg of the rows
        floatx16 p;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int sg = 2 * j + gg;
            const bf16x8 av = *(const bf16x8 *)(sx + l32 * 128 + 16 * (sg ^ (l32 & 7)));
            const int el = 32 * wave + l32;
            const bf16x8 bv = *(const bf16x8 *)(sw + el * 128 + 16 * (sg ^ (el & 7)));
            p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, j == 0 ? zero : p, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tot[i] += p[i];
        // x preparation: thread -> row tid/8, 16-byte segment tid&7 of the chunk
        if (do_prep) {
            const int row = tid >> 3, sg = tid & 7;
            const u32x4 v = *(const u32x4 *)(sx + row * 128 + 16 * (sg ^ (row & 7)));
            float s1 = 0.0f, s2 = 0.0f, mx = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s1 += bf16_lo(v[q]) + bf16_hi(v[q]);
                s2 = __builtin_fmaf(bf16_lo(v[q]), bf16_lo(v[q]), s2);
                s2 = __builtin_fmaf(bf16_hi(v[q]), bf16_hi(v[q]), s2);
                mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(v[q])), fabsf(bf16_hi(v[q]))));
            }
            s1v[c] = group_sum_dpp(s1, 8);
            s2v[c] = group_sum_dpp(s2, 8);
            mxv[c] = group_max_dpp8(mx);
            xpv[c] = to_f16x8(v);
        }
        if (do_norm) {                             // thread tid = router row e0 + tid
            const uint8_t *rw = sw + tid * 128;
#pragma unroll
            for (int sg = 0; sg < 8; ++sg) {
                // slots in a row-dependent order: eight lanes read eight banks
                const u32x4 v = *(const u32x4 *)(rw + 16 * (sg ^ (tid & 7)));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    wsq = __builtin_fmaf(bf16_lo(v[q]), bf16_lo(v[q]), wsq);
                    wsq = __builtin_fmaf(bf16_hi(v[q]), bf16_hi(v[q]), wsq);
                }
            }
        }
    }
    if (do_norm) wn2part[(size_t)sp * E + e0 + tid] = wsq;
    // the select kernel's superblock counters start at zero (stored after the
    // loop, like every store of this kernel)
    if (blockIdx.x == 0 && sp == 0 && blockIdx.z == 0)
        for (int i = tid; i < nzero; i += 256) zbuf[i] = 0;
    if (do_prep) {
        const int row = tid >> 3, sg = tid & 7;
        if (t0 + row < T) {
#pragma unroll
            for (int c = 0; c < MAXCH; ++c) {
                if (c >= nch) break;
                *(u32x4 *)(xp + (size_t)(t0 + row) * H + kbeg + 64 * c + 8 * sg) = xpv[c];
                if (sg == 0) {
                    const size_t gi = (size_t)(t0 + row) * G + kbeg / 64 + c;
                    xsum[gi] = s1v[c];
                    xsq[gi] = s2v[c];
                    xmx[gi] = mxv[c];
                }
            }
        }
    }
    float *out = part + (size_t)sp * T * E;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = t0 + 8 * (i >> 2) + 4 * gg + (i & 3);
        if (t < T) out[(size_t)t * E + e0 + 32 * wave + l32] = tot[i];
    }
}

// s_waitcnt vmcnt(n) for a wave-uniform n in 0..12
__device__ __forceinline__ void wait_vm_upto12(int n) {
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    }
}

// Per-wave LDS stage of the exact recompute: four 4 KB slots, one router row
// (or the token's x row) each, in 128-byte chunks of 64 inputs; 16-byte slot s
// of chunk c holds segment s ^ (c & 7) of the chunk, so that the 32 lanes
// reading one chunk each hit distinct banks.
constexpr int XS_SLOT = 4096;
constexpr int XS_WAVE = 4 * XS_SLOT;

// DMA of one row of H bf16 values into a 4 KB stage slot (LDS address dst) in the
// swizzled chunk layout: instruction j copies chunks 8 j .. 8 j + 7, lane l
// filling slot l & 7 of chunk 8 j + (l >> 3) (a chunk past the row: any valid one).
__device__ __forceinline__ void stage_row(const uint16_t *row, int H, int lane, uint32_t dst) {
    const int nch = H / 64, ipr = (nch + 7) >> 3;
    const int dch = lane >> 3, dseg = (lane & 7) ^ dch;
    for (int j = 0; j < ipr; ++j) {
        const int cc = 8 * j + dch < nch ? 8 * j + dch : 0;
        rdma16(row + 64 * cc + 8 * dseg, dst + (uint32_t)(1024 * j));
    }
}

// Fixed-order logits of the n experts elist[0..n) (n <= 256) of one token into
// out[0..n) (wave-local LDS); bv holds every expert's bias (expert e in lane e & 63,
// slot e >> 6).
// The token's x row is already in slot 3 of the wave's stage (stage /
// stage_lds: its generic and LDS addresses).  The router rows travel by DMA
// into slots 0-2 at once and into slot 3 once x is in registers; round r takes
// rows 4 r .. 4 r + 3 (slots 0-3) and then refills all four slots with the next
// round's rows.  Half h of the wave takes rows 4 r + h and 4 r + 2 + h, lane c
// of the half chunk c of both, each summed sequentially from its first product
// (two independent chains per lane).  The chunk partials of 8 rows collect in
// part (256 floats); after every second round lanes 0-7 add one row's 32
// partials each in chunk order, then its bias.
__device__ void exact_logits(const uint32_t *elist, int n, float *out, const float (&bv)[4],
                             const uint16_t *__restrict__ wr, int H, int lane, float *part,
                             const uint8_t *stage, uint32_t stage_lds) {
    const int c = lane & 31, hh = lane >> 5, nch = H / 64;
    const int ipr = (nch + 7) >> 3;               // DMA instructions per row (1 KB each)
    auto issue = [&](int i) {
        stage_row(wr + (size_t)elist[i] * H, H, lane, stage_lds + (uint32_t)(XS_SLOT * (i & 3)));
    };
    // vmcnt(0), in the form the compiler's own wait bookkeeping sees: x has landed,
    // and no load of the caller is in flight from here on, so the compiler adds no
    // waits of its own between the copies below and the explicit waits for them
    __builtin_amdgcn_s_waitcnt(0x0F70);
    const int pre = n < 3 ? n : 3;
    for (int i = 0; i < pre; ++i) issue(i);
    // while they travel: out[i] = the bias of elist[i] (expert e's sits in lane e & 63 of
    // bv, slot e >> 6)
    for (int g = 0; g < n; g += 64) {
        const int ci = g + lane;
        const int ee = ci < n ? (int)elist[ci] : 0;
        float b = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float bj = __shfl(bv[j], ee & 63);
            if ((ee >> 6) == j) b = bj;
        }
        if (ci < n) out[ci] = b;
    }
    u32x4 xv[8];
    if (c < nch) {
        const uint8_t *xs = stage + 3 * XS_SLOT + 128 * c;
#pragma unroll
        for (int q = 0; q < 8; ++q) xv[q] = *(const u32x4 *)(xs + 16 * (q ^ (c & 7)));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot 3 is refilled next
    int next = pre;
    if (next < n) issue(next++);
    for (int r = 0; 4 * r < n; ++r) {
        const int need = 4 * r + 4 < n ? 4 * r + 4 : n;
        wait_vm_upto12((next - need) * ipr);
        const int ia = 4 * r + hh, ib = ia + 2;
        if (c < nch) {
            const uint8_t *wa = stage + XS_SLOT * hh + 128 * c;
            const uint8_t *wb = stage + XS_SLOT * (2 + hh) + 128 * c;
            u32x4 va[8], vb[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                va[q] = *(const u32x4 *)(wa + 16 * (q ^ (c & 7)));
                vb[q] = *(const u32x4 *)(wb + 16 * (q ^ (c & 7)));
            }
            // sequential within the chunk, from its first product (each fma adds one exact
            // product); rows past n read a stale slot and are never used
            float sa = bf16_lo(xv[0][0]) * bf16_lo(va[0][0]);
            float sb = bf16_lo(xv[0][0]) * bf16_lo(vb[0][0]);
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (q > 0 || u > 0) {
                        sa = __builtin_fmaf(bf16_lo(xv[q][u]), bf16_lo(va[q][u]), sa);
                        sb = __builtin_fmaf(bf16_lo(xv[q][u]), bf16_lo(vb[q][u]), sb);
                    }
                    sa = __builtin_fmaf(bf16_hi(xv[q][u]), bf16_hi(va[q][u]), sa);
                    sb = __builtin_fmaf(bf16_hi(xv[q][u]), bf16_hi(vb[q][u]), sb);
                }
            part[32 * (ia & 7) + c] = sa;
            part[32 * (ib & 7) + c] = sb;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this round's slots are refilled next
        __builtin_amdgcn_wave_barrier();
        for (int u = 0; u < 4 && next < n; ++u) issue(next++);
        if ((r & 1) || 4 * r + 4 >= n) {
            // rows 8 g .. 8 g + 7 complete: lane l adds row 8 g + l's partials in chunk order
            const int i = 8 * (r >> 1) + lane;
            if (lane < 8 && i < n) {
                const float4 *pp = (const float4 *)(part + 32 * lane);
                float v[32];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float4 f = pp[q];
                    v[4 * q] = f.x;
                    v[4 * q + 1] = f.y;
                    v[4 * q + 2] = f.z;
                    v[4 * q + 3] = f.w;
                }
                float L = v[0];
#pragma unroll
                for (int q = 1; q < 32; ++q)
                    if (q < nch) L = L + v[q];
                out[i] = L + out[i];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// EXACT: every logit given in `exact` (fixed order); else the approximate partials.
template <bool EXACT>
__global__ __launch_bounds__(64 * TB) void route_select_kernel(
    const float *__restrict__ part, int S, const float *__restrict__ exact,
    const float *__restrict__ xsq, int G, const float *__restrict__ wn2,
    const float *__restrict__ bias, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ wr, int T, int H, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ tw, int32_t *__restrict__ blk_cnt, int32_t *__restrict__ lrank,
    int32_t *__restrict__ sup, const float *__restrict__ xmx, uint16_t *__restrict__ xp,
    float *__restrict__ xsum, float *__restrict__ tok) {
    __shared__ uint32_t mask[256];
    __shared__ int32_t sid[TB][8];
    __shared__ uint32_t cand_e[TB][256];
    __shared__ __attribute__((aligned(16))) float cand_l[TB][256];
    __shared__ __attribute__((aligned(16))) float scr[TB][64];
    __shared__ __attribute__((aligned(16))) float xpart[TB][256];   // exact recompute: 8 rows' chunk partials
    extern __shared__ __attribute__((aligned(1024))) uint8_t xstage[];   // [TB][XS_WAVE]
    const uint32_t xstage_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)xstage;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tl = wave, t = blockIdx.x * TB + tl;
    if (tid < 256) mask[tid] = 0u;
    __syncthreads();
    const uint8_t *stage = xstage + XS_WAVE * tl;
    const uint32_t stage_lds = xstage_lds + (uint32_t)(XS_WAVE * tl);
    if (t < T) {
        // the token's x row, for the fixed-order logits below, goes to slot 3 of the
        // wave's stage now, ahead of everything else
        if (!EXACT) stage_row(x + (size_t)t * H, H, lane, stage_lds + 3 * XS_SLOT);
        // ---- logits (approximate or exact) and their error radius
        float lt[4], dl[4];
        // every load of this phase goes out before the first wait: the token's
        // sums of squares and group maxima, all RS_SPLIT partials and norms (or
        // the exact logits), and the biases.  No load sits under a branch (a
        // branch between loads makes the compiler wait at it): out-of-range
        // lanes and a missing bias read a valid address and discard the value.
        float bv[4];
        const int gi = lane < G ? lane : 0;
        float ss = xsq[(size_t)t * G + gi];
        float xm = xmx[(size_t)t * G + gi];
        const float *bsrc = bias ? bias : (exact ? exact : wn2);   // >= E floats each
        if (EXACT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                bv[j] = bsrc[e];
                lt[j] = exact[(size_t)t * E + e];
                dl[j] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!bias) bv[j] = 0.0f;
        } else {
            float pv[4][RS_SPLIT], wv[4][RS_SPLIT];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                bv[j] = bsrc[e];
#pragma unroll
                for (int sp = 0; sp < RS_SPLIT; ++sp) {
                    pv[j][sp] = part[((size_t)sp * T + t) * E + e];
                    wv[j][sp] = wn2[(size_t)sp * E + e];
                }
            }
            if (lane >= G) ss = 0.0f;
            const float nx = sqrtf(wave_sum_f(ss));   // ||x||
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!bias) bv[j] = 0.0f;
                float v = pv[j][0], w2 = wv[j][0];
#pragma unroll
                for (int sp = 1; sp < RS_SPLIT; ++sp) {
                    v += pv[j][sp];
                    w2 += wv[j][sp];
                }
                lt[j] = v + bv[j];
                dl[j] = 0x1p-16f * (sqrtf(w2) * nx * 1.001f + fabsf(bv[j])) + 0x1p-100f;
            }
        }
        if (lane >= G) {
            ss = 0.0f;
            xm = 0.0f;
        }
        // ---- top-k of the (approximate) logits, ties to the lower index
        bool taken[4];
        uint32_t key[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            key[j] = ordered_key(lt[j]);
            taken[j] = false;
        }
        int my_pick = -1;
        float wl = 0.0f;   // the pick's logit (lanes < k)
        if (EXACT) {
            int pe;
            uint32_t pkey;
            wave_topk_radix(key, k, taken, pe, pkey, (uint32_t *)scr[tl]);
            my_pick = lane < k ? pe : -1;
            wl = lane < k ? key_to_float(pkey) : 0.0f;
        } else {
            // Every exact logit lies within d of its approximation.  An expert whose
            // interval [l - d, l + d] ends below m8, the lowest lower bound of the k
            // largest approximations, has an exact logit below all of theirs, so the
            // exact top-k lies among those k and the experts whose intervals reach m8.
            // These candidates get their fixed-order logits, and the top-k is taken
            // among the exact values (their order here does not matter).
            wave_topk_set(key, k, taken);
            uint32_t nk = 0u;   // max of ~key(l - d) over the k: ~key of the lowest bound
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t v = taken[j] ? ~ordered_key(lt[j] - dl[j]) : 0u;
                nk = v > nk ? v : nk;
            }
            const float m8 = key_to_float(~wave_umax(nk));
            int nc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool c = taken[j] || lt[j] + dl[j] >= m8;
                const uint64_t bal = __ballot(c);
                const int pos = nc + (int)__popcll(bal & ((1ull << lane) - 1ull));
                if (c) cand_e[tl][pos] = lane + 64 * j;
                nc += (int)__popcll(bal);
            }
            __builtin_amdgcn_wave_barrier();
            exact_logits(cand_e[tl], nc, cand_l[tl], bv, wr, H, lane, xpart[tl], stage, stage_lds);
            __builtin_amdgcn_wave_barrier();
            if (nc <= 64) {
                // rank of candidate `lane` by (exact logit desc, index asc)
                const bool live = lane < nc;
                const uint32_t ce = live ? cand_e[tl][lane] : 0xffffffffu;
                const float cl = live ? cand_l[tl][lane] : 0.0f;
                const uint32_t ck = live ? ordered_key(cl) : 0u;
                int rank = 0;
                for (int j = 0; j < nc; ++j) {
                    const uint32_t kj = __builtin_amdgcn_readlane(ck, j);
                    const uint32_t ej = __builtin_amdgcn_readlane(ce, j);
                    rank += (kj > ck || (kj == ck && ej < ce)) ? 1 : 0;
                }
                if (live && rank < k) {
                    ((uint32_t *)scr[tl])[rank] = ce;
                    scr[tl][8 + rank] = cl;
                }
                __builtin_amdgcn_wave_barrier();
                if (lane < k) {
                    my_pick = (int)((const uint32_t *)scr[tl])[lane];
                    wl = scr[tl][8 + lane];
                }
                __builtin_amdgcn_wave_barrier();
            } else {
                // more than 64 candidates: k rounds of a wave arg-max over them
                uint32_t ck[4];
                bool gone[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int ci = lane + 64 * j;
                    gone[j] = ci >= nc;
                    ck[j] = gone[j] ? 0u : ordered_key(cand_l[tl][ci]);
                }
                for (int p = 0; p < k; ++p) {
                    uint32_t m = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (!gone[j] && ck[j] > m) m = ck[j];
                    m = wave_umax(m);
                    // among the candidates holding the max key, the lowest expert index
                    uint32_t emin = 0xffffffffu;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (!gone[j] && ck[j] == m) {
                            const uint32_t ee = cand_e[tl][lane + 64 * j];
                            emin = ee < emin ? ee : emin;
                        }
                    emin = ~wave_umax(~emin);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (!gone[j] && ck[j] == m && cand_e[tl][lane + 64 * j] == emin) gone[j] = true;
                    if (lane == p) {
                        my_pick = (int)emin;
                        wl = key_to_float(m);
                    }
                }
            }
        }
        // ---- renormalised softmax over the k picks
        const float wk = topk_weight(wl, k);
        if (lane < k) {
            ids[(size_t)t * k + lane] = my_pick;
            tw[(size_t)t * k + lane] = wk;
            sid[tl][lane] = my_pick;
            atomicOr(&mask[my_pick], 1u << tl);
        }
        // ---- the token's range for the expert GEMM: x enters it as fp16 x 2^-e, with e = 0
        // unless max |x| is outside [2^-6, 2^14); then the fp16 copy and the group sums that
        // the router pass wrote are redone with the token's power of two (exact)
        const float xmax = key_to_float(wave_umax(ordered_key(xm)));
        const int e = x_exponent(xmax);
        if (e != 0) {
            const float sc = exp2i(-e);
            if (lane < G) {
                const u32x4 *src = (const u32x4 *)(x + (size_t)t * H + 64 * lane);
                u32x4 *dst = (u32x4 *)(xp + (size_t)t * H + 64 * lane);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const u32x4 v = src[q];
                    u32x4 o;
                    o.x = pack_f16x2(bf16_lo(v.x) * sc, bf16_hi(v.x) * sc);
                    o.y = pack_f16x2(bf16_lo(v.y) * sc, bf16_hi(v.y) * sc);
                    o.z = pack_f16x2(bf16_lo(v.z) * sc, bf16_hi(v.z) * sc);
                    o.w = pack_f16x2(bf16_lo(v.w) * sc, bf16_hi(v.w) * sc);
                    dst[q] = o;
                }
                xsum[(size_t)t * G + lane] *= sc;
            }
        }
        const float nxt = sqrtf(wave_sum_f(ss));
        if (lane == 0) {
            tok[2 * (size_t)t] = exp2i(e);
            tok[2 * (size_t)t + 1] = nxt;
        }
    }
    __syncthreads();
    if (tid < 256) {
        const int c = __popc(mask[tid]);
        blk_cnt[(size_t)blockIdx.x * E + tid] = c;
        // the block's counts into its superblock's (integer sums: order-independent)
        if (sup && c) atomicAdd(sup + (size_t)(blockIdx.x / kSupBlk) * E + tid, c);
    }
    if (tid < TB * k) {
        const int tl2 = tid / k, j = tid % k;
        const int t2 = blockIdx.x * TB + tl2;
        if (t2 < T) {
            const int e = sid[tl2][j];
            lrank[(size_t)t2 * k + j] = __popc(mask[e] & ((1u << tl2) - 1u));
        }
    }
}

void launch_router_fast(const uint16_t *x, const uint16_t *wr, int T, int H, int E, float *part,
                        float *wn2part, uint16_t *xp, float *xsum, float *xsq, float *xmx,
                        int32_t *zero, int nzero, hipStream_t s) {
    const int S = RS_SPLIT;       // H >= 256: every split holds at least one chunk
    static LdsLimit lim;
    lim.ensure((const void *)router_mfma_kernel, R_NST * R_STAGE);
    hipLaunchKernelGGL(router_mfma_kernel, dim3((T + RT_TOK - 1) / RT_TOK, S, 256 / RT_EH),
                       dim3(256), R_NST * R_STAGE, s, x, wr, T, H, E, S, part, xp, xsum, xsq,
                       wn2part, xmx, zero, nzero);
}

void launch_route_select(const float *part, const float *exact, const float *xsq,
                         const float *wn2, const float *bias, const uint16_t *x,
                         const uint16_t *wr, int T, int H, int E, int k, int32_t *ids, float *w,
                         int32_t *blk_cnt, int32_t *lrank, int32_t *sup, const float *xmx,
                         uint16_t *xp, float *xsum, float *tok, hipStream_t s) {
    const int S = RS_SPLIT;       // H >= 256: every split holds at least one chunk
    const dim3 grid((T + TB - 1) / TB), block(64 * TB);
    if (exact) {
        hipLaunchKernelGGL(route_select_kernel<true>, grid, block, 0, s, part, S, exact, xsq, H / 64,
                           wn2, bias, x, wr, T, H, E, k, ids, w, blk_cnt, lrank, sup, xmx, xp, xsum,
                           tok);
    } else {
        static LdsLimit lim;
        lim.ensure((const void *)route_select_kernel<false>, TB * XS_WAVE);
        hipLaunchKernelGGL(route_select_kernel<false>, grid, block, TB * XS_WAVE, s, part, S, exact,
                           xsq, H / 64, wn2, bias, x, wr, T, H, E, k, ids, w, blk_cnt, lrank, sup,
                           xmx, xp, xsum, tok);
    }
}

// ---------------------------------------------------------------------------
// Routing structures from the per-block counts: per expert an exclusive scan
// over token blocks (one workgroup per expert), then expert offsets and the
// block map (one workgroup), then the stable scatter (one thread per pick):
// row = offsets[e] + block_base[b][e] + rank, which orders rows by expert,
// then token.
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 256 threads of a workgroup (4 waves): a shuffle
// scan inside each wave, then the wave totals through LDS (wt: 4 entries); *total
// receives the sum over all threads.  Called by the whole workgroup.
__device__ unsigned long long block_scan_u64(unsigned long long v, int tid, unsigned long long *wt,
                                             unsigned long long *total) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) wt[wave] = v;
    __syncthreads();
    unsigned long long add = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if (w < wave) add += wt[w];
        tot += wt[w];
    }
    __syncthreads();
    *total = tot;
    return v + add;
}

__global__ __launch_bounds__(256) void scan_experts_kernel(int32_t *__restrict__ blk_cnt, int nTB,
                                                           int E, int32_t *__restrict__ counts) {
    __shared__ unsigned long long wt[4];
    const int e = blockIdx.x, tid = threadIdx.x;
    int run = 0;
    for (int b0 = 0; b0 < nTB; b0 += 256) {
        const int b = b0 + tid;
        const int v = b < nTB ? blk_cnt[(size_t)b * E + e] : 0;
        unsigned long long tot;
        const int inc = (int)block_scan_u64((unsigned long long)v, tid, wt, &tot);
        if (b < nTB) blk_cnt[(size_t)b * E + e] = run + inc - v;
        run += (int)tot;
    }
    if (tid == 0) counts[e] = run;
}

// Workgroup 0 of the scatter: expert offsets, the block map of at most BM rows per
// block, its size, and the GEMM schedule (thread tid = expert tid with cnt rows from
// row off; wt: the block scan's LDS scratch).  Called by the whole workgroup.
__device__ void publish_blocks(int tid, int cnt, int off, int BM, unsigned long long *wt,
                               int32_t *__restrict__ offsets, int32_t *__restrict__ blocks,
                               int32_t *__restrict__ num_blocks, int32_t *__restrict__ sched,
                               int32_t *__restrict__ qctl, int nslots) {
    const int nblk = (cnt + BM - 1) / BM;
    // GEMM schedule: blocks by cost class (32-row M tiles: 4, 3, 2, 1), then by
    // expert.  Four 16-bit class counters per expert are scanned as one word.
    const int last_rows = nblk ? cnt - (nblk - 1) * BM : 0;
    const int last_cls = nblk ? 4 - min(4, (last_rows + 31) >> 5) : 0;   // 0 = 4 tiles
    unsigned long long mine = 0;
    if (nblk) mine = (unsigned long long)(nblk - 1) + (1ull << (16 * last_cls));
    unsigned long long ntot, tot;
    const int bstart = (int)block_scan_u64((unsigned long long)nblk, tid, wt, &ntot) - nblk;
    const unsigned long long pre = block_scan_u64(mine, tid, wt, &tot) - mine;
    offsets[tid] = off;
    if (tid == 255) {
        offsets[256] = off + cnt;
        num_blocks[0] = bstart + nblk;
    }
    for (int i = 0; i < nblk; ++i) {
        int32_t *bp = blocks + 3 * (size_t)(bstart + i);
        bp[0] = tid;
        bp[1] = off + i * BM;
        bp[2] = min(BM, cnt - i * BM);
    }
    // the GEMMs' queue counters and the FFN's per-slot counts start at zero
    if (tid < QCTL_WORDS / QCTL_LINE) qctl[tid * QCTL_LINE] = 0;
    for (int i = tid; i < nslots; i += 256) qctl[QCTL_WORDS + i] = 0;
    int base[4];
    base[0] = 0;
    for (int c = 1; c < 4; ++c) base[c] = base[c - 1] + (int)((tot >> (16 * (c - 1))) & 0xFFFF);
    int p0 = base[0] + (int)(pre & 0xFFFF);
    for (int i = 0; i + 1 < nblk; ++i) sched[p0++] = bstart + i;
    if (nblk) {
        const int pl = last_cls == 0 ? p0 : base[last_cls] + (int)((pre >> (16 * last_cls)) & 0xFFFF);
        sched[pl] = bstart + nblk - 1;
    }
}

// Every workgroup scans the expert counts itself (256 values) to get the
// offsets; workgroup 0 also publishes offsets, the block map and its size.
// Then one thread per pick: row = offsets[e] + block_base[b][e] + rank.
__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ tw,
    const int32_t *__restrict__ blk_base, const int32_t *__restrict__ lrank,
    const int32_t *__restrict__ counts, int T, int E, int k, int BM,
    int32_t *__restrict__ offsets, int32_t *__restrict__ blocks, int32_t *__restrict__ num_blocks,
    int32_t *__restrict__ row_token, int32_t *__restrict__ tok_row, float *__restrict__ row_w,
    int32_t *__restrict__ sched, int32_t *__restrict__ qctl, int nslots) {
    __shared__ int s_off[256];
    __shared__ unsigned long long wt[4];
    const int tid = threadIdx.x;
    const int cnt = counts[tid];
    unsigned long long tot;
    const int off = (int)block_scan_u64((unsigned long long)cnt, tid, wt, &tot) - cnt;
    s_off[tid] = off;
    if (blockIdx.x == 0)
        publish_blocks(tid, cnt, off, BM, wt, offsets, blocks, num_blocks, sched, qctl, nslots);
    __syncthreads();
    const int idx = blockIdx.x * 256 + tid;
    if (idx >= T * k) return;
    const int t = idx / k;
    const int e = ids[idx];
    MOE_DBG(e >= 0 && e < E, DBG_ROUTE_INDEX);
    if (e < 0 || e >= E) return;
    const int r = s_off[e] + blk_base[(size_t)(t / TB) * E + e] + lrank[idx];
    MOE_DBG(r >= 0 && r < T * k, DBG_ROUTE_INDEX);
    if (r < 0 || r >= T * k) return;
    row_token[r] = t;
    tok_row[idx] = r;
    row_w[r] = tw[idx];
}

// The routing structures in one kernel for T <= 4096, one workgroup per 32 tokens
// (4 token blocks; 256 picks, one per thread), thread e standing for expert e in
// the scans.  route_select has added every token block's expert counts into the
// row of its superblock (kSupBlk consecutive blocks) in sup, so the base of
// expert e in block b is the sum of sup over the superblocks before b's plus
// blk_cnt over the blocks of b's superblock before b, and the expert counts are
// the column sums of sup: one batch of loads, then the same LDS scans as
// scatter_kernel.  Workgroup 0 also publishes counts, offsets, the block map
// and the GEMM schedule.
__global__ __launch_bounds__(256) void scatter1_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ tw,
    const int32_t *__restrict__ blk_cnt, const int32_t *__restrict__ sup,
    const int32_t *__restrict__ lrank, int T, int E, int k, int BM,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ blocks,
    int32_t *__restrict__ num_blocks, int32_t *__restrict__ row_token,
    int32_t *__restrict__ tok_row, float *__restrict__ row_w, int32_t *__restrict__ sched,
    int32_t *__restrict__ qctl, int nslots) {
    __shared__ int s_off[256];
    __shared__ int s_base[4][256];
    __shared__ unsigned long long wt[4];
    const int tid = threadIdx.x, e = tid;
    const int nTB = (T + TB - 1) / TB, nS = (nTB + kSupBlk - 1) / kSupBlk;
    const int b0 = blockIdx.x * 4, s0 = b0 / kSupBlk;
    // every load at once, none under a branch: rows past the end read a valid row
    // and are discarded
    const int idx = blockIdx.x * 256 + tid;
    const bool has = idx < T * k;
    const int ic = has ? idx : 0;
    const int pe = ids[ic], prk = lrank[ic];
    const float pw = tw[ic];
    int sv[kSupMax], iv[kSupBlk];
#pragma unroll
    for (int q = 0; q < kSupMax; ++q) sv[q] = sup[(size_t)(q < nS ? q : nS - 1) * E + e];
#pragma unroll
    for (int q = 0; q < kSupBlk; ++q) {
        const int b = s0 * kSupBlk + q;
        iv[q] = blk_cnt[(size_t)(b < nTB ? b : nTB - 1) * E + e];
    }
    int cnt = 0, run = 0;
#pragma unroll
    for (int q = 0; q < kSupMax; ++q) {
        const int v = q < nS ? sv[q] : 0;
        cnt += v;
        if (q < s0) run += v;
    }
#pragma unroll
    for (int q = 0; q < kSupBlk; ++q) {
        const int b = s0 * kSupBlk + q;
        if (b >= b0 && b < b0 + 4) s_base[b - b0][e] = run;
        if (b < b0 + 4 && b < nTB) run += iv[q];
    }
    unsigned long long tot;
    const int off = (int)block_scan_u64((unsigned long long)cnt, tid, wt, &tot) - cnt;
    s_off[tid] = off;
    if (blockIdx.x == 0) {
        counts[tid] = cnt;
        publish_blocks(tid, cnt, off, BM, wt, offsets, blocks, num_blocks, sched, qctl, nslots);
    }
    __syncthreads();
    if (!has) return;
    const int t = idx / k;
    MOE_DBG(pe >= 0 && pe < E, DBG_ROUTE_INDEX);
    if (pe < 0 || pe >= E) return;
    const int r = s_off[pe] + s_base[t / TB - b0][pe] + prk;
    MOE_DBG(r >= 0 && r < T * k, DBG_ROUTE_INDEX);
    if (r < 0 || r >= T * k) return;
    row_token[r] = t;
    tok_row[idx] = r;
    row_w[r] = pw;
}

void launch_scan_scatter(const int32_t *ids, const float *w, int32_t *blk_cnt,
                         const int32_t *sup, const int32_t *lrank, int T, int E, int k, int BM,
                         int32_t *counts, int32_t *offsets, int32_t *row_token, int32_t *tok_row,
                         float *row_w, int32_t *blocks, int32_t *num_blocks, int32_t *sched,
                         int32_t *qctl, int nslots, hipStream_t s) {
    const int nTB = (T + TB - 1) / TB;
    if (sup) {
        hipLaunchKernelGGL(scatter1_kernel, dim3((T * k + 255) / 256), dim3(256), 0, s, ids, w,
                           blk_cnt, sup, lrank, T, E, k, BM, counts, offsets, blocks, num_blocks,
                           row_token, tok_row, row_w, sched, qctl, nslots);
        return;
    }
    hipLaunchKernelGGL(scan_experts_kernel, dim3(E), dim3(256), 0, s, blk_cnt, nTB, E, counts);
    hipLaunchKernelGGL(scatter_kernel, dim3((T * k + 255) / 256), dim3(256), 0, s, ids, w, blk_cnt,
                       lrank, counts, T, E, k, BM, offsets, blocks, num_blocks, row_token,
                       tok_row, row_w, sched, qctl, nslots);
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t *__restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

void launch_zero_i32(int32_t *p, int n, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
}

// Activation preparation for the GEMM: fp16 copy of every row plus the group sums, one
// thread per (row, group of 64).
__global__ __launch_bounds__(256) void prep_act_kernel(const uint16_t *__restrict__ x, int rows,
                                                       int K, uint16_t *__restrict__ xp,
                                                       float *__restrict__ out,
                                                       float *__restrict__ sq,
                                                       float *__restrict__ mxo) {
    const int G = K / 64;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)rows * G) return;
    const size_t r = i / G, g = i % G;
    const u32x4 *p = (const u32x4 *)(x + r * K + g * 64);
    u32x4 *q = (u32x4 *)(xp + r * K + g * 64);
    float s = 0.0f, s2 = 0.0f, mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x4 v = p[j];
        s += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
             bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s2 = __builtin_fmaf(bf16_lo(v[q]), bf16_lo(v[q]), s2);
            s2 = __builtin_fmaf(bf16_hi(v[q]), bf16_hi(v[q]), s2);
            mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(v[q])), fabsf(bf16_hi(v[q]))));
        }
        q[j] = to_f16x8(v);
    }
    out[i] = s;
    if (sq) sq[i] = s2;
    if (mxo) mxo[i] = mx;
}

void launch_prep_act(const uint16_t *x, int rows, int K, uint16_t *xp, float *xsum, float *xsq,
                     float *xmx, hipStream_t s) {
    const size_t n = (size_t)rows * (K / 64);
    if (n == 0) return;
    hipLaunchKernelGGL(prep_act_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, rows,
                       K, xp, xsum, xsq, xmx);
}

MOE_DBG_READER(dbg_read_route)

}  // namespace moe
