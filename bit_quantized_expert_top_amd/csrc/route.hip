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
// Top-k per token (one wave per token) and the per-token-block half of the
// routing: each workgroup takes 64 consecutive tokens, records for every
// expert the set of its tokens that picked it as a 64-bit lane mask in LDS
// (an OR is order independent, so the masks are deterministic), and from
// the masks writes the block's expert histogram and the rank of each
// (token, pick) among the block's tokens of that expert (popcount of the
// lower mask bits).  Ranks in token order make the scatter stable.
// ---------------------------------------------------------------------------
constexpr int TB = 64;   // tokens per routing block

__device__ __forceinline__ uint32_t ordered_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);   // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__global__ __launch_bounds__(256) void topk_local_kernel(const float *__restrict__ logits, int T,
                                                         int E, int k, int32_t *__restrict__ ids,
                                                         float *__restrict__ tw,
                                                         int32_t *__restrict__ blk_cnt,
                                                         int32_t *__restrict__ lrank) {
    __shared__ unsigned long long mask[256];
    __shared__ int32_t sid[TB][8];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tb0 = blockIdx.x * TB;
    mask[tid] = 0ull;
    __syncthreads();
    for (int tl = wave; tl < TB; tl += 4) {
        const int t = tb0 + tl;
        if (t >= T) break;
        const float *l = logits + (size_t)t * E;
        uint64_t key[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            key[j] = ((uint64_t)ordered_key(l[e]) << 32) | (uint32_t)(0xffffu - e);
        }
        int my_pick = -1;
        float my_logit = 0.0f;
        for (int p = 0; p < k; ++p) {
            uint64_t best = key[0];
#pragma unroll
            for (int j = 1; j < 4; ++j) best = key[j] > best ? key[j] : best;
            best = wave_max_u64(best);
            const int e = 0xffff - (int)(best & 0xffffu);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (lane + 64 * j == e) key[j] = 0ull;
            if (lane == p) {
                // the winning key carries the logit: invert the order-preserving map
                const uint32_t kh = (uint32_t)(best >> 32);
                my_pick = e;
                my_logit = __uint_as_float((kh & 0x80000000u) ? (kh & 0x7fffffffu) : ~kh);
            }
        }
        // renormalised softmax over the k picks: exp(l_j - l_0) / sum
        const float lmax = __shfl(my_logit, 0);
        float pj = (lane < k) ? expf(my_logit - lmax) : 0.0f;
        float sum = pj;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane < k) {
            ids[(size_t)t * k + lane] = my_pick;
            tw[(size_t)t * k + lane] = pj / sum;
            sid[tl][lane] = my_pick;
            atomicOr(&mask[my_pick], 1ull << tl);
        }
    }
    __syncthreads();
    blk_cnt[(size_t)blockIdx.x * E + tid] = __popcll(mask[tid]);
    for (int idx = tid; idx < TB * k; idx += 256) {
        const int tl = idx / k, j = idx % k;
        const int t = tb0 + tl;
        if (t < T) {
            const int e = sid[tl][j];
            lrank[(size_t)t * k + j] = __popcll(mask[e] & ((1ull << tl) - 1ull));
        }
    }
}

void launch_topk_local(const float *logits, int T, int E, int k, int32_t *ids, float *w,
                       int32_t *blk_cnt, int32_t *lrank, hipStream_t s) {
    hipLaunchKernelGGL(topk_local_kernel, dim3((T + TB - 1) / TB), dim3(256), 0, s, logits, T, E,
                       k, ids, w, blk_cnt, lrank);
}

// ---------------------------------------------------------------------------
// Prefix scans, block map and stable scatter in one workgroup: per expert an
// exclusive scan of the token-block counts (written back in place), the
// expert histogram, its exclusive scan (offsets), the block map (blocks of at
// most BM consecutive rows of one expert, in expert order), and finally the
// scatter row = offsets[e] + block_base[b][e] + rank.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void scan_scatter_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ tw, int32_t *__restrict__ blk_cnt,
    const int32_t *__restrict__ lrank, int T, int E, int k, int BM, int max_blocks,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ row_token,
    int32_t *__restrict__ tok_row, float *__restrict__ row_w, int32_t *__restrict__ blocks,
    int32_t *__restrict__ num_blocks) {
    __shared__ int tmp[256];
    __shared__ int s_off[257];
    const int tid = threadIdx.x;
    const int nTB = (T + TB - 1) / TB;
    int cnt = 0, nblk = 0;
    if (tid < 256) {
        int run = 0;
        for (int b = 0; b < nTB; ++b) {
            const int c = blk_cnt[(size_t)b * E + tid];
            blk_cnt[(size_t)b * E + tid] = run;
            run += c;
        }
        cnt = run;
        counts[tid] = cnt;
        nblk = (cnt + BM - 1) / BM;
    }
    // the scans use the first 256 threads; the others wait at the barriers
    int off = 0, bstart = 0;
    {
        // expert offsets
        if (tid < 256) tmp[tid] = cnt;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            int a = 0;
            if (tid < 256 && tid >= o) a = tmp[tid - o];
            __syncthreads();
            if (tid < 256) tmp[tid] += a;
            __syncthreads();
        }
        if (tid < 256) off = tmp[tid] - cnt;
        __syncthreads();
        // block starts
        if (tid < 256) tmp[tid] = nblk;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            int a = 0;
            if (tid < 256 && tid >= o) a = tmp[tid - o];
            __syncthreads();
            if (tid < 256) tmp[tid] += a;
            __syncthreads();
        }
        if (tid < 256) bstart = tmp[tid] - nblk;
    }
    if (tid < 256) {
        s_off[tid] = off;
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
    }
    __syncthreads();
    for (int idx = tid; idx < T * k; idx += 1024) {
        const int t = idx / k;
        const int e = ids[idx];
        if (e < 0 || e >= E) continue;
        const int r = s_off[e] + blk_cnt[(size_t)(t / TB) * E + e] + lrank[idx];
        if (r < 0 || r >= T * k) continue;
        row_token[r] = t;
        tok_row[idx] = r;
        row_w[r] = tw[idx];
    }
}

void launch_scan_scatter(const int32_t *ids, const float *w, const int32_t *blk_cnt,
                         const int32_t *lrank, int T, int E, int k, int BM, int max_blocks,
                         int32_t *counts, int32_t *offsets, int32_t *row_token, int32_t *tok_row,
                         float *row_w, int32_t *blocks, int32_t *num_blocks, hipStream_t s) {
    hipLaunchKernelGGL(scan_scatter_kernel, dim3(1), dim3(1024), 0, s, ids, w,
                       const_cast<int32_t *>(blk_cnt), lrank, T, E, k, BM, max_blocks, counts,
                       offsets, row_token, tok_row, row_w, blocks, num_blocks);
}

// ---------------------------------------------------------------------------
// Group sums of a bf16 matrix: out[r][g] = sum of a[r][64g .. 64g+63] in fp32.
// The GEMMs feed exact 4-bit codes (plus a constant 128) to the MFMA and use
// these sums to remove that constant and to apply the per-group bias.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void group_sums_kernel(const uint16_t *__restrict__ a, int rows,
                                                         int K, float *__restrict__ out) {
    const int G = K / 64;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)rows * G) return;
    const size_t r = i / G, g = i % G;
    const u32x4 *p = (const u32x4 *)(a + r * K + g * 64);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x4 v = p[j];
        s += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
             bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
    }
    out[i] = s;
}

// Activation preparation for the GEMM: the 8-block permutation (0,4,1,5,2,6,3,7)
// of every row plus the group sums, one thread per (row, group of 64).
__global__ __launch_bounds__(256) void prep_act_kernel(const uint16_t *__restrict__ x, int rows,
                                                       int K, uint16_t *__restrict__ xp,
                                                       float *__restrict__ out) {
    const int G = K / 64;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)rows * G) return;
    const size_t r = i / G, g = i % G;
    const u32x4 *p = (const u32x4 *)(x + r * K + g * 64);
    u32x4 *q = (u32x4 *)(xp + r * K + g * 64);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x4 v = p[j];
        s += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
             bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
        u32x4 o;
        o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
        o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
        o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
        o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
        q[j] = o;
    }
    out[i] = s;
}

void launch_prep_act(const uint16_t *x, int rows, int K, uint16_t *xp, float *xsum, hipStream_t s) {
    const size_t n = (size_t)rows * (K / 64);
    if (n == 0) return;
    hipLaunchKernelGGL(prep_act_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, rows,
                       K, xp, xsum);
}

void launch_group_sums(const uint16_t *a, int rows, int K, float *out, hipStream_t s) {
    const size_t n = (size_t)rows * (K / 64);
    if (n == 0) return;
    hipLaunchKernelGGL(group_sums_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a,
                       rows, K, out);
}

}  // namespace moe
