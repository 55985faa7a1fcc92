// Batch-1 decode: one token through the router, top-8 and the nine selected
// experts (eight routed + the shared one).  At batch 1 there is no weight
// reuse, so the path is bound by how fast the selected experts' packed
// weights stream from HBM (mechatronicstore.cl, "Decode: mover menos bytes
// por token"; neuro-ai.ru, "Спекулятивное декодирование не взлетело").  Only
// the picked experts' rows are read; the expert ids never leave the device.
//
// Three short kernels:
//  1. router: one wave per expert computes its logit exactly in the fixed
//     order (sequential within each 64-chunk, then over chunks, then + bias),
//     so the ids need no certification step at batch 1;
//  2. gate/up: one wave per workgroup first takes the top-8 (logit
//     descending, index ascending) and the softmax weights restricted to them;
//     rows streamed with 16-byte loads, a wave keeps its slice of x
//     in registers for all its rows; codes become 128+q in bf16 with one
//     and-or per pair and meet x in packed bf16 dot products:
//        sum_k x_k (q_k s + b) = s (sum x (128 + q) - 128 sum x) + b sum x;
//     h = silu(gate) * up is written in fp16, 8-blocks permuted like the codes;
//  3. down: each workgroup stages h in LDS; codes become 1024+q in fp16 and
//     meet h in packed fp16 dot products; the nine slot results of an output
//     are summed in slot order with their routing weights.
#include "common.h"

namespace moe {

constexpr int DEC_ROWS_PER_WAVE = 4;   // gate/up rows (per lane group) handled by one wave

__device__ __forceinline__ uint32_t dec_and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
    return r;
}

// Sum of a row spread over LPR lanes (a power of two up to 64, groups aligned);
// the result is valid in every lane of the group.
__device__ __forceinline__ float row_total(float v, int LPR, int sub) {
    v = group_sum_dpp(v, LPR < 16 ? LPR : 16);
    if (LPR <= 16) return v;
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    if (LPR == 32) return sub == 0 ? r0 + r1 : r2 + r3;
    return (r0 + r1) + (r2 + r3);
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

// Top-k (k <= 8) of E <= 256 logits by (logit desc, index asc) and the weights
// exp(l - l_1) / sum, computed by one wave (all lanes end with the same picks).
__device__ void select_topk(const float *__restrict__ logits, int E, int k, int *pick_e,
                            float *pick_w) {
    const int lane = threadIdx.x & 63;
    uint32_t key[4];
    bool taken[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        key[j] = e < E ? ordered_key(logits[e]) : 0u;
        taken[j] = e >= E;
    }
    float pick_l[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (r >= k) break;
        uint32_t km;
        const int e = wave_argmax4(key, taken, &km);
        pick_e[r] = e;
        pick_l[r] = key_to_float(km);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (lane + 64 * j == e) taken[j] = true;
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

// 2. gate/up rows.  Wave 0 of every workgroup selects the experts (workgroup 0
// also writes them out); meanwhile all waves load their slice of x.  A lane
// group of LPR = H/32 lanes covers one row (each lane 32 consecutive inputs:
// four code words, half a quantisation group); a wave covers RPI = 64/LPR rows
// per step and DEC_ROWS_PER_WAVE steps, all of whose loads are issued before
// any arithmetic.
__global__ __launch_bounds__(256) void decode_gateup_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ logits, int H, int I, int k, int E,
    const uint8_t *__restrict__ pk, const uint8_t *__restrict__ pk_sh, int32_t *__restrict__ ids_out,
    float *__restrict__ tw_out, uint16_t *__restrict__ hbuf) {
    __shared__ int s_ids[8];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wave == 0) {
        int pe[8];
        float pw[8];
        select_topk(logits, E, k, pe, pw);
        if (lane < k) {
            int e = 0;
            float wv = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (r == lane) {
                    e = pe[r];
                    wv = pw[r];
                }
            s_ids[lane] = e;
            if (blockIdx.x == 0) {
                ids_out[lane] = e;
                tw_out[lane] = wv;
            }
        }
    }
    const int LPR = H / 32, RPI = 64 / LPR;
    const int sub = lane / LPR, lj = lane % LPR;
    const int kpos = 32 * lj, g = kpos / 64;
    const int G = H / 64;
    // x slice in pair order (0,4),(1,5),(2,6),(3,7) of each 8-block, and its sum
    uint32_t xp[16];
    float sx = 0.0f;
    {
        const u32x4 *px = (const u32x4 *)(x + kpos);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const u32x4 v = px[b];
            xp[4 * b + 0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
            xp[4 * b + 1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
            xp[4 * b + 2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
            xp[4 * b + 3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
#pragma unroll
            for (int r = 0; r < 4; ++r) sx += bf16_lo(v[r]) + bf16_hi(v[r]);
        }
    }
    __syncthreads();
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t cM = 0x000F000Fu, cC = 0x43004300u;
    asm volatile("" : "+v"(cM), "+v"(cC));
    const int R = (k + 1) * I;
    const int base = ((blockIdx.x * 4 + wave) * DEC_ROWS_PER_WAVE) * RPI;
    u32x4 wg[DEC_ROWS_PER_WAVE], wu[DEC_ROWS_PER_WAVE];
    uint16_t sgr[DEC_ROWS_PER_WAVE], bgr[DEC_ROWS_PER_WAVE], sur[DEC_ROWS_PER_WAVE],
        bur[DEC_ROWS_PER_WAVE];
#pragma unroll
    for (int it = 0; it < DEC_ROWS_PER_WAVE; ++it) {
        int row = base + it * RPI + sub;
        row = row < R ? row : R - 1;              // past the end: repeat the last row
        const int slot = row / I, i = row - slot * I;
        const bool sh = slot == k;
        int ex = sh ? 0 : s_ids[slot];
        ex = (ex < 0 || ex >= E) ? 0 : ex;
        // tile-layout block (tile i/128, group g); gate column cg, up column cg + 32
        const int j = i >> 7, cg = 64 * ((i & 127) >> 5) + (i & 31);
        const uint8_t *blk = sh ? pk_sh + ((size_t)j * G + g) * PK_BLOCK
                                : pk + (((size_t)ex * (I / 128) + j) * G + g) * PK_BLOCK;
        const int hh = lj & 1;                    // half of the group this lane covers
        wg[it] = *(const u32x4 *)(blk + 32 * cg + 16 * (hh ^ ((cg >> 3) & 1)));
        wu[it] = *(const u32x4 *)(blk + 32 * (cg + 32) + 16 * (hh ^ (((cg + 32) >> 3) & 1)));
        sgr[it] = *(const uint16_t *)(blk + PK_CODES + 2 * cg);
        bgr[it] = *(const uint16_t *)(blk + PK_CODES + 512 + 2 * cg);
        sur[it] = *(const uint16_t *)(blk + PK_CODES + 2 * (cg + 32));
        bur[it] = *(const uint16_t *)(blk + PK_CODES + 512 + 2 * (cg + 32));
    }
#pragma unroll
    for (int it = 0; it < DEC_ROWS_PER_WAVE; ++it) {
        const int row = base + it * RPI + sub;
        float dg = 0.0f, du = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const bf16x2 xv = __builtin_bit_cast(bf16x2, xp[4 * j + p]);
                const uint32_t cg = dec_and_or(wg[it][j] >> (4 * p), cM, cC);
                const uint32_t cu = dec_and_or(wu[it][j] >> (4 * p), cM, cC);
                dg = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cg), xv, dg, false);
                du = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cu), xv, du, false);
            }
        }
        float vg = bf16_to_f32(sgr[it]) * (dg - 128.0f * sx) + bf16_to_f32(bgr[it]) * sx;
        float vu = bf16_to_f32(sur[it]) * (du - 128.0f * sx) + bf16_to_f32(bur[it]) * sx;
        vg = row_total(vg, LPR, sub);
        vu = row_total(vu, LPR, sub);
        if (row < R && lj == 0) {
            const int slot = row / I, i = row - slot * I;
            const float hv = vg / (1.0f + expf(-vg)) * vu;
            hbuf[(size_t)slot * I + perm_pos(i)] = f32_to_f16(hv);
        }
    }
}

// 3. down.  Workgroup: 8 outputs; wave: 2 outputs x (k+1) slots = 2(k+1) rows,
// in batches of DOWN_STEPS steps of RPI rows (a lane group of LPR = I/32 lanes
// covers one row); the weight loads of a batch are issued before the h tile
// is needed.
constexpr int DOWN_STEPS = 5;
__global__ __launch_bounds__(256) void decode_down_kernel(
    const uint16_t *__restrict__ hbuf, int H, int I, const int32_t *__restrict__ ids,
    const float *__restrict__ tw, int k, int E, const uint8_t *__restrict__ pk,
    const uint8_t *__restrict__ pk_sh,
    float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    uint16_t *hs = (uint16_t *)dsm;                           // [(k+1)][I] fp16, permuted
    float *res = (float *)(dsm + (size_t)(k + 1) * I * 2);    // [4 waves][2 (k+1)]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const int LPR = I / 32, RPI = 64 / LPR;
    const int sub = lane / LPR, lj = lane % LPR;
    const int G = I / 64, g = lj / 2, hh = lj & 1;
    uint32_t cM = 0x000F000Fu, cC = 0x64006400u;
    asm volatile("" : "+v"(cM), "+v"(cC));
    const int nrow = 2 * (k + 1);                             // (output, slot) pairs of this wave
    const int n0 = blockIdx.x * 8 + 2 * wave;
    int sid[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) sid[r] = r < k ? ids[r] : 0;
    const int nh = (k + 1) * I / 8;                           // 16-byte units of h
    bool staged = false;
    for (int r0 = 0; r0 < nrow; r0 += DOWN_STEPS * RPI) {
        u32x4 wq[DOWN_STEPS];
        uint16_t sr[DOWN_STEPS], br[DOWN_STEPS];
#pragma unroll
        for (int st = 0; st < DOWN_STEPS; ++st) {
            int rr = r0 + st * RPI + sub;
            rr = rr < nrow ? rr : nrow - 1;
            const int n = min(n0 + rr / (k + 1), H - 1), slot = rr % (k + 1);
            const bool sh = slot == k;
            int ex = 0;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (r == slot) ex = sid[r];
            ex = (sh || ex < 0 || ex >= E) ? 0 : ex;
            // tile-layout block (tile n/256, group g), column n % 256
            const int j = n >> 8, c = n & 255;
            const uint8_t *blk = sh ? pk_sh + ((size_t)j * G + g) * PK_BLOCK
                                    : pk + (((size_t)ex * (H / 256) + j) * G + g) * PK_BLOCK;
            wq[st] = *(const u32x4 *)(blk + 32 * c + 16 * (hh ^ ((c >> 3) & 1)));
            sr[st] = *(const uint16_t *)(blk + PK_CODES + 2 * c);
            br[st] = *(const uint16_t *)(blk + PK_CODES + 512 + 2 * c);
        }
        if (!staged) {
            for (int u = tid; u < nh; u += 256) ((u32x4 *)hs)[u] = ((const u32x4 *)hbuf)[u];
            __syncthreads();
            staged = true;
        }
#pragma unroll
        for (int st = 0; st < DOWN_STEPS; ++st) {
            const int rr = r0 + st * RPI + sub;
            const int slot = (rr < nrow ? rr : nrow - 1) % (k + 1);
            const u32x4 *hp = (const u32x4 *)(hs + (size_t)slot * I + 32 * lj);
            float d = 0.0f, sh_sum = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 hv = hp[j];
                // the four h words as plain scalars (an element of the vector
                // bit-cast straight into the dot builtin selects the wrong word)
                const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t c = dec_and_or(wq[st][j] >> (4 * q), cM, cC);
                    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, c), __builtin_bit_cast(h2, hw[q]),
                                               d, false);
                    sh_sum += f16_lo(hw[q]) + f16_hi(hw[q]);
                }
            }
            float v = bf16_to_f32(sr[st]) * (d - 1024.0f * sh_sum) + bf16_to_f32(br[st]) * sh_sum;
            v = row_total(v, LPR, sub);
            if (rr < nrow && n0 + rr / (k + 1) < H && lj == 0) res[wave * nrow + rr] = v;
        }
    }
    __syncthreads();
    if (lane < 2) {
        const int n = n0 + lane;
        if (n < H) {
            float total = 0.0f;
            for (int slot = 0; slot < k; ++slot)
                total = __builtin_fmaf(tw[slot], res[wave * nrow + lane * (k + 1) + slot], total);
            total += res[wave * nrow + lane * (k + 1) + k];
            y[n] = total;
        }
    }
}

void launch_decode(const moe_shape &sh, const uint16_t *x, const moe_weights &w, int32_t *ids,
                   float *tw, float *y, void *scratch, hipStream_t s) {
    const int H = sh.H, I = sh.I, E = sh.E, k = sh.top_k;
    char *p = (char *)scratch;
    float *logits = (float *)p;         // [E]
    p += 4096;
    uint16_t *hbuf = (uint16_t *)p;     // fp16 [k+1][I]
    const PackLayout P = pack_layout(H, I, E);
    const uint8_t *pk = (const uint8_t *)w.packed;
    hipLaunchKernelGGL(decode_router_kernel, dim3((E + 3) / 4), dim3(256), 0, s, x, w.router_wt,
                       w.router_bias, H, E, logits);
    const int rows = (k + 1) * I, rpi = 64 / (H / 32);
    const int per_wg = 4 * DEC_ROWS_PER_WAVE * rpi;
    hipLaunchKernelGGL(decode_gateup_kernel, dim3((rows + per_wg - 1) / per_wg), dim3(256), 0, s,
                       x, logits, H, I, k, E, pk + P.gu, pk + P.sh_gu, ids, tw, hbuf);
    const size_t lds = (size_t)(k + 1) * I * 2 + 4 * 2 * (k + 1) * 4;
    hipLaunchKernelGGL(decode_down_kernel, dim3((H + 7) / 8), dim3(256), lds, s, hbuf, H, I, ids,
                       tw, k, E, pk + P.down, pk + P.sh_down, y);
}

size_t decode_scratch_bytes(int I, int k) { return 4096 + (size_t)(k + 1) * I * 2; }

}  // namespace moe
