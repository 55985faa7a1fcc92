// Decode: each token (up to 8 per call, independent problems in the same
// launches, token = blockIdx.y) through the router, top-8 and the nine selected
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
//  2. gate/up: a workgroup takes one slot and 8 gate + the 8 matching up
//     columns over all of K.  At one token every wave takes the top-8 itself
//     (logit descending, index ascending; softmax weights restricted to them),
//     which keeps a launch off the latency chain; with more tokens a small
//     kernel takes each token's top-8 once and the workgroups read the ids.
//     Then every wave issues all of its weight loads at once; the token's x is
//     loaded once per workgroup and read by the column lanes from LDS.
//     Codes become 128+q in bf16 with one and-or per pair and meet x in packed
//     bf16 dot products:
//        sum_k x_k (q_k s + b) = s (sum x (128 + q) - 128 sum x) + b sum x;
//     the two halves of a column meet by DPP, the waves' groups through LDS
//     in order, and h = silu(gate) * up is written in fp16;
//  3. down: a workgroup takes 8 outputs (a 256-byte run of every block of
//     their tile) for all nine slots and all groups; each lane loads the codes
//     of its (slot, group) pairs, the token's h block is loaded once per
//     workgroup and read from LDS, and codes become 1024+q in fp16.  The partial sums meet in LDS and are added per output
//     in a fixed order: groups, then slots in pick order with their routing
//     weights, then the shared expert.
#include "common.h"

namespace moe {


__device__ __forceinline__ uint32_t dec_and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
    return r;
}

// 1. logits[e] = sum over chunks c (in order) of sum_{k in chunk c} x_k w_ek (in order), + bias.
// One wave (one workgroup) per expert, so the 1 MB of router weights is read
// by E workgroups at once.  With a residual (res != NULL, a decode stack's layer
// after the first) the layer input is made here: x = bf16((res + yprev) /
// sqrt(mean((res + yprev)^2) + eps)); every wave computes it from the whole row
// (lane c holds elements 64 c .. 64 c + 63) and the expert-0 wave also writes it
// to u_out for the gate/up and down kernels.  res itself is updated by the
// gate/up kernel, after every wave here has read it.
__global__ __launch_bounds__(64) void decode_router_kernel(const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ wr,
                                                           const float *__restrict__ bias, int H,
                                                           float *__restrict__ logits,
                                                           const float *__restrict__ res,
                                                           const float *__restrict__ yprev, float eps,
                                                           uint16_t *__restrict__ u_out,
                                                           float *__restrict__ xn2) {
    const int lane = threadIdx.x;
    const int e = blockIdx.x;
    const int E = gridDim.x;
    const size_t t = blockIdx.y;   // token
    logits += t * E;
    const int G = H / 64;          // <= 32 chunks: lane c < G sums chunk c
    const int c = min(lane, G - 1);
    u32x4 xv[8], wv[8];
    {
        const u32x4 *pw = (const u32x4 *)(wr + (size_t)e * H + 64 * c);
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = pw[j];
    }
    if (res == nullptr) {
        const u32x4 *px = (const u32x4 *)(x + t * H + 64 * c);
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = px[j];
    } else {
        const floatx4 *pr = (const floatx4 *)(res + t * H + 64 * c);
        const floatx4 *py = (const floatx4 *)(yprev + t * H + 64 * c);
        floatx4 a[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) a[j] = pr[j] + py[j];
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) ss = __builtin_fmaf(a[j][q], a[j][q], ss);
        ss = lane < G ? ss : 0.0f;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            xv[j].x = pack_bf16x2(a[2 * j][0] * inv, a[2 * j][1] * inv);
            xv[j].y = pack_bf16x2(a[2 * j][2] * inv, a[2 * j][3] * inv);
            xv[j].z = pack_bf16x2(a[2 * j + 1][0] * inv, a[2 * j + 1][1] * inv);
            xv[j].w = pack_bf16x2(a[2 * j + 1][2] * inv, a[2 * j + 1][3] * inv);
        }
        if (e == 0 && lane < G) {
            u32x4 *pu = (u32x4 *)(u_out + t * H + 64 * lane);
#pragma unroll
            for (int j = 0; j < 8; ++j) pu[j] = xv[j];
        }
    }
    if (e == 0) {
        // the token's ||x||^2 for the gate/up kernel's h range bound (bf16 squares are
        // exact in fp32): off that kernel's latency chain
        float q2 = 0.0f;
        if (lane < G) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    q2 = __builtin_fmaf(bf16_lo(xv[j][r]), bf16_lo(xv[j][r]), q2);
                    q2 = __builtin_fmaf(bf16_hi(xv[j][r]), bf16_hi(xv[j][r]), q2);
                }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) q2 += __shfl_xor(q2, off);
        if (lane == 0) xn2[t] = q2;
    }
    float P = 0.0f;
    if (lane < G) {
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

// Top-k (k <= 8) of E = 256 logits by (logit desc, index asc), computed by one
// wave: lane p < k ends with pick p's expert and logit.  wl: 32 words of
// wave-local LDS.
__device__ void select_topk(const float *__restrict__ logits, int E, int k, int &pick_e,
                            float &pick_l, uint32_t *wl) {
    const int lane = threadIdx.x & 63;
    uint32_t key[4];
    bool taken[4];
    float lv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lv[j] = logits[min(lane + 64 * j, E - 1)];   // one round trip
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = lane + 64 * j < E ? ordered_key(lv[j]) : 0u;
    uint32_t pkey;
    wave_topk_radix(key, k, taken, pick_e, pkey, wl);
    pick_l = lane < k ? key_to_float(pkey) : 0.0f;
}

// scratch: the logits of every token, then the h rows and the h factors of every token's
// nine slots, each part 256-byte aligned (decode_scratch_size)
static size_t logits_bytes(int T, int E) { return ((size_t)T * E * 4 + 255) & ~(size_t)255; }
static size_t hbuf_bytes(int T, int I, int k) { return ((size_t)T * (k + 1) * I * 2 + 255) & ~(size_t)255; }

// 1b. (decode of two or more tokens) the top-k and weights of token blockIdx.x,
// once per token, for the gate/up and down workgroups to read.
__global__ __launch_bounds__(64) void decode_select_kernel(const float *__restrict__ logits, int E,
                                                           int k, int32_t *__restrict__ ids,
                                                           float *__restrict__ tw) {
    __shared__ uint32_t wl[32];
    const int t = blockIdx.x, lane = threadIdx.x;
    int pe;
    float pl;
    select_topk(logits + (size_t)t * E, E, k, pe, pl, wl);
    const float wv = topk_weight(pl, k);
    if (lane < k) {
        ids[(size_t)t * k + lane] = pe;
        tw[(size_t)t * k + lane] = wv;
    }
}

constexpr int DW = 8;                  // waves per decode workgroup
constexpr int NSLOT = 9;               // top-8 routed experts + the shared one (top_k is 8)
constexpr int DOUT = 8;                // outputs per decode workgroup (gate/up and down)
constexpr int DN_BATCH = 3;            // down: (slot, group) pairs per lane loaded at once
constexpr int DN_MAXP = NSLOT * 32;    // down: (slot, group) pairs for I <= 2048

// Nibble pair p (nibbles p and p + 4) of a tile-layout word holds the codes 2p and
// 2p + 1 and unpacks as two 16-bit values in a magic-number format (and-or with
// C = 128.0 bf16 pairs or 1024.0 fp16 pairs).  The matching x (or h) pair is word p
// of the 8-block: the words go into a scalar array, which the dot products read.
__device__ __forceinline__ void pair_words(const u32x4 v, uint32_t *o) {
    o[0] = v.x;
    o[1] = v.y;
    o[2] = v.z;
    o[3] = v.w;
}

// sum of lanes l and l ^ 1
__device__ __forceinline__ float pair_sum(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// 2. gate/up.  Workgroup (slot, 8 outputs i = 8 o .. 8 o + 7 of I): their
// gate and up columns are two 256-byte runs of every block of the slot's tile.
// Lane (gi, cc, ph) of wave w holds physical half ph of gate and up column cc
// of group 4 w + gi (+ 32 per further pass), so one load instruction of a wave
// covers four groups.  x is loaded before the selection, the weights right
// after it, all at once.
// at most 64 VGPRs: 8 waves per SIMD, so that four workgroups share a CU (small batches
// launch T x 576 workgroups)
__global__ __launch_bounds__(64 * DW) __attribute__((amdgpu_waves_per_eu(8, 8))) void decode_gateup_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ logits, int H, int I, int k, int E,
    GemmWeights gw, int32_t *__restrict__ ids_out, float *__restrict__ tw_out,
    uint16_t *__restrict__ hbuf, float *__restrict__ hfac, const float *__restrict__ xn2,
    bool picks_given, float *__restrict__ res, const float *__restrict__ yprev) {
    __shared__ float red[DW][DOUT][2];
    __shared__ uint32_t selw[DW][32];
    __shared__ u32x4 xs[256];                                     // the token's x, H <= 2048
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int G = H / 64, JT = I / 128, OPS = I / DOUT;
    // XCD-aware order: workgroups are dealt to the 8 XCDs round robin, and the ones on one
    // XCD take consecutive output groups, so the scale/bias lines they share (64 columns)
    // are fetched into one L2 rather than into all eight (OPS is a multiple of 16)
    const int slot = blockIdx.x / OPS, bl = blockIdx.x % OPS;
    const int o = (bl & 7) * (OPS >> 3) + (bl >> 3);
    {   // token blockIdx.y: its input row, logits, picks and h block
        const size_t t = blockIdx.y;
        x += t * H;
        logits += t * E;
        ids_out += t * k;
        tw_out += t * k;
        hbuf += t * NSLOT * I;
        hfac += t * NSLOT;
        // decode stack: the residual add the router kernel folded into this layer's input
        // is committed here, once every router wave has read res and yprev
        if (res != nullptr && blockIdx.x == 0)
            for (int i = 4 * threadIdx.x; i < H; i += 4 * 64 * DW) {
                floatx4 *pr = (floatx4 *)(res + t * H + i);
                *pr = *pr + *(const floatx4 *)(yprev + t * H + i);
            }
    }
    const int j = o >> 4, u = (o >> 2) & 3, v = o & 3;            // 8 o = 128 j + 32 u + 8 v
    const int gi = lane >> 4, cc = (lane >> 1) & 7, ph = lane & 1;
    const int lh = ph ^ (v & 1);                                  // logical half of my pieces
    const int tcg = 64 * u + 8 * v + cc;                          // my gate column; up is tcg + 32
    // my group g = 4 wave + gi (G <= 32: one pass of the 8 waves covers every group).  The
    // token's x (at most 4 KB) is loaded once per workgroup, 16 bytes per thread, and staged
    // in LDS after the weight loads are out; the eight column lanes of a group then read
    // their 64 bytes from there instead of each loading them from L2.
    const int g = 4 * wave + gi;
    const bool act = g < G;
    const int gc = min(g, G - 1);
    u32x4 xl = {0u, 0u, 0u, 0u};
    if ((int)threadIdx.x < H / 8) xl = *(const u32x4 *)(x + 8 * threadIdx.x);
    const float x2 = xn2[blockIdx.y];                             // ||x||^2 (router kernel)
    int ex = 0;
    if (slot < k && picks_given) {
        ex = ids_out[slot];                                       // written by decode_select_kernel
        MOE_DBG(ex >= 0 && ex < E, DBG_DECODE_ID);
        ex = (ex < 0 || ex >= E) ? 0 : ex;
    } else if (slot < k) {
        int pe;
        float pl;
        select_topk(logits, E, k, pe, pl, selw[wave]);
        ex = __builtin_amdgcn_readlane(pe, slot);
        MOE_DBG(ex >= 0 && ex < E, DBG_DECODE_ID);
        ex = (ex < 0 || ex >= E) ? 0 : ex;
        if (blockIdx.x == 0 && wave == 0) {
            const float wv = topk_weight(pl, k);
            if (lane < k) {
                ids_out[lane] = pe;
                tw_out[lane] = wv;
            }
        }
    }
    const uint8_t *tile = slot == k ? gw.pk_sh + (size_t)j * G * PK_BLOCK
                                    : gw.pk + ((size_t)ex * JT + j) * G * PK_BLOCK;
    const float *tcf = slot == k ? gw.colf_sh + (size_t)j * PK_COLF
                                 : gw.colf + ((size_t)ex * JT + j) * PK_COLF;
    // the columns' 2^-k and the expert's row-norm bound, for the eight output threads only
    // (lanes 0-7 of wave 0, output m = lane): the factor is a power of two, so applying it
    // to the reduced sums gives the same bits as applying it to every partial
    float kg = 1.0f, ku = 1.0f, nw = 0.0f;
    if (wave == 0) {
        const int tc = 64 * u + 8 * v + (lane & 7);
        kg = tcf[tc];
        ku = tcf[tc + 32];
        nw = gw.emeta[(size_t)(slot == k ? E : ex) * PK_EMETA];
    }
    u32x4 cw[2];
    uint16_t sv[2], bv[2];
    {
        const uint8_t *blk = tile + (size_t)gc * PK_BLOCK;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int tc = tcg + 32 * r;
            cw[r] = *(const u32x4 *)(blk + 32 * tc + 16 * ph);
            sv[r] = *(const uint16_t *)(blk + PK_CODES + 2 * tc);
            bv[r] = *(const uint16_t *)(blk + PK_CODES + 512 + 2 * tc);
        }
    }
    if ((int)threadIdx.x < H / 8) xs[threadIdx.x] = xl;
    __syncthreads();
    u32x4 xv[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) xv[qq] = xs[8 * gc + 4 * lh + qq];
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t cM = 0x000F000Fu, cC = 0x43004300u;
    asm volatile("" : "+v"(cM), "+v"(cC));
    float ag = 0.0f, au = 0.0f;
    if (act) {
        uint32_t xp[16];
        float sx = 0.0f;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            pair_words(xv[qq], xp + 4 * qq);
#pragma unroll
            for (int r = 0; r < 4; ++r) sx += bf16_lo(xv[qq][r]) + bf16_hi(xv[qq][r]);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float d = 0.0f;
            const uint32_t ww[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t c = dec_and_or(ww[qq] >> (4 * p), cM, cC);
                    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c),
                                                        __builtin_bit_cast(bf16x2, xp[4 * qq + p]), d, false);
                }
            // sum_k x_k (q_k s + b) = s (sum x (128 + q) - 128 sum x) + b sum x
            // (the block holds s and b times 2^k; the column factor 2^-k undoes it exactly,
            // after the reduction)
            const float val = bf16_to_f32(sv[r]) * (d - 128.0f * sx) + bf16_to_f32(bv[r]) * sx;
            if (r == 0) ag += val; else au += val;
        }
    }
    // sums over the two physical halves (lane bit 0) and the wave's four groups (lane bits
    // 4-5), then over the eight waves in wave order by the output lanes
    ag = pair_sum(ag);
    au = pair_sum(au);
    ag += __shfl_xor(ag, 16);
    au += __shfl_xor(au, 16);
    ag += __shfl_xor(ag, 32);
    au += __shfl_xor(au, 32);
    if (lane < 16 && ph == 0) {
        red[wave][cc][0] = ag;
        red[wave][cc][1] = au;
    }
    __syncthreads();
    if (threadIdx.x < DOUT) {
        const int m = threadIdx.x;
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int w = 0; w < DW; ++w) {
            gs += red[w][m][0];
            us += red[w][m][1];
        }
        gs *= kg;
        us *= ku;
        // h is kept as h 2^-f in fp16, f from the bound (row norm x ||x||)^2 on |h| (0 in
        // the usual range); every workgroup of the slot takes the same f, the first records 2^f
        const int f = h_exponent(nw, sqrtf(x2));
        hbuf[(size_t)slot * I + DOUT * o + m] = f32_to_f16(gs / (1.0f + expf(-gs)) * (us * exp2i(-f)));
        if (o == 0 && m == 0) hfac[slot] = exp2i(f);
    }
}

// 3. down.  Workgroup: 8 outputs n = 8 v' .. 8 v' + 7 of H (a 256-byte run of
// every block of their tile) for all nine slots and all groups of I.  Lane
// (sub, cc, ph) of wave w takes pair 4 (w + 8 it) + sub of the (slot, group)
// pairs, physical half ph of column cc; the pairs' partial sums meet in LDS and
// are added per output in a fixed order: groups, then slots in pick order with
// their routing weights, then the shared expert.
__global__ __launch_bounds__(64 * DW) void decode_down_kernel(
    const uint16_t *__restrict__ hbuf, const float *__restrict__ hfac, int H, int I,
    const int32_t *__restrict__ ids, const float *__restrict__ tw, int k, int E, GemmWeights gw,
    float *__restrict__ y) {
    __shared__ float part[DN_MAXP][DOUT];
    __shared__ float slot_sum[NSLOT][DOUT];
    extern __shared__ u32x4 hsh[];                                // the token's h block, (k+1) I fp16
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
    const int G = I / 64, JD = H / 256, NPAIR = (k + 1) * G;
    {   // token blockIdx.y: its h block, picks and output row
        const size_t t = blockIdx.y;
        hbuf += t * NSLOT * I;
        hfac += t * NSLOT;
        ids += t * k;
        tw += t * k;
        y += t * H;
    }
    // outputs 256 j + 8 v + (0..7); XCD-aware order: with the workgroups dealt to the 8 XCDs
    // round robin, the ones on one XCD share tile j and with it its scale/bias lines
    const int j = blockIdx.x % JD, v = blockIdx.x / JD;
    const int sub = lane >> 4, cc = (lane >> 1) & 7, ph = lane & 1;
    const int tc = 8 * v + cc;
    const int lh = ph ^ (v & 1);
    // the h block (9 KB at I = 512) is loaded once per workgroup, 16 bytes per thread and
    // pass, before the ids (it does not depend on them), and staged in LDS once the first
    // weight loads are out; every lane then reads its pairs' h values from LDS
    const int nh = (k + 1) * I / 8;
    constexpr int HCH = (NSLOT * 2048 / 8 + 64 * DW - 1) / (64 * DW);   // chunks per thread, I <= 2048
    u32x4 hl[HCH];
#pragma unroll
    for (int q = 0; q < HCH; ++q)
        if (tid + 64 * DW * q < nh) hl[q] = ((const u32x4 *)hbuf)[tid + 64 * DW * q];
    int sid[NSLOT];
    float sfac[NSLOT];     // per slot: routing weight (1 for the shared expert) times 2^f of its h
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
        const int e = s < k ? ids[s] : 0;
        MOE_DBG(e >= 0 && e < E, DBG_DECODE_ID);
        sid[s] = (e < 0 || e >= E) ? 0 : e;
        sfac[s] = (s < k ? tw[s] : 1.0f) * hfac[s];
    }
    // thread (slot tid / 8, output tid % 8), tid < 72: that slot's column factor 2^-k of the
    // output, applied to the slot's reduced sum (a power of two: the same bits as applying it
    // to every partial), loaded now and used at the end
    float kfm = 1.0f;
    if (tid < NSLOT * DOUT) {
        const int s = tid >> 3;
        int e = 0;
#pragma unroll
        for (int r = 0; r < NSLOT; ++r)
            if (r == s) e = sid[r];
        kfm = (s == k ? gw.colf_sh + (size_t)j * PK_COLF
                      : gw.colf + ((size_t)e * JD + j) * PK_COLF)[8 * v + (tid & 7)];
    }
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    uint32_t cM = 0x000F000Fu, cC = 0x64006400u;
    asm volatile("" : "+v"(cM), "+v"(cC));
    const int npass = (NPAIR + 4 * DW - 1) / (4 * DW);
    for (int it0 = 0; it0 < npass; it0 += DN_BATCH) {
        u32x4 cw[DN_BATCH], hv[DN_BATCH][4];
        uint16_t sv[DN_BATCH], bv[DN_BATCH];
        int pp[DN_BATCH], hcs[DN_BATCH];
#pragma unroll
        for (int b = 0; b < DN_BATCH; ++b) {
            const int p = 4 * (wave + DW * (it0 + b)) + sub;
            pp[b] = p;
            const int pc = min(p, NPAIR - 1);
            const int s = pc / G, g = pc - s * G;
            int e = 0;
#pragma unroll
            for (int r = 0; r < NSLOT; ++r)
                if (r == s) e = sid[r];
            const uint8_t *blk = (s == k ? gw.pk_sh + (size_t)j * G * PK_BLOCK
                                         : gw.pk + ((size_t)e * JD + j) * G * PK_BLOCK) +
                                 (size_t)g * PK_BLOCK;
            // pairs past the end load the last pair again (unconditional loads are
            // issued together) and are skipped below
            cw[b] = *(const u32x4 *)(blk + 32 * tc + 16 * ph);
            sv[b] = *(const uint16_t *)(blk + PK_CODES + 2 * tc);
            bv[b] = *(const uint16_t *)(blk + PK_CODES + 512 + 2 * tc);
            hcs[b] = s * I / 8 + 8 * g + 4 * lh;                       // its h values in LDS
        }
        if (it0 == 0) {
#pragma unroll
            for (int q = 0; q < HCH; ++q)
                if (tid + 64 * DW * q < nh) hsh[tid + 64 * DW * q] = hl[q];
            __syncthreads();
        }
#pragma unroll
        for (int b = 0; b < DN_BATCH; ++b)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) hv[b][qq] = hsh[hcs[b] + qq];
#pragma unroll
        for (int b = 0; b < DN_BATCH; ++b) {
            if (pp[b] >= NPAIR) continue;
            uint32_t hp[16];
            float shs = 0.0f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                pair_words(hv[b][qq], hp + 4 * qq);
#pragma unroll
                for (int r = 0; r < 4; ++r) shs += f16_lo(hv[b][qq][r]) + f16_hi(hv[b][qq][r]);
            }
            float d = 0.0f;
            const uint32_t ww[4] = {cw[b].x, cw[b].y, cw[b].z, cw[b].w};
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t c = dec_and_or(ww[qq] >> (4 * p), cM, cC);
                    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, c), __builtin_bit_cast(h2, hp[4 * qq + p]),
                                               d, false);
                }
            // sum_i h_i (q_i s + b) = s (sum h (1024 + q) - 1024 sum h) + b sum h
            const float val = pair_sum(bf16_to_f32(sv[b]) * (d - 1024.0f * shs) + bf16_to_f32(bv[b]) * shs);
            if (ph == 0) part[pp[b]][cc] = val;
        }
    }
    __syncthreads();
    if (tid < NSLOT * DOUT) {
        // each slot's sum over its groups, in group order, times its column factor
        const int s = tid >> 3, m = tid & 7;
        float a = 0.0f;
        for (int g = 0; g < G; ++g) a += part[s * G + g][m];
        slot_sum[s][m] = a * kfm;
    }
    __syncthreads();
    if (tid < DOUT) {
        // each slot's h was kept as h 2^-f: its weight (1 for the shared expert) times 2^f
        float sum = 0.0f;
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) sum = __builtin_fmaf(sfac[s], slot_sum[s][tid], sum);
        y[256 * j + DOUT * v + tid] = sum;
    }
}

void launch_decode(const moe_shape &sh, const uint16_t *x, const moe_weights &w, int32_t *ids,
                   float *tw, float *y, void *scratch, hipStream_t s, float *res, const float *yprev,
                   float eps, uint16_t *u_out) {
    const int T = sh.T, H = sh.H, I = sh.I, E = sh.E, k = sh.top_k;
    char *p = (char *)scratch;
    float *logits = (float *)p;                                   // [T][E]
    uint16_t *hbuf = (uint16_t *)(p + logits_bytes(T, E));        // fp16 [T][k+1][I]
    float *hfac = (float *)(p + logits_bytes(T, E) + hbuf_bytes(T, I, k));   // [T][k+1]
    float *xn2 = hfac + (size_t)T * (k + 1);                                  // [T]
    // the API admits top_k = 8, E <= 256, H <= 2048 (G <= 32), I <= 2048, T <= kDecodeMaxT
    if (k + 1 != NSLOT || E > 256 || H > 2048 || I > 2048 || T < 1 || T > kDecodeMaxT) return;
    const GemmWeights gu = gemm_weights(w.packed, H, I, E, true);
    const GemmWeights dn = gemm_weights(w.packed, H, I, E, false);
    // with a residual the router kernel makes the layer input and writes it to u_out
    const uint16_t *xin = res ? u_out : x;
    // every kernel takes token t = blockIdx.y; the tokens are independent problems
    hipLaunchKernelGGL(decode_router_kernel, dim3(E, T), dim3(64), 0, s, x, w.router_wt, w.router_bias,
                       H, logits, res, yprev, eps, u_out, xn2);
    // one token: every gate/up wave takes the top-k itself (no extra launch on the
    // latency chain); more tokens: the picks are taken once per token
    const bool picks_given = T > 1;
    if (picks_given)
        hipLaunchKernelGGL(decode_select_kernel, dim3(T), dim3(64), 0, s, logits, E, k, ids, tw);
    hipLaunchKernelGGL(decode_gateup_kernel, dim3((k + 1) * (I / DOUT), T), dim3(64 * DW), 0, s, xin,
                       logits, H, I, k, E, gu, ids, tw, hbuf, hfac, xn2, picks_given, res, yprev);
    hipLaunchKernelGGL(decode_down_kernel, dim3(H / DOUT, T), dim3(64 * DW), (size_t)(k + 1) * I * 2, s,
                       hbuf, hfac, H, I, ids, tw, k, E, dn, y);
}

size_t decode_scratch_bytes(int T, int H, int I, int k) {
    (void)H;
    return decode_scratch_size(T, I, k);
}

MOE_DBG_READER(dbg_read_decode)

}  // namespace moe
