// Grouped expert GEMMs over 4-bit affine weights on fp16 MFMA (gfx950).
//
// The pages rebuild 16-bit weights tile by tile inside the grouped GEMM and
// accumulate in FP32 (mechatronicstore.cl, "Prefill: pesos comprimidos y
// enrutamiento en la GPU").  Here the rebuilt weight is exact: with a bf16
// scale s (8 significant bits) and a code q in 0..15, (q - 8) * s needs at
// most 11 significant bits, so it is an fp16 number.  Splitting
//
//   w = q s + b = (q - 8) s + c,        c = b + 8 s   (per group, fp32),
//
// the contraction becomes
//
//   sum_k x_k w_k = sum_k x_k [(q_k - 8) s_g]  +  sum_g c_g xs_g,   xs_g = sum_{k in g} x_k
//
//  * each code word turns into four fp16 pairs (q - 8) s: one and-or drops a
//    nibble pair into the mantissa of 1024.0, one packed add removes 1032,
//    one packed multiply applies the scale, all exact;
//  * the activations enter the MFMA in fp16 (x is converted once, exactly for
//    |x| in the fp16 normal range; h is written in fp16 by the gate/up pass);
//  * the 32x32x16 fp16 MFMA accumulates straight into the fp32 result, so no
//    per-group rescaling is left on the vector ALU;
//  * the rank-G term sum_g c_g xs_g is zero whenever b = -8 s (the format's
//    symmetric case); otherwise a wave adds it with a small MFMA pass over
//    K = 3G of fp16 hi/lo splits: c_hi xs_hi + c_hi xs_lo + c_lo xs_hi.
//
// Element order: code pairs come out as k = (0,4), (1,5), (2,6), (3,7) of each
// 8-block, so activations are stored with every 8-block permuted to
// (0,4,1,5,2,6,3,7): x by the router's preparation pass, h by the gate/up
// epilogue.
//
// Tiles: a workgroup (4 waves) takes one routing block (up to 128 rows of one
// expert) and 256 weight columns: gate/up takes 128 columns of I from both
// projections (wave w owns gate and up columns 32w..32w+31, so SwiGLU stays
// inside a lane), down takes 256 columns of H.  Each wave computes all rows x
// its 64 columns.  Per 64-wide K step (one quantisation group) the activation
// rows, the code words, the scales and the biases are copied global->LDS by
// DMA (no registers) into a 3-deep ring, swizzled so that every MFMA operand
// read is free of bank conflicts.  Two workgroups share a CU.
#include "common.h"

#include <algorithm>

namespace moe {

constexpr int NW = 4;                        // waves per workgroup
constexpr int NTHR = 64 * NW;
constexpr int KC = 64;                       // K per stage: one quantisation group
constexpr int NSTAGE = 3;
constexpr int A_BYTES = kBM * KC * 2;        // [128 rows][8 x 16 B], 16 B slots XOR-swizzled
constexpr int B_BYTES = 256 * 32;            // [256 columns][2 x 16 B halves], halves swizzled
constexpr int STAGE = A_BYTES + B_BYTES;
// scales and biases travel in pairs of groups (one dword per column, copied on
// even chunks) through a 2-slot ring: [slot][s | b][256 columns] dwords
constexpr int PAIR_BYTES = 2 * 256 * 4;
constexpr int L_PAIR = NSTAGE * STAGE;
constexpr int L_TOTAL = L_PAIR + 2 * PAIR_BYTES;   // 77824: two workgroups per CU
constexpr int HS_LD = 272;                   // epilogue h tile row stride (bytes)
constexpr int YS_LD = 1056;                  // epilogue y tile row stride (bytes)
static_assert(kBM * HS_LD <= L_TOTAL && 32 * YS_LD <= L_TOTAL, "epilogue tiles fit the ring");

struct GemmArgs {
    const uint16_t *A;     // fp16 permuted activations: x [T][H] (gate/up) or h [rows][I] (down)
    const float *Asum;     // group sums of A rows: by token [T][G] or by row [rows][G]
    int K, G;
    int N;                 // rows of one projection: I (gate/up) or H (down)
    GemmProj p0, p1;       // routed projections: gate, up  |  down, -
    GemmProj s0, s1;       // the shared expert's
    const int32_t *blocks;
    const int32_t *num_blocks;
    const int32_t *sched;  // routed blocks in GEMM order
    int max_blocks;
    const int32_t *row_token;
    const float *row_w;
    int T, topk, E;
    int n_tiles;
    int n_shared;          // shared-expert M blocks (scheduled first)
    uint16_t *h;           // gate/up output, fp16 [T*topk + T][I]
    float *hsum;           // gate/up output, group sums of h [T*topk + T][I/64]
    float *y;
    uint16_t *stage;       // routed down outputs times their routing weight, bf16 [T*topk][H]
};

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
    return r;
}

// 8 codes of one word -> 8 fp16 weights (q - 8) * s, element order (0,4,1,5,2,6,3,7)
__device__ __forceinline__ f16x8 rebuild8(uint32_t w, uint32_t M, uint32_t C, f16x2 m1032,
                                          f16x2 ss) {
    const f16x2 p0 = (__builtin_bit_cast(f16x2, and_or(w, M, C)) + m1032) * ss;
    const f16x2 p1 = (__builtin_bit_cast(f16x2, and_or(w >> 4, M, C)) + m1032) * ss;
    const f16x2 p2 = (__builtin_bit_cast(f16x2, and_or(w >> 8, M, C)) + m1032) * ss;
    const f16x2 p3 = (__builtin_bit_cast(f16x2, and_or(w >> 12, M, C)) + m1032) * ss;
    u32x4 v;
    v.x = __builtin_bit_cast(uint32_t, p0);
    v.y = __builtin_bit_cast(uint32_t, p1);
    v.z = __builtin_bit_cast(uint32_t, p2);
    v.w = __builtin_bit_cast(uint32_t, p3);
    return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ floatx16 mfma16(f16x8 a, f16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Asynchronous global->LDS copies.  Lane i of the wave writes LDS bytes
// [lds + 16 i, +16) (dword form: [lds + 4 i, +4)).  Issued through inline assembly so that the compiler does not
// wait for them before every LDS read; completion is awaited explicitly
// (s_waitcnt vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}

// One tile: a routing block (or a shared-expert block) times 256 weight columns.
struct Tile {
    bool shared;
    int e, r0, nrows, ntile;
};

// activation source row of tile row m (rows past nrows repeat row 0)
template <int MODE>
__device__ __forceinline__ int src_row(const GemmArgs &a, const Tile &t, int m) {
    const int mm = m < t.nrows ? m : 0;
    if (MODE == 0) {
        const int tok = t.shared ? (t.r0 - a.T * a.topk + mm) : a.row_token[t.r0 + mm];
        return (tok >= 0 && tok < a.T) ? tok : 0;
    }
    return t.r0 + mm;
}

// projection and row of weight column bc (0..255) of the tile
template <int MODE>
__device__ __forceinline__ void column_of(const GemmArgs &a, const Tile &t, int bc, GemmProj &p,
                                          size_t &row) {
    const int w = bc >> 6, nt = (bc >> 5) & 1, l = bc & 31;
    int n;
    if (MODE == 0) {
        p = t.shared ? (nt ? a.s1 : a.s0) : (nt ? a.p1 : a.p0);
        n = t.ntile * 128 + 32 * w + l;
    } else {
        p = t.shared ? a.s0 : a.p0;
        n = t.ntile * 256 + 64 * w + 32 * nt + l;
    }
    row = (t.shared ? 0 : (size_t)t.e * a.N) + n;
}

template <int MODE, int MT>
__device__ void gemm_tile(const GemmArgs &a, const Tile &t, uint8_t *smem) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)smem;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));              // recomputed per item: nothing lane-dependent is hoisted
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, gg = lane >> 5;
    const int K = a.K, G = a.G, nch = K / KC;

    // ---- DMA sources of this thread
    // A: rows 32i + tid/8 (i = 0..3); 16 B slot tid&7 of a row holds its
    // segment slot ^ ((row >> 1) & 7)
    uint32_t aoff[4];
    {
        const int seg = (tid & 7) ^ ((tid >> 4) & 7);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 32 * i + (tid >> 3);
            aoff[i] = (uint32_t)src_row<MODE>(a, t, m) * (uint32_t)K + (uint32_t)(8 * seg);
        }
    }
    // B: columns 128i + tid/2 (i = 0, 1); LDS half tid&1 holds code words
    // 4 * ((tid&1) ^ ((col >> 3) & 1)) .. +3 of the group
    const uint32_t *qsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        GemmProj p;
        size_t row;
        column_of<MODE>(a, t, 128 * i + (tid >> 1), p, row);
        qsrc[i] = p.q + row * (size_t)(K / 8) + 4 * ((tid & 1) ^ ((tid >> 4) & 1));
    }
    // scale and bias of column tid
    const uint16_t *ssrc, *bsrc;
    {
        GemmProj p;
        size_t row;
        column_of<MODE>(a, t, tid, p, row);
        ssrc = p.s + row * (size_t)G;
        bsrc = p.b + row * (size_t)G;
    }
    auto issue = [&](int c) {
        const uint32_t base = lds0 + (uint32_t)((c % NSTAGE) * STAGE);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16(a.A + (size_t)aoff[i] + c * KC, base + (uint32_t)((i * 256 + wave * 64) * 16));
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16(qsrc[i] + c * 8, base + (uint32_t)(A_BYTES + (i * 256 + wave * 64) * 16));
        if ((c & 1) == 0) {                      // groups c, c+1 (G is even)
            const uint32_t pb = lds0 + (uint32_t)(L_PAIR + ((c >> 1) & 1) * PAIR_BYTES + wave * 256);
            dma4(ssrc + c, pb);
            dma4(bsrc + c, pb + 1024);
        }
    };
    // copies per thread: 8 for an even stage, 6 for an odd one.  Waiting for
    // "all but the newest n" with n = the count of the stage issued after it.

    issue(0);
    if (nch > 1) issue(1);

    floatx16 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][0][i] = acc[mt][1][i] = 0.0f;

    uint32_t cM = 0x000F000Fu, cC = 0x64006400u;
    asm volatile("" : "+v"(cM), "+v"(cC));       // keep the unpack constants in VGPRs
    const f16x2 m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const int sw = (l32 >> 1) & 7;
    const int swb = (l32 >> 3) & 1;
    bool nz = false;                             // any group with b != -8 s in my columns

    for (int c = 0; c < nch; ++c) {
        if (c + 1 >= nch)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (((c + 1) & 1) == 0)
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        __syncthreads();                         // stage c visible; stage c-1 no longer read
        if (c + 2 < nch) issue(c + 2);

        const uint8_t *sb = smem + (c % NSTAGE) * STAGE;
        u32x4 wq[2];
        f16x2 ss[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int bc = 64 * wave + 32 * nt + l32;
            wq[nt] = *(const u32x4 *)(sb + A_BYTES + bc * 32 + 16 * (gg ^ swb));
            const uint8_t *pr = smem + L_PAIR + ((c >> 1) & 1) * PAIR_BYTES + bc * 4;
            const uint32_t sv = *(const uint32_t *)pr, bv = *(const uint32_t *)(pr + 1024);
            const float sf = (c & 1) ? bf16_hi(sv) : bf16_lo(sv);
            nz |= ((c & 1) ? bf16_hi(bv) : bf16_lo(bv)) != -8.0f * sf;
            const _Float16 sh = (_Float16)sf;
            ss[nt] = f16x2{sh, sh};
        }
        const uint8_t *arow = sb + l32 * (KC * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f16x8 b0 = rebuild8(wq[0][j], cM, cC, m1032, ss[0]);
            const f16x8 b1 = rebuild8(wq[1][j], cM, cC, m1032, ss[1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f16x8 af =
                    *(const f16x8 *)(arow + mt * 32 * (KC * 2) + 16 * ((4 * gg + j) ^ sw));
                acc[mt][0] = mfma16(af, b0, acc[mt][0]);
                acc[mt][1] = mfma16(af, b1, acc[mt][1]);
            }
        }
    }

    // ---- rank-G term for groups whose bias is not -8 s (none for symmetric codes)
    if (__any(nz)) {
        const int K3 = 3 * G;
        int srcr[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) srcr[mt] = src_row<MODE>(a, t, 32 * mt + l32);
        const uint16_t *cs[2], *cb[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            GemmProj p;
            size_t row;
            column_of<MODE>(a, t, 64 * wave + 32 * nt + l32, p, row);
            cs[nt] = p.s + row * (size_t)G;
            cb[nt] = p.b + row * (size_t)G;
        }
        for (int j3 = 0; j3 < (K3 + 15) / 16; ++j3) {
            uint32_t bw[2][4], aw[MT][4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float bvals[2][2], avals[MT][2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    // operand slot k'' = 16 j3 + 8 gg + 2 e2 + hh: term tau, group g
                    const int kk = 16 * j3 + 8 * gg + 2 * e2 + hh;
                    const int tau = kk / G, g = kk - tau * G;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        float v = 0.0f;
                        if (tau < 3) {
                            const float cf = bf16_to_f32(cb[nt][g]) + 8.0f * bf16_to_f32(cs[nt][g]);
                            const float hi = (float)(_Float16)cf;
                            v = tau < 2 ? hi : (float)(_Float16)(cf - hi);
                        }
                        bvals[nt][hh] = v;
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        float v = 0.0f;
                        if (tau < 3) {
                            const float xs = a.Asum[(size_t)srcr[mt] * G + g];
                            const float hi = (float)(_Float16)xs;
                            v = tau == 1 ? (float)(_Float16)(xs - hi) : hi;
                        }
                        avals[mt][hh] = v;
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) bw[nt][e2] = pack_f16x2(bvals[nt][0], bvals[nt][1]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) aw[mt][e2] = pack_f16x2(avals[mt][0], avals[mt][1]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4 av = {aw[mt][0], aw[mt][1], aw[mt][2], aw[mt][3]};
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const u32x4 bv = {bw[nt][0], bw[nt][1], bw[nt][2], bw[nt][3]};
                    acc[mt][nt] = mfma16(__builtin_bit_cast(f16x8, av),
                                         __builtin_bit_cast(f16x8, bv), acc[mt][nt]);
                }
            }
        }
    }

    // ---- epilogue.  Accumulator element i of lane (l32, gg) is row
    // 8*(i/4) + 4*gg + i%4 of its 32-row tile, column l32 of the wave's n-tile.
    __syncthreads();                             // every wave is done with the ring
    if (MODE == 0) {
        // SwiGLU -> fp16 h tile in LDS [128 rows][128 columns], columns permuted
        const int pc = perm_pos(32 * wave + l32);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * mt + 8 * (i >> 2) + 4 * gg + (i & 3);
                const float g = acc[mt][0][i], u = acc[mt][1][i];
                const float hv = __fdividef(g, 1.0f + __expf(-g)) * u;
                *(uint16_t *)(smem + row * HS_LD + 2 * pc) = f32_to_f16(hv);
            }
        __syncthreads();
        // thread: row tid/2, 64-column half tid&1 -> 128 B of h and one group sum
        const int row = tid >> 1, half = tid & 1;
        if (row < t.nrows) {
            const uint8_t *src = smem + row * HS_LD + half * 128;
            uint16_t *dst = a.h + (size_t)(t.r0 + row) * a.N + t.ntile * 128 + half * 64;
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const u32x4 v = *(const u32x4 *)(src + 16 * q);
#pragma unroll
                for (int r = 0; r < 4; ++r) sum += f16_lo(v[r]) + f16_hi(v[r]);
                *(u32x4 *)(dst + 8 * q) = v;
            }
            a.hsum[(size_t)(t.r0 + row) * (a.N / 64) + t.ntile * 2 + half] = sum;
        }
    } else {
        const int Trk = a.T * a.topk;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (mt > 0) __syncthreads();
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rr = 8 * (i >> 2) + 4 * gg + (i & 3);
                    *(float *)(smem + rr * YS_LD + 4 * (64 * wave + 32 * nt + l32)) = acc[mt][nt][i];
                }
            __syncthreads();
            // thread: row tid/8 of the 32-row tile, 32 columns from (tid&7)*32
            const int rr = tid >> 3, seg = tid & 7;
            const int row = 32 * mt + rr;
            if (row < t.nrows) {
                const uint8_t *src = smem + rr * YS_LD + seg * 128;
                const int col = t.ntile * 256 + seg * 32;
                if (t.shared) {
                    float *dst = a.y + (size_t)(t.r0 - Trk + row) * a.N + col;
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        *(floatx4 *)(dst + 4 * q) = *(const floatx4 *)(src + 16 * q);
                } else {
                    // routed row: weighted output staged in bf16 (fp32 range; the combine adds in fp32)
                    uint16_t *dst = a.stage + (size_t)(t.r0 + row) * a.N + col;
                    const float wr = a.row_w[t.r0 + row];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const floatx4 v0 = *(const floatx4 *)(src + 32 * q);
                        const floatx4 v1 = *(const floatx4 *)(src + 32 * q + 16);
                        u32x4 o;
                        o.x = pack_bf16x2(wr * v0[0], wr * v0[1]);
                        o.y = pack_bf16x2(wr * v0[2], wr * v0[3]);
                        o.z = pack_bf16x2(wr * v1[0], wr * v1[1]);
                        o.w = pack_bf16x2(wr * v1[2], wr * v1[3]);
                        *(u32x4 *)(dst + 8 * q) = o;
                    }
                }
            }
        }
    }
}

// Persistent grid: workgroup g takes work items j = g, g + gridDim, ...  Item j
// is (slot, n-tile) with slot = 8 (j / 8 / n_tiles) + j % 8 and n-tile
// (j / 8) % n_tiles, so all n-tiles of one block (which share its activation
// rows) land on workgroups with the same g mod 8, i.e. on the same XCD.  Slots
// are the shared-expert blocks, then the routed blocks in the routing
// schedule's order (largest first), so every round of the grid takes items of
// similar cost and the tail is short.
template <int MODE>
__global__ __launch_bounds__(NTHR, 2) void q4_gemm_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int nb = min(a.num_blocks[0], a.max_blocks);
    const int S = a.n_shared + max(nb, 0);
    const int jend = ((S + 7) >> 3) * 8 * a.n_tiles;
    for (int j = blockIdx.x; j < jend; j += gridDim.x) {
        const int q = j >> 3;
        const int slot = (q / a.n_tiles) * 8 + (j & 7);
        if (slot >= S) continue;
        Tile t;
        t.ntile = q % a.n_tiles;
        t.shared = slot < a.n_shared;
        t.e = 0;
        if (!t.shared) {
            const int mb = a.sched[slot - a.n_shared];
            if (mb < 0 || mb >= nb) continue;
            t.e = a.blocks[3 * mb];
            t.r0 = a.blocks[3 * mb + 1];
            t.nrows = a.blocks[3 * mb + 2];
            // a malformed block map turns into a no-op, never an out-of-bounds access
            if (t.e < 0 || t.e >= a.E || t.r0 < 0 || t.nrows < 1 || t.nrows > kBM ||
                t.r0 + t.nrows > a.T * a.topk)
                continue;
        } else {
            t.r0 = a.T * a.topk + slot * kBM;
            t.nrows = min(kBM, a.T - slot * kBM);
        }
        __syncthreads();                         // the previous item is done with the LDS
        switch ((t.nrows + 31) >> 5) {
            case 1: gemm_tile<MODE, 1>(a, t, smem); break;
            case 2: gemm_tile<MODE, 2>(a, t, smem); break;
            case 3: gemm_tile<MODE, 3>(a, t, smem); break;
            default: gemm_tile<MODE, 4>(a, t, smem); break;
        }
    }
}

static int shared_blocks(int T) { return (T + kBM - 1) / kBM; }

// persistent grid: two workgroups per CU, never more than there are work items
static unsigned grid_for(int n_shared, int max_blocks, int n_tiles) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const long items = (long)((n_shared + max_blocks + 7) / 8) * 8 * n_tiles;
    return (unsigned)std::min<long>(items, 2L * cus);
}

// the GEMM needs more dynamic LDS than the default launch limit
template <int MODE>
static void allow_lds() {
    static bool done = false;
    if (!done) {
        (void)hipFuncSetAttribute((const void *)q4_gemm_kernel<MODE>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, L_TOTAL);
        done = true;
    }
}

void launch_gateup(const moe_shape &sh, const uint16_t *xp, const float *xsum, GemmProj gate,
                   GemmProj up, GemmProj sgate, GemmProj sup, const int32_t *blocks,
                   const int32_t *num_blocks, const int32_t *sched, int max_blocks,
                   const int32_t *row_token, uint16_t *h, float *hsum, hipStream_t s) {
    GemmArgs a{};
    a.A = xp;
    a.Asum = xsum;
    a.K = sh.H;
    a.G = sh.H / 64;
    a.N = sh.I;
    a.p0 = gate;
    a.p1 = up;
    a.s0 = sgate;
    a.s1 = sup;
    a.blocks = blocks;
    a.num_blocks = num_blocks;
    a.sched = sched;
    a.max_blocks = max_blocks;
    a.row_token = row_token;
    a.T = sh.T;
    a.topk = sh.top_k;
    a.E = sh.E;
    a.n_tiles = sh.I / 128;
    a.n_shared = shared_blocks(sh.T);
    a.h = h;
    a.hsum = hsum;
    allow_lds<0>();
    hipLaunchKernelGGL(q4_gemm_kernel<0>, dim3(grid_for(a.n_shared, max_blocks, a.n_tiles)),
                       dim3(NTHR), L_TOTAL, s, a);
}

// y[t] += sum_j stage[tok_row[t][j]] in pick order j = 0..k-1, in fp32: a fixed
// order, so the combined output is reproducible bit for bit.  One thread per 8
// outputs (16 bytes of each bf16 staging row).
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ stage,
                                                      const int32_t *__restrict__ tok_row, int T,
                                                      int H, int k, float *__restrict__ y) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t per = (size_t)H / 8;
    if (i >= (size_t)T * per) return;
    const size_t t = i / per, n = (i % per) * 8;
    float4 a0 = *(const float4 *)(y + t * H + n);
    float4 a1 = *(const float4 *)(y + t * H + n + 4);
    int rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = j < k ? tok_row[t * k + j] : -1;
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (rows[j] >= 0 && rows[j] < T * k) v[j] = *(const u32x4 *)(stage + (size_t)rows[j] * H + n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (rows[j] < 0 || rows[j] >= T * k) continue;
        a0.x += bf16_lo(v[j].x);
        a0.y += bf16_hi(v[j].x);
        a0.z += bf16_lo(v[j].y);
        a0.w += bf16_hi(v[j].y);
        a1.x += bf16_lo(v[j].z);
        a1.y += bf16_hi(v[j].z);
        a1.z += bf16_lo(v[j].w);
        a1.w += bf16_hi(v[j].w);
    }
    *(float4 *)(y + t * H + n) = a0;
    *(float4 *)(y + t * H + n + 4) = a1;
}

void launch_down(const moe_shape &sh, const uint16_t *h, const float *hsum, GemmProj down,
                 GemmProj sdown, const int32_t *blocks, const int32_t *num_blocks,
                 const int32_t *sched, int max_blocks,
                 const int32_t *row_token, const float *row_w, const int32_t *tok_row,
                 uint16_t *stage, float *y, hipStream_t s) {
    GemmArgs a{};
    a.A = h;
    a.Asum = hsum;
    a.K = sh.I;
    a.G = sh.I / 64;
    a.N = sh.H;
    a.p0 = down;
    a.s0 = sdown;
    a.blocks = blocks;
    a.num_blocks = num_blocks;
    a.sched = sched;
    a.max_blocks = max_blocks;
    a.row_token = row_token;
    a.row_w = row_w;
    a.T = sh.T;
    a.topk = sh.top_k;
    a.E = sh.E;
    a.n_tiles = sh.H / 256;
    a.n_shared = shared_blocks(sh.T);
    a.y = y;
    a.stage = stage;
    allow_lds<1>();
    // shared-expert blocks write y, routed blocks their weighted staging rows ...
    hipLaunchKernelGGL(q4_gemm_kernel<1>, dim3(grid_for(a.n_shared, max_blocks, a.n_tiles)),
                       dim3(NTHR), L_TOTAL, s, a);
    // ... then each token adds its eight routed rows
    const size_t n8 = (size_t)sh.T * sh.H / 8;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, stage,
                       tok_row, sh.T, sh.H, sh.top_k, y);
}

}  // namespace moe
