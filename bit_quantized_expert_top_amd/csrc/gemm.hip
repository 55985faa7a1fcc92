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
//    symmetric case); otherwise the item starts its accumulators with a small
//    fp32 MFMA pass (32x32x2, no rounding of c or of the group sums xs).
//
// Element order: the tile layout keeps each word's even codes in its low
// nibbles and its odd codes in the high ones, so the and-or pairs (p, p + 4)
// are the code pairs (2p, 2p + 1) and the weights come out in natural order;
// x and h are stored in natural order too.
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
#include <utility>

namespace moe {

constexpr int NW = 4;                        // waves per workgroup
constexpr int NTHR = 64 * NW;
constexpr int KC = 64;                       // K per stage: one quantisation group
// One ring stage holds, for one 64-wide K step:
//   A  [32 MT rows][8 x 16 B]      activations, 16 B slots XOR-swizzled
//   B  [256 columns][2 x 16 B]     code words, halves swizzled      } one tile-layout
//   S  [256] bf16 scales, [256] bf16 biases                          } block, as stored
// A block of fewer rows has a smaller stage and so more stages in flight.
constexpr int B_BYTES = PK_CODES;
constexpr int S_BYTES = PK_BLOCK - PK_CODES;
template <int MT> struct Ring {
    static constexpr int A_BYTES = MT * 32 * KC * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int NST = MT == 1 ? 5 : MT == 2 ? 4 : 3;   // stages
    static constexpr int AHEAD = NST - 1;                         // stages issued ahead
    static constexpr int PER = MT + 3;                            // copies per thread and stage
};
constexpr int L_TOTAL = 3 * Ring<4>::STAGE;  // 76800: two workgroups per CU
static_assert(Ring<1>::NST * Ring<1>::STAGE <= L_TOTAL && Ring<2>::NST * Ring<2>::STAGE <= L_TOTAL &&
                  Ring<3>::NST * Ring<3>::STAGE <= L_TOTAL, "rings fit");
static_assert((Ring<1>::AHEAD - 1) * Ring<1>::PER < 64 && (Ring<2>::AHEAD - 1) * Ring<2>::PER < 64,
              "vmcnt range");
constexpr int HS_LD = 272;                   // epilogue h tile row stride (bytes)
constexpr int YS_LD = 1056;                  // epilogue y tile row stride (bytes)
static_assert(kBM * HS_LD <= L_TOTAL && 64 * YS_LD <= L_TOTAL, "epilogue tiles fit the ring");

struct GemmArgs {
    const uint16_t *A;     // fp16 activations: x [T][H] (gate/up) or h [rows][I] (down)
    const float *Asum;     // group sums of A rows: by token [T][G] or by row [rows][G]
    int K, G;
    int N;                 // rows of one projection: I (gate/up) or H (down)
    const uint8_t *pk;     // routed experts' tile-layout blocks [E][n_tiles][G]
    const uint8_t *pk_sh;  // the shared expert's [n_tiles][G]
    const float *colf;     // routed experts' column factors [E][n_tiles][PK_COLF]
    const float *colf_sh;  // the shared expert's [n_tiles][PK_COLF]
    const float *emeta;    // per expert slot: [0] bounds the L2 norm of its gate and up rows
    const float *tok;      // gate/up: per token {2^e, ||x||} (x enters as fp16 x 2^-e)
    float *hexp;           // per h row 2^f (h stored as h 2^-f): gate/up writes, down reads
    const int32_t *blocks;
    const int32_t *num_blocks;
    const int32_t *sched;  // routed blocks by cost class (4, 3, 2, 1 M tiles), then expert
    int32_t *qctl;         // this GEMM's queue head [0] and finished-workgroup count [QCTL_LINE]
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

// 8 codes of one tile-layout word -> 8 fp16 weights (q - 8) * s in code order
// (nibbles (0,4), (1,5), (2,6), (3,7) hold the code pairs (0,1), (2,3), (4,5), (6,7)).
// Nibbles 0 and 4 of a byte pair (mask M1 = 0x000F000F) land as 1024 + q, nibbles
// 1 and 5 (M2 = 0x00F000F0) as 1024 + 16 q; subtracting 1032 resp. 1152 leaves q - 8 resp.
// 16 (q - 8), and the scale s resp. s / 16 (exact in fp16 for |s| >= 2^-13,
// as a subnormal at worst) gives (q - 8) s exactly: 13 operations per word.
__device__ __forceinline__ f16x8 rebuild8(uint32_t w, uint32_t M1, uint32_t M2, uint32_t C,
                                          f16x2 a1, f16x2 a2, f16x2 s1, f16x2 s16) {
    const uint32_t w8 = w >> 8;
    const f16x2 p0 = (__builtin_bit_cast(f16x2, and_or(w, M1, C)) + a1) * s1;
    const f16x2 p1 = (__builtin_bit_cast(f16x2, and_or(w, M2, C)) + a2) * s16;
    const f16x2 p2 = (__builtin_bit_cast(f16x2, and_or(w8, M1, C)) + a1) * s1;
    const f16x2 p3 = (__builtin_bit_cast(f16x2, and_or(w8, M2, C)) + a2) * s16;
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
// (s_waitcnt vmcnt) before the barrier that publishes a stage.  The compiler does not see the
// copy inside the asm, so the statement keeps the one wait state that gfx9 needs between an
// SALU write of M0 and an LDS DMA that reads it.
// COH: the copy carries the agent-scope cache policy (sc1), so it returns what an sc1 store
// on another XCD wrote, even where this XCD's L2 holds an older copy of the line.
template <bool COH = false> __device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
    if constexpr (COH)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off sc1" ::"v"(g), "s"(lds)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
                     : "memory", "m0");
}
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}

// The same copies with a wave-uniform base address in SGPRs and a per-lane
// 32-bit byte offset: the per-lane offsets stay fixed over the K loop and each
// K step only moves the scalar base.  The base may have been written by a VALU
// instruction just before (an SGPR reloaded from a spill lane); gfx9 needs 5 wait states
// between that write and a vector memory instruction reading the SGPR, which the statement
// keeps itself (s_nop 2, the M0 write, s_nop 0).
template <bool COH = false>
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds) {
    if constexpr (COH)
        asm volatile("s_nop 2\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 sc1" ::"v"(voff), "s"(sbase),
                     "s"(lds)
                     : "memory", "m0");
    else
        asm volatile("s_nop 2\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                     "s"(lds)
                     : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 2\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// Vector stores of the GEMM outputs.  COH: agent-scope policy (sc1), written through to
// memory: where the sc1 copies of a down item on any XCD read h, and measured faster for the
// down outputs of the one launch as well.  The compiler does not
// see a store inside the asm, so the 16-byte form keeps the wait states itself: a store of more
// than 8 bytes reads its data registers after it issues, and the next instructions must not
// overwrite them (2 wait states on gfx940 and later).
template <bool COH> __device__ __forceinline__ void store16(void *p, u32x4 v) {
    if constexpr (COH)
        asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 2" ::"v"(p), "v"(v) : "memory");
    else
        *(u32x4 *)p = v;
}
template <bool COH> __device__ __forceinline__ void store4(float *p, float v) {
    if constexpr (COH)
        asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
    else
        *p = v;
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// s_waitcnt vmcnt(n) for a compile-time n
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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
        MOE_DBG(tok >= 0 && tok < a.T, DBG_GEMM_TOKEN);
        return (tok >= 0 && tok < a.T) ? tok : 0;
    }
    return t.r0 + mm;
}

// One tile.  Thread 0 also takes the workgroup's next work item from the queue
// head during the main loop and leaves it in *s_next.
// Per-item values that the epilogue reads from LDS, copied in by DMA at the item's start:
// the 256 columns' 2^-k factors, two per-row values (gate/up: 2^e of the row's token and
// its ||x||; down: the routing weight and 2^f of the row's h), and the expert slot's
// row-norm bound (gate/up).
struct ItemLds {
    float *colk;   // [256]
    float *ra;     // [kBM]
    float *rb;     // [kBM]
    float *ne;     // [64], all equal
};

// COH (the one-launch FFN): h, its group sums and its row factors travel between XCDs, so the
// gate/up pass stores them and the down pass copies them with the agent-scope policy.
// pend >= 0: slot whose gate/up item this workgroup finished last and has not yet reported; its
// stores are awaited with the first stage (s_waitcnt vmcnt(0)) and done[pend] incremented.
template <int MODE, int MT, bool COH>
__device__ void gemm_tile(const GemmArgs &a, const Tile &t, uint8_t *smem, int *s_next,
                          const ItemLds &il, int32_t *done, int pend) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)smem;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));              // recomputed per item: nothing lane-dependent is hoisted
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, gg = lane >> 5;
    const int K = a.K, G = a.G, nch = K / KC;

    using RG = Ring<MT>;
    // ---- DMA sources of this thread
    // A: rows 32i + tid/8 (i < MT); 16 B slot tid&7 of a row holds its
    // segment slot ^ ((row >> 1) & 7)
    // (byte offsets from the wave-uniform bases, fixed over the K loop)
    uint32_t aoff[MT];
    {
        const int seg = (tid & 7) ^ ((tid >> 4) & 7);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int m = 32 * i + (tid >> 3);
            aoff[i] = ((uint32_t)src_row<MODE>(a, t, m) * (uint32_t)K + (uint32_t)(8 * seg)) * 2u;
        }
    }
    // B and S: the tile's block of K step c is one contiguous tile-layout
    // block, copied as stored: 16 B pieces tid and 256 + tid of the codes,
    // and dword lane of the wave's quarter of the scale/bias bytes
    const uint8_t *tb = t.shared ? a.pk_sh + (size_t)t.ntile * G * PK_BLOCK
                                 : a.pk + ((size_t)t.e * a.n_tiles + t.ntile) * G * PK_BLOCK;
    const uint32_t boff = 16u * (uint32_t)tid;
    const uint32_t soff = (uint32_t)(PK_CODES + 256 * wave + 4 * lane);
    // stage c into ring slot SLOT (c % NST, known at compile time)
    auto issue = [&](int c, auto SLOT) {
        constexpr uint32_t base = (uint32_t)(decltype(SLOT)::value * RG::STAGE);
        const uint8_t *ag = (const uint8_t *)a.A + (size_t)c * (KC * 2);
#pragma unroll
        for (int i = 0; i < MT; ++i)
            dma16s<COH && MODE == 1>(ag, aoff[i], lds0 + base + (uint32_t)((i * 256 + wave * 64) * 16));
        const uint8_t *blk = tb + (size_t)c * PK_BLOCK;
        dma16s(blk, boff, lds0 + base + (uint32_t)(RG::A_BYTES + wave * 64 * 16));
        dma16s(blk + 4096, boff, lds0 + base + (uint32_t)(RG::A_BYTES + (256 + wave * 64) * 16));
        dma4s(blk, soff, lds0 + base + (uint32_t)(RG::A_BYTES + B_BYTES + wave * 256));
    };
    floatx16 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][0][i] = acc[mt][1][i] = 0.0f;

    const float *tcolf = t.shared ? a.colf_sh + (size_t)t.ntile * PK_COLF
                                  : a.colf + ((size_t)t.e * a.n_tiles + t.ntile) * PK_COLF;
    // ---- rank-G term, for tiles with some group whose bias is not -8 s (a flag set at load
    // time; none for symmetric codes): sum_g c_g xs_g, with c = b + 8 s per column and group
    // (from the block's values, so at the column's 2^k like the main loop's weights) and xs
    // the rows' group sums.  It runs before the main loop, in the (still free) ring: the G
    // blocks' scale/bias sections (1 KB each) and the rows' group sums are copied in by DMA in
    // one round trip, then fp32 MFMA steps (32 x 32 x 2, fp32 operands: no rounding of c or xs,
    // no range limit) start the accumulators.
    if (__builtin_amdgcn_readfirstlane(((const int *)tcolf)[PK_TFLAG])) {
        // thread (row 32 i + tid / 8, p = tid % 8) copies the row's group sums g = p + 8 u
        const int per = (G + 7) / 8;
        const uint32_t sb0 = lds0, xs0 = lds0 + (uint32_t)(G * 1024);
        for (int g = wave; g < G; g += NW)
            dma16(tb + (size_t)g * PK_BLOCK + PK_CODES + 16 * lane, sb0 + (uint32_t)(1024 * g));
        {
            const int p = tid & 7;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                // row 32 i + tid / 8 of the tile: its source row (gate/up: the token, read back
                // from the A copy offsets instead of reloading row_token)
                const int srow = MODE == 0 ? (int)((aoff[i] >> 1) / (uint32_t)K)
                                           : src_row<MODE>(a, t, 32 * i + (tid >> 3));
                for (int u = 0; u < per; ++u) {
                    const int g = p + 8 * u;
                    if (g < G)
                        dma4<COH && MODE == 1>(a.Asum + (size_t)srow * G + g,
                             xs0 + (uint32_t)(4 * ((i * per + u) * 256 + 64 * wave)));
                }
            }
        }
        wait_vm<0>();
        __syncthreads();
        const uint8_t *sbl = smem;
        const float *xsl = (const float *)(smem + G * 1024);
        // k step j: groups 2 j and 2 j + 1; lane (l32, gg) supplies group 2 j + gg of row l32
        // (A) and of column l32 (B)
        for (int j = 0; j < (G + 1) / 2; ++j) {
            const int g = 2 * j + gg;
            float bv[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const uint8_t *sp = sbl + 1024 * min(g, G - 1) + 2 * (64 * wave + 32 * nt + l32);
                const float cf = __builtin_fmaf(8.0f, bf16_to_f32(*(const uint16_t *)sp),
                                                bf16_to_f32(*(const uint16_t *)(sp + 512)));
                bv[nt] = g < G ? cf : 0.0f;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float xs = g < G ? xsl[(mt * per + (g >> 3)) * 256 + 8 * l32 + (g & 7)] : 0.0f;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(xs, bv[nt], acc[mt][nt], 0, 0, 0);
            }
        }
        __syncthreads();                         // the staged operands are no longer read
    }

    // RG::PER copies per thread and stage, completing in order: stage c is in
    // once at most (stages issued after it) * PER copies are outstanding.
    // The epilogue's per-item values (ItemLds) are copied into LDS by DMA before the
    // stage copies (so older than all of them) and complete with the main loop's last
    // wait.  Plain loads would be waited for in the epilogue behind its own stores.
    {
        auto lds_of = [](const float *p) {
            return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
        };
        dma4(tcolf + tid, lds_of(il.colk) + (uint32_t)(256 * wave));
        if (wave < 2) {
            const int m = min(64 * wave + lane, t.nrows - 1);
            if (MODE == 0) {
                const int tok = src_row<MODE>(a, t, m);
                dma4(a.tok + 2 * (size_t)tok, lds_of(il.ra) + (uint32_t)(256 * wave));
                dma4(a.tok + 2 * (size_t)tok + 1, lds_of(il.rb) + (uint32_t)(256 * wave));
            } else {
                if (!t.shared) dma4(a.row_w + t.r0 + m, lds_of(il.ra) + (uint32_t)(256 * wave));
                dma4<COH>(a.hexp + t.r0 + m, lds_of(il.rb) + (uint32_t)(256 * wave));
            }
        } else if (MODE == 0 && wave == 2) {
            dma4(a.emeta + (size_t)(t.shared ? a.E : t.e) * PK_EMETA, lds_of(il.ne));
        }
    }
    static_for<RG::AHEAD>([&](auto P) {
        if (decltype(P)::value < nch) issue(decltype(P)::value, P);
    });

    uint32_t cM = 0x000F000Fu, cM2 = 0x00F000F0u, cC = 0x64006400u;
    asm volatile("" : "+v"(cM), "+v"(cM2), "+v"(cC));   // keep the unpack constants in VGPRs
    const f16x2 m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2 m1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const int sw = (l32 >> 1) & 7;
    const int swb = (l32 >> 3) & 1;
    int next = 0;

    // K loop unrolled by the ring depth, so that stage c's ring slot (c % NST)
    // and with it every LDS address of the step is a compile-time constant
    for (int c0 = 0; c0 < nch; c0 += RG::NST) {
        static_for<RG::NST>([&](auto U) {
            constexpr int u = decltype(U)::value;
            const int c = c0 + u;
            if (c >= nch) return;
            // stages issued after c: min(AHEAD - 1, nch - 1 - c)
            const int after = min(RG::AHEAD - 1, nch - 1 - c);
            const bool report = c == 0 && pend >= 0;   // also the last item's stores
            if (after <= 0 || report)
                wait_vm<0>();
            else if (after == 1)
                wait_vm<RG::PER>();
            else if (after == 2)
                wait_vm<(RG::AHEAD > 2 ? 2 : 0) * RG::PER>();
            else
                wait_vm<(RG::AHEAD > 3 ? 3 : 0) * RG::PER>();
            __syncthreads();                     // stage c visible; stage c-1 no longer read
            if (report && tid == 0)
                __hip_atomic_fetch_add(done + pend, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (c + RG::AHEAD < nch)             // into the slot of stage c-1
                issue(c + RG::AHEAD, std::integral_constant<int, (u + RG::AHEAD) % RG::NST>{});
            if (c == 1 && tid == 0) next = atomicAdd(&a.qctl[0], 1);   // overlaps the tile

            const uint8_t *sb = smem + u * RG::STAGE;
            u32x4 wq[2];
            f16x2 ss[2], ss16[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int bc = 64 * wave + 32 * nt + l32;
                wq[nt] = *(const u32x4 *)(sb + RG::A_BYTES + bc * 32 + 16 * (gg ^ swb));
                const uint8_t *pr = sb + RG::A_BYTES + B_BYTES + bc * 2;
                const float sf = bf16_to_f32(*(const uint16_t *)pr);
                const _Float16 sh = (_Float16)sf, sh16 = (_Float16)(sf * 0.0625f);
                ss[nt] = f16x2{sh, sh};
                ss16[nt] = f16x2{sh16, sh16};
            }
            const uint8_t *arow = sb + l32 * (KC * 2);
            // per 16-wide k slice j: the MT A fragments of slice j+1 are read together and
            // its two B fragments rebuilt while slice j runs its 2 MT MFMAs (both
            // double-buffered); the build's iterative-ILP scheduler keeps this order, so the
            // LDS latency hides behind the matrix core instead of stalling each MFMA pair
            auto a_frag = [&](int j, int mt) {
                return *(const f16x8 *)(arow + mt * 32 * (KC * 2) + 16 * ((4 * gg + j) ^ sw));
            };
            f16x8 af[2][MT], bf[2][2];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) af[0][mt] = a_frag(0, mt);
            bf[0][0] = rebuild8(wq[0][0], cM, cM2, cC, m1032, m1152, ss[0], ss16[0]);
            bf[0][1] = rebuild8(wq[1][0], cM, cM2, cC, m1032, m1152, ss[1], ss16[1]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cur = j & 1, nxt = cur ^ 1;
                if (j < 3) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) af[nxt][mt] = a_frag(j + 1, mt);
                    bf[nxt][0] = rebuild8(wq[0][j + 1], cM, cM2, cC, m1032, m1152, ss[0], ss16[0]);
                    bf[nxt][1] = rebuild8(wq[1][j + 1], cM, cM2, cC, m1032, m1152, ss[1], ss16[1]);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[mt][0] = mfma16(af[cur][mt], bf[cur][0], acc[mt][0]);
                    acc[mt][1] = mfma16(af[cur][mt], bf[cur][1], acc[mt][1]);
                }
            }
        });
    }

    if (tid == 0) *s_next = next;                // read after the caller's next barrier
    // ---- epilogue.  Accumulator element i of lane (l32, gg) is row
    // 8*(i/4) + 4*gg + i%4 of its 32-row tile, column l32 of the wave's n-tile.
    __syncthreads();                             // every wave is done with the ring
    if (MODE == 0) {
        // per row: the token's 2^e undoes the activation scale; h is stored as h 2^-f, f from
        // the bound (expert row norm x ||x||)^2 on |h| (0 in the usual range); 2^f is kept
        // per row for the down GEMM
        if (tid < kBM) {
            const int f = h_exponent(il.ne[0], il.rb[tid]);
            il.rb[tid] = exp2i(-f);
            if (t.ntile == 0 && tid < t.nrows) store4<COH>(a.hexp + t.r0 + tid, exp2i(f));
        }
        __syncthreads();
        // SwiGLU -> fp16 h tile in LDS [128 rows][128 columns]
        const int pc = 32 * wave + l32;
        const float kg = il.colk[64 * wave + l32], ku = il.colk[64 * wave + 32 + l32];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * mt + 8 * (i >> 2) + 4 * gg + (i & 3);
                const float al = il.ra[row];
                const float g = acc[mt][0][i] * (al * kg), u = acc[mt][1][i] * (al * ku);
                const float hv = __fdividef(g, 1.0f + __expf(-g)) * (u * il.rb[row]);
                *(uint16_t *)(smem + row * HS_LD + 2 * pc) = f32_to_f16(hv);
            }
        __syncthreads();
        // group sums: thread = row tid/2, 64-column half tid&1, summed in column order
        {
            const int row = tid >> 1, half = tid & 1;
            if (row < t.nrows) {
                const uint8_t *src = smem + row * HS_LD + half * 128;
                float sum = 0.0f;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const u32x4 v = *(const u32x4 *)(src + 16 * q);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sum += f16_lo(v[r]) + f16_hi(v[r]);
                }
                store4<COH>(a.hsum + (size_t)(t.r0 + row) * (a.N / 64) + t.ntile * 2 + half, sum);
            }
        }
        // h: 16 lanes per row, so that each store instruction writes whole 128-byte lines (the
        // sc1 stores are written through line by line)
#pragma unroll
        for (int q = 0; q < kBM * 16 / NTHR; ++q) {
            const int p = q * NTHR + tid, row = p >> 4, c16 = p & 15;
            if (row < t.nrows)
                store16<COH>(a.h + (size_t)(t.r0 + row) * a.N + t.ntile * 128 + 8 * c16,
                             *(const u32x4 *)(smem + row * HS_LD + 16 * c16));
        }
    } else {
        const int Trk = a.T * a.topk;
        // stores: 32 consecutive lanes write one row's 256 columns, so that every store
        // instruction covers whole 128-byte lines.  Routed rows (bf16): lane c8 takes columns
        // 8 c8 .. 8 c8 + 7, one 16-byte store.  Shared rows (fp32): columns 4 c8 .. 4 c8 + 3 and
        // 128 + 4 c8 .. 128 + 4 c8 + 3, two 16-byte stores each covering 512 contiguous bytes.
        const int c8 = tid & 31;
        const int cA = t.shared ? 4 * c8 : 8 * c8, cB = t.shared ? 128 + 4 * c8 : 8 * c8 + 4;
        const floatx4 k0 = *(const floatx4 *)(il.colk + cA);          // 2^-k per column
        const floatx4 k1 = *(const floatx4 *)(il.colk + cB);
        const int col0 = t.ntile * 256;
        // two m-tiles (64 rows) per pass through the LDS y tile
#pragma unroll
        for (int p = 0; p < (MT + 1) / 2; ++p) {
            if (p > 0) __syncthreads();
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int mt = 2 * p + h2;
                if (mt < MT) {
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int rr = 32 * h2 + 8 * (i >> 2) + 4 * gg + (i & 3);
                            *(float *)(smem + rr * YS_LD + 4 * (64 * wave + 32 * nt + l32)) = acc[mt][nt][i];
                        }
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int rr = (tid >> 5) + 8 * i;               // row of this pass's 64
                const int row = 64 * p + rr;
                if (2 * p + (rr >> 5) < MT && row < t.nrows) {
                    const uint8_t *src = smem + rr * YS_LD;
                    const floatx4 s0 = *(const floatx4 *)(src + 4 * cA);
                    const floatx4 s1 = *(const floatx4 *)(src + 4 * cB);
                    if (t.shared) {
                        const float hx = il.rb[row];
                        float *dst = a.y + (size_t)(t.r0 - Trk + row) * a.N + col0;
                        store16<COH>(dst + cA, __builtin_bit_cast(u32x4, s0 * (k0 * hx)));
                        store16<COH>(dst + cB, __builtin_bit_cast(u32x4, s1 * (k1 * hx)));
                    } else {
                        // routed row: weighted output staged in bf16 (fp32 range; the combine adds in fp32)
                        const float wr = il.ra[row] * il.rb[row];
                        const floatx4 v0 = s0 * k0, v1 = s1 * k1;
                        u32x4 o;
                        o.x = pack_bf16x2(wr * v0[0], wr * v0[1]);
                        o.y = pack_bf16x2(wr * v0[2], wr * v0[3]);
                        o.z = pack_bf16x2(wr * v1[0], wr * v1[1]);
                        o.w = pack_bf16x2(wr * v1[2], wr * v1[3]);
                        store16<COH>(a.stage + (size_t)(t.r0 + row) * a.N + col0 + cA, o);
                    }
                }
            }
        }
    }
}

// The tile of work item (slot, n-tile): slots are the shared-expert blocks, then the routed
// blocks in the routing schedule's order.  False for a malformed block map entry, which
// turns into a skipped item, never an out-of-bounds access.
__device__ __forceinline__ bool item_tile(const GemmArgs &a, int slot, int ntile, int nb, Tile &t) {
    t.ntile = ntile;
    t.shared = slot < a.n_shared;
    t.e = 0;
    if (t.shared) {
        t.r0 = a.T * a.topk + slot * kBM;
        t.nrows = min(kBM, a.T - slot * kBM);
        return true;
    }
    const int mb = a.sched[slot - a.n_shared];
    bool ok = mb >= 0 && mb < nb;
    if (ok) {
        t.e = a.blocks[3 * mb];
        t.r0 = a.blocks[3 * mb + 1];
        t.nrows = a.blocks[3 * mb + 2];
        ok = !(t.e < 0 || t.e >= a.E || t.r0 < 0 || t.nrows < 1 || t.nrows > kBM ||
               t.r0 + t.nrows > a.T * a.topk);
    }
    if (threadIdx.x == 0) MOE_DBG(ok, DBG_GEMM_BLOCK);
    return ok;
}

// one tile with the M-tile count of its rows
template <int MODE, bool COH>
__device__ __forceinline__ void run_tile(const GemmArgs &a, const Tile &t, uint8_t *smem, int *s_next,
                                         const ItemLds &il, int32_t *done, int pend) {
    switch ((t.nrows + 31) >> 5) {
        case 1: gemm_tile<MODE, 1, COH>(a, t, smem, s_next, il, done, pend); break;
        case 2: gemm_tile<MODE, 2, COH>(a, t, smem, s_next, il, done, pend); break;
        case 3: gemm_tile<MODE, 3, COH>(a, t, smem, s_next, il, done, pend); break;
        default: gemm_tile<MODE, 4, COH>(a, t, smem, s_next, il, done, pend); break;
    }
}

// Work items: (slot, n-tile) with the n-tile fastest, so the n-tiles of a
// block (which read the same activation rows) run side by side; slots are the
// shared-expert blocks, then the routed blocks in the routing schedule's order
// (cost class 4, 3, 2, 1 M tiles, each class by expert), i.e. longest first.
// Workgroup g takes item g, then items from one atomic head in that order, so
// the long items all start in the first round and the short ones fill in
// behind them wherever a workgroup comes free.
template <int MODE>
__global__ __launch_bounds__(NTHR, 2) void q4_gemm_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    __shared__ int s_next;
    __shared__ __attribute__((aligned(16))) float s_colk[256];
    __shared__ float s_ra[kBM], s_rb[kBM], s_ne[64];
    const ItemLds il{s_colk, s_ra, s_rb, s_ne};
    const int nb = min(max(a.num_blocks[0], 0), a.max_blocks);
    const int n_items = (a.n_shared + nb) * a.n_tiles;
    for (int k = blockIdx.x; k < n_items; k = (int)gridDim.x + s_next) {
        __syncthreads();                         // s_next has been read by every thread
        const int slot = k / a.n_tiles;
        Tile t;
        if (item_tile(a, slot, k - slot * a.n_tiles, nb, t))
            run_tile<MODE, false>(a, t, smem, &s_next, il, nullptr, -1);
        else if (threadIdx.x == 0)               // an empty item still takes the next one
            s_next = atomicAdd(&a.qctl[0], 1);
        __syncthreads();                         // s_next written; the tile is done with the LDS
    }
    // the last workgroup out re-arms the head for the next launch
    if (threadIdx.x == 0 && atomicAdd(&a.qctl[QCTL_LINE], 1) == (int)gridDim.x - 1) {
        atomicExch(&a.qctl[0], 0);
        atomicExch(&a.qctl[QCTL_LINE], 0);
    }
}

// Both GEMMs in one persistent launch.  One queue holds every gate/up item, then every down
// item (each part longest first, as above), so that workgroups freed by the last, short
// gate/up items start on the long down items instead of idling until the launch ends.
//
// A down item reads its block's h rows from all I/128 gate/up items of that slot, which may
// have run on any XCD; each XCD has its own L2.  The gate/up items therefore store h, its group
// sums and the row factors 2^f with the agent-scope policy (written through), the down items
// copy them with that policy (never served from a stale L2 line), and done[slot] counts the
// slot's finished gate/up items.  A workgroup reports a gate/up item once its stores are
// complete: at the first stage wait of its next gate/up item (s_waitcnt vmcnt(0) there), or
// before it takes a down item or leaves.  A down item's thread 0 then waits, with a bounded
// spin, until done[slot] reaches I/128.
//
// The wait ends: the queue hands out items in index order, and every gate/up item precedes
// every down item.  Of the unfinished items, the one with the lowest index waits for nothing
// (its gate/up items are finished, or it is a gate/up item), and its workgroup is running it
// or finishing an earlier item that also waits for nothing.  Workgroups start on static items
// (item = workgroup index) only within the gate/up part; the others take their first item from
// the head.
//
// done[] is zeroed by the routing pass and, for the next launch, by the last workgroup out.
__global__ __launch_bounds__(NTHR, 2) void q4_ffn_kernel(GemmArgs ag, GemmArgs ad, int32_t *done) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    __shared__ int s_next, s_last;
    __shared__ __attribute__((aligned(16))) float s_colk[256];
    __shared__ float s_ra[kBM], s_rb[kBM], s_ne[64];
    const ItemLds il{s_colk, s_ra, s_rb, s_ne};
    const int tid = threadIdx.x;
    const int nb = min(max(ag.num_blocks[0], 0), ag.max_blocks);
    const int nslot = ag.n_shared + nb;
    const int ng = nslot * ag.n_tiles, n_items = ng + nslot * ad.n_tiles;
    const int nstatic = min((int)gridDim.x, ng);
    int32_t *head = ag.qctl;                     // the same queue words in ad
    auto report = [&](int slot) {
        __hip_atomic_fetch_add(done + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    int pend = -1;                               // gate/up slot finished but not yet reported
    auto flush = [&]() {                         // whole workgroup; pend is uniform
        if (pend >= 0) {
            wait_vm<0>();                        // this wave's h stores are complete
            __syncthreads();                     // ... and every other wave's
            if (tid == 0) report(pend);
            pend = -1;
        }
    };
    if ((int)blockIdx.x >= nstatic) {
        if (tid == 0) s_next = atomicAdd(head, 1);
        __syncthreads();
    }
    for (int k = (int)blockIdx.x < nstatic ? (int)blockIdx.x : nstatic + s_next; k < n_items;
         k = nstatic + s_next) {
        __syncthreads();                         // s_next has been read by every thread
        Tile t;
        if (k < ng) {
            const int slot = k / ag.n_tiles;
            if (item_tile(ag, slot, k - slot * ag.n_tiles, nb, t)) {
                run_tile<0, true>(ag, t, smem, &s_next, il, done, pend);
                pend = slot;
            } else {
                flush();
                if (tid == 0) {
                    report(slot);                // nothing stored: reported at once
                    s_next = atomicAdd(head, 1);
                }
            }
        } else {
            const int kd = k - ng, slot = kd / ad.n_tiles;
            // the slot's count is read while the block is decoded (counts only grow, and a count
            // that is complete stays complete, so an early read is as good as a late one)
            int seen = 0;
            if (tid == 0) seen = __hip_atomic_load(done + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool ok = item_tile(ad, slot, kd - slot * ad.n_tiles, nb, t);
            flush();                             // never wait while holding a report
            if (ok) {
                if (tid == 0) {
                    int it = 0;
                    while (seen < ag.n_tiles && it < kFfnSpin) {
                        __builtin_amdgcn_s_sleep(2);
                        ++it;
                        seen = __hip_atomic_load(done + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    MOE_DBG(seen >= ag.n_tiles, DBG_FFN_WAIT);   // flagged only if it gave up
                }
                __syncthreads();                 // the slot's h is complete
                run_tile<1, true>(ad, t, smem, &s_next, il, done, -1);
            } else if (tid == 0) {
                s_next = atomicAdd(head, 1);
            }
        }
        __syncthreads();                         // s_next written; the tile is done with the LDS
    }
    flush();
    // the last workgroup out zeroes the counters and re-arms the head for the next launch
    if (tid == 0) s_last = atomicAdd(&head[QCTL_LINE], 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (s_last) {
        for (int i = tid; i < nslot; i += NTHR)
            __hip_atomic_store(done + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) {
            atomicExch(&head[0], 0);
            atomicExch(&head[QCTL_LINE], 0);
        }
    }
}

static int shared_blocks(int T) { return (T + kBM - 1) / kBM; }

// persistent grid: two workgroups per CU, never more than there are work items
static unsigned grid_for(int n_shared, int max_blocks, int n_tiles) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const long items = (long)(n_shared + max_blocks) * n_tiles;
    return (unsigned)std::max<long>(1, std::min<long>(items, 2L * cus));
}

// the GEMMs need more dynamic LDS than the default launch limit
template <const void *(*FN)()>
static void allow_lds() {
    static LdsLimit lim;
    lim.ensure(FN(), L_TOTAL);
}
template <int MODE> static const void *gemm_fn() { return (const void *)q4_gemm_kernel<MODE>; }
static const void *ffn_fn() { return (const void *)q4_ffn_kernel; }

static GemmArgs gateup_args(const moe_shape &sh, const uint16_t *xp, const float *xsum,
                            const float *tok, const GemmWeights &gw, const int32_t *blocks,
                            const int32_t *num_blocks, const int32_t *sched, int32_t *qctl,
                            int max_blocks, const int32_t *row_token, uint16_t *h, float *hsum,
                            float *hexp) {
    GemmArgs a{};
    a.A = xp;
    a.Asum = xsum;
    a.K = sh.H;
    a.G = sh.H / 64;
    a.N = sh.I;
    a.pk = gw.pk;
    a.pk_sh = gw.pk_sh;
    a.colf = gw.colf;
    a.colf_sh = gw.colf_sh;
    a.emeta = gw.emeta;
    a.tok = tok;
    a.hexp = hexp;
    a.blocks = blocks;
    a.num_blocks = num_blocks;
    a.sched = sched;
    a.qctl = qctl;
    a.max_blocks = max_blocks;
    a.row_token = row_token;
    a.T = sh.T;
    a.topk = sh.top_k;
    a.E = sh.E;
    a.n_tiles = sh.I / 128;
    a.n_shared = shared_blocks(sh.T);
    a.h = h;
    a.hsum = hsum;
    return a;
}

void launch_gateup(const moe_shape &sh, const uint16_t *xp, const float *xsum, const float *tok,
                   const GemmWeights &gw, const int32_t *blocks, const int32_t *num_blocks,
                   const int32_t *sched, int32_t *qctl, int max_blocks, const int32_t *row_token,
                   uint16_t *h, float *hsum, float *hexp, hipStream_t s) {
    const GemmArgs a = gateup_args(sh, xp, xsum, tok, gw, blocks, num_blocks, sched,
                                   qctl + QCTL_GATEUP, max_blocks, row_token, h, hsum, hexp);
    allow_lds<gemm_fn<0>>();
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
    {
        MOE_DBG(j >= k || (rows[j] >= 0 && rows[j] < T * k), DBG_COMBINE_ROW);
        if (rows[j] >= 0 && rows[j] < T * k) v[j] = *(const u32x4 *)(stage + (size_t)rows[j] * H + n);
    }
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

static GemmArgs down_args(const moe_shape &sh, const uint16_t *h, const float *hsum,
                          const float *hexp, const GemmWeights &gw, const int32_t *blocks,
                          const int32_t *num_blocks, const int32_t *sched, int32_t *qctl,
                          int max_blocks, const int32_t *row_token, const float *row_w,
                          uint16_t *stage, float *y) {
    GemmArgs a{};
    a.A = h;
    a.Asum = hsum;
    a.K = sh.I;
    a.G = sh.I / 64;
    a.N = sh.H;
    a.pk = gw.pk;
    a.pk_sh = gw.pk_sh;
    a.colf = gw.colf;
    a.colf_sh = gw.colf_sh;
    a.emeta = gw.emeta;
    a.hexp = (float *)hexp;
    a.blocks = blocks;
    a.num_blocks = num_blocks;
    a.sched = sched;
    a.qctl = qctl;
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
    return a;
}

// each token adds its k weighted routed rows to y
void launch_combine(const moe_shape &sh, const uint16_t *stage, const int32_t *tok_row, float *y,
                    hipStream_t s) {
    const size_t n8 = (size_t)sh.T * sh.H / 8;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, stage,
                       tok_row, sh.T, sh.H, sh.top_k, y);
}

void launch_down(const moe_shape &sh, const uint16_t *h, const float *hsum, const float *hexp,
                 const GemmWeights &gw, const int32_t *blocks, const int32_t *num_blocks,
                 const int32_t *sched, int32_t *qctl, int max_blocks,
                 const int32_t *row_token, const float *row_w, const int32_t *tok_row,
                 uint16_t *stage, float *y, bool combine, hipStream_t s) {
    const GemmArgs a = down_args(sh, h, hsum, hexp, gw, blocks, num_blocks, sched,
                                 qctl + QCTL_DOWN, max_blocks, row_token, row_w, stage, y);
    allow_lds<gemm_fn<1>>();
    // shared-expert blocks write y, routed blocks their weighted staging rows ...
    hipLaunchKernelGGL(q4_gemm_kernel<1>, dim3(grid_for(a.n_shared, max_blocks, a.n_tiles)),
                       dim3(NTHR), L_TOTAL, s, a);
    // ... then each token adds its eight routed rows (unless the caller's next kernel does)
    if (combine) launch_combine(sh, stage, tok_row, y, s);
}

void launch_ffn(const moe_shape &sh, const uint16_t *xp, const float *xsum, const float *tok,
                const GemmWeights &gwg, const GemmWeights &gwd, const int32_t *blocks,
                const int32_t *num_blocks, const int32_t *sched, int32_t *qctl, int max_blocks,
                const int32_t *row_token, const float *row_w, const int32_t *tok_row, uint16_t *h,
                float *hsum, float *hexp, uint16_t *stage, float *y, bool combine, hipStream_t s) {
    const GemmArgs ag = gateup_args(sh, xp, xsum, tok, gwg, blocks, num_blocks, sched,
                                    qctl + QCTL_FFN, max_blocks, row_token, h, hsum, hexp);
    const GemmArgs ad = down_args(sh, h, hsum, hexp, gwd, blocks, num_blocks, sched,
                                  qctl + QCTL_FFN, max_blocks, row_token, row_w, stage, y);
    allow_lds<ffn_fn>();
    hipLaunchKernelGGL(q4_ffn_kernel, dim3(grid_for(ag.n_shared, max_blocks, ag.n_tiles + ad.n_tiles)),
                       dim3(NTHR), L_TOTAL, s, ag, ad, qctl + QCTL_WORDS);
    if (combine) launch_combine(sh, stage, tok_row, y, s);
}

MOE_DBG_READER(dbg_read_gemm)

}  // namespace moe
