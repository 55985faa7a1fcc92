// Grouped expert GEMMs over 4-bit affine weights on bf16 MFMA (gfx950).
//
// The pages' design rebuilds bf16 weights tile by tile inside the grouped
// GEMM and accumulates in FP32 (mechatronicstore.cl, "Prefill: pesos
// comprimidos y enrutamiento en la GPU").  Rounding q*scale+bias to bf16
// loses up to 4 significant bits per weight, which on these layers leaves
// almost no margin under the output tolerance, so this kernel feeds the
// MFMA the exact codes instead and applies scale and bias in FP32:
//
//   sum_k x_k w_k = sum_g s_g * P_g  +  sum_g c_g * xs_g,
//   P_g = sum_{k in g} x_k (128 + q_k),   c_g = b_g - 128 s_g,   xs_g = sum_{k in g} x_k
//
//  * a code word becomes four bf16 pairs 128+q with one and-or each (the
//    nibble drops into the mantissa of 128.0): exact, 7 VALU ops per 8 codes;
//  * P_g comes from four 32x32x16 MFMA k-steps started from zero;
//  * the FP32 accumulator takes acc += s_g * P_g once per group;
//  * the rank-G term sum_g c_g xs_g is a small MFMA pass with K = 3G over
//    bf16 hi/lo splits: c_hi xs_hi + c_hi xs_lo + c_lo xs_hi.
//
// Element order: the code pairs come out as k = (0,4), (1,5), (2,6), (3,7) of
// each 8-block, so the activations are stored with every 8-block permuted to
// (0,4,1,5,2,6,3,7): x by the preparation pass, h by the gate/up epilogue.
//
// Tiles: a workgroup takes one routing block (up to 128 rows of one expert)
// and a slice of output columns; each of its 4 waves owns 64 output columns
// (gate/up: 32 gate + the 32 matching up columns, so SwiGLU is local to a
// lane) for all rows.  The activation rows of a 128-wide K chunk are copied
// global->LDS directly (no registers), double buffered, XOR-swizzled so the
// MFMA operand reads are bank-conflict free; the codes go straight from
// global memory to registers, each word used by exactly one wave.
#include "common.h"

namespace moe {

constexpr int KC = 128;                 // K per chunk: two quantisation groups
constexpr int A_ROW = 2 * KC;           // LDS bytes per staged activation row
constexpr int MAXG = 32;                // K <= 2048
constexpr int KB3_MAX = 3 * MAXG;       // K'' of the bias pass
constexpr int AB_LD = KB3_MAX + 8;      // bf16 per row of the bias-pass A operand
constexpr int NRING = 3;                // code/scale ring depth (chunks in flight)
constexpr int NWAVE = 8;                // waves per workgroup: 2 row halves x 4 column quarters
constexpr int B_NQ = 4096;              // bytes of codes per column quarter per chunk
constexpr int S_NQ = 256;               // bytes of scales per column quarter per chunk

// LDS map (bytes)
constexpr int L_A = 0;                                   // [2][128 rows][256 B] swizzled
constexpr int L_B = L_A + 2 * kBM * A_ROW;               // [NRING][4 nq][2 nt][2 groups][64 lanes][16 B]
constexpr int L_S = L_B + NRING * 4 * B_NQ;              // [NRING][4 nq][64 lanes][4 B]
constexpr int L_AB = L_S + NRING * 4 * S_NQ;             // [128 rows][AB_LD] bf16
constexpr int L_TOK = L_AB + kBM * AB_LD * 2;            // [128] int32 source rows
constexpr int L_TOTAL = L_TOK + kBM * 4;

struct GemmArgs {
    const uint16_t *A;     // permuted activations: x [T][H] (gate/up) or h [rows][I] (down)
    const float *Asum;     // group sums of A rows: by token [T][G] or by row [rows][G]
    int K, G;
    GemmProj p0, p1;       // routed projections: gate, up  |  down, -
    GemmProj s0, s1;       // the shared expert's
    int N;                 // rows per projection: I (gate/up) or H (down)
    const int32_t *blocks;
    const int32_t *num_blocks;
    int max_blocks;
    const int32_t *row_token;
    const float *row_w;
    int T, topk, E;
    int n_tiles;
    int n_shared;          // shared-expert M blocks (scheduled first)
    uint16_t *h;
    float *y;
    float *stage;          // routed down outputs times their routing weight [T*topk][H]
    int ldo;               // output row stride: I (h) or H (y)
};

// 8 codes of one word -> 8 bf16 values 128+q, element order (0,4,1,5,2,6,3,7):
// one v_and_or_b32 per pair (both constants in VGPRs, so no literal limits apply)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
    return r;
}
__device__ __forceinline__ bf16x8 codes_to_bf16x8(uint32_t w, uint32_t M, uint32_t C) {
    u32x4 v;
    v.x = and_or(w, M, C);
    v.y = and_or(w >> 4, M, C);
    v.z = and_or(w >> 8, M, C);
    v.w = and_or(w >> 12, M, C);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Asynchronous global->LDS copies.  Lane i of the wave writes LDS bytes
// [lds + 16 i, lds + 16 i + 16) (dword form: 4 i).  Issued through inline
// assembly so that the compiler does not wait for them before every LDS read;
// completion is awaited explicitly (s_waitcnt vmcnt) before the barrier that
// publishes a chunk.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}

template <int MODE>   // 0: gate/up + SwiGLU -> h ; 1: down -> y (shared) / staging (routed)
__global__ __launch_bounds__(512, 1) void q4_gemm_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    uint8_t *As = smem + L_A;
    uint16_t *abias = (uint16_t *)(smem + L_AB);
    int32_t *s_src = (int32_t *)(smem + L_TOK);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nq = wave & 3, mh = wave >> 2;       // column quarter, row half
    const int l32 = lane & 31, gg = lane >> 5;
    const int bid = (int)blockIdx.x / a.n_tiles;
    const int nt = (int)blockIdx.x % a.n_tiles;
    // shared-expert blocks first (full tiles), then the routed block map
    const bool shared = bid < a.n_shared;
    int e = 0, r0, nrows;
    if (!shared) {
        const int mb = bid - a.n_shared;
        if (mb >= a.num_blocks[0] || mb >= a.max_blocks) return;
        e = a.blocks[3 * mb];
        r0 = a.blocks[3 * mb + 1];
        nrows = a.blocks[3 * mb + 2];
        // a malformed block map turns into a no-op, never an out-of-bounds access
        if (e < 0 || e >= a.E || r0 < 0 || nrows < 1 || nrows > kBM || r0 + nrows > a.T * a.topk)
            return;
    } else {
        r0 = a.T * a.topk + bid * kBM;
        nrows = min(kBM, a.T - bid * kBM);
    }
    const int K = a.K, G = a.G;
    const int Trk = a.T * a.topk;
    const int nchunks = K / KC;

    // ---- this wave's two projection rows (one per 32-column n-tile)
    const GemmProj P0 = shared ? a.s0 : a.p0;
    const GemmProj P1 = shared ? (MODE == 0 ? a.s1 : a.s0) : (MODE == 0 ? a.p1 : a.p0);
    const size_t eoff = shared ? 0 : (size_t)e * a.N;
    int nrow[2];
    if (MODE == 0) {
        nrow[0] = nrow[1] = nt * 128 + 32 * nq + l32;
    } else {
        nrow[0] = nt * 256 + 64 * nq + l32;
        nrow[1] = nrow[0] + 32;
    }
    const uint32_t *qrow[2];
    const uint16_t *srow[2], *brow[2];
    {
        const GemmProj pp[2] = {P0, P1};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const size_t rr = eoff + nrow[q];
            qrow[q] = pp[q].q + rr * (K / 8) + 4 * gg;
            srow[q] = pp[q].s + rr * G;
            brow[q] = pp[q].b + rr * G;
        }
    }
    // codes of chunk c for column quarter nq: this wave copies n-tile mh (2 copies);
    // both waves copy the (identical) scales
    const uint32_t lB = lds0 + L_B + nq * B_NQ, lS = lds0 + L_S + nq * S_NQ;
    const uint32_t *my_q = mh ? qrow[1] : qrow[0];
    const uint16_t *my_srow = gg ? srow[1] : srow[0];     // lane L copies column (L>>5, L&31)
    auto copy_codes = [&](int c) {
        const int slot = c % NRING;
#pragma unroll
        for (int gm = 0; gm < 2; ++gm)
            dma16(my_q + c * 16 + gm * 8, lB + slot * 4 * B_NQ + (2 * mh + gm) * 1024);
        dma4(my_srow + 2 * c, lS + slot * 4 * S_NQ);
    };

    // ---- source rows of the tile (clamped: rows past nrows repeat row 0)
    if (tid < kBM) {
        const int mm = tid < nrows ? tid : 0;
        int src;
        if (MODE == 0) {
            const int t = shared ? (r0 - Trk + mm) : a.row_token[r0 + mm];
            src = (t >= 0 && t < a.T) ? t : 0;
        } else {
            src = r0 + mm;
        }
        s_src[tid] = src;
    }
    copy_codes(0);
    __syncthreads();

    // ---- activation chunk copies: wave w covers rows 16w .. 16w+15 in 4 copies of
    // 4 rows; lane L fills 16-byte slot L&15 of row L>>4, holding segment (L&15)^(row&15)
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4);
        const int segd = (lane & 15) ^ (row & 15);
        aoff[i] = (uint32_t)s_src[row] * (uint32_t)K + (uint32_t)(segd * 8);
    }
    auto copy_act = [&](int c, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16(a.A + (size_t)aoff[i] + c * KC,
                  lds0 + L_A + buf * kBM * A_ROW + (16 * wave + 4 * i) * A_ROW);
    };
    copy_act(0, 0);
    // issued last, so that "all but the newest 3 copies" below means chunk 0 complete
    if (nchunks > 1) copy_codes(1);

    // ---- group sums -> bias-pass A operand: [xs_hi | xs_lo | xs_hi | 0 pad].
    // Thread t owns a quarter row (G/4 <= 8 sums): all loads issued before use.
    const int KB3 = (3 * G + 15) & ~15;
    {
        const int m = tid >> 2, qt = tid & 3, qg = G >> 2, rem = G & 3;
        // quarters of G (G is even; the last quarter takes the remainder)
        const int g0 = qt * qg, cnt = qg + (qt == 3 ? rem : 0);
        const float *src = a.Asum + (size_t)s_src[m] * G + g0;
        float sv[10];
#pragma unroll
        for (int i = 0; i < 10; ++i)
            if (i < cnt) sv[i] = src[i];
        uint16_t *dst = abias + m * AB_LD + g0;
#pragma unroll
        for (int g = 0; g < 10; ++g) {
            if (g < cnt) {
                const uint16_t hi = f32_to_bf16(sv[g]);
                dst[g] = hi;
                dst[G + g] = f32_to_bf16(sv[g] - bf16_to_f32(hi));
                dst[2 * G + g] = hi;
            }
        }
        for (int c = 3 * G + qt; c < KB3; c += 4) abias[m * AB_LD + c] = 0;
    }

    // rows of this wave: 64*mh + 32*mt + ..., mt < MT
    const int MT = max(0, min(2, (nrows - 64 * mh + 31) >> 5));
    floatx16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][q][i] = 0.0f;

    // chunk 0 (activations + codes) and chunk 1 codes are in flight; wait for chunk 0
    if (nchunks > 1)
        asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const floatx16 zero = {};
    uint32_t cM = 0x000F000Fu, cC = 0x43004300u;
    asm volatile("" : "+v"(cM), "+v"(cC));   // keep the unpack constants in VGPRs
    for (int c = 0; c < nchunks; ++c) {
        const int cur = c & 1, slot = c % NRING;
        if (c + 1 < nchunks) copy_act(c + 1, cur ^ 1);
        if (c + 2 < nchunks) copy_codes(c + 2);
        const uint8_t *bsl = smem + L_B + slot * 4 * B_NQ + nq * B_NQ + lane * 16;
        const uint32_t *ssl = (const uint32_t *)(smem + L_S + slot * 4 * S_NQ + nq * S_NQ);
        const uint32_t sc0 = ssl[l32], sc1 = ssl[32 + l32];
        if (MT > 0) {
#pragma unroll
            for (int gm = 0; gm < 2; ++gm) {
                const float s0 = gm ? bf16_hi(sc0) : bf16_lo(sc0);
                const float s1 = gm ? bf16_hi(sc1) : bf16_lo(sc1);
                const u32x4 w0 = *(const u32x4 *)(bsl + (0 + gm) * 1024);
                const u32x4 w1 = *(const u32x4 *)(bsl + (2 + gm) * 1024);
                bf16x8 bfr[2][4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bfr[0][j] = codes_to_bf16x8(w0[j], cM, cC);
                    bfr[1][j] = codes_to_bf16x8(w1[j], cM, cC);
                }
                const uint8_t *abase = As + cur * kBM * A_ROW + (64 * mh + l32) * A_ROW;
                const int sw = l32 & 15;
                floatx16 p[2][2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    if (mt < MT) {
                        bf16x8 af[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            af[j] = *(const bf16x8 *)(abase + mt * 32 * A_ROW +
                                                      (((8 * gm + 4 * gg + j) ^ sw) << 4));
                        p[mt][0] = mfma32(af[0], bfr[0][0], zero);
                        p[mt][1] = mfma32(af[0], bfr[1][0], zero);
#pragma unroll
                        for (int j = 1; j < 4; ++j) {
                            p[mt][0] = mfma32(af[j], bfr[0][j], p[mt][0]);
                            p[mt][1] = mfma32(af[j], bfr[1][j], p[mt][1]);
                        }
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    if (mt < MT) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            acc[mt][0][i] = __builtin_fmaf(s0, p[mt][0][i], acc[mt][0][i]);
                            acc[mt][1][i] = __builtin_fmaf(s1, p[mt][1][i], acc[mt][1][i]);
                        }
                    }
                }
            }
        }
        // publish chunk c+1: its activations and codes must have landed (the
        // codes of chunk c+2, issued last, may still be in flight)
        if (c + 2 < nchunks)
            asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- rank-G term: sum_g c[n][g] * xs[m][g], c = b - 128 s, as MFMA over
    // K'' = 3G with A'' = [xs_hi | xs_lo | xs_hi] and B'' = [c_hi | c_hi | c_lo].
    // Scales and biases of this wave's 64 columns are staged in the (now free)
    // activation buffer: lane L holds column (L>>5, L&31).
    uint16_t *sb_s = (uint16_t *)(As + wave * 64 * 2 * MAXG * 2);
    uint16_t *sb_b = sb_s + 64 * MAXG;
    {
        const uint16_t *ps = gg ? srow[1] : srow[0];
        const uint16_t *pb = gg ? brow[1] : brow[0];
        if ((G & 7) == 0) {
            u32x4 vs[4], vb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (8 * i < G) {
                    vs[i] = *(const u32x4 *)(ps + 8 * i);
                    vb[i] = *(const u32x4 *)(pb + 8 * i);
                }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (8 * i < G) {
                    *(u32x4 *)(sb_s + lane * MAXG + 8 * i) = vs[i];
                    *(u32x4 *)(sb_b + lane * MAXG + 8 * i) = vb[i];
                }
        } else {
            for (int g = 0; g < G; ++g) {
                sb_s[lane * MAXG + g] = ps[g];
                sb_b[lane * MAXG + g] = pb[g];
            }
        }
    }
    __syncthreads();
    for (int j3 = 0; j3 < KB3 / 16; ++j3) {
        bf16x8 bb[2];
        const int kap0 = 16 * j3 + 8 * gg;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int col = q * 32 + l32;
            u32x4 pk = {0u, 0u, 0u, 0u};
            if ((G & 7) == 0) {
                // the 8 slots share one term tau and run over groups gam0 .. gam0+7
                const int tau = kap0 / G, gam0 = kap0 - tau * G;
                if (tau < 3) {
                    const u32x4 vs = *(const u32x4 *)(sb_s + col * MAXG + gam0);
                    const u32x4 vb = *(const u32x4 *)(sb_b + col * MAXG + gam0);
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) {
                        const float c0 = bf16_lo(vb[w2]) - 128.0f * bf16_lo(vs[w2]);
                        const float c1 = bf16_hi(vb[w2]) - 128.0f * bf16_hi(vs[w2]);
                        const uint32_t hi = pack_bf16x2(c0, c1);
                        pk[w2] = tau < 2 ? hi : pack_bf16x2(c0 - bf16_lo(hi), c1 - bf16_hi(hi));
                    }
                }
            } else {
                uint16_t v[8];
#pragma unroll
                for (int el = 0; el < 8; ++el) {
                    const int kap = kap0 + el;
                    const int tau = kap / G, gam = kap - tau * G;
                    uint16_t val = 0;
                    if (tau < 3) {
                        const float cf = bf16_to_f32(sb_b[col * MAXG + gam]) -
                                         128.0f * bf16_to_f32(sb_s[col * MAXG + gam]);
                        const uint16_t chi = f32_to_bf16(cf);
                        val = tau < 2 ? chi : f32_to_bf16(cf - bf16_to_f32(chi));
                    }
                    v[el] = val;
                }
                pk.x = v[0] | ((uint32_t)v[1] << 16);
                pk.y = v[2] | ((uint32_t)v[3] << 16);
                pk.z = v[4] | ((uint32_t)v[5] << 16);
                pk.w = v[6] | ((uint32_t)v[7] << 16);
            }
            bb[q] = __builtin_bit_cast(bf16x8, pk);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            if (mt < MT) {
                const bf16x8 af = *(const bf16x8 *)&abias[(64 * mh + 32 * mt + l32) * AB_LD +
                                                          16 * j3 + 8 * gg];
                acc[mt][0] = mfma32(af, bb[0], acc[mt][0]);
                acc[mt][1] = mfma32(af, bb[1], acc[mt][1]);
            }
        }
    }

    // ---- epilogue.  Accumulator element i of lane (l32, gg) is row
    // 8*(i/4) + 4*gg + i%4 of the 32-row tile, column l32.
    const int hcol = perm_pos(nrow[0]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        if (mt >= MT) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 64 * mh + 32 * mt + 8 * (i >> 2) + 4 * gg + (i & 3);
            if (row >= nrows) continue;
            if (MODE == 0) {
                const float g = acc[mt][0][i], u = acc[mt][1][i];
                const float hv = __fdividef(g, 1.0f + __expf(-g)) * u;
                a.h[(size_t)(r0 + row) * a.ldo + hcol] = f32_to_bf16(hv);
            } else {
                if (shared) {
                    const size_t t = (size_t)(r0 - Trk + row);
                    a.y[t * a.ldo + nrow[0]] = acc[mt][0][i];
                    a.y[t * a.ldo + nrow[1]] = acc[mt][1][i];
                } else {
                    // routing-weighted output of routed row r0+row, combined later
                    const float wr = a.row_w[r0 + row];
                    float *o = a.stage + (size_t)(r0 + row) * a.ldo;
                    o[nrow[0]] = wr * acc[mt][0][i];
                    o[nrow[1]] = wr * acc[mt][1][i];
                }
            }
        }
    }
}

static int shared_blocks(int T) { return (T + kBM - 1) / kBM; }

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
                   const int32_t *num_blocks, int max_blocks, const int32_t *row_token,
                   uint16_t *h, hipStream_t s) {
    GemmArgs a{};
    a.A = xp;
    a.Asum = xsum;
    a.K = sh.H;
    a.G = sh.H / 64;
    a.p0 = gate;
    a.p1 = up;
    a.s0 = sgate;
    a.s1 = sup;
    a.N = sh.I;
    a.blocks = blocks;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.row_token = row_token;
    a.T = sh.T;
    a.topk = sh.top_k;
    a.E = sh.E;
    a.n_tiles = sh.I / 128;
    a.n_shared = shared_blocks(sh.T);
    a.h = h;
    a.ldo = sh.I;
    allow_lds<0>();
    const int nmb = max_blocks + a.n_shared;
    hipLaunchKernelGGL(q4_gemm_kernel<0>, dim3(nmb * a.n_tiles), dim3(64 * NWAVE), L_TOTAL, s, a);
}

// y[t] += sum_j stage[tok_row[t][j]] in pick order j = 0..k-1: a fixed order, so
// the combined output is reproducible bit for bit.  One thread per 4 outputs.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ stage,
                                                      const int32_t *__restrict__ tok_row, int T,
                                                      int H, int k, float *__restrict__ y) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t per = (size_t)H / 4;
    if (i >= (size_t)T * per) return;
    const size_t t = i / per, n = (i % per) * 4;
    float4 acc = *(const float4 *)(y + t * H + n);
    for (int j = 0; j < k; ++j) {
        const int r = tok_row[t * k + j];
        if (r < 0 || r >= T * k) continue;
        const float4 v = *(const float4 *)(stage + (size_t)r * H + n);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    *(float4 *)(y + t * H + n) = acc;
}

void launch_down(const moe_shape &sh, const uint16_t *h, const float *hsum, GemmProj down,
                 GemmProj sdown, const int32_t *blocks, const int32_t *num_blocks, int max_blocks,
                 const int32_t *row_token, const float *row_w, const int32_t *tok_row,
                 float *stage, float *y, hipStream_t s) {
    GemmArgs a{};
    a.A = h;
    a.Asum = hsum;
    a.K = sh.I;
    a.G = sh.I / 64;
    a.p0 = down;
    a.s0 = sdown;
    a.N = sh.H;
    a.blocks = blocks;
    a.num_blocks = num_blocks;
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
    a.ldo = sh.H;
    allow_lds<1>();
    // shared-expert blocks write y, routed blocks their weighted staging rows ...
    const int nmb = max_blocks + a.n_shared;
    hipLaunchKernelGGL(q4_gemm_kernel<1>, dim3(nmb * a.n_tiles), dim3(64 * NWAVE), L_TOTAL, s, a);
    // ... then each token adds its eight routed rows
    const size_t n4 = (size_t)sh.T * sh.H / 4;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, stage,
                       tok_row, sh.T, sh.H, sh.top_k, y);
}

}  // namespace moe
