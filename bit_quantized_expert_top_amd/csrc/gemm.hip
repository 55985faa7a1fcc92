// Grouped expert GEMMs over 4-bit affine weights on bf16 MFMA (gfx950).
//
// The pages' design rebuilds bf16 weights tile by tile inside the grouped
// GEMM and accumulates in FP32 (mechatronicstore.cl, "Prefill: pesos
// comprimidos y enrutamiento en la GPU").  Rounding q*scale+bias to bf16
// loses up to 4 significant bits per weight, which on these layers leaves
// almost no margin under the output tolerance, so this kernel feeds the
// MFMA the exact codes instead and applies scale and bias in FP32:
//
//   sum_k x_k w_k = sum_g [ s_g * sum_{k in g} x_k q_k  +  b_g * sum_{k in g} x_k ]
//
//  * codes become bf16 values 128+q with one and-or per pair (the nibble
//    drops into the mantissa of 128.0), exact;
//  * each group's partial P_g = sum x (128+q) - 128 * sum x is produced by
//    four 32x32x16 MFMA k-steps whose accumulator starts at -128*sum(x) (a
//    per-row constant, so removing the 128 costs no instruction);
//  * the FP32 accumulator takes acc += s_g * P_g once per group;
//  * the bias term sum_g b_g * xs_g is one extra small MFMA pass with K =
//    2*groups: the bias values are exact bf16 and the group sums enter as a
//    bf16 hi+lo pair.
//
// Tiles: a workgroup takes one routing block (up to 128 rows of one expert)
// and a slice of output columns; each of its 4 waves owns 64 output columns
// (gate/up: 32 gate + the 32 matching up columns, so SwiGLU is local to a
// lane) for all 128 rows.  The activation rows of a 128-wide K chunk are
// staged in LDS (double buffered) and shared by the 4 waves; the codes go
// straight from global memory to registers, each word used by exactly one
// wave.
#include "common.h"

namespace moe {

constexpr int KC = 128;                 // K per chunk: two quantisation groups
constexpr int A_LD = 2 * KC + 16;       // LDS bytes per staged activation row (padded)
constexpr int MAXG = 64;                // K <= 4096
constexpr int AB_LD = 2 * MAXG + 8;     // bf16 per row of the bias-pass A operand

struct GemmArgs {
    const uint16_t *A;     // x [T][H] (gate/up) or h [rows][I] (down)
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
    int mb_begin;          // first M-block of this launch (shared blocks follow max_blocks)
    uint16_t *h;
    float *y;
    int ldo;               // output row stride: I (h) or H (y)
};

// 8 codes of one word -> 8 bf16 values 128+q, element order (0,4,1,5,2,6,3,7)
__device__ __forceinline__ bf16x8 codes_to_bf16x8(uint32_t w) {
    const uint32_t M = 0x000F000Fu, C = 0x43004300u;
    u32x4 v;
    v.x = (w & M) | C;
    v.y = ((w >> 4) & M) | C;
    v.z = ((w >> 8) & M) | C;
    v.w = ((w >> 12) & M) | C;
    return __builtin_bit_cast(bf16x8, v);
}

// 8 consecutive bf16 (x0..x7) -> order (0,4,1,5,2,6,3,7), matching the codes
__device__ __forceinline__ u32x4 permute_act(u32x4 a) {
    u32x4 o;
    o.x = __builtin_amdgcn_perm(a.z, a.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(a.z, a.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(a.w, a.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(a.w, a.y, 0x07060302u);
    return o;
}

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int MODE>   // 0: gate/up + SwiGLU -> h ; 1: down + routing-weighted combine -> y
__global__ __launch_bounds__(256, 1) void q4_gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t As[2][kBM * A_LD];
    __shared__ __attribute__((aligned(16))) float cinit[MAXG][kBM];
    __shared__ __attribute__((aligned(16))) uint16_t abias[kBM * AB_LD];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, gg = lane >> 5;
    const int mb = a.mb_begin + (int)blockIdx.x / a.n_tiles;
    const int nt = (int)blockIdx.x % a.n_tiles;
    const bool shared = mb >= a.max_blocks;
    int e = 0, r0, nrows;
    if (!shared) {
        if (mb >= a.num_blocks[0]) return;
        e = a.blocks[3 * mb];
        r0 = a.blocks[3 * mb + 1];
        nrows = a.blocks[3 * mb + 2];
        // a malformed block map turns into a no-op, never an out-of-bounds access
        if (e < 0 || e >= a.E || r0 < 0 || nrows < 1 || nrows > kBM || r0 + nrows > a.T * a.topk)
            return;
    } else {
        const int sb = mb - a.max_blocks;
        r0 = a.T * a.topk + sb * kBM;
        nrows = min(kBM, a.T - sb * kBM);
    }
    const int K = a.K, G = a.G;
    const int Trk = a.T * a.topk;

    // source row of A (and of its group sums) for tile row m
    auto src_row = [&](int m) -> int {
        const int mm = m < nrows ? m : 0;
        if (MODE == 0) {
            const int t = shared ? (r0 - Trk + mm) : a.row_token[r0 + mm];
            return (t >= 0 && t < a.T) ? t : 0;
        }
        return r0 + mm;
    };

    // ---- group sums -> LDS: -128*sum for the MFMA accumulator start, hi/lo bf16 for the bias pass
    const int KB2 = (2 * G + 15) & ~15;
    for (int idx = tid; idx < kBM * G; idx += 256) {
        const int m = idx / G, g = idx % G;
        const float sx = a.Asum[(size_t)src_row(m) * G + g];
        cinit[g][m] = -128.0f * sx;
        const uint16_t hi = f32_to_bf16(sx);
        const uint16_t lo = f32_to_bf16(sx - bf16_to_f32(hi));
        abias[m * AB_LD + g] = hi;
        abias[m * AB_LD + G + g] = lo;
    }
    for (int idx = tid; idx < kBM * (KB2 - 2 * G); idx += 256) {
        const int m = idx / (KB2 - 2 * G), c = idx % (KB2 - 2 * G);
        abias[m * AB_LD + 2 * G + c] = 0;
    }

    // ---- this thread's staged activation rows: 8 rows, one 16-byte segment each
    const int seg = tid & 15;
    const uint16_t *arow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) arow[i] = a.A + (size_t)src_row((tid >> 4) + 16 * i) * K + seg * 8;

    // ---- this wave's two projection rows (one per 32-column n-tile)
    const GemmProj P0 = shared ? a.s0 : a.p0;
    const GemmProj P1 = shared ? (MODE == 0 ? a.s1 : a.s0) : (MODE == 0 ? a.p1 : a.p0);
    const size_t eoff = shared ? 0 : (size_t)e * a.N;
    int nrow[2];
    if (MODE == 0) {
        nrow[0] = nrow[1] = nt * 128 + 32 * wave + l32;
    } else {
        nrow[0] = nt * 256 + 64 * wave + l32;
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

    const int MT = (nrows + 31) >> 5;
    const int nchunks = K / KC;
    floatx16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][q][i] = 0.0f;

    u32x4 areg[8];
    u32x4 bw[2][2], bwn[2][2];
    uint32_t sc[2], scn[2];

    auto load_a = [&](int c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) areg[i] = *(const u32x4 *)(arow[i] + c * KC);
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *(u32x4 *)(&As[buf][((tid >> 4) + 16 * i) * A_LD + seg * 16]) = permute_act(areg[i]);
    };
    auto load_b = [&](int c, u32x4 (&w)[2][2], uint32_t (&s)[2]) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int gm = 0; gm < 2; ++gm) w[q][gm] = *(const u32x4 *)(qrow[q] + c * 16 + gm * 8);
            s[q] = *(const uint32_t *)(srow[q] + 2 * c);
        }
    };

    load_a(0);
    load_b(0, bw, sc);
    store_a(0);
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int cur = c & 1;
        const bool more = c + 1 < nchunks;
        if (more) {
            load_a(c + 1);
            load_b(c + 1, bwn, scn);
        }
#pragma unroll
        for (int gm = 0; gm < 2; ++gm) {
            const int g = 2 * c + gm;
            const float s0 = gm ? bf16_hi(sc[0]) : bf16_lo(sc[0]);
            const float s1 = gm ? bf16_hi(sc[1]) : bf16_lo(sc[1]);
            bf16x8 bfr[2][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bfr[0][j] = codes_to_bf16x8(bw[0][gm][j]);
                bfr[1][j] = codes_to_bf16x8(bw[1][gm][j]);
            }
            const uint8_t *abase = &As[cur][l32 * A_LD + 128 * gm + 64 * gg];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (mt < MT) {
                    floatx16 cin;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const float4 v = *(const float4 *)&cinit[g][32 * mt + 8 * q4 + 4 * gg];
                        cin[4 * q4 + 0] = v.x;
                        cin[4 * q4 + 1] = v.y;
                        cin[4 * q4 + 2] = v.z;
                        cin[4 * q4 + 3] = v.w;
                    }
                    floatx16 p0 = cin, p1 = cin;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x8 af = *(const bf16x8 *)(abase + mt * 32 * A_LD + 16 * j);
                        p0 = mfma32(af, bfr[0][j], p0);
                        p1 = mfma32(af, bfr[1][j], p1);
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        acc[mt][0][i] = __builtin_fmaf(s0, p0[i], acc[mt][0][i]);
                        acc[mt][1][i] = __builtin_fmaf(s1, p1[i], acc[mt][1][i]);
                    }
                }
            }
        }
        if (more) {
            store_a(cur ^ 1);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                sc[q] = scn[q];
#pragma unroll
                for (int gm = 0; gm < 2; ++gm) bw[q][gm] = bwn[q][gm];
            }
        }
        __syncthreads();
    }

    // ---- bias term: sum_g b[n][g] * (hi + lo)[m][g] as MFMA over K'' = 2G (zero padded)
    for (int j2 = 0; j2 < KB2 / 16; ++j2) {
        bf16x8 bb[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint16_t v[8];
#pragma unroll
            for (int el = 0; el < 8; ++el) {
                const int kap = 16 * j2 + 8 * gg + el;
                v[el] = kap < G ? brow[q][kap] : (kap < 2 * G ? brow[q][kap - G] : (uint16_t)0);
            }
            u32x4 pk;
            pk.x = v[0] | ((uint32_t)v[1] << 16);
            pk.y = v[2] | ((uint32_t)v[3] << 16);
            pk.z = v[4] | ((uint32_t)v[5] << 16);
            pk.w = v[6] | ((uint32_t)v[7] << 16);
            bb[q] = __builtin_bit_cast(bf16x8, pk);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt < MT) {
                const bf16x8 af =
                    *(const bf16x8 *)&abias[(32 * mt + l32) * AB_LD + 16 * j2 + 8 * gg];
                acc[mt][0] = mfma32(af, bb[0], acc[mt][0]);
                acc[mt][1] = mfma32(af, bb[1], acc[mt][1]);
            }
        }
    }

    // ---- epilogue.  Accumulator element i of lane (l32, gg) is row
    // 8*(i/4) + 4*gg + i%4 of the 32-row tile, column l32.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        if (mt >= MT) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * mt + 8 * (i >> 2) + 4 * gg + (i & 3);
            if (row >= nrows) continue;
            if (MODE == 0) {
                const float g = acc[mt][0][i], u = acc[mt][1][i];
                const float hv = g / (1.0f + expf(-g)) * u;
                a.h[(size_t)(r0 + row) * a.ldo + nrow[0]] = f32_to_bf16(hv);
            } else {
                if (shared) {
                    const size_t t = (size_t)(r0 - Trk + row);
                    a.y[t * a.ldo + nrow[0]] = acc[mt][0][i];
                    a.y[t * a.ldo + nrow[1]] = acc[mt][1][i];
                } else {
                    const int tt = a.row_token[r0 + row];
                    if (tt < 0 || tt >= a.T) continue;
                    const size_t t = (size_t)tt;
                    const float wr = a.row_w[r0 + row];
                    unsafeAtomicAdd(a.y + t * a.ldo + nrow[0], wr * acc[mt][0][i]);
                    unsafeAtomicAdd(a.y + t * a.ldo + nrow[1], wr * acc[mt][1][i]);
                }
            }
        }
    }
}

static int shared_blocks(int T) { return (T + kBM - 1) / kBM; }

void launch_gateup(const moe_shape &sh, const uint16_t *x, const float *xsum, GemmProj gate,
                   GemmProj up, GemmProj sgate, GemmProj sup, const int32_t *blocks,
                   const int32_t *num_blocks, int max_blocks, const int32_t *row_token,
                   uint16_t *h, hipStream_t s) {
    GemmArgs a{};
    a.A = x;
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
    a.mb_begin = 0;
    a.h = h;
    a.ldo = sh.I;
    const int nmb = max_blocks + shared_blocks(sh.T);
    hipLaunchKernelGGL(q4_gemm_kernel<0>, dim3(nmb * a.n_tiles), dim3(256), 0, s, a);
}

void launch_down(const moe_shape &sh, const uint16_t *h, const float *hsum, GemmProj down,
                 GemmProj sdown, const int32_t *blocks, const int32_t *num_blocks, int max_blocks,
                 const int32_t *row_token, const float *row_w, float *y, hipStream_t s) {
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
    a.y = y;
    a.ldo = sh.H;
    // the shared expert first: plain stores initialise every y element ...
    a.mb_begin = max_blocks;
    hipLaunchKernelGGL(q4_gemm_kernel<1>, dim3(shared_blocks(sh.T) * a.n_tiles), dim3(256), 0, s,
                       a);
    // ... then the routed rows add their weighted outputs
    a.mb_begin = 0;
    hipLaunchKernelGGL(q4_gemm_kernel<1>, dim3(max_blocks * a.n_tiles), dim3(256), 0, s, a);
}

}  // namespace moe
