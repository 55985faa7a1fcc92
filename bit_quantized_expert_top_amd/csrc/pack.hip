// Tile layout of the expert weights.  The checkpoint stores each projection
// row by row (codes along K, then per-group scales and biases), so one 64-wide
// K step of a 256-column GEMM tile touches 256 separate 32-byte pieces of
// codes and 512 separate 2-byte scales and biases.  Regrouped once at load
// time, the same step is one contiguous block that a workgroup copies with a
// few whole-line loads (the pages rebuild weights tile by tile in the grouped
// GEMM and owe their decode bandwidth to coalesced reads: mechatronicstore.cl,
// "Prefill: pesos comprimidos y enrutamiento en la GPU" and "Decode: mover
// menos bytes por token").  The regrouping only moves bytes (and reorders the
// codes inside each 32-bit word, below).
#include "common.h"

#include <algorithm>

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

PackLayout pack_layout(int H, int I, int E) {
    PackLayout L{};
    const size_t gu_blocks = (size_t)(I / 128) * (H / 64);     // per expert
    const size_t dn_blocks = (size_t)(H / 256) * (I / 64);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.gu = take((size_t)E * gu_blocks * PK_BLOCK);
    L.sh_gu = take(gu_blocks * PK_BLOCK);
    L.down = take((size_t)E * dn_blocks * PK_BLOCK);
    L.sh_down = take(dn_blocks * PK_BLOCK);
    L.status = take(256);
    L.emeta = take((size_t)(E + 1) * PK_EMETA * 4);
    L.cgu = take((size_t)E * (I / 128) * PK_COLF * 4);
    L.csh_gu = take((size_t)(I / 128) * PK_COLF * 4);
    L.cdown = take((size_t)E * (H / 256) * PK_COLF * 4);
    L.csh_down = take((size_t)(H / 256) * PK_COLF * 4);
    L.total = off;
    return L;
}

GemmWeights gemm_weights(const void *packed, int H, int I, int E, bool gateup) {
    const PackLayout L = pack_layout(H, I, E);
    const uint8_t *p = (const uint8_t *)packed;
    GemmWeights g;
    g.pk = p + (gateup ? L.gu : L.down);
    g.pk_sh = p + (gateup ? L.sh_gu : L.sh_down);
    g.colf = (const float *)(p + (gateup ? L.cgu : L.cdown));
    g.colf_sh = (const float *)(p + (gateup ? L.csh_gu : L.csh_down));
    g.emeta = (const float *)(p + L.emeta);
    return g;
}

struct PackSrc {
    GemmProj p0, p1;    // gate, up (gate/up section) or down, - (down section)
};

// Column (tile j, column c) of projection row n: gate/up rows interleave in 32-column
// runs (gate row 128 j + 32 u + i is column 64 u + i, up row the same + 32); down row n
// is column n % 256 of tile n / 256.
__host__ __device__ inline void row_to_col(int gu, int proj, int n, int &j, int &c) {
    if (gu) {
        j = n / 128;
        const int w = n % 128;
        c = 64 * (w / 32) + 32 * proj + (w % 32);
    } else {
        j = n / 256;
        c = n % 256;
    }
}

// Load-time statistics, one wave per projection row (expert e, projection proj, row n):
// the power-of-two shift k of the row's scales, whether its tile needs the rank-G bias
// term, the row's L2
// norm (gate and up rows: folded into the expert slot's bound by an atomic max on the
// float's bits, which orders like the value for non-negative floats) and the validation
// flags.  The meta section must hold zeros beforehand.
__global__ __launch_bounds__(256) void pack_stats_kernel(PackSrc src, int nexp, int N, int K, int gu,
                                                        int slot0, float *__restrict__ colf,
                                                        float *__restrict__ emeta,
                                                        int32_t *__restrict__ status) {
    const int lane = threadIdx.x & 63;
    const size_t wrow = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nproj = gu ? 2 : 1;
    if (wrow >= (size_t)nexp * nproj * N) return;
    const int n = (int)(wrow % N);
    const int proj = (int)((wrow / N) % nproj);
    const int e = (int)(wrow / ((size_t)N * nproj));
    const GemmProj &q = proj ? src.p1 : src.p0;
    const int G = K / 64;
    const size_t row = (size_t)e * N + n;
    // scales and biases: lane g < G holds group g (G <= 32)
    float sv = 0.0f, bv = 0.0f;
    if (lane < G) {
        sv = bf16_to_f32(q.s[row * G + lane]);
        bv = bf16_to_f32(q.b[row * G + lane]);
    }
    bool bad_nf = lane < G && (!__builtin_isfinite(sv) || !__builtin_isfinite(bv));
    float smax = (lane < G && __builtin_isfinite(sv)) ? fabsf(sv) : 0.0f;
    float smin = (lane < G && __builtin_isfinite(sv) && sv != 0.0f) ? fabsf(sv) : INFINITY;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        smax = fmaxf(smax, __shfl_xor(smax, off));
        smin = fminf(smin, __shfl_xor(smin, off));
    }
    const int k = smax > 0.0f ? 10 - ilog2f(smax) : 0;
    const float kmul = exp2i(k);
    // every nonzero |s| 2^k at least 2^-13: (q - 8) s 2^k / 16 is then an exact fp16 value
    const bool bad_span = smax > 0.0f && smin * kmul < 0x1p-13f;
    const float bk = bv * kmul;
    const bool bad_bias = lane < G && __builtin_isfinite(bv) && !(fabsf(bk) < 0x1.fep127f);
    // a group with b != -8 s: the row's tile needs the rank-G bias term
    const bool affine = __any(lane < G && bv != -8.0f * sv);
    if (lane == 0) {
        int j, c;
        row_to_col(gu, proj, n, j, c);
        const int JT = gu ? N / 128 : N / 256;
        float *cf = colf + ((size_t)e * JT + j) * PK_COLF;
        cf[c] = exp2i(-k);
        if (affine) atomicOr((int *)(cf + PK_TFLAG), 1);
    }
    const int flags = (__any(bad_nf) ? PK_BAD_NONFINITE : 0) | (bad_span ? PK_BAD_SCALE_SPAN : 0) |
                      (__any(bad_bias) ? PK_BAD_BIAS_RANGE : 0);
    if (lane == 0 && flags) atomicOr(status, flags);
    if (!gu) return;
    // L2 norm of the row's weights q s + b (fp32, the bound adds a margin for rounding)
    float ss = 0.0f;
    const uint32_t *qr = q.q + row * (size_t)(K / 8);
    for (int wi = lane; wi < K / 8; wi += 64) {
        const uint32_t wd = qr[wi];
        const int g = wi / 8;
        const float s_g = __shfl(sv, g), b_g = __shfl(bv, g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float w = __builtin_fmaf((float)((wd >> (4 * i)) & 0xFu), s_g, b_g);
            ss = __builtin_fmaf(w, w, ss);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) {
        const float nrm = sqrtf(ss) * 1.001f;
        if (__builtin_isfinite(nrm))
            atomicMax((unsigned int *)(emeta + (size_t)(slot0 + e) * PK_EMETA), __float_as_uint(nrm));
        else
            atomicOr(status, PK_BAD_NONFINITE);
    }
}

// Code order inside a tile-layout word: the even codes 0, 2, 4, 6 of the
// checkpoint word go to nibbles 0-3 (the low half), the odd codes 1, 3, 5, 7 to
// nibbles 4-7.  The kernels unpack a word as the nibble pairs (p, p + 4), p = 0..3
// (one and-or with mask 0x000F000F per pair, shifted by 4 p), which in this order
// are the code pairs (2p, 2p + 1): weights come out in natural order and meet
// activations (x, h) stored in natural order.
__device__ __forceinline__ uint32_t unzip_codes(uint32_t w) {
    uint32_t r = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        r |= ((w >> (8 * m)) & 0xFu) << (4 * m);             // code 2m   -> nibble m
        r |= ((w >> (8 * m + 4)) & 0xFu) << (4 * m + 16);    // code 2m+1 -> nibble m + 4
    }
    return r;
}

// One thread per 16-byte piece of codes; the first 256 threads of a block
// also move the block's scales and biases, times the column's 2^k.  Block b
// of a section is (expert, tile j, group g) with g fastest; N = rows per
// expert, K = inputs.
__global__ __launch_bounds__(256) void pack_kernel(PackSrc src, int nexp, int N, int K, int gu,
                                                   const float *__restrict__ colf,
                                                   uint8_t *__restrict__ dst) {
    const int G = K / 64, JT = gu ? N / 128 : N / 256;
    const size_t npieces = (size_t)nexp * JT * G * 512;
    for (size_t p = (size_t)blockIdx.x * 256 + threadIdx.x; p < npieces;
         p += (size_t)gridDim.x * 256) {
        const size_t b = p >> 9;
        const int pp = (int)(p & 511);
        const int g = (int)(b % G);
        const size_t ej = b / G;
        const int j = (int)(ej % JT), e = (int)(ej / JT);
        uint8_t *blk = dst + b * PK_BLOCK;
        // codes: piece pp = column pp/2, half pp&1, which holds code words
        // 4 * (half ^ ((column >> 3) & 1)) .. +3 of the group
        {
            const int c = pp >> 1, hh = pp & 1;
            const GemmProj &q = (gu && ((c >> 5) & 1)) ? src.p1 : src.p0;
            const int n = gu ? 128 * j + 32 * (c >> 6) + (c & 31) : 256 * j + c;
            const size_t row = (size_t)e * N + n;
            const u32x4 v = *(const u32x4 *)(q.q + row * (size_t)(K / 8) + 8 * g + 4 * (hh ^ ((c >> 3) & 1)));
            u32x4 o;
            o.x = unzip_codes(v.x);
            o.y = unzip_codes(v.y);
            o.z = unzip_codes(v.z);
            o.w = unzip_codes(v.w);
            *(u32x4 *)(blk + 16 * pp) = o;
        }
        if (pp < 256) {
            const int c = pp;
            const GemmProj &q = (gu && ((c >> 5) & 1)) ? src.p1 : src.p0;
            const int n = gu ? 128 * j + 32 * (c >> 6) + (c & 31) : 256 * j + c;
            const size_t row = (size_t)e * N + n;
            // 2^k = 1 / colk: a power of two, so the products are exact bf16 values
            const float kmul = 1.0f / colf[((size_t)e * JT + j) * PK_COLF + c];
            ((uint16_t *)(blk + PK_CODES))[c] = f32_to_bf16(bf16_to_f32(q.s[row * G + g]) * kmul);
            ((uint16_t *)(blk + PK_CODES + 512))[c] = f32_to_bf16(bf16_to_f32(q.b[row * G + g]) * kmul);
        }
    }
}

__global__ void pack_zero_kernel(uint32_t *__restrict__ p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__global__ void pack_status_copy_kernel(const int32_t *__restrict__ src, int32_t *__restrict__ dst) {
    if (threadIdx.x == 0) dst[0] = src[0];
}

void launch_pack(const moe_shape &sh, const moe_weights &w, uint8_t *dst, int32_t *status,
                 hipStream_t s) {
    const PackLayout L = pack_layout(sh.H, sh.I, sh.E);
    auto gp = [](const moe_q4 &p) { return GemmProj{p.q, p.scale, p.bias}; };
    int32_t *st = (int32_t *)(dst + L.status);
    float *emeta = (float *)(dst + L.emeta);
    // the meta section starts at zero: status, expert bounds, tile flags (a fill kernel,
    // not a memset)
    const size_t nz = (L.total - L.status) / 4;
    hipLaunchKernelGGL(pack_zero_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, s,
                       (uint32_t *)st, nz);
    auto stats = [&](PackSrc src, int nexp, int N, int K, int gu, int slot0, size_t coff) {
        const size_t rows = (size_t)nexp * (gu ? 2 : 1) * N;
        hipLaunchKernelGGL(pack_stats_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, src,
                           nexp, N, K, gu, slot0, (float *)(dst + coff), emeta, st);
    };
    auto run = [&](PackSrc src, int nexp, int N, int K, int gu, size_t off, size_t coff) {
        const size_t npieces = (size_t)nexp * (gu ? N / 128 : N / 256) * (K / 64) * 512;
        const unsigned grid = (unsigned)std::min<size_t>((npieces + 255) / 256, 65536);
        hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, src, nexp, N, K, gu,
                           (const float *)(dst + coff), dst + off);
    };
    const PackSrc gu{gp(w.gate), gp(w.up)}, sgu{gp(w.sh_gate), gp(w.sh_up)};
    const PackSrc dn{gp(w.down), gp(w.down)}, sdn{gp(w.sh_down), gp(w.sh_down)};
    stats(gu, sh.E, sh.I, sh.H, 1, 0, L.cgu);
    stats(sgu, 1, sh.I, sh.H, 1, sh.E, L.csh_gu);
    stats(dn, sh.E, sh.H, sh.I, 0, 0, L.cdown);
    stats(sdn, 1, sh.H, sh.I, 0, sh.E, L.csh_down);
    run(gu, sh.E, sh.I, sh.H, 1, L.gu, L.cgu);
    run(sgu, 1, sh.I, sh.H, 1, L.sh_gu, L.csh_gu);
    run(dn, sh.E, sh.H, sh.I, 0, L.down, L.cdown);
    run(sdn, 1, sh.H, sh.I, 0, L.sh_down, L.csh_down);
    if (status) hipLaunchKernelGGL(pack_status_copy_kernel, dim3(1), dim3(64), 0, s, st, status);
}

}  // namespace moe
