// Tile layout of the expert weights.  The checkpoint stores each projection
// row by row (codes along K, then per-group scales and biases), so one 64-wide
// K step of a 256-column GEMM tile touches 256 separate 32-byte pieces of
// codes and 512 separate 2-byte scales and biases.  Regrouped once at load
// time, the same step is one contiguous block that a workgroup copies with a
// few whole-line loads (the pages rebuild weights tile by tile in the grouped
// GEMM and owe their decode bandwidth to coalesced reads: mechatronicstore.cl,
// "Prefill: pesos comprimidos y enrutamiento en la GPU" and "Decode: mover
// menos bytes por token").  The regrouping only moves bytes.
#include "common.h"

#include <algorithm>

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

PackLayout pack_layout(int H, int I, int E) {
    PackLayout L{};
    const size_t gu_blocks = (size_t)(I / 128) * (H / 64);     // per expert
    const size_t dn_blocks = (size_t)(H / 256) * (I / 64);
    size_t off = 0;
    L.gu = off;
    off = align256(off + (size_t)E * gu_blocks * PK_BLOCK);
    L.sh_gu = off;
    off = align256(off + gu_blocks * PK_BLOCK);
    L.down = off;
    off = align256(off + (size_t)E * dn_blocks * PK_BLOCK);
    L.sh_down = off;
    off = align256(off + dn_blocks * PK_BLOCK);
    L.total = off;
    return L;
}

struct PackSrc {
    GemmProj p0, p1;    // gate, up (gate/up section) or down, - (down section)
};

// One thread per 16-byte piece of codes; the first 256 threads of a block
// also move the block's scales and biases.  Block b of a section is
// (expert, tile j, group g) with g fastest; N = rows per expert, K = inputs.
__global__ __launch_bounds__(256) void pack_kernel(PackSrc src, int nexp, int N, int K, int gu,
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
            *(u32x4 *)(blk + 16 * pp) = v;
        }
        if (pp < 256) {
            const int c = pp;
            const GemmProj &q = (gu && ((c >> 5) & 1)) ? src.p1 : src.p0;
            const int n = gu ? 128 * j + 32 * (c >> 6) + (c & 31) : 256 * j + c;
            const size_t row = (size_t)e * N + n;
            ((uint16_t *)(blk + PK_CODES))[c] = q.s[row * G + g];
            ((uint16_t *)(blk + PK_CODES + 512))[c] = q.b[row * G + g];
        }
    }
}

void launch_pack(const moe_shape &sh, const moe_weights &w, uint8_t *dst, hipStream_t s) {
    const PackLayout L = pack_layout(sh.H, sh.I, sh.E);
    auto gp = [](const moe_q4 &p) { return GemmProj{p.q, p.scale, p.bias}; };
    auto run = [&](PackSrc src, int nexp, int N, int K, int gu, size_t off) {
        const size_t npieces = (size_t)nexp * (gu ? N / 128 : N / 256) * (K / 64) * 512;
        const unsigned grid = (unsigned)std::min<size_t>((npieces + 255) / 256, 65536);
        hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, src, nexp, N, K, gu, dst + off);
    };
    run(PackSrc{gp(w.gate), gp(w.up)}, sh.E, sh.I, sh.H, 1, L.gu);
    run(PackSrc{gp(w.sh_gate), gp(w.sh_up)}, 1, sh.I, sh.H, 1, L.sh_gu);
    run(PackSrc{gp(w.down), gp(w.down)}, sh.E, sh.H, sh.I, 0, L.down);
    run(PackSrc{gp(w.sh_down), gp(w.sh_down)}, 1, sh.H, sh.I, 0, L.sh_down);
}

}  // namespace moe
