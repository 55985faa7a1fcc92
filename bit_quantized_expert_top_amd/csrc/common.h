// Shared device helpers and internal launcher declarations of libmoeq4.
// gfx950 (CDNA4) only: wave64, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe_q4.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 64;      // quantisation group along K
constexpr int kBM = 128;        // rows per routing block (GEMM M tile)
constexpr int kTB = 8;          // tokens per routing token block (one wave each)
constexpr int kSupBlk = 16;      // token blocks per superblock of the single-pass routing scan
constexpr int kSupMax = 32;      // superblocks of the single-pass scan (T <= 4096)
constexpr int kDecodeMaxT = 8;  // moe_decode: tokens per call (each an independent GEMV problem)

// Decode scratch for T tokens (E = 256 experts, k + 1 slots): the router logits, the h
// rows, and the per-slot h factors followed by each token's ||x||^2, each part rounded
// up to 256 bytes.
constexpr size_t decode_scratch_size(int T, int I, int k) {
    return (((size_t)T * 256 * 4 + 255) & ~(size_t)255) +
           (((size_t)T * (k + 1) * I * 2 + 255) & ~(size_t)255) +
           (((size_t)T * (k + 2) * 4 + 255) & ~(size_t)255);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// fp32 -> fp16 bits, round to nearest even
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t v) {
    return (float)__builtin_bit_cast(f16x2, v)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
    return (float)__builtin_bit_cast(f16x2, v)[1];
}

// Monotone uint32 key of a float (larger float -> larger key; -0 ranks with +0)
// and its inverse.
__device__ __forceinline__ uint32_t ordered_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);   // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t kh) {
    return __uint_as_float((kh & 0x80000000u) ? (kh & 0x7fffffffu) : ~kh);
}


// Wave-wide unsigned max, returned in every lane: DPP steps inside each row of
// 16 lanes (xor 1, xor 2, half-row mirror, row mirror), then the four row
// results read as scalars.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    v = dpp_umax<0xB1>(v);
    v = dpp_umax<0x4E>(v);
    v = dpp_umax<0x141>(v);
    v = dpp_umax<0x140>(v);
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

// Largest key among 4 per lane (key[j] belongs to expert lane + 64 j; taken
// entries excluded), ties to the lowest expert index.  Returns the expert.
__device__ __forceinline__ int wave_argmax4(const uint32_t (&key)[4], const bool (&taken)[4],
                                            uint32_t *kmax) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (!taken[j] && key[j] > m) m = key[j];
    m = wave_umax(m);
    *kmax = m;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t b = __ballot(!taken[j] && key[j] == m);
        if (b) return 64 * j + __builtin_ctzll(b);
    }
    return -1;
}

// The k <= 8 largest of the wave's 256 keys (key[j] belongs to expert lane + 64 j),
// ties to the lower expert index.  A bitwise search from the top bit finds the
// k-th largest key value T (stopping early once exactly k keys reach the
// candidate); the picks are the keys above T and the lowest-index keys equal to
// T.  wave_topk_set marks them in taken[j]; wave_topk_radix also ranks them by
// (key desc, index asc) through wave-local LDS (wl: 32 words), so that lane p < k
// ends with pick p.
__device__ inline void wave_topk_set(const uint32_t (&key)[4], int k, bool (&taken)[4]) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t lo = 0;                     // #(key >= lo) >= k throughout
    bool exact = false;                  // #(key >= lo) == k
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = lo | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt += (int)__popcll(__ballot(key[j] >= cand));
        if (cnt >= k) {
            lo = cand;
            if (cnt == k) {
                exact = true;
                break;
            }
        }
    }
    if (exact) {
#pragma unroll
        for (int j = 0; j < 4; ++j) taken[j] = key[j] >= lo;
    } else {
        // lo is the k-th largest value: every key above it, then keys equal to it
        // in ascending expert index (j, then lane) until k are taken
        int need = k;
#pragma unroll
        for (int j = 0; j < 4; ++j) need -= (int)__popcll(__ballot(key[j] > lo));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint64_t eq = __ballot(key[j] == lo);
            const bool mine = key[j] == lo && (int)__popcll(eq & below) < need;
            taken[j] = key[j] > lo || mine;
            need -= min((int)__popcll(eq), max(need, 0));
        }
    }
}

__device__ inline void wave_topk_radix(const uint32_t (&key)[4], int k, bool (&taken)[4], int &pick_e,
                                uint32_t &pick_key, uint32_t *wl) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    wave_topk_set(key, k, taken);
    // compact the picks (any order), then rank them
    int base = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t bal = __ballot(taken[j]);
        if (taken[j]) {
            const int pos = base + (int)__popcll(bal & below);
            wl[pos] = (uint32_t)(lane + 64 * j);
            wl[8 + pos] = key[j];
        }
        base += (int)__popcll(bal);
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < k) {
        const uint32_t ep = wl[lane], kp = wl[8 + lane];
        int rk = 0;
        for (int q = 0; q < k; ++q) {
            const uint32_t eq = wl[q], kq = wl[8 + q];
            rk += (kq > kp || (kq == kp && eq < ep)) ? 1 : 0;
        }
        wl[16 + rk] = ep;
        wl[24 + rk] = kp;
    }
    __builtin_amdgcn_wave_barrier();
    pick_e = lane < k ? (int)wl[16 + lane] : -1;
    pick_key = lane < k ? wl[24 + lane] : 0u;
    __builtin_amdgcn_wave_barrier();
}

// Routing weight of pick p, held by lane p < k (k <= 8) with its fixed-order logit l:
// the softmax over all experts renormalised over the picks, i.e.
//   w_p = exp(l_p - l_0) / sum_{j<k} exp(l_j - l_0),
// evaluated in fp64 (the differences of two fp32 logits are exact there) and rounded
// once to fp32.  Lanes >= k return 0.  Every lane of the wave must call it.
__device__ inline float topk_weight(float l, int k) {
    const int lane = threadIdx.x & 63;
    const float l0 = __shfl(l, 0);
    const double p = lane < k ? exp((double)l - (double)l0) : 0.0;
    double s = p;
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);      // lanes 0..7: the sum over the (at most 8) picks
    return lane < k ? (float)(p / s) : 0.0f;
}

// Sum over aligned groups of n lanes (n = 1, 2, 4, 8 or 16) with DPP; every
// lane of a group ends with the group's sum.
__device__ __forceinline__ float group_sum_dpp(float v, int n) {
    if (n >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if (n >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    if (n >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if (n >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// Maximum over aligned groups of 8 lanes with DPP; every lane of a group ends with it.
__device__ __forceinline__ float group_max_dpp8(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    return v;
}

// GEMM work queues (int32 words of the workspace's qctl area): per GEMM launch a
// queue head and a finished-workgroup count, then (one-launch FFN) a finished
// gate/up item count per slot.  The routing scatter zeroes them all; each
// launch's last workgroup zeroes its own again.  Every queue counter has a
// 128-byte line of its own (atomics on one shared line serialise).
constexpr int QCTL_LINE = 32;                       // words per counter
constexpr int QCTL_GATEUP = 0;                      // head, then finished count
constexpr int QCTL_DOWN = 2 * QCTL_LINE;            // same for the down GEMM
constexpr int QCTL_FFN = 4 * QCTL_LINE;             // same for the one-launch FFN
constexpr int QCTL_WORDS = 6 * QCTL_LINE;           // then the FFN's per-slot counts
// bounded wait of a one-launch FFN down item for its slot's gate/up items (s_sleep 2 rounds,
// each with a round trip to memory: about a second)
constexpr int kFfnSpin = 1 << 20;

// Tile layout of the expert weights: one block per (tile of 256 columns, group
// of 64 inputs), codes then scales then biases (the block format is documented
// with moe_pack_weights).
constexpr int PK_BLOCK = 9216;
constexpr int PK_CODES = 8192;      // byte offset of the scales; biases at +512
// Per projection row (one GEMM column), a power-of-two factor written at load time:
//  colk = 2^-k: the block holds scale and bias times 2^k, with k chosen so that the
//         row's largest |scale| times 2^k lies in [2^10, 2^11); the rebuilt fp16
//         weights (q - 8) s 2^k are then exact whenever the row's nonzero scales span
//         at most 2^23, whatever their absolute size; results are multiplied by colk.
// They are stored per tile: [colk of the 256 columns][flags], the flags word (int32 at
// float index PK_TFLAG) nonzero when some column of the tile has a group with b != -8 s
// (the tile needs the rank-G bias term).
constexpr int PK_COLF = 260;        // floats of column factors and flags per tile (16-byte multiple)
constexpr int PK_TFLAG = 256;
// Load-time validation flags (the status word of the meta section)
constexpr int PK_BAD_NONFINITE = 1;     // a scale or bias is NaN or infinite
constexpr int PK_BAD_SCALE_SPAN = 2;    // a row's nonzero scales span more than 2^23
constexpr int PK_BAD_BIAS_RANGE = 4;    // a bias times 2^k leaves the bf16 range
constexpr int PK_EMETA = 4;         // floats per expert slot in the meta section
struct PackLayout {
    size_t gu, sh_gu, down, sh_down;        // tile-layout blocks of the four sections
    size_t status;                          // int32 validation flags (one 256-byte line)
    size_t emeta;                           // float [E+1][PK_EMETA]: [0] bounds the L2 norm
                                            // of every gate and up row of the expert slot
    size_t cgu, csh_gu, cdown, csh_down;    // column factors, per tile [PK_COLF] floats
    size_t total;
};
PackLayout pack_layout(int H, int I, int E);
// column c of a gate/up block of tile j: projection (c >> 5) & 1 (0 gate,
// 1 up), row 128 j + 32 (c >> 6) + (c & 31); of a down block: row 256 j + c
void launch_pack(const moe_shape &sh, const moe_weights &w, uint8_t *dst, int32_t *status,
                 hipStream_t s);

// Device index checks of the MOE_DEBUG build.  Wherever a kernel meets an index that the
// routing structures should never hold (an expert id, row, token or block out of range) it
// already clamps or skips it; the debug build also records what it met in a status word of
// the translation unit (moe_debug_status reads and clears them all).  Vector atomics only.
constexpr uint32_t DBG_ROUTE_INDEX = 1;     // scatter: pick expert or row out of range
constexpr uint32_t DBG_GEMM_BLOCK = 2;      // grouped GEMM: malformed block map entry
constexpr uint32_t DBG_GEMM_TOKEN = 4;      // grouped GEMM: row token out of range
constexpr uint32_t DBG_COMBINE_ROW = 8;     // combine: a pick's row out of range
constexpr uint32_t DBG_DECODE_ID = 16;      // decode: a pick's expert id out of range
constexpr uint32_t DBG_FFN_WAIT = 32;       // one-launch FFN: a down item's wait timed out
#ifdef MOE_DEBUG
static __device__ uint32_t dbg_word;
#define MOE_DBG(cond, bit)                           \
    do {                                             \
        if (!(cond)) atomicOr(&dbg_word, (bit));     \
    } while (0)
// host: read (and clear) this translation unit's status word
#define MOE_DBG_READER(name)                                                          \
    uint32_t name(bool clear) {                                                       \
        uint32_t v = 0;                                                               \
        if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(dbg_word), sizeof v, 0,                \
                                hipMemcpyDeviceToHost) != hipSuccess)                 \
            return 0x80000000u;                                                       \
        if (clear) {                                                                  \
            const uint32_t z = 0;                                                     \
            (void)hipMemcpyToSymbol(HIP_SYMBOL(dbg_word), &z, sizeof z, 0,            \
                                    hipMemcpyHostToDevice);                           \
        }                                                                             \
        return v;                                                                     \
    }
#else
#define MOE_DBG(cond, bit) ((void)0)
#define MOE_DBG_READER(name) \
    uint32_t name(bool) { return 0; }
#endif
uint32_t dbg_read_route(bool clear);
uint32_t dbg_read_gemm(bool clear);
uint32_t dbg_read_decode(bool clear);
uint32_t dbg_read_misc(bool clear);

// A kernel's dynamic-LDS limit raised once per device (thread-safe: a host thread's
// first launch on a device sets it, concurrent first launches wait for that).
struct LdsLimit {
    static constexpr int kMaxDevices = 64;
    std::once_flag once[kMaxDevices];
    void ensure(const void *fn, int bytes) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
            (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
            return;
        }
        std::call_once(once[dev], [&] {
            (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        });
    }
};

// Workspace layout (byte offsets), shared by route/gemm/decode.  All host-known.
struct WsLayout {
    size_t logits;      // fp32 [T][E]            (used when routing.logits == NULL)
    size_t xsum;        // fp32 [T][H/64]         group sums of x
    size_t xp;          // fp16 [T][H]            x in fp16 (times the token's 2^-e)
    size_t xsq;         // fp32 [T][H/64]         group sums of x^2
    size_t part;        // fp32 [4][T][E]         K-split approximate router logits
    size_t wn2;         // fp32 [4][E]            squared norms of the router rows, per K split
    size_t hsum;        // fp32 [T*k + T][I/64]   group sums of h (fp16 values)
    size_t stage;       // bf16 [T*k][H]          routed down outputs times routing weight
    size_t blk_cnt;     // int32 [T/kTB][E]       per token-block expert counts / bases
    size_t lrank;       // int32 [T][k]           rank of (t,j) inside its token block
    size_t sup;         // int32 [T/(kTB kSupBlk)][E] per superblock expert counts (T <= 4096)
    size_t sched;       // int32 [max_blocks]     GEMM order of the routed blocks (by cost class)
    size_t qctl;        // int32 [QCTL_WORDS + ffn_slots]  GEMM work-queue counters, FFN slot counts
    size_t xmx;         // fp32 [T][H/64]         group maxima of |x|
    size_t tok;         // fp32 [T][2]            per token: 2^e (x enters the GEMM as x 2^-e), ||x||
    size_t hexp;        // fp32 [T*k + T]         per h row: 2^f (h is stored as h 2^-f)
    size_t dec;         // decode scratch
    size_t total;
};

WsLayout ws_layout(int T, int H, int I, int E, int k);
int max_blocks_for(int T, int E, int k);
// work-item slots of the GEMMs: shared-expert blocks plus at most max_blocks_for routed blocks
int ffn_slots(int T, int E, int k);

// ---- launchers (defined in the .hip files; all asynchronous) ----
void launch_router_logits(const uint16_t *x, const uint16_t *wr_t, const float *bias, int T, int H,
                          int E, float *logits, hipStream_t s);
void launch_router_fast(const uint16_t *x, const uint16_t *wr, int T, int H, int E, float *part,
                        float *wn2part, uint16_t *xp, float *xsum, float *xsq, float *xmx,
                        int32_t *zero, int nzero, hipStream_t s);
void launch_route_select(const float *part, const float *exact, const float *xsq,
                         const float *wn2, const float *bias, const uint16_t *x,
                         const uint16_t *wr, int T, int H, int E, int k, int32_t *ids, float *w,
                         int32_t *blk_cnt, int32_t *lrank, int32_t *sup, const float *xmx,
                         uint16_t *xp, float *xsum, float *tok, hipStream_t s);
// sup != NULL (T <= 4096): one kernel from the superblock counts; else a per-expert
// scan kernel, then the scatter
void launch_scan_scatter(const int32_t *ids, const float *w, int32_t *blk_cnt,
                         const int32_t *sup, const int32_t *lrank, int T, int E, int k, int BM,
                         int32_t *counts, int32_t *offsets, int32_t *row_token, int32_t *tok_row,
                         float *row_w, int32_t *blocks, int32_t *num_blocks, int32_t *sched,
                         int32_t *qctl, int nslots, hipStream_t s);
void launch_zero_i32(int32_t *p, int n, hipStream_t s);
void launch_prep_act(const uint16_t *x, int rows, int K, uint16_t *xp, float *xsum, float *xsq,
                     float *xmx, hipStream_t s);

struct GemmProj {
    const uint32_t *q;
    const uint16_t *s;
    const uint16_t *b;
};

// The expert weights of one GEMM: tile-layout blocks and column factors of the routed
// experts and of the shared expert, and the per-expert meta (gate/up only).
struct GemmWeights {
    const uint8_t *pk, *pk_sh;
    const float *colf, *colf_sh;
    const float *emeta;
};
GemmWeights gemm_weights(const void *packed, int H, int I, int E, bool gateup);

void launch_gateup(const moe_shape &sh, const uint16_t *x, const float *xsum, const float *tok,
                   const GemmWeights &gw, const int32_t *blocks, const int32_t *num_blocks,
                   const int32_t *sched, int32_t *qctl, int max_blocks, const int32_t *row_token,
                   uint16_t *h, float *hsum, float *hexp, hipStream_t s);
void launch_down(const moe_shape &sh, const uint16_t *h, const float *hsum, const float *hexp,
                 const GemmWeights &gw, const int32_t *blocks, const int32_t *num_blocks,
                 const int32_t *sched, int32_t *qctl, int max_blocks,
                 const int32_t *row_token, const float *row_w, const int32_t *tok_row,
                 uint16_t *stage, float *y, bool combine, hipStream_t s);
// gate/up and down in one persistent launch, then (combine) the combine
void launch_ffn(const moe_shape &sh, const uint16_t *xp, const float *xsum, const float *tok,
                const GemmWeights &gwg, const GemmWeights &gwd, const int32_t *blocks,
                const int32_t *num_blocks, const int32_t *sched, int32_t *qctl, int max_blocks,
                const int32_t *row_token, const float *row_w, const int32_t *tok_row, uint16_t *h,
                float *hsum, float *hexp, uint16_t *stage, float *y, bool combine, hipStream_t s);
// y[t] += the k staged routed rows of token t, in pick order (fp32)
void launch_combine(const moe_shape &sh, const uint16_t *stage, const int32_t *tok_row, float *y,
                    hipStream_t s);
// r += (y + the k staging rows of each token, in pick order); u = bf16(RMSNorm(r))
void launch_combine_residual_norm(int T, int H, int k, float eps, float *r, const float *y,
                                  const uint16_t *stage, const int32_t *tok_row, uint16_t *u,
                                  hipStream_t s);

// Power-of-two helpers for the range normalisation: 2^n as a float (n clamped to the
// normal range), and floor(log2 |v|) of a finite nonzero float.
__host__ __device__ inline float exp2i(int n) {
    n = n < -126 ? -126 : (n > 127 ? 127 : n);
    union { uint32_t u; float f; } c;
    c.u = (uint32_t)(n + 127) << 23;
    return c.f;
}
__device__ inline int ilog2f(float v) {
    const uint32_t u = __float_as_uint(v) & 0x7fffffffu;
    if (u >= 0x00800000u) return (int)(u >> 23) - 127;
    return -127 - __builtin_clz(u) + 9;        // subnormal: 2^-149 .. 2^-127
}

// Exponent f of the power of two that brings h = silu(g) u into the fp16 range: with
// |g|, |u| <= nw ||x|| (Cauchy-Schwarz, nw bounding the L2 norm of every gate and up row)
// and |silu(g)| <= |g|, |h| <= B = (nw ||x||)^2.  f = 0 while B lies in [2^-2, 2^15);
// otherwise f is the exponent with B 2^-f in [2^14, 2^15) (up to rounding), so h 2^-f
// stays below 65504 and its bulk above the fp16 subnormals.
__device__ inline int h_exponent(float nw, float nx) {
    if (!(nw > 0.0f) || !(nx > 0.0f)) return 0;
    const int a = ilog2f(nw) + ilog2f(nx);              // nw nx in [2^a, 2^(a+2))
    int eb;                                             // B < 2^eb
    if (a > 60 || a < -60) {
        eb = 2 * a + 4;
    } else {
        const float p = nw * nx;                        // no overflow or underflow here
        const float B = p * p;
        if (B >= 0.25f && B < 32768.0f) return 0;
        eb = ilog2f(B) + 1;
    }
    const int f = eb - 15;
    return f < -100 ? -100 : (f > 100 ? 100 : f);
}

// Exponent e of the power of two that brings a token's activations into the fp16 range
// of the expert GEMM: 0 while max |x| lies in [2^-6, 2^14) (bf16 values down to 2^-17
// convert exactly), otherwise the e with max |x| 2^-e in [2^13, 2^14).
__device__ inline int x_exponent(float xmax) {
    if (!(xmax > 0.0f) || (xmax >= 0x1p-6f && xmax < 16384.0f)) return 0;
    return ilog2f(xmax) - 13;
}

// res == NULL: decode x.  Otherwise x is ignored and the input is bf16(RMSNorm(res + yprev)),
// written to u_out; res <- res + yprev (a decode stack's residual step).
void launch_decode(const moe_shape &sh, const uint16_t *x, const moe_weights &w, int32_t *ids,
                   float *tw, float *y, void *scratch, hipStream_t s, float *res = nullptr,
                   const float *yprev = nullptr, float eps = 0.0f, uint16_t *u_out = nullptr);

void launch_rmsnorm_residual(int T, int H, float eps, float *r, const float *y, uint16_t *u,
                             hipStream_t s);
void launch_dequant(const GemmProj &p, int N, int K, uint16_t *out, hipStream_t s);

}  // namespace moe
