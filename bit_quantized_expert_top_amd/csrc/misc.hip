// Residual add + RMSNorm between stacked layers, and the dequantisation test hook.
#include "common.h"

namespace moe {

// r <- r + y; u = bf16(r * rsqrt(mean(r^2) + eps)), unit weight.  One workgroup per row,
// thread tid on elements 4 tid + 1024 j.  COMBINE: y holds only the shared expert's part
// of the layer output, and the row's k routed rows are added to it first, from the bf16
// staging rows in pick order, exactly as the combine kernel does; the sum is used and
// never stored.  Both forms therefore give the same bits.
template <bool COMBINE>
__global__ __launch_bounds__(256) void residual_norm_kernel(int H, float eps, float *__restrict__ r,
                                                            const float *__restrict__ y,
                                                            uint16_t *__restrict__ u,
                                                            const uint16_t *__restrict__ stage,
                                                            const int32_t *__restrict__ tok_row,
                                                            int T, int k) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    float *rr = r + row * H;
    const float *yy = y + row * H;
    int rows[8];
    if (COMBINE) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            rows[j] = j < k ? tok_row[row * k + j] : -1;
            MOE_DBG(j >= k || (rows[j] >= 0 && rows[j] < T * k), DBG_COMBINE_ROW);
            if (rows[j] >= T * k) rows[j] = -1;
        }
    }
    float ss = 0.0f;
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        float4 a = *(const float4 *)(rr + i);
        float4 b = *(const float4 *)(yy + i);
        if (COMBINE) {
            uint2 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (rows[j] >= 0) v[j] = *(const uint2 *)(stage + (size_t)rows[j] * H + i);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (rows[j] < 0) continue;
                b.x += bf16_lo(v[j].x);
                b.y += bf16_hi(v[j].x);
                b.z += bf16_lo(v[j].y);
                b.w += bf16_hi(v[j].y);
            }
        }
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
        *(float4 *)(rr + i) = a;
        // explicit fmas in element order: nothing left for the compiler to contract, so
        // both forms of the kernel round identically
        ss = __builtin_fmaf(a.x, a.x, ss);
        ss = __builtin_fmaf(a.y, a.y, ss);
        ss = __builtin_fmaf(a.z, a.z, ss);
        ss = __builtin_fmaf(a.w, a.w, ss);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        const float4 a = *(const float4 *)(rr + i);
        uint2 o;
        o.x = pack_bf16x2(a.x * inv, a.y * inv);
        o.y = pack_bf16x2(a.z * inv, a.w * inv);
        *(uint2 *)(u + row * H + i) = o;
    }
}

void launch_rmsnorm_residual(int T, int H, float eps, float *r, const float *y, uint16_t *u,
                             hipStream_t s) {
    hipLaunchKernelGGL(residual_norm_kernel<false>, dim3(T), dim3(256), 0, s, H, eps, r, y, u,
                       nullptr, nullptr, T, 0);
}

void launch_combine_residual_norm(int T, int H, int k, float eps, float *r, const float *y,
                                  const uint16_t *stage, const int32_t *tok_row, uint16_t *u,
                                  hipStream_t s) {
    hipLaunchKernelGGL(residual_norm_kernel<true>, dim3(T), dim3(256), 0, s, H, eps, r, y, u, stage,
                       tok_row, T, k);
}

// out[n][k] = bf16_rne(fma(code, scale, bias)) in fp32
__global__ __launch_bounds__(256) void dequant_kernel(GemmProj p, int N, int K,
                                                      uint16_t *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;   // one word
    const size_t W = (size_t)K / 8;
    if (i >= (size_t)N * W) return;
    const size_t n = i / W, wd = i % W;
    const uint32_t w = p.q[i];
    const size_t g = n * (K / 64) + (wd * 8) / 64;
    const float s = bf16_to_f32(p.s[g]), b = bf16_to_f32(p.b[g]);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float w0 = __builtin_fmaf((float)((w >> (8 * j)) & 0xFu), s, b);
        const float w1 = __builtin_fmaf((float)((w >> (8 * j + 4)) & 0xFu), s, b);
        o[j] = pack_bf16x2(w0, w1);
    }
    *(uint4 *)(out + n * K + wd * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

void launch_dequant(const GemmProj &p, int N, int K, uint16_t *out, hipStream_t s) {
    const size_t words = (size_t)N * K / 8;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, p,
                       N, K, out);
}

MOE_DBG_READER(dbg_read_misc)

}  // namespace moe
