// Residual add + RMSNorm between stacked layers, and the dequantisation test hook.
#include "common.h"

namespace moe {

// r <- r + y; u = bf16(r * rsqrt(mean(r^2) + eps)), unit weight.  One workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_residual_kernel(int H, float eps, float *__restrict__ r,
                                                               const float *__restrict__ y,
                                                               uint16_t *__restrict__ u) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    float *rr = r + row * H;
    const float *yy = y + row * H;
    float ss = 0.0f;
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        float4 a = *(const float4 *)(rr + i);
        const float4 b = *(const float4 *)(yy + i);
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
        *(float4 *)(rr + i) = a;
        ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
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
    hipLaunchKernelGGL(rmsnorm_residual_kernel, dim3(T), dim3(256), 0, s, H, eps, r, y, u);
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

}  // namespace moe
