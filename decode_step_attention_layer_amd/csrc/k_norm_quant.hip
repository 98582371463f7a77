// k_norm_quant.hip — RMSNorm and Q8_0 activation quantization for gfx950.
//
// RMSNorm (C-Kernel-Engine "mega_fused_attention_decode_q5_0.c", MAIN KERNEL
// STEP 1): one workgroup per token, y = x * gamma / sqrt(mean(x^2) + eps).
// Q8_0 (the quantize_row_q8_0 call before each projection): one 32-element
// block per half-wave, bit-exact with the fp32 definition (see ck_device.hpp).
#include "ck_device.hpp"
#include "ck_gemv_common.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

constexpr int kNormThreads = 256;

// Sum of x^2 over D elements by the whole workgroup, returned to every thread.
__device__ float block_sumsq(const float *x, int D, float *red) {
    float s = 0.0f;
    for (int i = threadIdx.x; i < D; i += kNormThreads) s += x[i] * x[i];
    s = group_sum<32>(s);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[2 * wave] = s;
    if (lane == 32) red[2 * wave + 1] = s;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 2 * (kNormThreads / kWave); i++) t += red[i];
    return t;
}

__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(const float *__restrict__ x,
                                                          const float *__restrict__ gamma,
                                                          float *__restrict__ y, int D, float eps) {
    __shared__ float red[2 * kNormThreads / kWave];
    const float *xs = x + (size_t)blockIdx.x * D;
    float *ys = y + (size_t)blockIdx.x * D;
    float ss = block_sumsq(xs, D, red);
    float r = 1.0f / sqrtf(ss / (float)D + eps);
    for (int i = threadIdx.x; i < D; i += kNormThreads) ys[i] = xs[i] * r * gamma[i];
}

// Writes one Q8_0 block from the 32 lanes of a half-wave (lane j = element j).
__device__ __forceinline__ void store_q8_0_block(uint8_t *blk, int j, float x) {
    int code;
    uint16_t dbits;
    quantize_q8_0_half(x, code, dbits);
    blk[2 + j] = (uint8_t)(int8_t)code;
    if (j == 0) {
        blk[0] = (uint8_t)(dbits & 0xFF);
        blk[1] = (uint8_t)(dbits >> 8);
    }
}

__global__ __launch_bounds__(256) void k_quantize_q8_0(const float *__restrict__ x,
                                                       uint8_t *__restrict__ y,
                                                       long long nblocks) {
    const int lane = threadIdx.x & 63;
    const long long blk = ((long long)blockIdx.x * 256 + threadIdx.x) >> 5;
    const int j = lane & 31;
    const bool ok = blk < nblocks;
    float v = ok ? x[blk * kQK + j] : 0.0f;
    int code;
    uint16_t dbits;
    quantize_q8_0_half(v, code, dbits);
    if (ok) {
        uint8_t *b = y + blk * kQ8Bytes;
        b[2 + j] = (uint8_t)(int8_t)code;
        if (j == 0) {
            b[0] = (uint8_t)(dbits & 0xFF);
            b[1] = (uint8_t)(dbits >> 8);
        }
    }
}

// RMSNorm and quantization of one token per workgroup (the layer's fused
// variant when its single-kernel first half does not fit): the normalized row
// is written to xn and its Q8_0 blocks to xq, with the same row function as
// the fused first half.
// With an activation image (xi.base set) the blocks also go there, and
// workgroup 0 writes its zero scales.
__global__ __launch_bounds__(kGemvThreads) void k_rmsnorm_quant(const float *__restrict__ x,
                                                                const float *__restrict__ gamma,
                                                                float *__restrict__ xn,
                                                                uint8_t *__restrict__ xq, int D,
                                                                float eps, XImage xi) {
    __shared__ float red[2 * kGemvThreads / kWave];
    const size_t s = blockIdx.x;
    const int nb = D / kQK;
    if (xi.base && s == 0) ximage_zero_pads(xi, 0, nb, threadIdx.x, kGemvThreads);
    norm_quant_row(x + s * D, gamma, D, eps, red,
                   [&](int c, float4 v, uint32_t packed, uint16_t dbits, int) {
                       reinterpret_cast<float4 *>(xn + s * D)[c] = v;
                       uint8_t *blk = xq + (s * nb + (c >> 3)) * kQ8Bytes;
                       uint16_t *dst = reinterpret_cast<uint16_t *>(blk + 2 + 4 * (c & 7));
                       dst[0] = (uint16_t)(packed & 0xFFFF);
                       dst[1] = (uint16_t)(packed >> 16);
                       if ((c & 7) == 0) *reinterpret_cast<uint16_t *>(blk) = dbits;
                       if (xi.base) ximage_put(xi, (int)s, c >> 3, c & 7, packed, dbits);
                   });
}

}  // namespace

hipError_t launch_rmsnorm(const float *x, const float *gamma, float *y, int m, int D, float eps,
                          hipStream_t st) {
    hipLaunchKernelGGL(k_rmsnorm, dim3(m), dim3(kNormThreads), 0, st, x, gamma, y, D, eps);
    return hipGetLastError();
}

hipError_t launch_quantize_q8_0(const float *x, uint8_t *y, long long nblocks, hipStream_t st) {
    long long grid = (nblocks + 7) / 8;
    hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)grid), dim3(256), 0, st, x, y, nblocks);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_quant(const float *x, const float *gamma, float *xn, uint8_t *xq, int m,
                                int D, float eps, hipStream_t st, uint32_t *ximg) {
    const XImage xi{ximg, m, D / kQK};
    hipLaunchKernelGGL(k_rmsnorm_quant, dim3(m), dim3(kGemvThreads), 0, st, x, gamma, xn, xq, D,
                       eps, xi);
    return hipGetLastError();
}

}  // namespace ck
