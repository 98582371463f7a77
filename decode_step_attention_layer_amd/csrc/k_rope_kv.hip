// k_rope_kv.hip — RoPE and KV-cache append for gfx950.
//
// RoPE (C-Kernel-Engine "mega_fused_attention_decode_q5_0.c", helper "RoPE
// application (inline)"): rotate-half pairing, element i with element
// i + hd/2 of every q and k head, by row `pos` of the cos/sin tables.
// KV append (MAIN KERNEL STEP 6; paged addressing as the block tables of the
// metrale "prefill_attn_a.rs" paged decode launchers).
#include "ck_device.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

__global__ __launch_bounds__(256) void k_rope(float *__restrict__ q, float *__restrict__ k,
                                              const float *__restrict__ cos_tab,
                                              const float *__restrict__ sin_tab, Positions pos,
                                              int H, int KV, int hd) {
    const int s = blockIdx.y;
    const int half = hd >> 1;
    const int nq = q ? H * half : 0;
    const int nk = k ? KV * half : 0;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nq + nk) return;
    float *base;
    int pair;
    if (i < nq) {
        base = q + (size_t)s * H * hd;
        pair = i;
    } else {
        base = k + (size_t)s * KV * hd;
        pair = i - nq;
    }
    const int head = pair / half, d = pair % half;
    float *x = base + (size_t)head * hd;
    const int p = pos.get(s);
    if (p < 0) return;
    const float c = cos_tab[(size_t)p * half + d];
    const float sn = sin_tab[(size_t)p * half + d];
    const float a = x[d], b = x[d + half];
    x[d] = a * c - b * sn;
    x[d + half] = a * sn + b * c;
}

__global__ __launch_bounds__(256) void k_kv_append(CacheView c, const float *__restrict__ k,
                                                   const float *__restrict__ v, Positions pos) {
    const int s = blockIdx.y;
    const int n = c.kv_heads * c.head_dim;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int g = i / c.head_dim, d = i % c.head_dim;
    const int p = pos.get(s);
    if (p < 0) return;
    long long off = cache_row(c, s, g, p);
    if (off < 0) return;  // unmapped page: nothing is written, attention reports NaN
    cache_put(c, true, off + d, k[(size_t)s * n + i]);
    cache_put(c, false, off + d, v[(size_t)s * n + i]);
}

// RoPE of q and k plus the append of (rotated k, v) at the token's position,
// one launch: threads [0, H*hd/2) rotate q pairs; the next KV*hd/2 rotate k
// pairs and store both halves into the k buffer and the cache; the last
// KV*hd copy v into the cache.
__global__ __launch_bounds__(256) void k_rope_append(float *__restrict__ q, float *__restrict__ k,
                                                     const float *__restrict__ v,
                                                     const float *__restrict__ cos_tab,
                                                     const float *__restrict__ sin_tab,
                                                     CacheView c, Positions pos, int H,
                                                     unsigned *zero, int nzero, int zstride) {
    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < nzero; i += blockDim.x)
            __hip_atomic_store(zero + (size_t)i * zstride, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
    const int s = blockIdx.y;
    const int KV = c.kv_heads, hd = c.head_dim, half = hd >> 1;
    const int nq = H * half, nk = KV * half, nv = KV * hd;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int p = pos.get(s);
    if (p < 0) return;
    if (i < nq + nk) {
        const bool isq = i < nq;
        const int pair = isq ? i : i - nq;
        const int head = pair / half, d = pair % half;
        float *x = (isq ? q + (size_t)s * H * hd : k + (size_t)s * KV * hd) + (size_t)head * hd;
        const float cs = cos_tab[(size_t)p * half + d];
        const float sn = sin_tab[(size_t)p * half + d];
        const float a = x[d], b = x[d + half];
        const float ra = a * cs - b * sn, rb = a * sn + b * cs;
        x[d] = ra;
        x[d + half] = rb;
        if (!isq) {
            long long off = cache_row(c, s, head, p);
            if (off >= 0) {
                cache_put(c, true, off + d, ra);
                cache_put(c, true, off + d + half, rb);
            }
        }
    } else if (i < nq + nk + nv) {
        const int e = i - nq - nk;
        const int head = e / hd, d = e % hd;
        long long off = cache_row(c, s, head, p);
        if (off >= 0) cache_put(c, false, off + d, v[(size_t)s * nv + e]);
    }
}

}  // namespace

hipError_t launch_rope_append(float *q, float *k, const float *v, const float *cos_tab,
                              const float *sin_tab, const CacheView &c, const Positions &pos, int m,
                              int H, hipStream_t st, unsigned *zero, int nzero, int zstride) {
    const int n = H * (c.head_dim / 2) + c.kv_heads * (c.head_dim / 2) + c.kv_heads * c.head_dim;
    hipLaunchKernelGGL(k_rope_append, dim3((n + 255) / 256, m), dim3(256), 0, st, q, k, v, cos_tab,
                       sin_tab, c, pos, H, zero, zero ? nzero : 0, zstride);
    return hipGetLastError();
}

hipError_t launch_rope(float *q, float *k, const float *cos_tab, const float *sin_tab,
                       const Positions &pos, int m, int H, int KV, int hd, hipStream_t st) {
    int n = (q ? H : 0) * (hd / 2) + (k ? KV : 0) * (hd / 2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_rope, dim3((n + 255) / 256, m), dim3(256), 0, st, q, k, cos_tab, sin_tab,
                       pos, H, KV, hd);
    return hipGetLastError();
}

hipError_t launch_kv_append(const CacheView &c, const float *k, const float *v,
                            const Positions &pos, int m, hipStream_t st) {
    int n = c.kv_heads * c.head_dim;
    hipLaunchKernelGGL(k_kv_append, dim3((n + 255) / 256, m), dim3(256), 0, st, c, k, v, pos);
    return hipGetLastError();
}

}  // namespace ck
