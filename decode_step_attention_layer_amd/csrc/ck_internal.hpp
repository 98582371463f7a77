// ck_internal.hpp — argument structs and launchers shared between the kernel
// translation units and the C-ABI entry points (ck_api.cpp). Host-side only
// declarations plus the by-value kernel argument structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ck.h"
#include "ck_device.hpp"

namespace ck {

constexpr int kMaxSeqs = CK_MAX_SEQS;

// Token positions: host values copied into the kernel arguments, or (dev not
// null) a device array read by the kernels, so that a captured launch can be
// replayed for the next token. A device position outside [0, limit) reads as
// -1: that sequence then writes nothing to the cache and attends no token
// (its outputs are undefined), and nothing is accessed out of bounds.
struct Positions {
    int32_t p[kMaxSeqs];
    const int32_t *dev;
    int limit;
    __device__ __forceinline__ int get(int s) const {
        if (!dev) return p[s];
        const int v = dev[s];
        return (v >= 0 && v < limit) ? v : -1;
    }
};

// Cache view passed by value to kernels (mirrors ck_kv_cache).
struct CacheView {
    void *k;
    void *v;
    const int32_t *table;
    int kv_heads, head_dim, capacity, page_size, max_pages, num_pages;
    int dtype;                // CK_KV_*
    float k_scale, v_scale;   // fp8
    int window;               // 0 = every token, else the last `window` positions
    int ring;                 // contiguous ring: token t in slot t % capacity
};

// First token a sequence of L tokens attends under a window (0 = none).
__host__ __device__ __forceinline__ int window_start(int L, int window) {
    return (window > 0 && L > window) ? L - window : 0;
}

// Stores element idx of K (is_k) or V from an fp32 value, in the cache's type.
__device__ __forceinline__ void cache_put(const CacheView &c, bool is_k, long long idx, float x) {
    void *base = is_k ? c.k : c.v;
    if (c.dtype == CK_KV_BF16) {
        static_cast<uint16_t *>(base)[idx] = f32_to_bf16(x);
    } else if (c.dtype == CK_KV_FP8_E4M3) {
        static_cast<uint8_t *>(base)[idx] = f32_to_e4m3(x / (is_k ? c.k_scale : c.v_scale));
    } else {
        static_cast<float *>(base)[idx] = x;
    }
}

// Four consecutive elements (idx a multiple of 4) of a cache whose element
// type DT is known at compile time: the raw load, then the conversion to
// fp32 (split, so that loads can be issued ahead of their use).
template <int DT>
struct CacheRaw4 {
    typedef uint4 type;      // fp32: 16 bytes
};
template <>
struct CacheRaw4<CK_KV_BF16> {
    typedef uint2 type;      // 8 bytes
};
template <>
struct CacheRaw4<CK_KV_FP8_E4M3> {
    typedef uint32_t type;   // 4 bytes
};

template <int DT>
__device__ __forceinline__ typename CacheRaw4<DT>::type cache_raw4(const CacheView &c, bool is_k,
                                                                   long long idx) {
    typedef typename CacheRaw4<DT>::type R;
    const void *base = is_k ? c.k : c.v;
    if constexpr (DT == CK_KV_BF16)
        return *reinterpret_cast<const R *>(static_cast<const uint16_t *>(base) + idx);
    else if constexpr (DT == CK_KV_FP8_E4M3)
        return *reinterpret_cast<const R *>(static_cast<const uint8_t *>(base) + idx);
    else
        return *reinterpret_cast<const R *>(static_cast<const float *>(base) + idx);
}

template <int DT>
__device__ __forceinline__ typename CacheRaw4<DT>::type cache_raw4_zero() {
    if constexpr (DT == CK_KV_BF16) return make_uint2(0u, 0u);
    else if constexpr (DT == CK_KV_FP8_E4M3) return 0u;
    else return make_uint4(0u, 0u, 0u, 0u);
}

template <int DT>
__device__ __forceinline__ float4 cache_cvt4(const CacheView &c, bool is_k,
                                             typename CacheRaw4<DT>::type r) {
    if constexpr (DT == CK_KV_BF16) {
        return make_float4(bf16_to_f32(r.x & 0xFFFFu), bf16_to_f32(r.x >> 16),
                           bf16_to_f32(r.y & 0xFFFFu), bf16_to_f32(r.y >> 16));
    } else if constexpr (DT == CK_KV_FP8_E4M3) {
        // v_cvt_pk_f32_fp8 decodes OCP E4M3 on gfx950 (checked against the
        // format's definition over all 256 codes, NaN included)
        const float sc = is_k ? c.k_scale : c.v_scale;
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)r, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)r, true);
        return make_float4(lo[0] * sc, lo[1] * sc, hi[0] * sc, hi[1] * sc);
    } else {
        return make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                           __uint_as_float(r.w));
    }
}

// Element offset of (seq, kv head, token) in the K (or V) buffer, or -1 if the
// token's page is unmapped or out of range. Shared by the kernels.
__device__ __forceinline__ long long cache_row(const CacheView &c, int s, int g, int t) {
    if (c.page_size == 0) {
        const int slot = c.ring ? t % c.capacity : t;
        return (((long long)s * c.kv_heads + g) * c.capacity + slot) * (long long)c.head_dim;
    }
    int page = c.table[(long long)s * c.max_pages + t / c.page_size];
    if (page < 0 || page >= c.num_pages) return -1;
    return (((long long)page * c.kv_heads + g) * c.page_size + t % c.page_size) *
           (long long)c.head_dim;
}

// One GEMV output segment: rows [0, rows) of a weight matrix.
struct GemvSeg {
    const uint8_t *W;
    const float *bias;      // nullable
    const float *residual;  // nullable, [m][rows]
    float *y;               // [m][rows]
    int rows;
    int is_q5;              // 1: Q5_0 weights, 0: Q8_0 weights
    int wg_begin;           // first workgroup of this segment
    int pad;
};

struct GemvArgs {
    GemvSeg seg[3];
    int nseg;
    const uint8_t *xq;      // [m][K/32] Q8_0 blocks
    int K;
    int m;
    const uint32_t *ximg;   // nullable: the same blocks as an activation image (below)
};

// The batched matrix-core GEMV's LDS image of m tokens' Q8_0 activation
// blocks, written by the kernel that quantizes them so that the GEMV copies
// it with 16-byte loads instead of unpacking 34-byte blocks: the codes
// [nb][m][8 words] (block-major), then the scales [nb][16] as fp32 (the
// fp16 scale's value), zero for the token slots from m to 15. One buffer of
// ximage_bytes(m, nb) bytes, 16-byte aligned.
struct XImage {
    uint32_t *base;         // nullable: no image
    int m, nb;
};
__host__ __device__ __forceinline__ size_t ximage_bytes(int m, int nb) {
    return (size_t)nb * (32 * (size_t)m + 64);
}
// Whether the GEMV takes an image of m tokens x nb blocks (it loads at most
// five 16-byte pieces per thread of its 512 ahead of the weights).
__host__ __device__ __forceinline__ bool ximage_fits(int m, int nb) {
    return (size_t)nb * (2 * m + 4) <= 5 * 512;
}
// Element group `sub` (codes 4sub..4sub+3, packed) of block `blk` of token
// `tok`, and the block's scale on sub 0.
__device__ __forceinline__ void ximage_put(const XImage &xi, int tok, int blk, int sub,
                                           uint32_t packed, uint16_t dbits) {
    xi.base[((size_t)blk * xi.m + tok) * 8 + sub] = packed;
    if (sub == 0) {
        float *sc = reinterpret_cast<float *>(xi.base + (size_t)xi.m * xi.nb * 8);
        sc[blk * 16 + tok] = half_bits_to_float(dbits);
    }
}
// The zero scales of token slots m..15 of blocks [b0, b1), by one
// workgroup's threads.
__device__ __forceinline__ void ximage_zero_pads(const XImage &xi, int b0, int b1, int tid,
                                                 int nthreads) {
    float *sc = reinterpret_cast<float *>(xi.base + (size_t)xi.m * xi.nb * 8);
    for (int i = b0 * 16 + tid; i < b1 * 16; i += nthreads)
        if ((i & 15) >= xi.m) sc[i] = 0.0f;
}

// Launchers. Each returns hipSuccess or the launch error.
hipError_t launch_rmsnorm(const float *x, const float *gamma, float *y, int m, int D,
                          float eps, hipStream_t st);
hipError_t launch_quantize_q8_0(const float *x, uint8_t *y, long long nblocks, hipStream_t st);
hipError_t launch_rmsnorm_quant(const float *x, const float *gamma, float *xn, uint8_t *xq,
                                int m, int D, float eps, hipStream_t st, uint32_t *ximg = nullptr);
bool gemv_shape_supported(int K);
bool qkv_shape_supported(int D, int m);
hipError_t launch_qkv(const float *x, const float *gamma, float eps, int D, int H, int KV, int hd,
                      int m, const uint8_t *wq, const uint8_t *wk, const uint8_t *wv,
                      const float *bq, const float *bk, const float *bv, const float *cos_tab,
                      const float *sin_tab, const Positions &pos, const CacheView &c, float *q,
                      float *k, float *v, float *xn, uint8_t *xq, hipStream_t st,
                      unsigned *zero = nullptr, int nzero = 0, int zstride = 1);
hipError_t launch_gemv(const GemvArgs &a, hipStream_t st);
// Small-M GEMV on the int8 matrix cores (k_gemv_mfma.hip): batches of 4..16
// tokens; same arguments and results as launch_gemv.
bool gemv_mfma_supported(int K, int m);
hipError_t launch_gemv_mfma(GemvArgs a, hipStream_t st);
// The epilogue of a Q/K/V projection launch whose segments are q, k and v
// in that order: RoPE of q and k (rotate-half pairs, table row pos), then k
// and v appended to the cache at pos; a token with an invalid position keeps
// its unrotated q and k and appends nothing (as launch_rope_append).
struct QkvEpi {
    const float *cos_tab, *sin_tab;   // [rows][hd/2]
    Positions pos;
    CacheView c;
    int hd;
};
hipError_t launch_gemv_mfma_qkv(GemvArgs a, const QkvEpi &e, hipStream_t st);
hipError_t launch_rope(float *q, float *k, const float *cos_tab, const float *sin_tab,
                       const Positions &pos, int m, int H, int KV, int hd, hipStream_t st);
hipError_t launch_kv_append(const CacheView &c, const float *k, const float *v,
                            const Positions &pos, int m, hipStream_t st);
// zero/nzero/zstride (optional): words this launch clears (zero[i * zstride],
// i < nzero), the counters of the attention + merge + O launch that follows.
hipError_t launch_rope_append(float *q, float *k, const float *v, const float *cos_tab,
                              const float *sin_tab, const CacheView &c, const Positions &pos, int m,
                              int H, hipStream_t st, unsigned *zero = nullptr, int nzero = 0,
                              int zstride = 1);

// Attention geometry: tokens per chunk and chunks per (sequence, KV head).
struct AttnPlan {
    int chunk;
    int nchunks;
};
// Tokens per step of the attention kernel that runs a query group of G heads
// over a cache of type dtype (CK_KV_*), on the matrix cores if `matrix`;
// dtype < 0: whichever runs (a common multiple of their steps), for plans
// that another call must reproduce without knowing the cache.
int attn_step(int G, int dtype, bool matrix);
// Whether the attention launch of m sequences with query groups of G heads
// runs on the matrix cores: with no selection, groups over 4 heads attending
// an fp32 cache, and every group of a single sequence attending a bf16 or
// fp8 cache.
bool attn_matrix_path(int G, int dtype, int m, bool selection);
// The split of the attended tokens. An explicit chunk_req is used as given
// (every kernel masks the rows past a chunk); the automatic chunk is a whole
// number of `step`s sized for the kernel: with `matrix`, about one
// workgroup per compute unit, otherwise about two.
AttnPlan attn_plan(int KV, int G, int max_tokens, long long total_tokens, int chunk_req, int step,
                   bool matrix);
int attn_max_chunks(int KV, int G, int max_tokens, int chunk_req);
// Tokens attended over all sequences (host positions), under a window.
long long total_tokens(const Positions &p, int m, int window);
bool attn_shape_supported(int G, int hd);
bool attn_chunks_supported(int nchunks);
size_t attn_partials_bytes(int m, int H, int hd, int nchunks);
// The attention launch's work items: first[s] is sequence s's first item,
// first[m] (returned) the count. Host positions give each sequence exactly
// its chunks; device positions (or a selection, when `uniform`) give every
// sequence plan.nchunks items, those past its length returning at once.
int attn_first(const Positions &pos, int window, const AttnPlan &plan, int m, bool uniform,
               int *first);
// Sparse attention: per sequence, topk token positions (device, [m][topk],
// -1 = absent) replace the sequence's tokens; sink (device, [H], nullable)
// holds logits that join the softmax denominator only.
struct SparseSel {
    const int32_t *sel;
    int topk;
    const float *sink;
};
hipError_t launch_attn_partial(const float *q, const CacheView &c, const Positions &pos, int m,
                               int H, float scale, const AttnPlan &plan, void *partials,
                               hipStream_t st, const SparseSel *sp = nullptr);
// ximg (nullable, with out_q8): the output's Q8_0 blocks also as an
// activation image of m tokens x H*hd/32 blocks.
hipError_t launch_attn_merge(const void *partials, const Positions &pos, int window, int m,
                             int H, int KV, int hd, const AttnPlan &plan, float *out,
                             uint8_t *out_q8, hipStream_t st, const SparseSel *sp = nullptr,
                             uint32_t *ximg = nullptr);
hipError_t launch_attention(const float *q, const CacheView &c, const Positions &pos, float *out,
                            uint8_t *out_q8, int m, int H, float scale, const AttnPlan &plan,
                            void *partials, hipStream_t st, const SparseSel *sp = nullptr,
                            uint32_t *ximg = nullptr);

// Attention + merge + Q8_0 + O projection in one launch (k_ato.hip): the
// second launch of the two-launch layer. Its counters (ato_counter_words)
// must be zero when it starts: the launch before it clears them.
size_t ato_counter_words(int m, int KV);  // words of the counter region
int ato_counters(int m, int KV);          // counters in it, ato_counter_stride() words apart
int ato_counter_stride();
size_t ato_status_word(int m, int KV);    // word index of the status word
bool ato_supported(int H, int hd, int nchunks);
hipError_t launch_ato(const float *q, const CacheView &c, const Positions &pos, int m, int H,
                      float scale, const AttnPlan &plan, void *partials, float *attn_out,
                      uint8_t *aq, void *aqx, const uint8_t *wo, const float *bo,
                      const float *residual, float *out, int D, unsigned *cnt, hipStream_t st);

// A plain streaming read of `bytes` (a multiple of 16) by nwg workgroups
// (k_probe.hip); sink: nwg words, written only for an impossible value.
hipError_t launch_read_probe(const void *src, size_t bytes, unsigned *sink, int nwg,
                             hipStream_t st);

// Persistent decode step (k_step.hip): every layer of a step in one launch.
struct StepLayer {
    const uint8_t *wq, *wk, *wv, *wo;
    const float *bq, *bk, *bv, *bo, *gamma;
    float *kc, *vc;
    const int32_t *table;
};

struct StepLaunch {
    int L, D, H, KV, hd, m;
    float eps, scale;
    const float *cos_tab, *sin_tab;
    Positions pos;
    int capacity, page_size, max_pages, num_pages;
    AttnPlan plan;
    const float *x;
    float *out;
    float *xbuf, *q, *k, *v, *po, *pml, *attn, *xn;
    unsigned *aqx;
    uint8_t *aq, *xq;
    unsigned *cnt;
    int num_cus;
    StepLayer layers[CK_MAX_STEP_LAYERS];
};

bool step_supported(int D, int H, int KV, int hd, int m, int nchunks);
size_t step_counter_words(int L, int m, int KV);
hipError_t launch_step(const StepLaunch &sl, hipStream_t st);
int num_cus();

}  // namespace ck
