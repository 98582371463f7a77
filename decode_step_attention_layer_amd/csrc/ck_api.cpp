// ck_api.cpp — the C ABI of libck.so (declared in include/ck.h): argument
// validation on the host, workspace layout, and the launch sequence of the
// decode layer (C-Kernel-Engine "mega_fused_attention_decode_q5_0.c", MAIN
// KERNEL steps 1-8). Nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/ck.h"
#include "ck_gemv_common.hpp"
#include "ck_internal.hpp"

using namespace ck;

namespace {

bool al(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int hip_rc(hipError_t e) { return e == hipSuccess ? CK_OK : CK_EHIP; }

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }


// Validates the cache descriptor and builds the kernel view.
int cache_view(const ck_kv_cache *kv, CacheView *out) {
    if (!kv || !kv->k || !kv->v || kv->kv_heads <= 0 || kv->head_dim <= 0) return CK_EINVAL;
    if (kv->dtype != CK_KV_F32 && kv->dtype != CK_KV_BF16 && kv->dtype != CK_KV_FP8_E4M3)
        return CK_EINVAL;
    if (kv->dtype == CK_KV_FP8_E4M3 &&
        !(kv->k_scale > 0.0f && kv->k_scale < INFINITY && kv->v_scale > 0.0f &&
          kv->v_scale < INFINITY))
        return CK_EINVAL;
    if (!al(kv->k, 16) || !al(kv->v, 16) || kv->head_dim % 4) return CK_EINVAL;
    if (kv->page_size < 0 || kv->window < 0 || (kv->ring != 0 && kv->ring != 1)) return CK_EINVAL;
    if (kv->page_size == 0) {
        if (kv->capacity <= 0) return CK_EINVAL;
        // a ring holds the last `capacity` tokens: the window may not reach further
        if (kv->ring && (kv->window < 1 || kv->window > kv->capacity)) return CK_EINVAL;
    } else {
        if (kv->ring) return CK_EINVAL;
        if (!kv->page_table || kv->max_pages_per_seq <= 0 || kv->num_pages <= 0) return CK_EINVAL;
        if (!al(kv->page_table, 4)) return CK_EINVAL;
    }
    out->k = kv->k;
    out->v = kv->v;
    out->table = kv->page_table;
    out->kv_heads = kv->kv_heads;
    out->head_dim = kv->head_dim;
    out->capacity = kv->capacity;
    out->page_size = kv->page_size;
    out->max_pages = kv->max_pages_per_seq;
    out->num_pages = kv->num_pages;
    out->dtype = kv->dtype;
    out->k_scale = kv->k_scale;
    out->v_scale = kv->v_scale;
    out->window = kv->window;
    out->ring = kv->ring;
    return CK_OK;
}

// Token capacity of one sequence of the cache (positions must stay below); a
// ring has no bound of its own.
long long cache_tokens(const ck_kv_cache *kv) {
    if (kv->page_size == 0 && kv->ring) return 1LL << 30;
    return kv->page_size == 0 ? (long long)kv->capacity
                              : (long long)kv->page_size * kv->max_pages_per_seq;
}

// Most tokens one sequence attends when the longest has max_len tokens.
int attended(int max_len, int window) { return max_len - window_start(max_len, window); }

int read_positions(const int32_t *pos_host, int m, long long limit, Positions *p, int *max_tokens) {
    if (!pos_host || m < 1 || m > CK_MAX_SEQS) return CK_EINVAL;
    int mx = 0;
    memset(p, 0, sizeof(*p));
    p->dev = nullptr;
    p->limit = (int)(limit < (1LL << 30) ? limit : (1LL << 30));
    for (int s = 0; s < m; s++) {
        if (pos_host[s] < 0 || pos_host[s] >= limit) return CK_EINVAL;
        p->p[s] = pos_host[s];
        if (pos_host[s] + 1 > mx) mx = pos_host[s] + 1;
    }
    *max_tokens = mx;
    return CK_OK;
}

}  // namespace

namespace ck {
long long total_tokens(const Positions &p, int m, int window) {
    long long t = 0;
    for (int s = 0; s < m; s++) t += attended(p.p[s] + 1, window);
    return t;
}
}  // namespace ck

namespace {

// Where a layer or step takes its positions from: a host array (validated
// here) or a device array read by the kernels (bounded by max_ctx).
struct PosIn {
    const int32_t *host;
    const int32_t *dev;
    int max_ctx;
};

int resolve_positions(const PosIn &in, int m, long long limit, Positions *p, int *mx,
                      long long *total) {
    if (in.host) {
        const int rc = read_positions(in.host, m, limit, p, mx);
        if (rc) return rc;
        *total = total_tokens(*p, m, 0);
        return CK_OK;
    }
    if (!in.dev || in.max_ctx < 1 || m < 1 || m > CK_MAX_SEQS || !al(in.dev, 4)) return CK_EINVAL;
    memset(p, 0, sizeof(*p));
    const long long lim = in.max_ctx < limit ? in.max_ctx : limit;
    p->dev = in.dev;
    p->limit = (int)lim;
    *mx = (int)lim;
    *total = (long long)m * lim;
    return CK_OK;
}

// Batches of 4 or more tokens use the matrix-core GEMV where it applies; the
// vector GEMV serves everything else.
hipError_t gemv_any(const GemvArgs &g, hipStream_t st) {
    return gemv_mfma_supported(g.K, g.m) ? launch_gemv_mfma(g, st) : launch_gemv(g, st);
}

struct WsLayout {
    size_t xn, xq, q, k, v, attn, aq, aqx, xqi, aqi, cnt, part, total;
};

WsLayout ws_layout(const ck_layer_desc *d, int max_ctx) {
    const size_t m = d->m, D = d->D, HD = (size_t)d->H * d->head_dim,
                 KD = (size_t)d->KV * d->head_dim;
    WsLayout w;
    size_t o = 0;
    w.xn = o; o = up256(o + sizeof(float) * m * D);
    w.xq = o; o = up256(o + m * (D / CK_QK) * CK_Q8_0_BYTES);
    w.q = o; o = up256(o + sizeof(float) * m * HD);
    w.k = o; o = up256(o + sizeof(float) * m * KD);
    w.v = o; o = up256(o + sizeof(float) * m * KD);
    w.attn = o; o = up256(o + sizeof(float) * m * HD);
    w.aq = o; o = up256(o + m * (HD / CK_QK) * CK_Q8_0_BYTES);
    // the two-launch variant: the staged Q8_0 blocks of the attention output
    // and the counters of its second launch (the status word last)
    w.aqx = o; o = up256(o + m * (HD / CK_QK) * sizeof(XBlock));
    // the batched projections' activation images of xq and aq
    w.xqi = o; o = up256(o + ximage_bytes((int)m, (int)(D / CK_QK)));
    w.aqi = o; o = up256(o + ximage_bytes((int)m, (int)(HD / CK_QK)));
    w.cnt = o; o = up256(o + sizeof(unsigned) * ato_counter_words(d->m, d->KV));
    const int maxc = attn_max_chunks(d->KV, d->H / d->KV, max_ctx, d->attn_chunk);
    w.part = o; o = up256(o + attn_partials_bytes(d->m, d->H, d->head_dim, maxc));
    w.total = o;
    return w;
}

int check_desc(const ck_layer_desc *d) {
    if (!d) return CK_EINVAL;
    if (d->D <= 0 || d->H <= 0 || d->KV <= 0 || d->head_dim <= 0 || d->m < 1 || d->m > CK_MAX_SEQS)
        return CK_EINVAL;
    if (d->D % CK_QK || (d->H * d->head_dim) % CK_QK || d->head_dim % 2 || d->H % d->KV)
        return CK_EINVAL;
    if (d->variant != CK_VARIANT_CHAIN && d->variant != CK_VARIANT_FUSED &&
        d->variant != CK_VARIANT_PERSISTENT && d->variant != CK_VARIANT_TWO_LAUNCH)
        return CK_EINVAL;
    if (d->attn_chunk < 0 || !(d->eps >= 0.0f)) return CK_EINVAL;
    if (!attn_shape_supported(d->H / d->KV, d->head_dim)) return CK_EUNSUPPORTED;
    if (!gemv_shape_supported(d->D) || !gemv_shape_supported(d->H * d->head_dim))
        return CK_EUNSUPPORTED;
    return CK_OK;
}

int gemv_common(const void *W, const void *xq, const float *bias, const float *residual, float *y,
                int rows, int K, int m, void *stream, int is_q5) {
    if (!W || !xq || !y || rows <= 0 || K <= 0 || K % CK_QK || m < 1) return CK_EINVAL;
    if (!al(W, 4) || !al(xq, 2) || !al(y, 4) || (bias && !al(bias, 4)) ||
        (residual && !al(residual, 4)))
        return CK_EINVAL;
    if (!gemv_shape_supported(K)) return CK_EUNSUPPORTED;
    GemvArgs a;
    memset(&a, 0, sizeof(a));
    a.nseg = 1;
    a.seg[0].W = static_cast<const uint8_t *>(W);
    a.seg[0].bias = bias;
    a.seg[0].residual = residual;
    a.seg[0].y = y;
    a.seg[0].rows = rows;
    a.seg[0].is_q5 = is_q5;
    a.xq = static_cast<const uint8_t *>(xq);
    a.K = K;
    a.m = m;
    return hip_rc(gemv_any(a, (hipStream_t)stream));
}

// Workspace of a whole step: the ping-pong layer outputs, then either the
// persistent kernel's buffers or one ck_decode_layer workspace.
struct StepWs {
    size_t xbuf, xn, xq, q, k, v, attn, aqx, aq, po, pml, cnt, layer, total;
    int maxc;
};

StepWs step_layout(const ck_layer_desc *d, int layers, int max_ctx) {
    const size_t m = d->m, D = d->D, HD = (size_t)d->H * d->head_dim,
                 KD = (size_t)d->KV * d->head_dim;
    StepWs w;
    memset(&w, 0, sizeof(w));
    size_t o = 0;
    w.xbuf = o; o = up256(o + sizeof(float) * 2 * m * D);
    w.maxc = attn_max_chunks(d->KV, d->H / d->KV, max_ctx, d->attn_chunk);
    if (d->variant == CK_VARIANT_PERSISTENT) {
        // intermediates (offsets independent of the layer count and the
        // context), then the counters (the status word's offset does not
        // depend on the context), then the partials
        w.xn = o; o = up256(o + sizeof(float) * m * D);
        w.xq = o; o = up256(o + m * (D / CK_QK) * CK_Q8_0_BYTES);
        w.q = o; o = up256(o + sizeof(float) * m * HD);
        w.k = o; o = up256(o + sizeof(float) * m * KD);
        w.v = o; o = up256(o + sizeof(float) * m * KD);
        w.attn = o; o = up256(o + sizeof(float) * m * HD);
        w.aqx = o; o = up256(o + sizeof(unsigned) * 10 * m * (HD / CK_QK));
        w.aq = o; o = up256(o + m * (HD / CK_QK) * CK_Q8_0_BYTES);
        w.cnt = o; o = up256(o + sizeof(unsigned) * step_counter_words(layers, d->m, d->KV));
        w.po = o; o = up256(o + sizeof(float) * m * d->H * (size_t)w.maxc * d->head_dim);
        w.pml = o; o = up256(o + sizeof(float) * m * d->H * (size_t)w.maxc * 2);
    } else {
        w.layer = o; o = up256(o + ws_layout(d, max_ctx).total);
    }
    w.total = o;
    return w;
}

}  // namespace

extern "C" {

const char *ck_strerror(int code) {
    switch (code) {
        case CK_OK: return "ok";
        case CK_EINVAL: return "invalid argument";
        case CK_ENOSPC: return "workspace too small";
        case CK_EUNSUPPORTED: return "shape not supported";
        case CK_EHIP: return "HIP runtime error";
    }
    return "unknown error";
}

int ck_version(void) { return (0 << 16) | 2; }

int ck_read_probe(const void *src, size_t bytes, void *sink, void *stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 || !al(src, 16) || !al(sink, 4))
        return CK_EINVAL;
    // a few workgroups per compute unit, each over one contiguous slice
    const int nwg = 4 * num_cus();
    return hip_rc(launch_read_probe(src, bytes, static_cast<unsigned *>(sink), nwg,
                                    (hipStream_t)stream));
}

int ck_rmsnorm(const float *x, const float *gamma, float *y, int m, int D, float eps, void *stream) {
    if (!x || !gamma || !y || m < 1 || D <= 0 || !(eps >= 0.0f)) return CK_EINVAL;
    if (!al(x, 4) || !al(gamma, 4) || !al(y, 4)) return CK_EINVAL;
    return hip_rc(launch_rmsnorm(x, gamma, y, m, D, eps, (hipStream_t)stream));
}

int ck_quantize_q8_0(const float *x, void *y, int m, int K, void *stream) {
    if (!x || !y || m < 1 || K <= 0 || K % CK_QK) return CK_EINVAL;
    if (!al(x, 4) || !al(y, 2)) return CK_EINVAL;
    return hip_rc(launch_quantize_q8_0(x, static_cast<uint8_t *>(y), (long long)m * (K / CK_QK),
                                       (hipStream_t)stream));
}

int ck_gemv_q5_0_q8_0(const void *W, const void *xq, const float *bias, const float *residual,
                      float *y, int rows, int K, int m, void *stream) {
    return gemv_common(W, xq, bias, residual, y, rows, K, m, stream, 1);
}

int ck_gemv_q8_0_q8_0(const void *W, const void *xq, const float *bias, const float *residual,
                      float *y, int rows, int K, int m, void *stream) {
    return gemv_common(W, xq, bias, residual, y, rows, K, m, stream, 0);
}

int ck_rope(float *q, float *k, const float *cos_tab, const float *sin_tab, int tab_rows,
            const int32_t *pos_host, int m, int H, int KV, int hd, void *stream) {
    if ((!q && !k) || !cos_tab || !sin_tab || tab_rows <= 0 || hd <= 0 || hd % 2) return CK_EINVAL;
    if ((q && H <= 0) || (k && KV <= 0)) return CK_EINVAL;
    Positions p;
    int mx;
    int rc = read_positions(pos_host, m, tab_rows, &p, &mx);
    if (rc) return rc;
    return hip_rc(launch_rope(q, k, cos_tab, sin_tab, p, m, q ? H : 0, k ? KV : 0, hd,
                              (hipStream_t)stream));
}

int ck_kv_append(const ck_kv_cache *kv, const float *k, const float *v, const int32_t *pos_host,
                 int m, void *stream) {
    CacheView c;
    int rc = cache_view(kv, &c);
    if (rc) return rc;
    if (!k || !v) return CK_EINVAL;
    Positions p;
    int mx;
    rc = read_positions(pos_host, m, cache_tokens(kv), &p, &mx);
    if (rc) return rc;
    return hip_rc(launch_kv_append(c, k, v, p, m, (hipStream_t)stream));
}

size_t ck_attn_workspace_size(int m, int H, int KV, int hd, int max_tokens, int chunk) {
    if (m < 1 || H <= 0 || KV <= 0 || H % KV || hd <= 0 || max_tokens < 1 || chunk < 0) return 0;
    return attn_partials_bytes(m, H, hd, attn_max_chunks(KV, H / KV, max_tokens, chunk));
}

int ck_attn_decode_gqa(const float *q, const ck_kv_cache *kv, const int32_t *pos_host, float *out,
                       int m, int H, float scale, int chunk, void *ws, size_t ws_bytes,
                       void *stream) {
    CacheView c;
    int rc = cache_view(kv, &c);
    if (rc) return rc;
    if (!q || !out || !ws || H <= 0 || chunk < 0 || H % c.kv_heads) return CK_EINVAL;
    if (!al(q, 16) || !al(out, 4) || !al(ws, 16)) return CK_EINVAL;
    if (!attn_shape_supported(H / c.kv_heads, c.head_dim)) return CK_EUNSUPPORTED;
    Positions p;
    int mx;
    rc = read_positions(pos_host, m, cache_tokens(kv), &p, &mx);
    if (rc) return rc;
    const int G = H / c.kv_heads;
    const bool matrix = attn_matrix_path(G, c.dtype, m, false);
    AttnPlan pl = attn_plan(c.kv_heads, G, attended(mx, c.window), total_tokens(p, m, c.window),
                            chunk, attn_step(G, c.dtype, matrix), matrix);
    if (!attn_chunks_supported(pl.nchunks)) return CK_EUNSUPPORTED;
    if (ws_bytes < attn_partials_bytes(m, H, c.head_dim, pl.nchunks)) return CK_ENOSPC;
    return hip_rc(launch_attention(q, c, p, out, nullptr, m, H, scale, pl, ws, (hipStream_t)stream));
}

int ck_attn_partial(const float *q, const ck_kv_cache *kv, const int32_t *pos_host, int m, int H,
                    float scale, int chunk, void *partials, size_t bytes, void *stream) {
    CacheView c;
    int rc = cache_view(kv, &c);
    if (rc) return rc;
    if (!q || !partials || H <= 0 || chunk < 0 || H % c.kv_heads) return CK_EINVAL;
    if (!al(q, 16) || !al(partials, 16)) return CK_EINVAL;
    if (!attn_shape_supported(H / c.kv_heads, c.head_dim)) return CK_EUNSUPPORTED;
    Positions p;
    int mx;
    rc = read_positions(pos_host, m, cache_tokens(kv), &p, &mx);
    if (rc) return rc;
    // the merge reproduces this plan without the cache type
    AttnPlan pl = attn_plan(c.kv_heads, H / c.kv_heads, attended(mx, c.window),
                            total_tokens(p, m, c.window), chunk, attn_step(H / c.kv_heads, -1, false),
                            false);
    if (!attn_chunks_supported(pl.nchunks)) return CK_EUNSUPPORTED;
    if (bytes < attn_partials_bytes(m, H, c.head_dim, pl.nchunks)) return CK_ENOSPC;
    return hip_rc(launch_attn_partial(q, c, p, m, H, scale, pl, partials, (hipStream_t)stream));
}

int ck_attn_merge(const void *partials, size_t bytes, const int32_t *pos_host, int m, int H,
                  int KV, int hd, int chunk, int window, float *out, void *out_q8,
                  void *stream) {
    if (!partials || !out || H <= 0 || KV <= 0 || H % KV || chunk < 0 || window < 0)
        return CK_EINVAL;
    if (!al(partials, 16) || !al(out, 16) || (out_q8 && !al(out_q8, 2))) return CK_EINVAL;
    if (!attn_shape_supported(H / KV, hd)) return CK_EUNSUPPORTED;
    Positions p;
    int mx;
    int rc = read_positions(pos_host, m, 1LL << 30, &p, &mx);
    if (rc) return rc;
    AttnPlan pl = attn_plan(KV, H / KV, attended(mx, window), total_tokens(p, m, window), chunk,
                            attn_step(H / KV, -1, false), false);
    if (!attn_chunks_supported(pl.nchunks)) return CK_EUNSUPPORTED;
    if (bytes < attn_partials_bytes(m, H, hd, pl.nchunks)) return CK_ENOSPC;
    return hip_rc(launch_attn_merge(partials, p, window, m, H, KV, hd, pl, out,
                                    static_cast<uint8_t *>(out_q8), (hipStream_t)stream));
}

int ck_attn_sparse(const float *q, const ck_kv_cache *kv, const int32_t *pos_host,
                   const int32_t *sel, int topk, const float *sink, float *out, int m, int H,
                   float scale, int chunk, void *ws, size_t ws_bytes, void *stream) {
    CacheView c;
    int rc = cache_view(kv, &c);
    if (rc) return rc;
    if (!q || !out || !ws || !sel || topk < 1 || H <= 0 || chunk < 0 || H % c.kv_heads)
        return CK_EINVAL;
    if (!al(q, 16) || !al(out, 4) || !al(ws, 16) || !al(sel, 4) || (sink && !al(sink, 4)))
        return CK_EINVAL;
    if (!attn_shape_supported(H / c.kv_heads, c.head_dim)) return CK_EUNSUPPORTED;
    Positions p;
    int mx;
    rc = read_positions(pos_host, m, cache_tokens(kv), &p, &mx);
    if (rc) return rc;
    const AttnPlan pl = attn_plan(c.kv_heads, H / c.kv_heads, topk, (long long)m * topk, chunk,
                                  attn_step(H / c.kv_heads, c.dtype, false), false);
    if (!attn_chunks_supported(pl.nchunks)) return CK_EUNSUPPORTED;
    if (ws_bytes < attn_partials_bytes(m, H, c.head_dim, pl.nchunks)) return CK_ENOSPC;
    const SparseSel sp{sel, topk, sink};
    return hip_rc(launch_attention(q, c, p, out, nullptr, m, H, scale, pl, ws, (hipStream_t)stream,
                                   &sp));
}

size_t ck_decode_step_workspace_size(const ck_layer_desc *desc, int layers, int max_ctx) {
    if (check_desc(desc) != CK_OK || max_ctx < 1 || layers < 1 || layers > CK_MAX_STEP_LAYERS)
        return 0;
    return step_layout(desc, layers, max_ctx).total;
}

long ck_decode_step_status_offset(const ck_layer_desc *desc, int layers) {
    if (check_desc(desc) != CK_OK || layers < 1 || layers > CK_MAX_STEP_LAYERS ||
        desc->variant != CK_VARIANT_PERSISTENT)
        return -1;
    StepWs w = step_layout(desc, layers, 1);
    return (long)(w.cnt + sizeof(unsigned) * (step_counter_words(layers, desc->m, desc->KV) - 1));
}

}  // extern "C"

namespace {

// phases: 1 = steps 1-6 (RMSNorm through the KV append; q, k, v left in the
// workspace), 2 = steps 7-8 (attention through the O projection, from them),
// 3 = the whole layer.
int decode_layer_impl(const ck_layer_desc *desc, const ck_layer_weights *w, const ck_kv_cache *kv,
                      const float *x, const float *residual, const PosIn &pin, float *out,
                      void *ws, size_t ws_bytes, void *stream, const SparseSel *sp = nullptr,
                      int phases = 3);

// The attention split of the persistent step: fp32 caches without a window,
// the vector kernel's step.
AttnPlan persistent_attn_plan(const ck_layer_desc &d, int mx, long long total) {
    const int G = d.H / d.KV;
    return attn_plan(d.KV, G, mx, total, d.attn_chunk, attn_step(G, CK_KV_F32, false), false);
}

int decode_step_impl(const ck_layer_desc *desc, const ck_layer_weights *w, const ck_kv_cache *kv,
                     int layers, const float *x, const PosIn &pin, float *out, void *ws,
                     size_t ws_bytes, void *stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    const ck_layer_desc &d = *desc;
    if (!w || !kv || layers < 1 || layers > CK_MAX_STEP_LAYERS) return CK_EINVAL;
    if (!x || !out || !ws || x == out || !al(x, 16) || !al(out, 16) || !al(ws, 256))
        return CK_EINVAL;
    CacheView c0;
    rc = cache_view(&kv[0], &c0);
    if (rc) return rc;
    if (c0.kv_heads != d.KV || c0.head_dim != d.head_dim) return CK_EINVAL;
    for (int l = 0; l < layers; l++) {
        const ck_layer_weights &wl = w[l];
        if (!wl.wq || !wl.wk || !wl.wv || !wl.wo || !wl.gamma) return CK_EINVAL;
        if (!al(wl.wq, 4) || !al(wl.wk, 4) || !al(wl.wv, 4) || !al(wl.wo, 4) || !al(wl.gamma, 16))
            return CK_EINVAL;
        CacheView cl;
        rc = cache_view(&kv[l], &cl);
        if (rc) return rc;
        if (cl.kv_heads != c0.kv_heads || cl.head_dim != c0.head_dim ||
            cl.capacity != c0.capacity || cl.page_size != c0.page_size ||
            cl.max_pages != c0.max_pages || cl.num_pages != c0.num_pages)
            return CK_EINVAL;
    }
    if (!w[0].rope_cos || !w[0].rope_sin) return CK_EINVAL;
    Positions p;
    int mx;
    long long total;
    long long limit = w[0].rope_rows;
    for (int l = 0; l < layers; l++)
        if (cache_tokens(&kv[l]) < limit) limit = cache_tokens(&kv[l]);
    rc = resolve_positions(pin, d.m, limit, &p, &mx, &total);
    if (rc) return rc;
    StepWs L = step_layout(desc, layers, mx);
    const AttnPlan plan = persistent_attn_plan(d, mx, total);
    if (ws_bytes < L.total) return CK_ENOSPC;
    hipStream_t st = (hipStream_t)stream;
    uint8_t *base = static_cast<uint8_t *>(ws);
    float *xbuf = reinterpret_cast<float *>(base + L.xbuf);
    const size_t md = (size_t)d.m * d.D;

    if (d.variant != CK_VARIANT_PERSISTENT) {
        const float *cur = x;
        for (int l = 0; l < layers; l++) {
            float *dst = (l == layers - 1) ? out : xbuf + (size_t)(l & 1) * md;
            ck_layer_weights wl = w[l];
            wl.rope_cos = w[0].rope_cos;
            wl.rope_sin = w[0].rope_sin;
            wl.rope_rows = w[0].rope_rows;
            rc = decode_layer_impl(desc, &wl, &kv[l], cur, cur, pin, dst, base + L.layer,
                                   ws_bytes - L.layer, stream);
            if (rc) return rc;
            cur = dst;
        }
        return CK_OK;
    }

    if (!step_supported(d.D, d.H, d.KV, d.head_dim, d.m, plan.nchunks)) return CK_EUNSUPPORTED;
    // fp32 caches without window or ring only
    for (int l = 0; l < layers; l++)
        if (kv[l].dtype != CK_KV_F32 || kv[l].window != 0 || kv[l].ring) return CK_EUNSUPPORTED;
    StepLaunch sl;
    memset(&sl, 0, sizeof(sl));
    sl.L = layers;
    sl.D = d.D;
    sl.H = d.H;
    sl.KV = d.KV;
    sl.hd = d.head_dim;
    sl.m = d.m;
    sl.eps = d.eps;
    sl.scale = 1.0f / sqrtf((float)d.head_dim);
    sl.cos_tab = w[0].rope_cos;
    sl.sin_tab = w[0].rope_sin;
    sl.pos = p;
    sl.capacity = c0.capacity;
    sl.page_size = c0.page_size;
    sl.max_pages = c0.max_pages;
    sl.num_pages = c0.num_pages;
    sl.plan = plan;
    sl.x = x;
    sl.out = out;
    sl.xbuf = xbuf;
    sl.q = reinterpret_cast<float *>(base + L.q);
    sl.k = reinterpret_cast<float *>(base + L.k);
    sl.v = reinterpret_cast<float *>(base + L.v);
    sl.attn = reinterpret_cast<float *>(base + L.attn);
    sl.xn = reinterpret_cast<float *>(base + L.xn);
    sl.xq = base + L.xq;
    sl.aqx = reinterpret_cast<unsigned *>(base + L.aqx);
    sl.aq = base + L.aq;
    sl.po = reinterpret_cast<float *>(base + L.po);
    sl.pml = reinterpret_cast<float *>(base + L.pml);
    sl.cnt = reinterpret_cast<unsigned *>(base + L.cnt);
    sl.num_cus = num_cus();
    for (int l = 0; l < layers; l++) {
        StepLayer &s = sl.layers[l];
        s.wq = static_cast<const uint8_t *>(w[l].wq);
        s.wk = static_cast<const uint8_t *>(w[l].wk);
        s.wv = static_cast<const uint8_t *>(w[l].wv);
        s.wo = static_cast<const uint8_t *>(w[l].wo);
        s.bq = w[l].bq;
        s.bk = w[l].bk;
        s.bv = w[l].bv;
        s.bo = w[l].bo;
        s.gamma = w[l].gamma;
        s.kc = static_cast<float *>(kv[l].k);
        s.vc = static_cast<float *>(kv[l].v);
        s.table = kv[l].page_table;
    }
    return hip_rc(launch_step(sl, st));
}

}  // namespace

extern "C" {

int ck_decode_step(const ck_layer_desc *desc, const ck_layer_weights *w, const ck_kv_cache *kv,
                   int layers, const float *x, const int32_t *pos_host, float *out, void *ws,
                   size_t ws_bytes, void *stream) {
    if (!pos_host) return CK_EINVAL;
    return decode_step_impl(desc, w, kv, layers, x, PosIn{pos_host, nullptr, 0}, out, ws,
                            ws_bytes, stream);
}

int ck_decode_step_devpos(const ck_layer_desc *desc, const ck_layer_weights *w,
                          const ck_kv_cache *kv, int layers, const float *x,
                          const int32_t *pos_dev, int max_ctx, float *out, void *ws,
                          size_t ws_bytes, void *stream) {
    if (!pos_dev) return CK_EINVAL;
    return decode_step_impl(desc, w, kv, layers, x, PosIn{nullptr, pos_dev, max_ctx}, out, ws,
                            ws_bytes, stream);
}

size_t ck_decode_layer_workspace_size(const ck_layer_desc *desc, int max_ctx) {
    if (check_desc(desc) != CK_OK || max_ctx < 1) return 0;
    if (desc->variant == CK_VARIANT_PERSISTENT) return step_layout(desc, 1, max_ctx).total;
    return ws_layout(desc, max_ctx).total;
}

long ck_decode_layer_ws_offset(const ck_layer_desc *desc, int max_ctx, const char *name) {
    if (check_desc(desc) != CK_OK || max_ctx < 1 || !name) return -1;
    if (desc->variant == CK_VARIANT_PERSISTENT) {
        // a one-layer step's workspace
        StepWs sw = step_layout(desc, 1, max_ctx);
        if (!strcmp(name, "xn")) return (long)sw.xn;
        if (!strcmp(name, "xq")) return (long)sw.xq;
        if (!strcmp(name, "q")) return (long)sw.q;
        if (!strcmp(name, "k")) return (long)sw.k;
        if (!strcmp(name, "v")) return (long)sw.v;
        if (!strcmp(name, "attn")) return (long)sw.attn;
        if (!strcmp(name, "aq")) return (long)sw.aq;
        return -1;
    }
    WsLayout w = ws_layout(desc, max_ctx);
    if (!strcmp(name, "status"))
        return desc->variant == CK_VARIANT_TWO_LAUNCH
                   ? (long)(w.cnt + sizeof(unsigned) * ato_status_word(desc->m, desc->KV))
                   : -1;
    if (!strcmp(name, "xn")) return (long)w.xn;
    if (!strcmp(name, "xq")) return (long)w.xq;
    if (!strcmp(name, "q")) return (long)w.q;
    if (!strcmp(name, "k")) return (long)w.k;
    if (!strcmp(name, "v")) return (long)w.v;
    if (!strcmp(name, "attn")) return (long)w.attn;
    if (!strcmp(name, "aq")) return (long)w.aq;
    return -1;
}

}  // extern "C"

namespace {

// The attention split of one non-persistent layer call: it covers each
// sequence's window only, or its selection. The chain and fused layers launch
// the attention kernel (on the matrix cores for some shapes); the two-launch
// layer plans for its own vector attention.
AttnPlan layer_attn_plan(const ck_layer_desc &d, const CacheView &c, const Positions &p, int mx,
                         const SparseSel *sp) {
    const int amx = sp ? sp->topk : attended(mx, c.window);
    const long long atot = sp ? (long long)d.m * sp->topk
                              : (p.dev ? (long long)d.m * amx : total_tokens(p, d.m, c.window));
    const int G = d.H / d.KV;
    const bool matrix = (d.variant == CK_VARIANT_CHAIN || d.variant == CK_VARIANT_FUSED) &&
                        attn_matrix_path(G, c.dtype, d.m, sp != nullptr);
    return attn_plan(d.KV, G, amx, atot, d.attn_chunk, attn_step(G, c.dtype, matrix), matrix);
}

int decode_layer_impl(const ck_layer_desc *desc, const ck_layer_weights *w, const ck_kv_cache *kv,
                      const float *x, const float *residual, const PosIn &pin, float *out,
                      void *ws, size_t ws_bytes, void *stream, const SparseSel *sp, int phases) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (phases < 1 || phases > 3) return CK_EINVAL;
    if ((sp || phases != 3) && desc->variant == CK_VARIANT_PERSISTENT) return CK_EUNSUPPORTED;
    if (desc->variant == CK_VARIANT_PERSISTENT) {
        // a one-layer persistent step; its residual is its input
        if (residual != x) return CK_EINVAL;
        return decode_step_impl(desc, w, kv, 1, x, pin, out, ws, ws_bytes, stream);
    }
    const ck_layer_desc &d = *desc;
    if (!w || !w->wq || !w->wk || !w->wv || !w->wo || !w->gamma || !w->rope_cos || !w->rope_sin)
        return CK_EINVAL;
    if (!al(w->wq, 4) || !al(w->wk, 4) || !al(w->wv, 4) || !al(w->wo, 4)) return CK_EINVAL;
    if (!x || !out || !ws || !al(x, 4) || !al(out, 4) || !al(ws, 256)) return CK_EINVAL;
    if (residual && !al(residual, 4)) return CK_EINVAL;
    if (x == out) return CK_EINVAL;
    CacheView c;
    rc = cache_view(kv, &c);
    if (rc) return rc;
    if (c.kv_heads != d.KV || c.head_dim != d.head_dim) return CK_EINVAL;
    Positions p;
    int mx;
    long long total;
    long long limit = cache_tokens(kv);
    if (w->rope_rows < limit) limit = w->rope_rows;
    rc = resolve_positions(pin, d.m, limit, &p, &mx, &total);
    if (rc) return rc;
    WsLayout L = ws_layout(desc, mx);
    const AttnPlan plan = layer_attn_plan(d, c, p, mx, sp);
    if (!attn_chunks_supported(plan.nchunks)) return CK_EUNSUPPORTED;
    if (ws_bytes < L.part + attn_partials_bytes(d.m, d.H, d.head_dim, plan.nchunks))
        return CK_ENOSPC;

    hipStream_t st = (hipStream_t)stream;
    uint8_t *base = static_cast<uint8_t *>(ws);
    float *xn = reinterpret_cast<float *>(base + L.xn);
    uint8_t *xq = base + L.xq;
    float *q = reinterpret_cast<float *>(base + L.q);
    float *k = reinterpret_cast<float *>(base + L.k);
    float *v = reinterpret_cast<float *>(base + L.v);
    float *attn = reinterpret_cast<float *>(base + L.attn);
    uint8_t *aq = base + L.aq;
    void *part = base + L.part;
    const int HD = d.H * d.head_dim, KD = d.KV * d.head_dim;
    const float scale = 1.0f / sqrtf((float)d.head_dim);
    // the two-launch layer: Q/K/V (clearing the counters of the second
    // launch), then attention + merge + O in one launch; selections and
    // shapes it does not take run as the fused variant
    const bool two = d.variant == CK_VARIANT_TWO_LAUNCH && !sp &&
                     ato_supported(d.H, d.head_dim, plan.nchunks);
    const bool fused = d.variant == CK_VARIANT_FUSED || d.variant == CK_VARIANT_TWO_LAUNCH;
    unsigned *cnt = reinterpret_cast<unsigned *>(base + L.cnt);
    const int ncnt = two ? ato_counters(d.m, d.KV) : 0;
    const int zstride = ato_counter_stride();
    // the fused batched layer hands its projections activation images (the
    // two-launch variant's O projection is inside its second launch)
    const bool img_x = fused && gemv_mfma_supported(d.D, d.m) && ximage_fits(d.m, d.D / CK_QK);
    const bool img_a = fused && !two && gemv_mfma_supported(HD, d.m) && ximage_fits(d.m, HD / CK_QK);
    uint32_t *xqi = img_x ? reinterpret_cast<uint32_t *>(base + L.xqi) : nullptr;
    uint32_t *aqi = img_a ? reinterpret_cast<uint32_t *>(base + L.aqi) : nullptr;

    hipError_t e;
    if (!(phases & 1)) {
        // steps 7-8 only: q, k and v are in the workspace already
    } else if (fused && qkv_shape_supported(d.D, d.m)) {
        // steps 1-6 in one kernel: RMSNorm, Q8_0, Q/K/V projections + bias,
        // RoPE, KV append
        e = launch_qkv(x, w->gamma, d.eps, d.D, d.H, d.KV, d.head_dim, d.m,
                       static_cast<const uint8_t *>(w->wq), static_cast<const uint8_t *>(w->wk),
                       static_cast<const uint8_t *>(w->wv), w->bq, w->bk, w->bv, w->rope_cos,
                       w->rope_sin, p, c, q, k, v, xn, xq, st, cnt, ncnt, zstride);
        if (e != hipSuccess) return CK_EHIP;
    } else {
        // steps 1-2: RMSNorm and the one Q8_0 quantization shared by Q, K and V
        if (fused) {
            e = launch_rmsnorm_quant(x, w->gamma, xn, xq, d.m, d.D, d.eps, st, xqi);
        } else {
            e = launch_rmsnorm(x, w->gamma, xn, d.m, d.D, d.eps, st);
            if (e == hipSuccess)
                e = launch_quantize_q8_0(xn, xq, (long long)d.m * (d.D / CK_QK), st);
        }
        if (e != hipSuccess) return CK_EHIP;

        // steps 2-4: Q, K (Q5_0) and V (Q8_0) projections with bias, one launch
        GemvArgs g;
        memset(&g, 0, sizeof(g));
        g.nseg = 3;
        g.seg[0] = GemvSeg{static_cast<const uint8_t *>(w->wq), w->bq, nullptr, q, HD, 1, 0, 0};
        g.seg[1] = GemvSeg{static_cast<const uint8_t *>(w->wk), w->bk, nullptr, k, KD, 1, 0, 0};
        g.seg[2] = GemvSeg{static_cast<const uint8_t *>(w->wv), w->bv, nullptr, v, KD, 0, 0, 0};
        g.xq = xq;
        g.K = d.D;
        g.m = d.m;
        g.ximg = xqi;
        // the fused layer on the matrix cores (no counters to clear): RoPE
        // and the append (steps 5-6) in the projection's epilogue
        const bool epi = fused && ncnt == 0 && xqi;
        if (epi) {
            const QkvEpi ep{w->rope_cos, w->rope_sin, p, c, d.head_dim};
            e = launch_gemv_mfma_qkv(g, ep, st);
        } else {
            e = gemv_any(g, st);
        }
        if (e != hipSuccess) return CK_EHIP;

        // steps 5-6: RoPE on q and k, then the append of (k, v) at pos
        if (epi) {
            // done in the projection's epilogue
        } else if (fused) {
            e = launch_rope_append(q, k, v, w->rope_cos, w->rope_sin, c, p, d.m, d.H, st, cnt,
                                   ncnt, zstride);
        } else {
            e = launch_rope(q, k, w->rope_cos, w->rope_sin, p, d.m, d.H, d.KV, d.head_dim, st);
            if (e == hipSuccess) e = launch_kv_append(c, k, v, p, d.m, st);
        }
        if (e != hipSuccess) return CK_EHIP;
    }

    if (!(phases & 2)) return CK_OK;
    if (two) {
        // steps 7-8 in one launch: attention, merge + Q8_0, O projection +
        // bo + residual
        return hip_rc(launch_ato(q, c, p, d.m, d.H, scale, plan, part, attn, aq, base + L.aqx,
                                 static_cast<const uint8_t *>(w->wo), w->bo, residual, out, d.D,
                                 cnt, st));
    }

    // step 7: attention over pos + 1 tokens, or the selection (fused: the
    // merge also quantizes)
    e = launch_attention(q, c, p, attn, fused ? aq : nullptr, d.m, d.H, scale, plan, part, st, sp,
                         aqi);
    if (e != hipSuccess) return CK_EHIP;
    if (!fused) {
        e = launch_quantize_q8_0(attn, aq, (long long)d.m * (HD / CK_QK), st);
        if (e != hipSuccess) return CK_EHIP;
    }

    // step 8: O projection (Q5_0) + bo + residual
    GemvArgs o;
    memset(&o, 0, sizeof(o));
    o.nseg = 1;
    o.seg[0] = GemvSeg{static_cast<const uint8_t *>(w->wo), w->bo, residual, out, d.D, 1, 0, 0};
    o.xq = aq;
    o.K = HD;
    o.m = d.m;
    o.ximg = aqi;
    return hip_rc(gemv_any(o, st));
}

}  // namespace

extern "C" {

int ck_decode_layer(const ck_layer_desc *desc, const ck_layer_weights *w, const ck_kv_cache *kv,
                    const float *x, const float *residual, const int32_t *pos_host, float *out,
                    void *ws, size_t ws_bytes, void *stream) {
    if (!pos_host) return CK_EINVAL;
    return decode_layer_impl(desc, w, kv, x, residual, PosIn{pos_host, nullptr, 0}, out, ws,
                             ws_bytes, stream);
}

int ck_decode_layer_sparse(const ck_layer_desc *desc, const ck_layer_weights *w,
                           const ck_kv_cache *kv, const float *x, const float *residual,
                           const int32_t *pos_host, const int32_t *pos_dev, int max_ctx,
                           const int32_t *sel, int topk, const float *sink, float *out,
                           void *ws, size_t ws_bytes, void *stream) {
    if (!sel || topk < 1 || !al(sel, 4) || (sink && !al(sink, 4))) return CK_EINVAL;
    if (!pos_host == !pos_dev) return CK_EINVAL;     // exactly one source of positions
    const SparseSel sp{sel, topk, sink};
    const PosIn pin = pos_host ? PosIn{pos_host, nullptr, 0} : PosIn{nullptr, pos_dev, max_ctx};
    return decode_layer_impl(desc, w, kv, x, residual, pin, out, ws, ws_bytes, stream, &sp);
}

int ck_decode_layer_attn_plan(const ck_layer_desc *desc, const ck_kv_cache *kv,
                              const int32_t *pos_host, int topk, int *chunk, int *nchunks) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!pos_host || !chunk || !nchunks || topk < 0) return CK_EINVAL;
    const ck_layer_desc &d = *desc;
    CacheView c;
    rc = cache_view(kv, &c);
    if (rc) return rc;
    if (c.kv_heads != d.KV || c.head_dim != d.head_dim) return CK_EINVAL;
    // the persistent step takes fp32 caches without window or ring, and no
    // selection
    if (d.variant == CK_VARIANT_PERSISTENT &&
        (topk || c.dtype != CK_KV_F32 || c.window != 0 || c.ring))
        return CK_EUNSUPPORTED;
    Positions p;
    int mx;
    long long total;
    rc = resolve_positions(PosIn{pos_host, nullptr, 0}, d.m, cache_tokens(kv), &p, &mx, &total);
    if (rc) return rc;
    AttnPlan pl;
    if (d.variant == CK_VARIANT_PERSISTENT) {
        pl = persistent_attn_plan(d, mx, total);
    } else {
        const SparseSel sp{nullptr, topk, nullptr};
        pl = layer_attn_plan(d, c, p, mx, topk ? &sp : nullptr);
    }
    *chunk = pl.chunk;
    *nchunks = pl.nchunks;
    return CK_OK;
}

int ck_decode_layer_part(const ck_layer_desc *desc, const ck_layer_weights *w,
                         const ck_kv_cache *kv, const float *x, const float *residual,
                         const int32_t *pos_host, float *out, void *ws, size_t ws_bytes, int part,
                         void *stream) {
    if (!pos_host || (part != 1 && part != 2)) return CK_EINVAL;
    return decode_layer_impl(desc, w, kv, x, residual, PosIn{pos_host, nullptr, 0}, out, ws,
                             ws_bytes, stream, nullptr, part);
}

int ck_decode_layer_devpos(const ck_layer_desc *desc, const ck_layer_weights *w,
                           const ck_kv_cache *kv, const float *x, const float *residual,
                           const int32_t *pos_dev, int max_ctx, float *out, void *ws,
                           size_t ws_bytes, void *stream) {
    if (!pos_dev) return CK_EINVAL;
    return decode_layer_impl(desc, w, kv, x, residual, PosIn{nullptr, pos_dev, max_ctx}, out,
                             ws, ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------- allocation-free layer --
// The workspace of ck_decode_layer_noalloc: a library-owned device array of
// CK_NOALLOC_SCRATCH_BYTES. Every GPU the library runs on holds its own copy
// at its own address until the process ends. In host code `scratch` only
// names the array; its device address comes from hipGetSymbolAddress, taken
// once per device (with that device current) and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[CK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device).
int scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CK_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CK_EHIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return CK_OK;
}

}  // namespace

extern "C" {

int ck_decode_layer_noalloc(const ck_layer_desc *desc, const ck_layer_weights *w,
                            const ck_kv_cache *kv, const float *x, const float *residual,
                            const int32_t *pos_host, float *out, void *stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!pos_host) return CK_EINVAL;
    int mx = 0;
    for (int s = 0; s < desc->m; s++) {
        if (pos_host[s] < 0) return CK_EINVAL;
        if (pos_host[s] + 1 > mx) mx = pos_host[s] + 1;
    }
    // the workspace this call needs, against the array's size (before any
    // device call, so that a refusal touches nothing)
    const size_t need = ck_decode_layer_workspace_size(desc, mx);
    if (need == 0) return CK_EINVAL;
    if (need > (size_t)CK_NOALLOC_SCRATCH_BYTES) return CK_ENOSPC;
    void *ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    return decode_layer_impl(desc, w, kv, x, residual, PosIn{pos_host, nullptr, 0}, out, ws,
                             (size_t)CK_NOALLOC_SCRATCH_BYTES, stream);
}

size_t ck_decode_layer_noalloc_limit(void) { return (size_t)CK_NOALLOC_SCRATCH_BYTES; }

}  // extern "C"
