/*
 * ck.h — C ABI of libck.so, the MI355X (gfx950) decode-step attention layer.
 *
 * The layer is the one on the C-Kernel-Engine page
 * "mega_fused_attention_decode_q5_0.c" (MAIN KERNEL, steps 1-8): RMSNorm,
 * Q8_0 activation quantization, Q/K/O projections with Q5_0 weights and the V
 * projection with Q8_0 weights (each plus bias), RoPE, KV-cache append,
 * grouped-query decode attention, O projection, residual add. The paged cache
 * follows the metrale page "prefill_attn_a.rs" (paged_decode_attn_*: block
 * tables, block size); the attention is split over tokens and merged with a
 * log-sum-exp pass.
 *
 * Conventions for every entry point:
 *  - Pointers named *_host are host memory; every other pointer is device
 *    memory (hipMalloc'd or a torch CUDA tensor), 16-byte aligned.
 *  - The caller owns every buffer: weights, cache, inputs, outputs and the
 *    workspace. The library never allocates, frees or synchronizes. (The one
 *    exception is ck_decode_layer_noalloc, whose workspace is a device array
 *    the library owns; see there.)
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; results are valid after the stream is synchronized.
 *  - Arguments are validated on the host before anything is launched. The
 *    return value is CK_OK or a negative CK_E* code; on an error nothing has
 *    been enqueued. A launch failure reported by the runtime returns CK_EHIP.
 *  - The library keeps no state between calls and is safe to call from
 *    several host threads on different streams (ck_decode_layer_noalloc
 *    excepted: its calls on one GPU share one workspace).
 *  - m, the number of tokens (one per sequence), is at most CK_MAX_SEQS.
 *
 * Block layouts (little-endian, packed, no padding), 32 values per block:
 *   Q8_0, 34 B: fp16 d | int8 q[32]                 value_j = d * q_j
 *   Q5_0, 22 B: fp16 d | uint8 qh[4] | uint8 qs[16] value_j = d * (code_j - 16)
 *     code_j = (j < 16 ? qs[j] & 15 : qs[j-16] >> 4) | ((qh32 >> j) & 1) << 4
 *   A weight matrix [rows][K] is rows * K/32 blocks, row-major (row = output).
 */
#ifndef CK_H
#define CK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CK_OK 0
#define CK_EINVAL (-1)        /* bad pointer, size, position or alignment */
#define CK_ENOSPC (-2)        /* workspace too small */
#define CK_EUNSUPPORTED (-3)  /* shape not built into this library */
#define CK_EHIP (-4)          /* the HIP runtime reported an error */

#define CK_MAX_SEQS 16
#define CK_QK 32
#define CK_Q8_0_BYTES 34
#define CK_Q5_0_BYTES 22

/* KV cache, fp32.
 * page_size == 0: contiguous, k/v are [m][kv_heads][capacity][head_dim]
 *   (the page's [KV][capacity][head_dim] per sequence, sequences stacked).
 * page_size  > 0: paged, k/v are pools [num_pages][kv_heads][page_size][head_dim];
 *   token t of sequence s is in page page_table[s*max_pages_per_seq + t/page_size]
 *   (device int32, -1 = unmapped) at slot t % page_size. A page id outside
 *   [0, num_pages) is never dereferenced: the attention of that sequence
 *   returns NaN. */
typedef struct ck_kv_cache {
    void *k;                     /* elements of type dtype, 16-byte aligned */
    void *v;
    int32_t kv_heads;
    int32_t head_dim;            /* a multiple of 4 */
    int32_t capacity;            /* contiguous: tokens per sequence */
    int32_t page_size;           /* 0 = contiguous */
    const int32_t *page_table;   /* device, [m][max_pages_per_seq] */
    int32_t max_pages_per_seq;
    int32_t num_pages;
    int32_t dtype;               /* CK_KV_F32 (0, the default), CK_KV_BF16, CK_KV_FP8_E4M3 */
    float k_scale, v_scale;      /* CK_KV_FP8_E4M3: value = e4m3(code) * scale (fp32) */
    int32_t window;              /* sliding window: 0 = attend every token; W > 0 = only
                                    tokens t > pos - W (the last W positions) */
    int32_t ring;                /* 1 = ring buffer (contiguous only; 1 <= window <=
                                    capacity): token t lives in slot t % capacity */
} ck_kv_cache;

/* Sliding window and ring buffer. A window W attends, for a sequence at
 * position pos, the tokens max(0, pos + 1 - W) .. pos (the sliding_window
 * argument of the metrale page's paged decode attention, where 0 means the
 * whole sequence). A ring cache is the window ring of the spark_model page's
 * decode body: a contiguous cache of `capacity` slots per (sequence, KV head)
 * in which the append writes token pos at slot pos % capacity, overwriting
 * the token capacity positions back. Since the window never reaches further
 * back than capacity tokens, a ring needs 1 <= window <= capacity (otherwise
 * CK_EINVAL); positions are then bounded only by rope_rows. A ring or window
 * applies to the chain and fused variants and to the attention calls; the
 * persistent variant returns CK_EUNSUPPORTED for either. */

/* Element types of the cache (the bf16 and fp8 caches of the metrale page's
 * paged_decode_attn_bf16 / paged_decode_attn_fp8, whose fp8 variant takes one
 * k_scale and one v_scale). FP8 is OCP E4M3 (bias 7, largest finite 448,
 * S.1111.111 the only NaN). A store rounds to nearest, ties to even; an fp8
 * store encodes fp32(x / scale) and saturates at +-448 (NaN -> 0x7F). The
 * attention attends the value each element encodes (fp8: the code's value
 * times the scale). One sequence over a bf16 or fp8 cache is attended on the
 * bf16 matrix cores: the values exact, q and the probabilities as two bf16
 * terms each (about 16 significant bits per product), fp32 sums. */
#define CK_KV_F32 0
#define CK_KV_BF16 1
#define CK_KV_FP8_E4M3 2

#define CK_VARIANT_CHAIN 0       /* one kernel per step (the unfused chain) */
#define CK_VARIANT_FUSED 1       /* steps fused into four kernels per layer */
#define CK_VARIANT_PERSISTENT 2  /* every layer of a step in one persistent kernel */
#define CK_VARIANT_TWO_LAUNCH 3  /* two launches per layer: RMSNorm + Q8_0 + Q/K/V + RoPE +
                                    append; then attention, merge + Q8_0 and the O
                                    projection in one launch whose workgroups hand over
                                    through device-coherent counters (sparse selections and
                                    shapes it does not take run as CK_VARIANT_FUSED) */

#define CK_MAX_STEP_LAYERS 32

typedef struct ck_layer_desc {
    int32_t D;          /* model width (RMSNorm, Q/K/V input, O output) */
    int32_t H;          /* query heads */
    int32_t KV;         /* KV heads; H % KV == 0, query head h reads KV head h*KV/H */
    int32_t head_dim;   /* even; H*head_dim and D multiples of 32 */
    int32_t m;          /* tokens, one per sequence, 1..CK_MAX_SEQS */
    float eps;          /* RMSNorm epsilon */
    int32_t variant;    /* CK_VARIANT_* */
    int32_t attn_chunk; /* tokens per attention split; 0 = choose for the GPU */
} ck_layer_desc;

typedef struct ck_layer_weights {
    const void *wq;            /* Q5_0 [H*hd][D] */
    const void *wk;            /* Q5_0 [KV*hd][D] */
    const void *wv;            /* Q8_0 [KV*hd][D] */
    const void *wo;            /* Q5_0 [D][H*hd] */
    const float *bq, *bk, *bv, *bo;   /* biases, each nullable (= no bias) */
    const float *gamma;        /* RMSNorm weight [D] */
    const float *rope_cos;     /* [rope_rows][hd/2]: cos of the angle of (position, pair) */
    const float *rope_sin;     /* [rope_rows][hd/2] */
    int32_t rope_rows;         /* every position must be < rope_rows */
} ck_layer_weights;

/* Human-readable name of a return code. */
const char *ck_strerror(int code);

/* Library version, (major << 16) | minor. */
int ck_version(void);

/* Step 1 — RMSNorm of m rows of D fp32: y = x * gamma / sqrt(mean(x^2) + eps).
 * x, y: [m][D]; gamma: [D]. y may alias x. */
int ck_rmsnorm(const float *x, const float *gamma, float *y, int m, int D,
               float eps, void *stream);

/* Q8_0 quantization of m rows of K fp32 (K % 32 == 0) into m*K/32 blocks
 * (the quantization done before every projection; MAIN KERNEL, steps 2-4 and
 * 8). Per block: d = amax/127, q = round-half-away-from-zero(x * (1/d)) with
 * fp32 operations, stored scale = binary16(d) rounded to nearest even. */
int ck_quantize_q8_0(const float *x, void *y, int m, int K, void *stream);

/* Block GEMV (helper "Q5_0 GEMV with inline processing"; step 8 for the O
 * projection): for each token s < m and row r < rows,
 *   y[s][r] = sum_b d_w * d_x * (integer block dot) + bias[r] (+ residual[s][r]).
 * W: [rows][K/32] blocks; xq: [m][K/32] Q8_0 blocks; bias [rows] and residual
 * [m][rows] nullable; y: [m][rows]; y may alias residual. K % 32 == 0. */
int ck_gemv_q5_0_q8_0(const void *W, const void *xq, const float *bias,
                      const float *residual, float *y, int rows, int K, int m,
                      void *stream);
int ck_gemv_q8_0_q8_0(const void *W, const void *xq, const float *bias,
                      const float *residual, float *y, int rows, int K, int m,
                      void *stream);

/* Step 5 — rotate-half RoPE in place (helper "RoPE application (inline)"):
 * within every head of q ([m][H][hd]) and k ([m][KV][hd]), element i and
 * element i + hd/2 are rotated by row pos_host[s] of the tables. q or k may
 * be NULL. Every pos_host[s] must lie in [0, tab_rows). */
int ck_rope(float *q, float *k, const float *cos_tab, const float *sin_tab,
            int tab_rows, const int32_t *pos_host, int m, int H, int KV, int hd,
            void *stream);

/* Step 6 — KV append: the new token's k and v ([m][KV][hd], k already
 * rotated) are written at position pos_host[s] of sequence s (a ring cache:
 * slot pos_host[s] % capacity). */
int ck_kv_append(const ck_kv_cache *kv, const float *k, const float *v,
                 const int32_t *pos_host, int m, void *stream);

/* Workspace bytes ck_attn_decode_gqa needs for m sequences of at most
 * max_tokens attended tokens each (under a window W: at most W), with the
 * given split (0 = automatic). */
size_t ck_attn_workspace_size(int m, int H, int KV, int hd, int max_tokens, int chunk);

/* Step 7 — grouped-query decode attention: for each sequence s and query head
 * h, softmax(scale * q_h . K_g[t]) . V_g over tokens t <= pos_host[s] (under
 * the cache's window W only t > pos_host[s] - W), with g = h*KV/H. q, out: [m][H][hd]. Tokens are split into chunks of `chunk`
 * tokens (0 = automatic); each chunk's online-softmax partial goes to the
 * workspace (at least ck_attn_workspace_size bytes, any contents) and a
 * second kernel merges them by log-sum-exp. Calls that share a workspace must
 * not overlap in time. */
int ck_attn_decode_gqa(const float *q, const ck_kv_cache *kv, const int32_t *pos_host,
                       float *out, int m, int H, float scale, int chunk,
                       void *ws, size_t ws_bytes, void *stream);

/* The two passes of ck_attn_decode_gqa as separate calls, for callers that
 * produce or merge partials themselves (e.g. token-sharded caches: partials of
 * several shards merged in one pass). ck_attn_partial writes, per chunk of
 * `chunk` tokens and query head, the chunk's running max (log2 units), sum of
 * exponentials and unnormalized output into `partials` (layout: outputs
 * [m][KV][nchunks][H/KV][hd] fp32, then (max, sum) pairs, each region
 * 256-byte aligned; nchunks is fixed by (m, KV, the most tokens a sequence
 * attends, chunk); chunk c of a sequence covers its attended tokens
 * [c*chunk, (c+1)*chunk) counted from the window's first token).
 * ck_attn_merge combines them by log-sum-exp into out ([m][H][hd]) and, when
 * out_q8 is not NULL, also writes the Q8_0 blocks of out (the quantization
 * done before the O projection). Both validate like ck_attn_decode_gqa; the
 * merge must see the same pos_host, m, H, KV, hd and chunk as the partial,
 * and as window the window of the partial's cache (0 = none). An explicit
 * chunk is used as given. The automatic split (chunk 0) of this pair depends
 * on neither the cache type nor the kernel, so it can differ from
 * ck_attn_decode_gqa's, which sizes chunks for the kernel that runs (the
 * matrix-core kernels for query groups over 4 heads on an fp32 cache and for
 * one sequence over a bf16 or fp8 cache, whole steps of the vector kernel
 * otherwise): with equal explicit chunks the two give identical bits. */
int ck_attn_partial(const float *q, const ck_kv_cache *kv, const int32_t *pos_host, int m, int H,
                    float scale, int chunk, void *partials, size_t bytes, void *stream);
int ck_attn_merge(const void *partials, size_t bytes, const int32_t *pos_host, int m, int H,
                  int KV, int hd, int chunk, int window, float *out, void *out_q8,
                  void *stream);

/* Sparse attention over a selection (the spark_model page's sparse_attn,
 * with selections padded by -1 as in its decode_fixed_topk): for each
 * sequence s and query head h (KV head g = h*KV/H),
 *   out_h = sum_e exp(s_e) V_g[t_e] / (exp(sink_h) + sum_e exp(s_e)),
 *   s_e = scale * q_h . K_g[t_e],
 * over the entries t_e = sel[s*topk + e], e < topk, that are not -1. A -1
 * entry adds nothing, so padding a selection with -1 changes no result;
 * duplicates each count. sel: device int32 [m][topk]; sink: device fp32 [H]
 * logits that join the denominator only (the usual attention sink), or NULL
 * for none. Every entry other than -1 must be a token of its sequence
 * (0 <= t <= pos_host[s]) that the cache holds: an entry past the sequence,
 * on an unmapped page or already overwritten in a ring makes that sequence's
 * outputs NaN (nothing is read out of bounds). With no entry and no sink the
 * output is zero. The cache's window is not applied: the selection is the
 * attended set. q, out: [m][H][hd]. Workspace: at least
 * ck_attn_workspace_size(m, H, KV, hd, topk, chunk) bytes. */
int ck_attn_sparse(const float *q, const ck_kv_cache *kv, const int32_t *pos_host,
                   const int32_t *sel, int topk, const float *sink, float *out, int m, int H,
                   float scale, int chunk, void *ws, size_t ws_bytes, void *stream);

/* The decode layer (as ck_decode_layer) with ck_attn_sparse's attention in
 * place of step 7, over sel [m][topk] and sink [H] (nullable), both device
 * arrays; a selection may include the position being appended. Positions:
 * exactly one of pos_host (host array) and pos_dev (device array, bounded by
 * max_ctx as in ck_decode_layer_devpos). With sel, sink and pos_dev on the
 * device and topk fixed (-1-padded selections), one captured call serves
 * every token. Workspace: ck_decode_layer_workspace_size(desc, n) bytes with
 * n at least the larger of topk and the largest position + 1. Chain and
 * fused variants; the persistent variant returns CK_EUNSUPPORTED. */
int ck_decode_layer_sparse(const ck_layer_desc *desc, const ck_layer_weights *w,
                           const ck_kv_cache *kv, const float *x, const float *residual,
                           const int32_t *pos_host, const int32_t *pos_dev, int max_ctx,
                           const int32_t *sel, int topk, const float *sink, float *out,
                           void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes ck_decode_layer needs when every position is < max_ctx. */
size_t ck_decode_layer_workspace_size(const ck_layer_desc *desc, int max_ctx);

/* The whole layer, steps 1-8, for m tokens sharing the weights:
 *   xn = RMSNorm(x); xq = Q8_0(xn); q = Wq xq + bq; k = Wk xq + bk; v = Wv xq + bv
 *   RoPE(q, k, pos); cache[pos] = (k, v); a = attention over pos + 1 tokens
 *   out = Wo Q8_0(a) + bo + residual
 * x, residual, out: [m][D]; residual nullable; out may alias residual but not
 * x. pos_host: [m] host positions. ws: at least
 * ck_decode_layer_workspace_size bytes of device memory. With
 * CK_VARIANT_PERSISTENT the layer runs as a one-layer ck_decode_step, which
 * requires residual == x (else CK_EINVAL). */
int ck_decode_layer(const ck_layer_desc *desc, const ck_layer_weights *w,
                    const ck_kv_cache *kv, const float *x, const float *residual,
                    const int32_t *pos_host, float *out, void *ws, size_t ws_bytes,
                    void *stream);

/* The attention split a layer call plans for the given host positions
 * (ck_decode_layer, its devpos form at those positions, the step's layers;
 * topk > 0: ck_decode_layer_sparse with that many selected tokens): *chunk
 * tokens per chunk and *nchunks chunks for the longest sequence. Passing
 * *chunk to ck_attn_partial or ck_attn_decode_gqa runs the attention as the
 * layer does. Host-side only; CK_EINVAL / CK_EUNSUPPORTED as the layer call
 * would for the descriptor, cache and positions (with the persistent
 * variant: a selection, or a cache other than fp32 without window or ring,
 * CK_EUNSUPPORTED). */
int ck_decode_layer_attn_plan(const ck_layer_desc *desc, const ck_kv_cache *kv,
                              const int32_t *pos_host, int topk, int *chunk, int *nchunks);

/* The layer of ck_decode_layer in two calls on the same workspace, for
 * callers that interleave other work with the halves or time them apart:
 * part 1 runs steps 1-6 (RMSNorm, Q8_0, Q/K/V projections, RoPE, KV append)
 * and leaves q, k and v in the workspace; part 2 runs steps 7-8 (attention,
 * Q8_0 of its output, O projection + bias + residual) from them. Same
 * arguments as ck_decode_layer in both calls (part 1 does not write out;
 * part 2 does not read x); part 1 then part 2 on one stream, with nothing
 * else using the workspace in between, equals ck_decode_layer. Chain, fused
 * and two-launch variants (CK_EUNSUPPORTED for the persistent one). */
int ck_decode_layer_part(const ck_layer_desc *desc, const ck_layer_weights *w,
                         const ck_kv_cache *kv, const float *x, const float *residual,
                         const int32_t *pos_host, float *out, void *ws, size_t ws_bytes, int part,
                         void *stream);

/* A whole decode step: `layers` layers of the same shape, layer l reading the
 * previous layer's output (x for layer 0) with that input as its residual:
 *   x_{l+1} = ck_decode_layer(layer l, x_l, residual = x_l),  out = x_layers.
 * w and kv are arrays of `layers` entries (1..CK_MAX_STEP_LAYERS); every
 * layer's cache has the same geometry and every layer uses the RoPE tables of
 * w[0]. With desc->variant == CK_VARIANT_PERSISTENT the step runs as one
 * persistent kernel (plus a counter-clearing kernel) in which HBM streams
 * continue across layer and phase boundaries; it requires H*head_dim == D <=
 * 4096, D % 64 == 0, head_dim 64 or 128 and H/KV <= 8 (else CK_EUNSUPPORTED).
 * The other variants run ck_decode_layer per layer. If a persistent step
 * cannot complete (its bounded waits time out), the launch still ends, out
 * is undefined, and the status word (ck_decode_step_status_offset) is set.
 * ws: at least ck_decode_step_workspace_size bytes, 256-byte aligned; out
 * must not alias x. Calls that share a workspace must not overlap. */
size_t ck_decode_step_workspace_size(const ck_layer_desc *desc, int layers, int max_ctx);
int ck_decode_step(const ck_layer_desc *desc, const ck_layer_weights *w, const ck_kv_cache *kv,
                   int layers, const float *x, const int32_t *pos_host, float *out,
                   void *ws, size_t ws_bytes, void *stream);
/* Device-resident positions (the graph-capturable decode loop of the
 * spark_model page attn_v41/decode.rs: the per-token position lives in device
 * memory and the launch arguments stay constant): as ck_decode_layer and
 * ck_decode_step, but the m positions are read by the
 * kernels from pos_dev (device memory, int32[m], 4-byte aligned) when they
 * run, so that one captured launch sequence serves every later token: the
 * caller advances pos_dev between replays (for example with a kernel in the
 * same graph). The attention's chunk plan is sized for max_ctx attended
 * tokens per sequence (the workspace: ck_decode_layer_workspace_size /
 * ck_decode_step_workspace_size with the same max_ctx). Positions must lie in
 * [0, min(max_ctx, cache capacity, rope_rows)); the host cannot check them:
 * a sequence whose position is outside that range appends nothing, attends no
 * token and gets undefined outputs, and nothing is accessed out of bounds.
 * Host-side validation of everything else as in the host-position calls. */
int ck_decode_layer_devpos(const ck_layer_desc *desc, const ck_layer_weights *w,
                           const ck_kv_cache *kv, const float *x, const float *residual,
                           const int32_t *pos_dev, int max_ctx, float *out, void *ws,
                           size_t ws_bytes, void *stream);
int ck_decode_step_devpos(const ck_layer_desc *desc, const ck_layer_weights *w,
                          const ck_kv_cache *kv, int layers, const float *x,
                          const int32_t *pos_dev, int max_ctx, float *out, void *ws,
                          size_t ws_bytes, void *stream);

/* Byte offset in the step workspace of the uint32 status word: zero after
 * a persistent step that completed, non-zero after one whose waits timed out
 * (read it after synchronizing). -1 for an invalid desc or a variant other
 * than CK_VARIANT_PERSISTENT. */
long ck_decode_step_status_offset(const ck_layer_desc *desc, int layers);

/* Workspace layout of ck_decode_layer, so that callers (tests) can read the
 * intermediates after a call: byte offsets into ws, or -1 if the variant does
 * not keep that intermediate in the workspace. Names: "xn", "xq", "q", "k",
 * "v", "attn", "aq". For CK_VARIANT_PERSISTENT they are the offsets in the
 * workspace of a step (they do not depend on the number of layers), where
 * the intermediates of the step's last layer remain. */
long ck_decode_layer_ws_offset(const ck_layer_desc *desc, int max_ctx, const char *name);
/* "status" (CK_VARIANT_TWO_LAUNCH only, else -1): the uint32 status word of
 * the layer's second launch, zero after a call whose waits completed and
 * non-zero if one timed out (read it after synchronizing). */

/* Measurement utility: a plain streaming read of `bytes` (a multiple of 16)
 * at src with 16-byte non-temporal loads, four workgroups per compute unit
 * each over one contiguous slice: the achievable HBM read bandwidth to set
 * beside the nominal peak. sink: device memory of 4 * (4 * compute units)
 * bytes, written only in the impossible case that the folded words match a
 * fixed pattern. */
int ck_read_probe(const void *src, size_t bytes, void *sink, void *stream);

/* Allocation-free decode layer, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): ck_decode_layer, same arguments, results and variants,
 * with the workspace taken from a device array the library owns instead of
 * a caller's buffer. The array holds CK_NOALLOC_SCRATCH_BYTES (16 MiB); each
 * GPU the library runs on keeps its own copy until the process ends. A call
 * whose workspace (ck_decode_layer_workspace_size at the largest position
 * + 1) exceeds that returns CK_ENOSPC before touching the device. The call
 * allocates and frees nothing; the first call on a device looks up the
 * array's device address (hipGetSymbolAddress) once. Nothing in the array
 * has to start at zero: what a call's kernels count they clear themselves.
 * Every call on one GPU shares that GPU's array and leaves it holding the
 * last call's intermediates: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialized by the caller. */
#define CK_NOALLOC_SCRATCH_BYTES (16u << 20)
int ck_decode_layer_noalloc(const ck_layer_desc *desc, const ck_layer_weights *w,
                            const ck_kv_cache *kv, const float *x, const float *residual,
                            const int32_t *pos_host, float *out, void *stream);
/* CK_NOALLOC_SCRATCH_BYTES as built into the library. */
size_t ck_decode_layer_noalloc_limit(void);

#ifdef __cplusplus
}
#endif
#endif
