/*
 * oracle.h — plain, single-threaded C model of the single-token (decode)
 * transformer attention layer: RMSNorm, Q8_0 activation quantization,
 * Q5_0/Q8_0 block GEMVs with bias, rotate-half RoPE, KV-cache append,
 * grouped-query attention over the cached tokens, O projection and residual.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the checker for the HIP path.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code, header, table or helper with the HIP path.
 *
 * Semantics follow the C-Kernel-Engine page "mega_fused_attention_decode_q5_0.c"
 * (the serial kernel: helpers "Q5_0 GEMV with inline processing", "RoPE
 * application (inline)", and MAIN KERNEL steps 1-8). The paged cache follows
 * the metrale page "prefill_attn_a.rs" (paged_decode_attn_*: block tables,
 * block size). Readings of points those pages leave open are listed in the
 * repository design notes and repeated at each function in oracle.c.
 *
 * Byte layouts (little-endian, packed, no padding):
 *   Q8_0 block, 34 B: fp16 d | 32 x int8 q            value_j = d * q_j
 *   Q5_0 block, 22 B: fp16 d | 4 B qh | 16 B qs       value_j = d * (q_j - 16)
 *     q_j = low nibble (qs[j] for j < 16, qs[j-16] >> 4 for j >= 16)
 *           | bit j of qh (little-endian uint32) << 4
 *
 * Parity pins: every function is pinned by the CPU tests (tests/test_oracle_*.py)
 * against closed forms, textbook/library routines, invariants or float64 brute
 * force. Nothing in this library is "parity unpinned" except the question of
 * whether the Q5_0/Q8_0 byte conventions match any external file format.
 */
#ifndef DSAL_ORACLE_H
#define DSAL_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_QK 32
#define ORC_Q8_0_BYTES 34
#define ORC_Q5_0_BYTES 22

/* ---- IEEE-754 binary16 codec ------------------------------------------ */
float    orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f);   /* round to nearest, ties to even */

/* ---- decoding of single blocks (used by the pins) ---------------------- */
void orc_dequantize_q8_0(const uint8_t *blocks, float *out, int K);
void orc_dequantize_q5_0(const uint8_t *blocks, float *out, int K);

/* ---- the steps of the layer -------------------------------------------- */
void orc_rmsnorm(const float *x, const float *gamma, float *y, int D, float eps);
void orc_quantize_q8_0(const float *x, uint8_t *out, int K);
void orc_gemv_q5_0(const uint8_t *W, const uint8_t *xq, const float *bias,
                   const float *residual, float *y, int rows, int K);
void orc_gemv_q8_0(const uint8_t *W, const uint8_t *xq, const float *bias,
                   const float *residual, float *y, int rows, int K);
void orc_rope(float *q, float *k, const float *cos_tab, const float *sin_tab,
              int pos, int H, int KV, int hd);

/* ---- cache element codecs (the bf16 and fp8 KV caches) ----------------- */
float    orc_bf16_to_f32(uint16_t b);   /* exact */
uint16_t orc_f32_to_bf16(float f);      /* round to nearest, ties to even; NaN stays NaN */
float    orc_e4m3_to_f32(uint8_t c);    /* OCP FP8 E4M3: bias 7, no infinities, S.1111.111 = NaN */
uint8_t  orc_f32_to_e4m3(float f);      /* nearest, ties to even, saturating at +-448; NaN -> 0x7F */

/* KV cache. page_size == 0: contiguous, [m][KV][capacity][hd] (sequence s at
 * s*KV*capacity*hd). page_size > 0: pools [num_pages][KV][page_size][hd],
 * token t of sequence s lives in page page_table[s*max_pages_per_seq + t/page_size]
 * at slot t % page_size. K and V use separate buffers of the same layout.
 * Sliding window: window > 0 attends the tokens t >= L - window only; with
 * ring = 1 a contiguous cache is a ring of `capacity` slots (token t in slot
 * t % capacity), which then holds the last `capacity` tokens.
 * Element type (dtype): fp32; bf16; or FP8 E4M3 codes with one scale per
 * tensor, value = fp32(e4m3(code) * k_scale) (k_scale for K, v_scale for V),
 * stored code = e4m3(fp32(x / scale)). */
#define ORC_KV_F32 0
#define ORC_KV_BF16 1
#define ORC_KV_FP8_E4M3 2
typedef struct {
    void *k;                 /* elements of type dtype */
    void *v;
    int kv_heads;
    int head_dim;
    int capacity;            /* tokens per sequence (contiguous); unused if paged */
    int page_size;
    const int32_t *page_table;
    int max_pages_per_seq;
    int num_pages;
    int dtype;               /* ORC_KV_* */
    float k_scale, v_scale;  /* FP8 only */
    int ring;                /* contiguous only: token t lives in slot t % capacity */
    int window;              /* > 0: attention reads only the last `window` tokens */
} orc_cache;

/* Returns 0, or -1 if the token has no valid home (page id out of range). */
int orc_kv_append(const orc_cache *c, int seq, int pos, const float *k, const float *v);

/* Attention of H query heads (q: [H][hd]) over tokens 0..L-1 of sequence `seq`.
 * Query head h reads KV head h*KV/H. out: [H][hd]. probs (nullable): [H][L],
 * the softmax weights. Returns 0, or -1 if a page id is out of range. */
int orc_attention(const float *q, const orc_cache *c, int seq, int L, int H,
                  float *out, double *probs);

/* Whole layer for m tokens (one per sequence), sharing the weights. */
typedef struct {
    int D, H, KV, hd, m;
    float eps;
} orc_dims;

typedef struct {
    const uint8_t *wq, *wk, *wv, *wo;       /* Q5_0, Q5_0, Q8_0, Q5_0 */
    const float *bq, *bk, *bv, *bo;         /* nullable */
    const float *gamma;
    const float *rope_cos, *rope_sin;       /* [rope_rows][hd/2] */
    int rope_rows;
} orc_weights;

/* Optional intermediates, each [m][...] and nullable. */
typedef struct {
    float   *xn;        /* [m][D]        RMSNorm output                */
    uint8_t *xq;        /* [m][D/32*34]  Q8_0 of xn                    */
    float   *q_pre;     /* [m][H*hd]     Q projection before RoPE      */
    float   *k_pre;     /* [m][KV*hd]                                  */
    float   *q;         /* [m][H*hd]     after RoPE                    */
    float   *k;         /* [m][KV*hd]    after RoPE                    */
    float   *v;         /* [m][KV*hd]                                  */
    float   *attn;      /* [m][H*hd]     attention output              */
    uint8_t *aq;        /* [m][H*hd/32*34] Q8_0 of attn                */
} orc_trace;

/* Returns 0, -1 on a bad argument or an out-of-range page or position. */
int orc_decode_layer(const orc_dims *dims, const orc_weights *w, const orc_cache *c,
                     const float *x, const float *residual, const int32_t *pos,
                     float *out, orc_trace *trace);

/* Sparse attention over a selection: sel[topk] token positions of sequence
 * seq (-1 = absent), sink[H] logits joining the denominator only (NULL = no
 * sink). out[h] = sum_e exp(s_e) V[sel_e] / (exp(sink_h) + sum_e exp(s_e)).
 * Returns -1 for an entry >= L or a row the cache does not hold. */
int orc_attention_sparse(const float *q, const orc_cache *c, int seq, int L, int H,
                         const int32_t *sel, int topk, const float *sink, float *out);

/* The decode layer with the sparse attention in place of step 7: sel is
 * [m][topk] (per sequence), sink [H] or NULL. */
int orc_decode_layer_sparse(const orc_dims *dims, const orc_weights *w, const orc_cache *c,
                            const float *x, const float *residual, const int32_t *pos,
                            const int32_t *sel, int topk, const float *sink,
                            float *out, orc_trace *tr);

#ifdef __cplusplus
}
#endif
#endif
