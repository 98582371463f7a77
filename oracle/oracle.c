/*
 * oracle.c — the plain single-threaded C oracle of the decode-step attention
 * layer. TEST INFRASTRUCTURE ONLY: it is the checker for the HIP path, loaded
 * by the tests, the smoke check and the benchmark's CPU-baseline leg, never by
 * the product path. It shares no code with the HIP path.
 *
 * Precision: values cross stage boundaries as fp32 (the page's serial kernel
 * keeps q, k, v, the attention output and the layer output in float buffers,
 * MAIN KERNEL scratch layout); every reduction inside a stage is carried in
 * double. The Q8_0 activation quantizer is the one step that is defined in
 * fp32 operations, because its bytes are a bit-exact contract.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off (no fused multiply-add, no
 * fast-math), so every float operation below rounds exactly as written.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== *
 * binary16 codec, written from the IEEE-754 definition of the format:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent field 0
 * holds the subnormals (fraction * 2^-24), field 31 holds inf/NaN.
 * ======================================================================== */

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);
}

/* Round a non-negative double that is an exact multiple of 2^-k (small k)
 * to the nearest integer, ties to even. */
static double round_half_even(double y)
{
    double fl = floor(y);
    double diff = y - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f)) return (uint16_t)(sign | 0x7e00);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    /* 65504 is the largest finite half; halfway to the next step (65536) is
     * 65520, which rounds to even = overflow. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    int ex;
    frexp(a, &ex);              /* a = fr * 2^ex, fr in [0.5, 1) */
    int E = ex - 1;             /* a in [2^E, 2^(E+1)) */
    if (E < -14) {
        /* subnormal range: the quantum is 2^-24 */
        double n = round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);   /* n == 1024 is the smallest normal */
    }
    double n = round_half_even(ldexp(a, 10 - E));   /* in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; E += 1; }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

/* ======================================================================== *
 * Block decoding.
 * ======================================================================== */

static float block_scale(const uint8_t *blk)
{
    return orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* The 5-bit code of element j of a Q5_0 block: low nibble from qs (byte j for
 * the first 16 elements, the high nibble of byte j-16 for the rest), fifth bit
 * from bit j of the little-endian 32-bit qh word. */
static int q5_code(const uint8_t *blk, int j)
{
    const uint8_t *qh = blk + 2;
    const uint8_t *qs = blk + 6;
    uint32_t hbits = (uint32_t)qh[0] | ((uint32_t)qh[1] << 8) |
                     ((uint32_t)qh[2] << 16) | ((uint32_t)qh[3] << 24);
    int lo = (j < 16) ? (qs[j] & 0x0f) : (qs[j - 16] >> 4);
    int hi = (int)((hbits >> j) & 1u);
    return lo | (hi << 4);
}

static int q8_code(const uint8_t *blk, int j)
{
    return (int)(int8_t)blk[2 + j];
}

void orc_dequantize_q8_0(const uint8_t *blocks, float *out, int K)
{
    for (int b = 0; b < K / ORC_QK; b++) {
        const uint8_t *blk = blocks + (size_t)b * ORC_Q8_0_BYTES;
        double d = block_scale(blk);
        for (int j = 0; j < ORC_QK; j++)
            out[b * ORC_QK + j] = (float)(d * q8_code(blk, j));
    }
}

void orc_dequantize_q5_0(const uint8_t *blocks, float *out, int K)
{
    for (int b = 0; b < K / ORC_QK; b++) {
        const uint8_t *blk = blocks + (size_t)b * ORC_Q5_0_BYTES;
        double d = block_scale(blk);
        for (int j = 0; j < ORC_QK; j++)
            out[b * ORC_QK + j] = (float)(d * (q5_code(blk, j) - 16));
    }
}

/* ======================================================================== *
 * Step 1 — RMSNorm of one token over all D features
 * (mega_fused_attention_decode_q5_0.c, MAIN KERNEL, STEP 1: T = 1, the norm
 * runs over the whole aligned embedding width). Reading: y = x * gamma /
 * sqrt(mean(x^2) + eps), gamma applied as is (no +1 offset).
 * ======================================================================== */
void orc_rmsnorm(const float *x, const float *gamma, float *y, int D, float eps)
{
    double ss = 0.0;
    for (int i = 0; i < D; i++)
        ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)D + (double)eps);
    for (int i = 0; i < D; i++)
        y[i] = (float)((double)x[i] * r * (double)gamma[i]);
}

/* ======================================================================== *
 * Q8_0 activation quantization (the quantize_row_q8_0 call made before every
 * GEMV: helper "Q5_0 GEMV with inline processing" and MAIN KERNEL STEP 8).
 * The page shows the call, not the body; the reading, in fp32 operations:
 *   amax = max |x_j| over the 32-element block
 *   d    = amax / 127                (one correctly rounded fp32 division)
 *   id   = d != 0 ? 1 / d : 0        (one correctly rounded fp32 division)
 *   q_j  = round-half-away-from-zero(x_j * id)   (one fp32 multiply)
 *   stored scale = binary16(d), rounded to nearest even; q uses the fp32 d.
 * ======================================================================== */
void orc_quantize_q8_0(const float *x, uint8_t *out, int K)
{
    for (int b = 0; b < K / ORC_QK; b++) {
        const float *xb = x + (size_t)b * ORC_QK;
        uint8_t *blk = out + (size_t)b * ORC_Q8_0_BYTES;
        float amax = 0.0f;
        for (int j = 0; j < ORC_QK; j++) {
            float a = fabsf(xb[j]);
            if (a > amax) amax = a;
        }
        float d = amax / 127.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        uint16_t dh = orc_f32_to_f16(d);
        blk[0] = (uint8_t)(dh & 0xff);
        blk[1] = (uint8_t)(dh >> 8);
        for (int j = 0; j < ORC_QK; j++) {
            float scaled = xb[j] * id;
            float r = roundf(scaled);        /* C roundf: halves away from zero */
            blk[2 + j] = (uint8_t)(int8_t)(int)r;
        }
    }
}

/* ======================================================================== *
 * Block GEMVs (helper "Q5_0 GEMV with inline processing": for every output
 * row, a quantized dot over K/32 blocks, then out = dot + bias; MAIN KERNEL
 * STEP 8 adds the residual after the bias: out = dot + bo + residual).
 * Per block the dot is d_w * d_x * S with S = sum_j w_j * x_j an exact
 * integer (w_j = q_j - 16 for Q5_0, the int8 code for Q8_0); the sum over
 * blocks is carried in double and rounded to fp32 once, then the bias and
 * the residual are added in fp32 in that order.
 * ======================================================================== */
static void gemv_blocks(const uint8_t *W, int wbytes, int is_q5, const uint8_t *xq,
                        const float *bias, const float *residual, float *y,
                        int rows, int K)
{
    const int nb = K / ORC_QK;
    for (int r = 0; r < rows; r++) {
        double acc = 0.0;
        for (int b = 0; b < nb; b++) {
            const uint8_t *wb = W + ((size_t)r * nb + b) * wbytes;
            const uint8_t *xb = xq + (size_t)b * ORC_Q8_0_BYTES;
            long s = 0;
            for (int j = 0; j < ORC_QK; j++) {
                int wj = is_q5 ? (q5_code(wb, j) - 16) : q8_code(wb, j);
                s += (long)wj * q8_code(xb, j);
            }
            acc += (double)block_scale(wb) * (double)block_scale(xb) * (double)s;
        }
        float dot = (float)acc;
        float o = dot + (bias ? bias[r] : 0.0f);
        if (residual) o = o + residual[r];
        y[r] = o;
    }
}

void orc_gemv_q5_0(const uint8_t *W, const uint8_t *xq, const float *bias,
                   const float *residual, float *y, int rows, int K)
{
    gemv_blocks(W, ORC_Q5_0_BYTES, 1, xq, bias, residual, y, rows, K);
}

void orc_gemv_q8_0(const uint8_t *W, const uint8_t *xq, const float *bias,
                   const float *residual, float *y, int rows, int K)
{
    gemv_blocks(W, ORC_Q8_0_BYTES, 0, xq, bias, residual, y, rows, K);
}

/* ======================================================================== *
 * RoPE, rotate-half pairing (helper "RoPE application (inline)"): within each
 * head of q (H heads) and k (KV heads), element i and element i + hd/2 form a
 * pair that is rotated by the angle whose cosine and sine are row `pos`,
 * column i of the tables ([rows][hd/2]). v is not rotated. The rotation is
 * evaluated in double and rounded to fp32.
 * ======================================================================== */
static void rope_heads(float *x, int nheads, int hd, const float *c, const float *s)
{
    const int half = hd / 2;
    for (int h = 0; h < nheads; h++) {
        float *xh = x + (size_t)h * hd;
        for (int i = 0; i < half; i++) {
            double a = xh[i], b = xh[i + half];
            xh[i] = (float)(a * (double)c[i] - b * (double)s[i]);
            xh[i + half] = (float)(a * (double)s[i] + b * (double)c[i]);
        }
    }
}

void orc_rope(float *q, float *k, const float *cos_tab, const float *sin_tab,
              int pos, int H, int KV, int hd)
{
    const float *c = cos_tab + (size_t)pos * (hd / 2);
    const float *s = sin_tab + (size_t)pos * (hd / 2);
    if (q) rope_heads(q, H, hd, c, s);
    if (k) rope_heads(k, KV, hd, c, s);
}

/* ======================================================================== *
 * KV cache addressing. Contiguous: the page's cache layout [KV][capacity][hd]
 * per sequence (MAIN KERNEL STEP 6), sequences stacked. Paged: the block
 * table of the metrale paged decode launchers, one entry per page of
 * page_size tokens; the page pool is [pages][KV][page_size][hd] (reading: the
 * head-major order of the contiguous layout, kept inside each page).
 * Ring (contiguous only): token t in slot t % capacity.
 * Returns the float offset of (seq, kv head, token), or -1 if unmapped.
 * ======================================================================== */
static long cache_row(const orc_cache *c, int seq, int g, int t)
{
    const long hd = c->head_dim;
    if (c->page_size == 0) {
        if (t < 0 || (!c->ring && t >= c->capacity)) return -1;
        /* ring (the window ring of the spark_model page's decode_body, written
         * at pos % window): slot t % capacity */
        const int slot = c->ring ? t % c->capacity : t;
        return (((long)seq * c->kv_heads + g) * c->capacity + slot) * hd;
    }
    if (c->ring) return -1;
    int lp = t / c->page_size;
    if (t < 0 || lp >= c->max_pages_per_seq) return -1;
    int page = c->page_table[(long)seq * c->max_pages_per_seq + lp];
    if (page < 0 || page >= c->num_pages) return -1;
    return (((long)page * c->kv_heads + g) * c->page_size + t % c->page_size) * hd;
}

/* ======================================================================== *
 * Cache element codecs for the reduced-precision caches of the metrale
 * paged decode launchers (paged_decode_attn_bf16 / _fp8, whose fp8 variant
 * takes one k_scale and one v_scale). The pages name the types but not the
 * FP8 flavour or the rounding of the store; readings: FP8 = OCP E4M3 (bias
 * 7, no infinities, S.1111.111 the only NaN code, largest finite 448), value
 * = code value x scale in fp32; storing rounds x / scale (fp32 division) to
 * the nearest code, ties to even, saturating at +-448 (a cache stays
 * finite), NaN -> 0x7F. bf16 = the top half of binary32, stored with
 * round-to-nearest-even.
 * ======================================================================== */
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);            /* quiet NaN, sign kept */
    /* add half an ulp of bf16 (minus one when the kept lsb is 0): ties to even */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float orc_e4m3_to_f32(uint8_t c)
{
    const int sgn = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);                 /* subnormal: m * 2^-6 / 8 */
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(sgn ? -v : v);
}

uint8_t orc_f32_to_e4m3(float f)
{
    if (isnan(f)) return 0x7F;
    const uint8_t sgn = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (a >= 448.0) return sgn | 0x7E;                     /* saturate (inf included) */
    /* the representable magnitudes are k * 2^(E-3) for the binade's exponent
     * E (E >= -6; the subnormals share E = -6): scale, round half to even,
     * and let a rounded-up mantissa of 16 carry into the next binade */
    int E;
    frexp(a, &E);                                          /* a = f * 2^E, f in [0.5, 1) */
    E -= 1;                                                /* a in [2^E, 2^(E+1)) */
    if (a == 0.0 || E < -6) E = -6;
    double q = ldexp(a, 3 - E);                            /* exact: a power-of-two scaling */
    double r = floor(q);
    double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;
    double v = ldexp(r, E - 3);
    if (v >= 448.0) return sgn | 0x7E;
    /* encode v exactly */
    if (v < ldexp(1.0, -6)) return sgn | (uint8_t)(int)ldexp(v, 9);   /* subnormal code */
    int e;
    frexp(v, &e);
    e -= 1;
    int m = (int)(ldexp(v, 3 - e) - 8.0);
    return sgn | (uint8_t)(((e + 7) << 3) | m);
}

/* element i of K (is_k) or V as the attention reads it */
static double cache_value(const orc_cache *c, int is_k, long i)
{
    const void *p = is_k ? c->k : c->v;
    switch (c->dtype) {
    case ORC_KV_BF16: return (double)orc_bf16_to_f32(((const uint16_t *)p)[i]);
    case ORC_KV_FP8_E4M3: {
        const float sc = is_k ? c->k_scale : c->v_scale;
        return (double)(orc_e4m3_to_f32(((const uint8_t *)p)[i]) * sc);   /* fp32 product */
    }
    default: return (double)((const float *)p)[i];
    }
}

static void cache_store(const orc_cache *c, int is_k, long i, float x)
{
    void *p = is_k ? c->k : c->v;
    switch (c->dtype) {
    case ORC_KV_BF16: ((uint16_t *)p)[i] = orc_f32_to_bf16(x); break;
    case ORC_KV_FP8_E4M3: {
        const float sc = is_k ? c->k_scale : c->v_scale;
        ((uint8_t *)p)[i] = orc_f32_to_e4m3(x / sc);                      /* fp32 division */
        break;
    }
    default: ((float *)p)[i] = x; break;
    }
}

/* STEP 6 — store the new token's k and v (after RoPE) at position pos. */
int orc_kv_append(const orc_cache *c, int seq, int pos, const float *k, const float *v)
{
    for (int g = 0; g < c->kv_heads; g++) {
        long off = cache_row(c, seq, g, pos);
        if (off < 0) return -1;
        for (int d = 0; d < c->head_dim; d++) {
            cache_store(c, 1, off + d, k[(size_t)g * c->head_dim + d]);
            cache_store(c, 0, off + d, v[(size_t)g * c->head_dim + d]);
        }
    }
    return 0;
}

/* ======================================================================== *
 * STEP 7 — decode attention with grouped KV heads. Query head h reads KV head
 * h*KV/H (the mapping the page states for the GQA-aware decode kernel) and
 * attends all L = pos + 1 cached tokens, the new one included. Scale
 * 1/sqrt(hd) (the inv_sqrt_d / hd^-0.5 of the other two pages; the first page
 * does not show it). Two passes in double: scores and their maximum, then
 * exp-weights, their sum and the weighted sum of V; one division at the end.
 * ======================================================================== */
int orc_attention(const float *q, const orc_cache *c, int seq, int L, int H,
                  float *out, double *probs)
{
    const int KV = c->kv_heads, hd = c->head_dim;
    /* sliding window (the metrale page's sliding_window: 0 = the whole
     * sequence, else only the last `window` positions): tokens [t0, L) */
    const int t0 = (c->window > 0 && L > c->window) ? L - c->window : 0;
    /* a ring keeps only the last `capacity` tokens: older ones are gone */
    if (c->ring && L - t0 > c->capacity) return -1;
    const double scale = 1.0 / sqrt((double)hd);
    double *score = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)hd);
    if (!score || !acc) { free(score); free(acc); return -1; }
    int rc = 0;
    for (int h = 0; h < H && rc == 0; h++) {
        const int g = h * KV / H;
        const float *qh = q + (size_t)h * hd;
        double mx = -INFINITY;
        for (int t = t0; t < L; t++) {
            long off = cache_row(c, seq, g, t);
            if (off < 0) { rc = -1; break; }
            double s = 0.0;
            for (int d = 0; d < hd; d++)
                s += (double)qh[d] * cache_value(c, 1, off + d);
            score[t] = s * scale;
            if (score[t] > mx) mx = score[t];
        }
        if (rc) break;
        double denom = 0.0;
        for (int d = 0; d < hd; d++) acc[d] = 0.0;
        for (int t = t0; t < L; t++) {
            long off = cache_row(c, seq, g, t);
            double p = exp(score[t] - mx);
            score[t] = p;
            denom += p;
            for (int d = 0; d < hd; d++)
                acc[d] += p * cache_value(c, 0, off + d);
        }
        for (int d = 0; d < hd; d++)
            out[(size_t)h * hd + d] = (float)(acc[d] / denom);
        if (probs)
            for (int t = 0; t < L; t++)
                probs[(size_t)h * L + t] = t < t0 ? 0.0 : score[t] / denom;
    }
    free(score);
    free(acc);
    return rc;
}

/* ======================================================================== *
 * The whole layer, STEP 1 through STEP 8 of the page's MAIN KERNEL, once per
 * token (m tokens, one per sequence, sharing the weights):
 *   xn = RMSNorm(x); xq = Q8_0(xn)  (one quantization feeds Q, K and V)
 *   q = Wq.xq + bq; k = Wk.xq + bk (Q5_0); v = Wv.xq + bv (Q8_0)
 *   RoPE(q, k, pos); cache[pos] = (k, v); a = attention over pos + 1 tokens
 *   aq = Q8_0(a); out = Wo.aq + bo + residual (Q5_0)
 * The page quantizes the same normalized input once per projection; the
 * three quantizations are identical, so one is kept.
 * ======================================================================== */
/* ======================================================================== *
 * Sparse attention over a selection (the spark_model page's sparse_attn and
 * decode_fixed_topk): for each sequence, `topk` token positions of its cache
 * (-1 = absent: the entry is skipped, so padding changes nothing) and, per
 * query head, a sink logit that joins the softmax denominator only (reading:
 * the usual attention sink, a virtual token with a learned logit and a zero
 * value). With s_e = scale * q_h . K_g[sel_e] over the present entries,
 *   out_h = sum_e exp(s_e) V_g[sel_e] / (exp(sink_h) + sum_e exp(s_e)).
 * An entry past the sequence (>= L), or whose row the cache does not hold,
 * is an error; duplicates each count. The window setting is not applied:
 * the selection is the attended set.
 * ======================================================================== */
int orc_attention_sparse(const float *q, const orc_cache *c, int seq, int L, int H,
                         const int32_t *sel, int topk, const float *sink, float *out)
{
    const int KV = c->kv_heads, hd = c->head_dim;
    const double scale = 1.0 / sqrt((double)hd);
    double *score = (double *)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)hd);
    if (!score || !acc) { free(score); free(acc); return -1; }
    int rc = 0;
    for (int e = 0; e < topk && rc == 0; e++) {
        const int t = sel[e];
        if (t < 0) continue;
        if (t >= L || (c->ring && t < L - c->capacity)) rc = -1;
    }
    for (int h = 0; h < H && rc == 0; h++) {
        const int g = h * KV / H;
        const float *qh = q + (size_t)h * hd;
        double mx = sink ? (double)sink[h] : -INFINITY;
        for (int e = 0; e < topk; e++) {
            if (sel[e] < 0) continue;
            long off = cache_row(c, seq, g, sel[e]);
            if (off < 0) { rc = -1; break; }
            double sc = 0.0;
            for (int d = 0; d < hd; d++)
                sc += (double)qh[d] * cache_value(c, 1, off + d);
            score[e] = sc * scale;
            if (score[e] > mx) mx = score[e];
        }
        if (rc) break;
        double denom = sink ? exp((double)sink[h] - mx) : 0.0;
        for (int d = 0; d < hd; d++) acc[d] = 0.0;
        for (int e = 0; e < topk; e++) {
            if (sel[e] < 0) continue;
            long off = cache_row(c, seq, g, sel[e]);
            double p = exp(score[e] - mx);
            denom += p;
            for (int d = 0; d < hd; d++)
                acc[d] += p * cache_value(c, 0, off + d);
        }
        /* nothing present and no sink: an empty softmax, output zero */
        for (int d = 0; d < hd; d++)
            out[(size_t)h * hd + d] = denom > 0.0 ? (float)(acc[d] / denom) : 0.0f;
    }
    free(score);
    free(acc);
    return rc;
}

static int decode_layer(const orc_dims *dm, const orc_weights *w, const orc_cache *c,
                        const float *x, const float *residual, const int32_t *pos,
                        const int32_t *sel, int topk, const float *sink,
                        float *out, orc_trace *tr)
{
    const int D = dm->D, H = dm->H, KV = dm->KV, hd = dm->hd;
    const int HD = H * hd, KD = KV * hd;
    if (D % ORC_QK || HD % ORC_QK || hd % 2 || KV <= 0 || H % KV) return -1;
    if (c->kv_heads != KV || c->head_dim != hd) return -1;

    float *xn = (float *)malloc(sizeof(float) * D);
    uint8_t *xq = (uint8_t *)malloc((size_t)D / ORC_QK * ORC_Q8_0_BYTES);
    float *q = (float *)malloc(sizeof(float) * HD);
    float *k = (float *)malloc(sizeof(float) * KD);
    float *v = (float *)malloc(sizeof(float) * KD);
    float *a = (float *)malloc(sizeof(float) * HD);
    uint8_t *aq = (uint8_t *)malloc((size_t)HD / ORC_QK * ORC_Q8_0_BYTES);
    int rc = (xn && xq && q && k && v && a && aq) ? 0 : -1;

    for (int s = 0; s < dm->m && rc == 0; s++) {
        const float *xs = x + (size_t)s * D;
        const int p = pos[s];
        if (p < 0 || p >= w->rope_rows) { rc = -1; break; }

        orc_rmsnorm(xs, w->gamma, xn, D, dm->eps);
        orc_quantize_q8_0(xn, xq, D);
        orc_gemv_q5_0(w->wq, xq, w->bq, NULL, q, HD, D);
        orc_gemv_q5_0(w->wk, xq, w->bk, NULL, k, KD, D);
        orc_gemv_q8_0(w->wv, xq, w->bv, NULL, v, KD, D);
        if (tr && tr->q_pre) memcpy(tr->q_pre + (size_t)s * HD, q, sizeof(float) * HD);
        if (tr && tr->k_pre) memcpy(tr->k_pre + (size_t)s * KD, k, sizeof(float) * KD);
        orc_rope(q, k, w->rope_cos, w->rope_sin, p, H, KV, hd);
        if (orc_kv_append(c, s, p, k, v)) { rc = -1; break; }
        if (sel) {
            if (orc_attention_sparse(q, c, s, p + 1, H, sel + (size_t)s * topk, topk, sink, a)) {
                rc = -1;
                break;
            }
        } else if (orc_attention(q, c, s, p + 1, H, a, NULL)) {
            rc = -1;
            break;
        }
        orc_quantize_q8_0(a, aq, HD);
        orc_gemv_q5_0(w->wo, aq, w->bo, residual ? residual + (size_t)s * D : NULL,
                      out + (size_t)s * D, D, HD);

        if (tr) {
            if (tr->xn) memcpy(tr->xn + (size_t)s * D, xn, sizeof(float) * D);
            if (tr->xq) memcpy(tr->xq + (size_t)s * D / ORC_QK * ORC_Q8_0_BYTES, xq,
                               (size_t)D / ORC_QK * ORC_Q8_0_BYTES);
            if (tr->q) memcpy(tr->q + (size_t)s * HD, q, sizeof(float) * HD);
            if (tr->k) memcpy(tr->k + (size_t)s * KD, k, sizeof(float) * KD);
            if (tr->v) memcpy(tr->v + (size_t)s * KD, v, sizeof(float) * KD);
            if (tr->attn) memcpy(tr->attn + (size_t)s * HD, a, sizeof(float) * HD);
            if (tr->aq) memcpy(tr->aq + (size_t)s * HD / ORC_QK * ORC_Q8_0_BYTES, aq,
                               (size_t)HD / ORC_QK * ORC_Q8_0_BYTES);
        }
    }
    free(xn); free(xq); free(q); free(k); free(v); free(a); free(aq);
    return rc;
}

int orc_decode_layer(const orc_dims *dm, const orc_weights *w, const orc_cache *c,
                     const float *x, const float *residual, const int32_t *pos,
                     float *out, orc_trace *tr)
{
    return decode_layer(dm, w, c, x, residual, pos, NULL, 0, NULL, out, tr);
}

int orc_decode_layer_sparse(const orc_dims *dm, const orc_weights *w, const orc_cache *c,
                            const float *x, const float *residual, const int32_t *pos,
                            const int32_t *sel, int topk, const float *sink,
                            float *out, orc_trace *tr)
{
    if (!sel || topk < 0) return -1;
    return decode_layer(dm, w, c, x, residual, pos, sel, topk, sink, out, tr);
}
