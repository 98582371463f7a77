// k_step.hip — the whole decode step (every layer) in one persistent launch.
//
// Per layer (C-Kernel-Engine "mega_fused_attention_decode_q5_0.c", MAIN
// KERNEL steps 1-8) the work is a list of items:
//   QKV  row groups of Wq | Wk | Wv: RMSNorm + Q8_0 of the layer input
//        (recomputed per item from L2), block dots, bias, RoPE, KV append;
//   ATT  one (sequence, KV head, token chunk): split-K flash-decode partial;
//   MRG  one (sequence, query head): log-sum-exp merge + Q8_0 of the output;
//   O    row groups of Wo: block dots + bias + residual = the layer output.
// Items of all layers form one global sequence; workgroup w takes items
// w, w + NWG, w + 2 NWG, ... in order. An item waits only for items earlier
// in the sequence (QKV of layer l on O of layer l-1, ATT on QKV, MRG on the
// ATT chunks of its KV head, O on MRG), so the smallest unfinished item can
// always proceed while every workgroup is resident; the grid is sized from
// the occupancy so that they are. What an item can load before its
// dependency is met (weight rows, the first K/V tile of a chunk that does not
// hold the new token) is loaded before it waits, so HBM streams across phase
// and layer boundaries.
//
// Cross-workgroup data (q/k/v, the appended cache row, partials, the
// quantized attention output, layer outputs) is written and read with
// relaxed device-scope atomic accesses, which the compiler issues as plain
// loads/stores with device-level coherence (no L2 write-back or invalidate);
// a producer waits for its stores to complete (s_waitcnt), passes a barrier,
// then increments the item counter; a consumer reads the counter (bounded
// spin with sleep) before reading the data. Every wait is bounded: on time-out
// the workgroup sets a shared abort word and leaves, and every other wait
// sees it and leaves too, so the launch always ends; the host reads the
// abort word to report a failed step.
#include <string.h>

#include "ck_device.hpp"
#include "ck_gemv_common.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

constexpr int NT = 512;
constexpr int NW = NT / kWave;
constexpr int kTileS = 64;
constexpr int kMaxGS = 8;
constexpr int kMaxChunksS = 1024;
constexpr float kLog2eS = 1.4426950408889634f;
constexpr unsigned kMaxSpins = 1u << 18;

// The thread index behind an empty volatile asm: values derived from it are
// computed inside each item instead of being hoisted out of the persistent
// loop, where they would stay live (and spill) across every item type.
__device__ __forceinline__ int item_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

struct StepArgs {
    int L, D, H, KV, hd, m;
    float eps, scale;
    const float *cos_tab, *sin_tab;
    Positions pos;
    int capacity, page_size, max_pages, num_pages;
    int chunk, nchunks;
    const float *x;           // [m][D] step input
    float *out;               // [m][D] step output
    float *xbuf;              // [2][m][D] layer outputs (ping-pong)
    float *q, *k, *v;         // [m][H*hd], [m][KV*hd], [m][KV*hd]
    float *po, *pml;          // partials
    float *attn;              // [m][H*hd]
    float *xn;                // [m][D] normalized input of the last layer
    uint8_t *xq;              // [m][D/32] its Q8_0 blocks
    unsigned *aqx;            // [m*H*hd/32][10] staged Q8_0 blocks: codes, d, sum
    uint8_t *aq;              // [m][H*hd/32] canonical Q8_0 blocks (last layer)
    unsigned *cnt;            // counters [L][cstride], then the abort word
    int cstride;
    int nq_items, nk_items, na_items, nm_items, no_items;
    StepLayer layer[CK_MAX_STEP_LAYERS];
};

struct Ctx {
    const StepArgs &a;
    int l;                    // layer
    unsigned *c;              // this layer's counters
    unsigned *abort_word;
};

// Waits until *cnt >= target (thread 0 spins; the result is broadcast).
// Returns false on abort or time-out.
__device__ bool wait_ge(unsigned *cnt, unsigned target, unsigned *abort_word, int *flag) {
    if (threadIdx.x == 0) {
        int ok = 1;
        unsigned spins = 0;
        while (ld_cu(cnt) < target) {
            if (ld_cu(abort_word) != 0u) { ok = 0; break; }
            if (++spins > kMaxSpins) { st_cu(abort_word, 1u); ok = 0; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        *flag = ok;
    }
    __syncthreads();
    const bool ok = *flag != 0;
    __syncthreads();
    return ok;
}

// Publishes this workgroup's coherent stores, then counts the item done.
__device__ void signal(unsigned *cnt) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ long long cache_off(const StepArgs &a, const StepLayer &ly, int s, int g,
                                               int t) {
    if (a.page_size == 0) return (((long long)s * a.KV + g) * a.capacity + t) * (long long)a.hd;
    const int page = ly.table[(long long)s * a.max_pages + t / a.page_size];
    if (page < 0 || page >= a.num_pages) return -1;
    return (((long long)page * a.KV + g) * a.page_size + t % a.page_size) * (long long)a.hd;
}

// Physical row of logical row r of a rotated segment (pairs i, i + hd/2).
__device__ __forceinline__ int rope_row_s(int r, int hd) {
    const int half = hd >> 1, p = r >> 1;
    return (p / half) * hd + (p % half) + (r & 1) * half;
}

// RMSNorm + Q8_0 of one row (read coherently when another workgroup of this
// launch wrote it) into XBlocks (512 threads); xn_out / xq_out, when not
// null, receive the normalized row and its Q8_0 blocks.
__device__ void norm_quant_c(const float *x, bool coherent, const float *gamma, int D, float eps,
                             float *red, XBlock *xs, float *xn_out, uint8_t *xq_out) {
    const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
    const int n4 = D / 4;                       // chunks of 4; D <= 4096: <= 2 per thread
    float4 xv[2], gv[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int c = tid + i * NT;
        if (c < n4) {
            xv[i] = coherent ? ld_c4(x + 4 * c) : reinterpret_cast<const float4 *>(x)[c];
            gv[i] = reinterpret_cast<const float4 *>(gamma)[c];
        } else {
            xv[i] = gv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; i++)
        ss += (xv[i].x * xv[i].x + xv[i].y * xv[i].y) + (xv[i].z * xv[i].z + xv[i].w * xv[i].w);
    ss = group_sum<32>(ss);
    if (lane == 0) red[2 * wave] = ss;
    if (lane == 32) red[2 * wave + 1] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < 2 * NW; i++) tot += red[i];
    const float r = 1.0f / sqrtf(tot / (float)D + eps);
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int c = tid + i * NT;
        if (c < n4) {
            const float4 v = make_float4(xv[i].x * r * gv[i].x, xv[i].y * r * gv[i].y,
                                         xv[i].z * r * gv[i].z, xv[i].w * r * gv[i].w);
            uint32_t packed;
            uint16_t dbits;
            quantize_q8_0_x4_codes(v, packed, dbits);
            float cs = (float)(int8_t)(packed & 0xFF) + (float)(int8_t)((packed >> 8) & 0xFF) +
                       (float)(int8_t)((packed >> 16) & 0xFF) + (float)(int8_t)(packed >> 24);
            cs = group_sum<8>(cs);
            XBlock &xb = xs[c >> 3];
            xb.c[c & 7] = (int)packed;
            if ((c & 7) == 0) {
                xb.d = half_bits_to_float(dbits);
                xb.sum = (int)cs;
            }
            if (xn_out) {
                reinterpret_cast<float4 *>(xn_out)[c] = v;
                uint8_t *blk = xq_out + (size_t)(c >> 3) * kQ8Bytes;
                uint16_t *dst = reinterpret_cast<uint16_t *>(blk + 2 + 4 * (c & 7));
                dst[0] = (uint16_t)(packed & 0xFFFF);
                dst[1] = (uint16_t)(packed >> 16);
                if ((c & 7) == 0) *reinterpret_cast<uint16_t *>(blk) = dbits;
            }
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------- QKV item --
template <int LPR>
__device__ void qkv_item(const Ctx &cx, int item, XBlock *xs, float *red, int *flag) {
    constexpr bool PAIRED = true;
    constexpr int R = 2;
    constexpr int RPW = kWave / LPR;
    using F5 = Fmt<true, PAIRED>;
    using F8 = Fmt<false, PAIRED>;
    constexpr int WORDS = F8::words;   // room for either format
    const StepArgs &a = cx.a;
    const StepLayer &ly = a.layer[cx.l];
    const int seg = item < a.nq_items ? 0 : (item < a.nq_items + a.nk_items ? 1 : 2);
    const int wg_in_seg = seg == 0 ? item : (seg == 1 ? item - a.nq_items
                                                      : item - a.nq_items - a.nk_items);
    const bool q5 = seg < 2;
    const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPR, rsel = lane / LPR;
    const int D = a.D, nb = D / kQK, hd = a.hd;
    const int nunits = nb / 2;
    const size_t row_bytes = (size_t)nb * (q5 ? kQ5Bytes : kQ8Bytes);
    const int ubytes = q5 ? F5::bytes : F8::bytes;
    const uint8_t *W = seg == 0 ? ly.wq : (seg == 1 ? ly.wk : ly.wv);
    const float *bias = seg == 0 ? ly.bq : (seg == 1 ? ly.bk : ly.bv);
    const int rows = (seg == 0 ? a.H : a.KV) * hd;
    const bool rotate = seg < 2;
    const int row0 = (wg_in_seg * NW + wave) * (RPW * R);

    uint32_t wr[R][WORDS];
#pragma unroll
    for (int it = 0; it < R; it++) {
        const int lr = row0 + it * RPW + rsel;
        const int pr = rotate ? rope_row_s(lr, hd) : lr;
        if (lr < rows && sub < nunits) {
            const uint8_t *p = W + (size_t)pr * row_bytes + (size_t)sub * ubytes;
            if (q5) load_unit<true, true>(p, wr[it]);
            else load_unit<false, true>(p, wr[it]);
        } else {
#pragma unroll
            for (int i = 0; i < WORDS; i++) wr[it][i] = 0;
        }
    }
    // the layer input: the step input, or the previous layer's output
    if (cx.l > 0) {
        unsigned *prev = a.cnt + (size_t)(cx.l - 1) * a.cstride;
        if (!wait_ge(prev + 2, (unsigned)a.no_items, cx.abort_word, flag)) return;
    }
    const float *xin = cx.l == 0 ? a.x : a.xbuf + (size_t)((cx.l - 1) & 1) * a.m * D;
    // the last layer's first item also leaves xn and xq in the workspace
    // (one writer only: two workgroups of different XCDs writing the same
    // lines with plain stores would leave whichever L2 writes back last)
    const bool trace = item == 0 && cx.l == a.L - 1;
    for (int s = 0; s < a.m; s++)
        norm_quant_c(xin + (size_t)s * D, cx.l > 0, ly.gamma, D, a.eps, red, xs + s * nb,
                     trace ? a.xn + (size_t)s * D : nullptr,
                     trace ? a.xq + (size_t)s * nb * kQ8Bytes : nullptr);

    const int half = hd >> 1;
    for (int s = 0; s < a.m; s++) {
        XBlock xb[2];
        if (sub < nunits) {
            xb[0] = xs[s * nb + 2 * sub];
            xb[1] = xs[s * nb + 2 * sub + 1];
        } else {
            xb[0] = xb[1] = XBlock{{0, 0, 0, 0, 0, 0, 0, 0}, 0.0f, 0, {0, 0}};
        }
        float val[R];
#pragma unroll
        for (int it = 0; it < R; it++) {
            float acc = q5 ? unit_dot<true, true>(wr[it], xb, 0.0f)
                           : unit_dot<false, true>(wr[it], xb, 0.0f);
            acc = row_reduce<LPR>(acc);
            const int lr = row0 + it * RPW + rsel;
            const int pr = rotate ? rope_row_s(lr, hd) : lr;
            val[it] = acc + ((bias && lr < rows) ? bias[pr] : 0.0f);
        }
        const int pv = a.pos.get(s);
        const int p = max(pv, 0);
#pragma unroll
        for (int it = 0; it < R; it++) {
            const int lr = row0 + it * RPW + rsel;
            const int pr = rotate ? rope_row_s(lr, hd) : lr;
            float o = val[it];
            if (rotate) {
                float other;
                if constexpr (LPR == kWave) other = val[it ^ 1];
                else other = __shfl_xor(val[it], LPR);
                const int i = (lr >> 1) % half;
                const float cs = a.cos_tab[(size_t)p * half + i];
                const float sn = a.sin_tab[(size_t)p * half + i];
                o = (lr & 1) ? other * sn + val[it] * cs : val[it] * cs - other * sn;
            }
            if (sub == 0 && lr < rows) {
                if (seg == 0) {
                    st_c(a.q + (size_t)s * rows + pr, o);
                } else {
                    st_c((seg == 1 ? a.k : a.v) + (size_t)s * rows + pr, o);
                    const long long off = pv >= 0 ? cache_off(a, ly, s, pr / hd, p) : -1;
                    if (off >= 0) st_c((seg == 1 ? ly.kc : ly.vc) + off + pr % hd, o);
                }
            }
        }
    }
    signal(cx.c + 0);
}

// ------------------------------------------------------------- ATT item --
template <int HD>
struct AttSmem {
    static constexpr int stride = HD + 4;
    float kv[2 * kTileS * stride];
    float q[kMaxGS * HD];
    float p[kTileS * kMaxGS];
    float alpha[kMaxGS];
    int bad;
};

template <int HD>
__device__ void att_item(const Ctx &cx, int item, void *lds, int *flag) {
    constexpr int C4 = HD / 4;
    constexpr int NLD = kTileS * C4 / NT;
    constexpr int ROWS_PER_LD = NT / C4;
    constexpr int NTG = NT / C4;
    constexpr int TPG = kTileS / NTG;
    constexpr int S = AttSmem<HD>::stride;
    AttSmem<HD> &sm = *reinterpret_cast<AttSmem<HD> *>(lds);
    const StepArgs &a = cx.a;
    const StepLayer &ly = a.layer[cx.l];
    const int KV = a.KV, H = a.H, G = H / KV;
    const int cidx = item % a.nchunks;
    const int g = (item / a.nchunks) % KV;
    const int s = item / (a.nchunks * KV);
    const int pos = a.pos.get(s);
    const int L = pos + 1;
    const int t0 = cidx * a.chunk;
    if (t0 >= L) return;                              // no such chunk for this sequence
    const int t1 = min(L, t0 + a.chunk);
    const int tid = item_tid(), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float *sk = sm.kv;
    float *sv = sm.kv + kTileS * S;
    const int ld_col = tid % C4, ld_row = tid / C4;
    float4 kreg[NLD], vreg[NLD];
    int bad = 0;
    // rows before pos were written by earlier launches: plain loads; the row
    // at pos was appended in this launch: coherent loads
    auto fetch = [&](int st) {
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int t = st + ld_row + i * ROWS_PER_LD;
            long long off = -1;
            if (t < t1) {
                off = cache_off(a, ly, s, g, t);
                if (off < 0) bad = 1;
            }
            if (off >= 0 && t != pos) {
                kreg[i] = *reinterpret_cast<const float4 *>(ly.kc + off + 4 * ld_col);
                vreg[i] = *reinterpret_cast<const float4 *>(ly.vc + off + 4 * ld_col);
            } else if (off >= 0) {
                kreg[i] = ld_c4(ly.kc + off + 4 * ld_col);
                vreg[i] = ld_c4(ly.vc + off + 4 * ld_col);
            } else {
                kreg[i] = vreg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };
    const bool has_new = t1 == L;                      // this chunk holds the new token
    if (!has_new) fetch(t0);                           // prefetch before the dependency
    if (!wait_ge(cx.c + 0, (unsigned)(a.nq_items + 2 * a.nk_items), cx.abort_word, flag)) return;
    if (has_new) fetch(t0);

    const float qs = a.scale * kLog2eS;
    const float *qg = a.q + ((size_t)s * H + (size_t)g * G) * HD;
    for (int i = tid; i < G * HD; i += NT) sm.q[i] = ld_c(qg + i) * qs;
    if (tid == 0) sm.bad = 0;
    __syncthreads();
    if (bad) sm.bad = 1;

    float m_run = -INFINITY, l_lane = 0.0f;
    const int pv_col = tid % C4, pv_tg = tid / C4;
    float4 o[kMaxGS];
#pragma unroll
    for (int j = 0; j < kMaxGS; j++) o[j] = make_float4(0.f, 0.f, 0.f, 0.f);

    for (int st = t0; st < t1; st += kTileS) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int r = ld_row + i * ROWS_PER_LD;
            *reinterpret_cast<float4 *>(&sk[r * S + 4 * ld_col]) = kreg[i];
            *reinterpret_cast<float4 *>(&sv[r * S + 4 * ld_col]) = vreg[i];
        }
        __syncthreads();
        if (st + kTileS < t1) {
            fetch(st + kTileS);
            if (bad) sm.bad = 1;
        }
        if (wave < G) {
            const float *krow = &sk[lane * S];
            const float *qrow = &sm.q[wave * HD];
            float sc0 = 0.0f, sc1 = 0.0f;
#pragma unroll 8
            for (int d = 0; d < HD; d += 8) {
                const float4 k0 = *reinterpret_cast<const float4 *>(krow + d);
                const float4 k1 = *reinterpret_cast<const float4 *>(krow + d + 4);
                const float4 q0 = *reinterpret_cast<const float4 *>(qrow + d);
                const float4 q1 = *reinterpret_cast<const float4 *>(qrow + d + 4);
                sc0 = fmaf(k0.x, q0.x, sc0); sc0 = fmaf(k0.y, q0.y, sc0);
                sc0 = fmaf(k0.z, q0.z, sc0); sc0 = fmaf(k0.w, q0.w, sc0);
                sc1 = fmaf(k1.x, q1.x, sc1); sc1 = fmaf(k1.y, q1.y, sc1);
                sc1 = fmaf(k1.z, q1.z, sc1); sc1 = fmaf(k1.w, q1.w, sc1);
            }
            const float sv2 = (st + lane < t1) ? sc0 + sc1 : -INFINITY;
            const float m_new = fmaxf(m_run, wave_max(sv2));
            const float alpha = exp2f(m_run - m_new);
            const float pr = exp2f(sv2 - m_new);
            l_lane = l_lane * alpha + pr;
            m_run = m_new;
            sm.p[lane * kMaxGS + wave] = pr;
            if (lane == 0) sm.alpha[wave] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMaxGS; j++) {
            if (j < G) {
                const float al = sm.alpha[j];
                o[j].x *= al; o[j].y *= al; o[j].z *= al; o[j].w *= al;
            }
        }
#pragma unroll
        for (int i = 0; i < TPG; i++) {
            const int r = pv_tg + i * NTG;
            const float4 vv = *reinterpret_cast<const float4 *>(&sv[r * S + 4 * pv_col]);
            const float4 p0 = *reinterpret_cast<const float4 *>(&sm.p[r * kMaxGS]);
            const float4 p1 = *reinterpret_cast<const float4 *>(&sm.p[r * kMaxGS + 4]);
            const float pj[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int j = 0; j < kMaxGS; j++) {
                if (j < G) {
                    o[j].x = fmaf(pj[j], vv.x, o[j].x);
                    o[j].y = fmaf(pj[j], vv.y, o[j].y);
                    o[j].z = fmaf(pj[j], vv.z, o[j].z);
                    o[j].w = fmaf(pj[j], vv.w, o[j].w);
                }
            }
        }
    }
    __syncthreads();

    float *red = sm.kv;   // [NW][G][HD]
    static_assert(NW * kMaxGS * HD <= 2 * kTileS * (HD + 4), "reduction buffer");
#pragma unroll
    for (int j = 0; j < kMaxGS; j++) {
        if (j < G) {
#pragma unroll
            for (int sh = C4; sh < kWave; sh <<= 1) {
                o[j].x += __shfl_xor(o[j].x, sh);
                o[j].y += __shfl_xor(o[j].y, sh);
                o[j].z += __shfl_xor(o[j].z, sh);
                o[j].w += __shfl_xor(o[j].w, sh);
            }
            if (lane < C4)
                *reinterpret_cast<float4 *>(&red[(wave * G + j) * HD + 4 * lane]) = o[j];
        }
    }
    const float lsum = wave_sum(l_lane);
    __syncthreads();
    const size_t grp = (size_t)s * KV + g;
    const size_t part = grp * a.nchunks + cidx;
    for (int e = tid; e < G * HD; e += NT) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; w++) acc += red[w * G * HD + e];
        st_c(a.po + part * G * HD + e, acc);
    }
    if (wave < G && lane == 0) {
        st_c(a.pml + (part * G + wave) * 2 + 0, m_run);
        st_c(a.pml + (part * G + wave) * 2 + 1, sm.bad ? NAN : lsum);
    }
    signal(cx.c + 3 + grp);
}

// ------------------------------------------------------------- MRG item --
template <int HD>
__device__ void mrg_item(const Ctx &cx, int item, float *lds, int *flag, bool last_layer) {
    constexpr int C4 = HD / 4;
    constexpr int CG = NT / C4;
    float *w_s = lds;                                  // [kMaxChunksS]
    float *red = lds + kMaxChunksS;                    // [NW]
    float4 *part = reinterpret_cast<float4 *>(lds + kMaxChunksS + 16);   // [NW][C4]
    const StepArgs &a = cx.a;
    const int H = a.H, KV = a.KV, G = H / KV;
    const int h = item % H, s = item / H;
    const int g = h / G, j = h % G;
    const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
    const int L = a.pos.get(s) + 1;
    const int nc = (L + a.chunk - 1) / a.chunk;
    const size_t grp = (size_t)s * KV + g;
    if (!wait_ge(cx.c + 3 + grp, (unsigned)nc, cx.abort_word, flag)) return;
    const size_t base = grp * a.nchunks;

    float mx = -INFINITY;
    for (int c = tid; c < nc; c += NT) mx = fmaxf(mx, ld_c(a.pml + ((base + c) * G + j) * 2));
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++) M = fmaxf(M, red[i]);
    __syncthreads();
    float den = 0.0f;
    for (int c = tid; c < nc; c += NT) {
        const size_t pj = (base + c) * G + j;
        const float w = exp2f(ld_c(a.pml + pj * 2) - M);
        w_s[c] = w;
        den = fmaf(w, ld_c(a.pml + pj * 2 + 1), den);
    }
    den = wave_sum(den);
    if (lane == 0) red[wave] = den;
    __syncthreads();
    float Dn = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; i++) Dn += red[i];

    const int d4 = tid % C4, cg = tid / C4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = cg; c < nc; c += CG) {
        const float4 v = ld_c4(a.po + ((base + c) * G + j) * HD + 4 * d4);
        const float w = w_s[c];
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
    }
#pragma unroll
    for (int sh = C4; sh < kWave; sh <<= 1) {
        acc.x += __shfl_xor(acc.x, sh);
        acc.y += __shfl_xor(acc.y, sh);
        acc.z += __shfl_xor(acc.z, sh);
        acc.w += __shfl_xor(acc.w, sh);
    }
    if (lane < C4) part[wave * C4 + lane] = acc;
    __syncthreads();
    if (tid < C4) {
        float4 t = part[tid];
#pragma unroll
        for (int w = 1; w < NW; w++) {
            const float4 u = part[w * C4 + tid];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        const float inv = 1.0f / Dn;
        const float4 v = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
        const size_t oi = ((size_t)s * H + h) * HD + 4 * tid;
        st_c(a.attn + oi, v.x);
        st_c(a.attn + oi + 1, v.y);
        st_c(a.attn + oi + 2, v.z);
        st_c(a.attn + oi + 3, v.w);
        uint32_t packed;
        uint16_t dbits;
        quantize_q8_0_x4_codes(v, packed, dbits);
        float cs = (float)(int8_t)(packed & 0xFF) + (float)(int8_t)((packed >> 8) & 0xFF) +
                   (float)(int8_t)((packed >> 16) & 0xFF) + (float)(int8_t)(packed >> 24);
        cs = group_sum<8>(cs);
        const size_t b = oi / kQK;
        unsigned *xb = a.aqx + b * 10;
        st_cu(xb + (tid & 7), packed);
        if ((tid & 7) == 0) {
            st_cu(xb + 8, __float_as_uint(half_bits_to_float(dbits)));
            st_cu(xb + 9, (unsigned)(int)cs);
        }
        if (last_layer) {
            uint8_t *blk = a.aq + b * kQ8Bytes;
            uint16_t *dst = reinterpret_cast<uint16_t *>(blk + 2 + 4 * (tid & 7));
            dst[0] = (uint16_t)(packed & 0xFFFF);
            dst[1] = (uint16_t)(packed >> 16);
            if ((tid & 7) == 0) *reinterpret_cast<uint16_t *>(blk) = dbits;
        }
    }
    signal(cx.c + 1);
}

// --------------------------------------------------------------- O item --
template <int LPR>
__device__ void o_item(const Ctx &cx, int item, XBlock *xs, int *flag) {
    constexpr int R = 2;
    constexpr int RPW = kWave / LPR;
    using F = Fmt<true, true>;
    const StepArgs &a = cx.a;
    const StepLayer &ly = a.layer[cx.l];
    const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPR, rsel = lane / LPR;
    const int HD = a.H * a.hd, D = a.D;
    const int nb = HD / kQK, nunits = nb / 2;
    const size_t row_bytes = (size_t)nb * kQ5Bytes;
    const int row0 = (item * NW + wave) * (RPW * R);
    uint32_t wr[R][F::words];
#pragma unroll
    for (int it = 0; it < R; it++) {
        const int row = row0 + it * RPW + rsel;
        if (row < D && sub < nunits)
            load_unit<true, true>(ly.wo + (size_t)row * row_bytes + (size_t)sub * F::bytes, wr[it]);
        else
#pragma unroll
            for (int i = 0; i < F::words; i++) wr[it][i] = 0;
    }
    if (!wait_ge(cx.c + 1, (unsigned)(a.m * a.H), cx.abort_word, flag)) return;
    // the quantized attention output, staged coherently
    for (int b = tid; b < a.m * nb; b += NT) {
        const unsigned *src = a.aqx + (size_t)b * 10;
        XBlock xb;
#pragma unroll
        for (int i = 0; i < 8; i++) xb.c[i] = (int)ld_cu(src + i);
        xb.d = __uint_as_float(ld_cu(src + 8));
        xb.sum = (int)ld_cu(src + 9);
        xb.pad[0] = xb.pad[1] = 0;
        xs[b] = xb;
    }
    __syncthreads();
    const bool last = cx.l == a.L - 1;
    const float *res = cx.l == 0 ? a.x : a.xbuf + (size_t)((cx.l - 1) & 1) * a.m * D;
    float *dst = last ? a.out : a.xbuf + (size_t)(cx.l & 1) * a.m * D;
    for (int s = 0; s < a.m; s++) {
        XBlock xb[2];
        if (sub < nunits) {
            xb[0] = xs[s * nb + 2 * sub];
            xb[1] = xs[s * nb + 2 * sub + 1];
        } else {
            xb[0] = xb[1] = XBlock{{0, 0, 0, 0, 0, 0, 0, 0}, 0.0f, 0, {0, 0}};
        }
#pragma unroll
        for (int it = 0; it < R; it++) {
            float acc = unit_dot<true, true>(wr[it], xb, 0.0f);
            acc = row_reduce<LPR>(acc);
            const int row = row0 + it * RPW + rsel;
            if (sub == 0 && row < D) {
                float o = acc + (ly.bo ? ly.bo[row] : 0.0f);
                const float r = cx.l == 0 ? res[(size_t)s * D + row] : ld_c(res + (size_t)s * D + row);
                o = o + r;
                st_c(dst + (size_t)s * D + row, o);
            }
        }
    }
    signal(cx.c + 2);
}

// ---------------------------------------------------------------- kernel --
template <int HD, int LPR>
__global__ __launch_bounds__(NT, 4) void k_step(StepArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float red[2 * NW];
    __shared__ int flag;
    unsigned *abort_word = a.cnt + (size_t)a.L * a.cstride;
    const int per_layer = a.nq_items + 2 * a.nk_items + a.na_items + a.nm_items + a.no_items;
    const long long total = (long long)per_layer * a.L;
    // an abort is seen by every later wait, which then returns at once
    for (long long gi = blockIdx.x; gi < total; gi += gridDim.x) {
        const int l = (int)(gi / per_layer);
        int r = (int)(gi % per_layer);
        Ctx cx{a, l, a.cnt + (size_t)l * a.cstride, abort_word};
        const int nqkv = a.nq_items + 2 * a.nk_items;
        if (r < nqkv) {
            qkv_item<LPR>(cx, r, reinterpret_cast<XBlock *>(lds), red, &flag);
        } else if ((r -= nqkv) < a.na_items) {
            att_item<HD>(cx, r, lds, &flag);
        } else if ((r -= a.na_items) < a.nm_items) {
            mrg_item<HD>(cx, r, reinterpret_cast<float *>(lds), &flag, l == a.L - 1);
        } else {
            r -= a.nm_items;
            o_item<LPR>(cx, r, reinterpret_cast<XBlock *>(lds), &flag);
        }
        __syncthreads();   // LDS is reused by the next item
    }
}

__global__ void k_step_clear(unsigned *cnt, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        cnt[i] = 0u;
}

template <int HD>
size_t step_lds(int m, int D) {
    size_t att = sizeof(AttSmem<HD>);
    size_t xs = sizeof(XBlock) * (size_t)m * (D / kQK);
    size_t mrg = sizeof(float) * (kMaxChunksS + 16) + sizeof(float4) * NW * (HD / 4);
    size_t mx = att > xs ? att : xs;
    return mx > mrg ? mx : mrg;
}

static_assert(sizeof(StepArgs) <= 4096, "kernel arguments");

// Resident workgroups per CU of one instance at one LDS size, queried once
// per (device, instance, LDS size).
template <int HD, int LPR>
hipError_t resident_per_cu(size_t lds, int *per_cu) {
    constexpr int kDevs = 16, kSlots = 8;
    static int dev_of[kDevs * kSlots], lds_of[kDevs * kSlots], val_of[kDevs * kSlots];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kDevs) {
        for (int i = dev * kSlots; i < (dev + 1) * kSlots; i++)
            if (val_of[i] > 0 && lds_of[i] == (int)lds && dev_of[i] == dev) {
                *per_cu = val_of[i];
                return hipSuccess;
            }
    }
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, k_step<HD, LPR>, NT, lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kDevs && *per_cu > 0) {
        for (int i = dev * kSlots; i < (dev + 1) * kSlots; i++)
            if (val_of[i] == 0) {
                dev_of[i] = dev;
                lds_of[i] = (int)lds;
                val_of[i] = *per_cu;
                break;
            }
    }
    return hipSuccess;
}

template <int HD, int LPR>
hipError_t launch_step_t(StepArgs &a, int grid_max, hipStream_t st) {
    const size_t lds = step_lds<HD>(a.m, a.D);
    int per_cu = 0;
    hipError_t e = resident_per_cu<HD, LPR>(lds, &per_cu);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    int grid = per_cu * grid_max;
    hipLaunchKernelGGL((k_step<HD, LPR>), dim3(grid), dim3(NT), lds, st, a);
    return hipGetLastError();
}

}  // namespace

bool step_supported(int D, int H, int KV, int hd, int m, int nchunks) {
    if (H * hd != D || D % 64 != 0 || D > 4096) return false;
    if (!(hd == 64 || hd == 128) || H % KV != 0 || H / KV > kMaxGS) return false;
    if (nchunks > kMaxChunksS) return false;
    const int nb = D / kQK;
    if (sizeof(XBlock) * (size_t)m * nb > 64 * 1024) return false;
    return true;
}

// Counter words a step needs (the layers' counters + the abort word).
size_t step_counter_words(int L, int m, int KV) { return (size_t)L * (3 + m * KV) + 1; }

hipError_t launch_step(const StepLaunch &sl, hipStream_t st) {
    StepArgs a;
    memset(&a, 0, sizeof(a));
    a.L = sl.L;
    a.D = sl.D;
    a.H = sl.H;
    a.KV = sl.KV;
    a.hd = sl.hd;
    a.m = sl.m;
    a.eps = sl.eps;
    a.scale = sl.scale;
    a.cos_tab = sl.cos_tab;
    a.sin_tab = sl.sin_tab;
    a.pos = sl.pos;
    a.capacity = sl.capacity;
    a.page_size = sl.page_size;
    a.max_pages = sl.max_pages;
    a.num_pages = sl.num_pages;
    a.chunk = sl.plan.chunk;
    a.nchunks = sl.plan.nchunks;
    a.x = sl.x;
    a.out = sl.out;
    a.xbuf = sl.xbuf;
    a.q = sl.q;
    a.k = sl.k;
    a.v = sl.v;
    a.po = sl.po;
    a.pml = sl.pml;
    a.attn = sl.attn;
    a.xn = sl.xn;
    a.xq = sl.xq;
    a.aqx = sl.aqx;
    a.aq = sl.aq;
    a.cnt = sl.cnt;
    a.cstride = 3 + sl.m * sl.KV;
    const int nb = sl.D / kQK;
    const int nunits = nb / 2;
    const int lpr = nunits <= 4 ? 4 : (nunits <= 16 ? 16 : 64);
    const int rows_per_item = NW * (kWave / lpr) * 2;
    a.nq_items = (sl.H * sl.hd + rows_per_item - 1) / rows_per_item;
    a.nk_items = (sl.KV * sl.hd + rows_per_item - 1) / rows_per_item;
    a.na_items = sl.m * sl.KV * sl.plan.nchunks;
    a.nm_items = sl.m * sl.H;
    a.no_items = (sl.D + rows_per_item - 1) / rows_per_item;
    for (int i = 0; i < sl.L; i++) a.layer[i] = sl.layers[i];
    const int nwords = (int)step_counter_words(sl.L, sl.m, sl.KV);
    hipLaunchKernelGGL(k_step_clear, dim3((nwords + 255) / 256), dim3(256), 0, st, sl.cnt, nwords);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int cus = sl.num_cus;
    if (sl.hd == 64) {
        if (lpr == 4) return launch_step_t<64, 4>(a, cus, st);
        if (lpr == 16) return launch_step_t<64, 16>(a, cus, st);
        return launch_step_t<64, 64>(a, cus, st);
    }
    if (lpr == 4) return launch_step_t<128, 4>(a, cus, st);
    if (lpr == 16) return launch_step_t<128, 16>(a, cus, st);
    return launch_step_t<128, 64>(a, cus, st);
}

}  // namespace ck
