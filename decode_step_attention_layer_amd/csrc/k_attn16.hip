// k_attn16.hip — split-K GQA decode attention over bf16 and fp8 caches on the
// bf16 matrix cores of gfx950.
//
// What it computes is the attention of the C-Kernel-Engine page
// "mega_fused_attention_decode_q5_0.c" (MAIN KERNEL STEP 7) over the reduced
// caches of the metrale page "prefill_attn_a.rs" (paged_decode_attn_bf16 /
// _fp8, one k_scale and one v_scale): the same grid, chunks and partials as
// k_attn, for any query group up to 8 heads, no selection.
//
// A wave takes 32 tokens a step. v_mfma_f32_16x16x32_bf16 (lane l supplies
// A[l%16][8(l/16)+e] and B[8(l/16)+e][l%16], e < 8, and receives
// D[4(l/16)+r][l%16], r < 4; checked on the device) computes
//   S^T[token][head] = sum_d K[token][d] q[head][d]      (2 x HD/32 per 16 tokens)
//   O^T[dim][head]  += sum_t V[t][dim] P[t][head]        (2 x HD/16 per 32 tokens)
// with the group's heads in the 16 columns (padding columns repeat the last
// head and are never read). K and V enter exactly: bf16 values as stored,
// fp8 E4M3 codes decoded to bf16 (their 3-bit significands fit; K codes by
// the hardware's fp8-to-bf16 pair conversion, V codes through fp32), the scales
// applied to q (k_scale) and to the chunk's output (v_scale). q (scaled to
// log2 units) and the probabilities P enter as two bf16 terms each, a high
// part and the bf16 of the remainder (for bf16 caches never zero, see
// bf16_split2), so each product keeps about 16 bits of significand: two
// MFMAs per contraction step, fp32 accumulation.
//
// Lane (hl = l % 16, kq = l / 16):
//   scores: for the 16-token half mb of the step, K of token 16mb + hl at
//     dims 32kb + 8kq + e (bf16: the four lanes of a row read 64 adjacent
//     bytes per load) or KQ*kq + 8kb + e (fp8: kq's contiguous quarter of
//     the row; a contraction may visit its index in any order), q of head
//     hl at the same dims; the lane receives the scores of tokens
//     16mb + 4kq + r;
//   value sums: its A operand for output tile T is V of the 8 tokens
//     16(e/4) + 4kq + e%4 (e < 8) at dim VT*hl + T, so that its B operand is
//     exactly the 8 probabilities it computed (no exchange between lanes);
//     the 8 rows' VT-dim slices are loaded whole (16 lanes read a full row
//     per instruction) and regrouped in registers, one byte permute per
//     operand word; the lane ends holding, for head hl, dims
//     VT*(4kq + r) + T.
// Every load of a step is issued before its arithmetic (a scheduling
// barrier keeps them together). Only a wave's last step can reach past the
// chunk: its tokens there re-read the chunk's last row, their scores masked
// (bf16: their V rows zeroed too); every other step runs unmasked with one
// address. The waves' online-softmax states are combined through LDS as in
// the fp32 matrix-core kernel.
#include "ck_attn_common.hpp"

namespace ck {

namespace {

using namespace attn;

typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One word of two bf16: the upper (HI) or lower halves of the words lo and
// hi, lo's in the low half (one byte permute).
template <bool HI>
__device__ __forceinline__ uint32_t pack_halves(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, HI ? 0x07060302u : 0x05040100u);
}

// x and y rounded to nearest even bf16 (one conversion), x in the low half.
__device__ __forceinline__ uint32_t bf16x2_rne(float x, float y) {
    const f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// x and y as high bf16 terms (hi) and the bf16 of their remainders (lo). With
// NZ a remainder of zero becomes the smallest positive bf16 (2^-133): an
// infinite cache value times the low term then stays infinite instead of
// becoming NaN (inf x 0), as in the fp32 arithmetic; against a finite value
// it adds less than an fp32 rounding (a single token's output is still its V
// exactly). fp8 caches hold no infinity and take plain remainders.
template <bool NZ>
__device__ __forceinline__ void bf16_split2(float x, float y, uint32_t &hi, uint32_t &lo) {
    hi = bf16x2_rne(x, y);
    lo = bf16x2_rne(x - __uint_as_float(hi << 16), y - __uint_as_float(hi & 0xFFFF0000u));
    if constexpr (NZ) {
        if (!(lo & 0x7FFFu)) lo = (lo & 0xFFFF0000u) | 1u;
        if (!(lo & 0x7FFF0000u)) lo = (lo & 0xFFFFu) | 0x10000u;
    }
}

// Two fp8 E4M3 codes (bytes 2*HI, 2*HI + 1 of w) decoded to fp32 (exact).
template <bool HI>
__device__ __forceinline__ f32x2 fp8_pair(uint32_t w) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
    return f32x2{f[0], f[1]};
}

// The same codes as a pair of bf16 in one word, in one conversion (an fp8
// value is exact in bf16, and the conversion's scale is one).
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

template <int NB, bool NT>
__device__ __forceinline__ void load_bytes(const uint8_t *p, uint32_t *w) {
    static_assert(NB == 4 || NB == 8 || NB == 16, "load size");
    if constexpr (NB == 16) {
        const u4v v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p))
                         : *reinterpret_cast<const u4v *>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (NB == 8) {
        const u2v v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u2v *>(p))
                         : *reinterpret_cast<const u2v *>(p);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = NT ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p))
                  : *reinterpret_cast<const uint32_t *>(p);
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u4v v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8, v);
}

template <int HD, int G, int NW, bool PAGED, int DT, bool STREAM>
__device__ __forceinline__ bool attn_item_mfma16(const AttnArgs &a, int item, int g,
                                                 SmemM<HD, G, NW> &sm) {
    static_assert(HD == 64 || HD == 128, "head size");
    static_assert(G >= 1 && G <= 16 && NW >= 1 && NW <= 8, "query group, waves");
    static_assert(DT == CK_KV_BF16 || DT == CK_KV_FP8_E4M3, "reduced caches");
    constexpr int NT = NW * kWave;
    constexpr int EB = DT == CK_KV_BF16 ? 2 : 1;   // bytes per element
    constexpr int KQ = HD / 4;                     // K dims per lane (contiguous)
    constexpr int KB = HD / 32;                    // 8-dim k-blocks per lane and half
    constexpr int KW = KQ * EB / 4;                // words of a lane's K slice
    constexpr int VT = HD / 16;                    // V dims per lane per row; output tiles
    constexpr int VW = VT * EB / 4;                // words of a lane's V slice of one row
    constexpr int KLOAD = KQ * EB >= 16 ? 16 : KQ * EB;
    constexpr int VLOAD = VT * EB;
    int s = 0;
    while (s + 1 < a.m && item >= a.first[s + 1]) s++;
    const int cidx = item - a.first[s];
    const int L = a.pos.get(s) + 1;
    const int t0 = window_start(L, a.c.window) + cidx * a.chunk;
    if (t0 >= L) return false;       // device positions: items past this sequence's chunks
    const int t1 = min(L, t0 + a.chunk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane & 15, kq = lane >> 4;
    const int KV = a.c.kv_heads;

    if (tid == 0) sm.bad = 0;
    int pg0 = 0;
    bool pages_in_lds = false;
    if (PAGED) {
        const int ps = a.c.page_size;
        pg0 = t0 / ps;
        const int npg = (t1 - 1) / ps - pg0 + 1;
        pages_in_lds = npg <= kPagesLds;
        if (pages_in_lds)
            for (int i = tid; i < npg; i += NT)
                sm.pages[i] = a.c.table[(long long)s * a.c.max_pages + pg0 + i];
    }
    __syncthreads();
    const size_t seq_base = PAGED ? 0 : ((size_t)s * KV + g) * a.c.capacity * HD;
    const int slot0 = (!PAGED && a.c.ring) ? t0 % a.c.capacity : t0;
    bool bad = false;
    // element offset of token t's row (t0 <= t < t1); an unmapped page reads
    // page 0 of the pool and marks the chunk bad
    auto row_off = [&](int t) -> long long {
        if constexpr (PAGED) {
            long long off = -1;
            if (pages_in_lds) {
                const int ps = a.c.page_size;
                const int page = sm.pages[t / ps - pg0];
                if (page >= 0 && page < a.c.num_pages)
                    off = (((long long)page * KV + g) * ps + t % ps) * (long long)HD;
            } else {
                off = cache_row(a.c, s, g, t);
            }
            if (off < 0) bad = true;
            return off < 0 ? 0 : off;
        } else {
            // a chunk's tokens are consecutive and fit in the ring: its first
            // slot, then at most one wrap
            int slot = slot0 + (t - t0);
            if (slot >= a.c.capacity) slot -= a.c.capacity;
            return (long long)(seq_base + (size_t)slot * HD);
        }
    };
    const uint8_t *Kc = static_cast<const uint8_t *>(a.c.k);
    const uint8_t *Vc = static_cast<const uint8_t *>(a.c.v);

    // a step's loads: K of tokens tb + 16mb + hl (the lane's K dims), V of
    // tokens tb + 16(e/4) + 4kq + e%4 (the lane's VT dims). FULL:
    // all 32 tokens lie in the chunk and in consecutive slots of a
    // contiguous cache, so every row is the step's first row plus a constant
    // (one address a step, the rest immediate offsets); otherwise each row
    // is located on its own, rows past the chunk re-reading its last row.
    // The lane's K dims, in 16-byte pieces. bf16: piece i is elements
    // 32i + 8kq .. + 7 of the row (k-slice i), so that the four lanes of a
    // row read 64 adjacent bytes per load instruction and consecutive
    // instructions stay on one 128-byte line (with each lane's quarter of
    // the row contiguous, every instruction touched both lines of 16 rows,
    // and streamed lines were fetched again: 8% over the K and V bytes, and
    // 31.0 against 24.3 us at long context). fp8: the row's kq-th quarter
    // (its one 128-byte line; interleaved pieces measured the same); q takes
    // the same dims.
    constexpr bool KI = DT == CK_KV_BF16;
    constexpr int NKP = KQ * EB / KLOAD;            // K pieces per row and lane
    static_assert(KLOAD == 16, "16-byte K pieces");
    auto kpiece = [&](int i) { return KI ? 32 * i : 16 * i; };   // elements
    const int k_lane0 = KI ? 8 * kq : KQ * kq;
    const int k_lane = hl * HD + k_lane0;       // element offsets from the step's first row
    const int v_lane = 4 * kq * HD + VT * hl;
    auto load_step = [&](auto full, int tb, uint32_t (&kw)[2][KW], uint32_t (&vw)[8][VW]) {
        constexpr bool FULL = decltype(full)::value;
        if constexpr (FULL && !PAGED) {
            const long long base = (long long)seq_base + (long long)(slot0 + (tb - t0)) * HD;
            const uint8_t *kp = Kc + (base + k_lane) * EB;
            const uint8_t *vp = Vc + (base + v_lane) * EB;
#pragma unroll
            for (int mb = 0; mb < 2; mb++)
#pragma unroll
                for (int i = 0; i < NKP; i++)
                    load_bytes<KLOAD, STREAM>(kp + (16 * mb * HD + kpiece(i)) * EB,
                                              &kw[mb][i * KLOAD / 4]);
#pragma unroll
            for (int e = 0; e < 8; e++)
                load_bytes<VLOAD, STREAM>(vp + (16 * (e >> 2) + (e & 3)) * HD * EB, vw[e]);
        } else {
#pragma unroll
            for (int mb = 0; mb < 2; mb++) {
                const uint8_t *kp =
                    Kc + (row_off(min(tb + 16 * mb + hl, t1 - 1)) + k_lane0) * EB;
#pragma unroll
                for (int i = 0; i < NKP; i++)
                    load_bytes<KLOAD, STREAM>(kp + kpiece(i) * EB, &kw[mb][i * KLOAD / 4]);
            }
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int t = tb + 16 * (e >> 2) + 4 * kq + (e & 3);
                const uint8_t *vp = Vc + (row_off(min(t, t1 - 1)) + VT * hl) * EB;
                load_bytes<VLOAD, STREAM>(vp, vw[e]);
            }
        }
    };

    // q of head hl at the lane's K dims, loaded before the first step's
    // loads and split after them (nothing waits for q before K/V are in
    // flight); fp8: the K scale folded in
    float qf[KQ];
    {
        // qf[8kb + e] is q at the dim of k-slice kb, element e
        const float *qh = a.q + ((size_t)s * a.H + (size_t)g * G + min(hl, G - 1)) * HD + k_lane0;
#pragma unroll
        for (int i = 0; i < KQ; i += 4) {
            const int d = KI ? 32 * (i >> 3) + (i & 7) : i;
            const float4 v = *reinterpret_cast<const float4 *>(qh + d);
            qf[i] = v.x;
            qf[i + 1] = v.y;
            qf[i + 2] = v.z;
            qf[i + 3] = v.w;
        }
    }
    constexpr bool kNZ = DT == CK_KV_BF16;   // see bf16_split2
    const int nstep = (t1 - t0 + 31) / 32;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 o[VT];
#pragma unroll
    for (int T = 0; T < VT; T++) o[T] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 qh8[KB], ql8[KB];
    // One online-softmax step over the 32 tokens at tb; FULL: all of them in
    // the chunk (nothing to mask).
    auto compute_step = [&](auto full, int tb, uint32_t (&kw)[2][KW], uint32_t (&vw)[8][VW]) {
        constexpr bool FULL = decltype(full)::value;
        // scores of tokens tb + 16mb + 4kq + r for head hl
        f32x4 sc[2];
#pragma unroll
        for (int mb = 0; mb < 2; mb++) {
            sc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; kb++) {
                bf16x8 kop;
                if constexpr (DT == CK_KV_BF16) {
                    kop = as_bf16x8(kw[mb][4 * kb], kw[mb][4 * kb + 1], kw[mb][4 * kb + 2],
                                    kw[mb][4 * kb + 3]);
                } else {
                    const uint32_t w0 = kw[mb][2 * kb], w1 = kw[mb][2 * kb + 1];
                    kop = as_bf16x8(fp8_pair_bf16<false>(w0), fp8_pair_bf16<true>(w0),
                                    fp8_pair_bf16<false>(w1), fp8_pair_bf16<true>(w1));
                }
                sc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qh8[kb], sc[mb], 0, 0, 0);
                sc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, ql8[kb], sc[mb], 0, 0, 0);
            }
        }
        float sv[2][4];
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                sv[mb][r] = (FULL || tb + 16 * mb + 4 * kq + r < t1) ? sc[mb][r] : -INFINITY;
        float mt = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
            mt = fmaxf(mt, fmaxf(fmaxf(sv[mb][0], sv[mb][1]), fmaxf(sv[mb][2], sv[mb][3])));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m_run, mt);
        const float mr = mn == -INFINITY ? 0.0f : mn;
        const float alpha = exp2f(m_run - mr);
        // the lane's 8 probabilities are its B operand: element e is
        // token 16(e/4) + 4kq + e%4
        float p[8], ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            p[e] = exp2f(sv[e >> 2][e & 3] - mr);
            ps += p[e];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        m_run = mn;
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; i++) bf16_split2<kNZ>(p[2 * i], p[2 * i + 1], ph[i], pl[i]);
        const bf16x8 ph8 = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
        const bf16x8 pl8 = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
        for (int T = 0; T < VT; T++) o[T] *= alpha;
        // V of the 8 tokens, two dims (VT*hl + T2, + 1) at a time: the pair
        // of each row, then the A operands of tiles T2 and T2 + 1, rows 2d and
        // 2d + 1 in word d (one byte permute a word). A bf16 row past the
        // chunk is zeroed (it may hold an infinity, and 0 x inf is NaN); an
        // fp8 one needs nothing: its probability is exactly zero and its
        // value finite, or a NaN that the chunk's own last row holds too.
        bool ok[8];
#pragma unroll
        for (int e = 0; e < 8; e++) ok[e] = FULL || tb + 16 * (e >> 2) + 4 * kq + (e & 3) < t1;
#pragma unroll
        for (int T2 = 0; T2 < VT; T2 += 2) {
            uint32_t lo[8], hi[8];   // rows' values at dims T2 (lo) and T2 + 1 (hi)
#pragma unroll
            for (int e = 0; e < 8; e++) {
                if constexpr (DT == CK_KV_BF16) {
                    const uint32_t w = ok[e] ? vw[e][T2 >> 1] : 0u;
                    lo[e] = w;
                    hi[e] = w;
                } else {
                    const f32x2 f = ((T2 >> 1) & 1) ? fp8_pair<true>(vw[e][T2 >> 2])
                                                    : fp8_pair<false>(vw[e][T2 >> 2]);
                    lo[e] = __float_as_uint(f[0]);
                    hi[e] = __float_as_uint(f[1]);
                }
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                uint32_t aw[4];
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    if constexpr (DT == CK_KV_BF16)
                        aw[d] = h ? pack_halves<true>(hi[2 * d], hi[2 * d + 1])
                                  : pack_halves<false>(lo[2 * d], lo[2 * d + 1]);
                    else
                        aw[d] = h ? pack_halves<true>(hi[2 * d], hi[2 * d + 1])
                                  : pack_halves<true>(lo[2 * d], lo[2 * d + 1]);
                }
                const bf16x8 vop = as_bf16x8(aw[0], aw[1], aw[2], aw[3]);
                o[T2 + h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, ph8, o[T2 + h], 0, 0, 0);
                o[T2 + h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pl8, o[T2 + h], 0, 0, 0);
            }
        }
    };
    const std::integral_constant<bool, true> kFull;
    const std::integral_constant<bool, false> kPart;
    // A wave's steps are wave, wave + NW, .... Only a wave's last step can
    // be partial (the chunk's last), and the fast addressing needs a
    // contiguous cache (no pages, no ring); every other step takes the full
    // path. bf16: the next step's loads go out before the current one is
    // computed, so that they land meanwhile. Two register sets take turns (a
    // copy from one to the other would wait for the loads in flight), and
    // the last steps are peeled off, so that no load inside the loop is
    // conditional (a conditional one makes the waits after it wait for every
    // load). fp8 (half the bytes a step, more decode work) measured faster
    // one step at a time.
    constexpr bool kPrefetch = DT == CK_KV_BF16;
    const bool fast = !PAGED && !a.c.ring;
    const int n = wave < nstep ? (nstep - 1 - wave) / NW + 1 : 0;
    if (n > 0) {
        auto at = [&](int i) { return t0 + 32 * (wave + i * NW); };
        // load and compute of a wave's step i: the fast forms for all but the last
        auto ld = [&](int i, uint32_t (&kw)[2][KW], uint32_t (&vw)[8][VW]) {
            if (fast && i + 1 < n) load_step(kFull, at(i), kw, vw);
            else load_step(kPart, at(i), kw, vw);
        };
        auto cp = [&](int i, uint32_t (&kw)[2][KW], uint32_t (&vw)[8][VW]) {
            if (i + 1 < n) compute_step(kFull, at(i), kw, vw);
            else compute_step(kPart, at(i), kw, vw);
        };
        uint32_t k0[2][KW], v0[8][VW], k1[2][KW], v1[8][VW];
        ld(0, k0, v0);
        __builtin_amdgcn_sched_barrier(0);
        // q split after the first step's loads are out (its wait is for q only)
        {
            const float qs = a.scale * kLog2e * (DT == CK_KV_FP8_E4M3 ? a.c.k_scale : 1.0f);
#pragma unroll
            for (int kb = 0; kb < KB; kb++) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    bf16_split2<kNZ>(qf[8 * kb + 2 * i] * qs, qf[8 * kb + 2 * i + 1] * qs, hw[i],
                                     lw[i]);
                qh8[kb] = as_bf16x8(hw[0], hw[1], hw[2], hw[3]);
                ql8[kb] = as_bf16x8(lw[0], lw[1], lw[2], lw[3]);
            }
        }
        if constexpr (kPrefetch) {
            int i = 0;
            for (; i + 2 < n; i += 2) {
                ld(i + 1, k1, v1);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(kFull, at(i), k0, v0);
                ld(i + 2, k0, v0);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(kFull, at(i + 1), k1, v1);
            }
            if (i + 1 < n) {
                ld(i + 1, k1, v1);
                __builtin_amdgcn_sched_barrier(0);
                compute_step(kFull, at(i), k0, v0);
                compute_step(kPart, at(i + 1), k1, v1);
            } else {
                compute_step(kPart, at(i), k0, v0);
            }
        } else {
            cp(0, k0, v0);
            for (int i = 1; i < n; i++) {
                ld(i, k0, v0);
                __builtin_amdgcn_sched_barrier(0);
                cp(i, k0, v0);
            }
        }
    }

    // the waves' states through LDS: o[T][r] is dim VT*(4kq + r) + T
    if (bad) sm.bad = 1;
    if (hl < G) {
#pragma unroll
        for (int r = 0; r < 4; r++)
#pragma unroll
            for (int T = 0; T < VT; T += 4)
                *reinterpret_cast<float4 *>(&sm.ro[wave][hl][VT * (4 * kq + r) + T]) =
                    make_float4(o[T][r], o[T + 1][r], o[T + 2][r], o[T + 3][r]);
        if (kq == 0) {
            sm.rm[wave][hl] = m_run;
            sm.rl[wave][hl] = l_run;
        }
    }
    __syncthreads();
    // every thread weighs the waves' states of its own output slice; fp8:
    // the V scale applied to the weighted sum of code values
    const size_t part = ((size_t)s * KV + g) * a.nchunks + cidx;
    const bool any_bad = sm.bad != 0;
    const float vsc = DT == CK_KV_FP8_E4M3 ? a.c.v_scale : 1.0f;
    for (int i4 = tid; i4 < G * HD / 4; i4 += NT) {
        const int j = i4 / (HD / 4), c = 4 * (i4 % (HD / 4));
        float M = sm.rm[0][j];
#pragma unroll
        for (int w = 1; w < NW; w++) M = fmaxf(M, sm.rm[w][j]);
        const float Mr = M == -INFINITY ? 0.0f : M;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float ls = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; w++) {
            const float wt = exp2f(sm.rm[w][j] - Mr);
            ls = fmaf(sm.rl[w][j], wt, ls);
            const float4 v = *reinterpret_cast<const float4 *>(&sm.ro[w][j][c]);
            acc = make_float4(fmaf(v.x, wt, acc.x), fmaf(v.y, wt, acc.y), fmaf(v.z, wt, acc.z),
                              fmaf(v.w, wt, acc.w));
        }
        float *po = &a.po[part * G * HD + (size_t)j * HD + c];
        po[0] = acc.x * vsc;
        po[1] = acc.y * vsc;
        po[2] = acc.z * vsc;
        po[3] = acc.w * vsc;
        if (c == 0) {
            a.pml[(part * G + j) * 2 + 0] = M;
            a.pml[(part * G + j) * 2 + 1] = any_bad ? NAN : ls;
        }
    }
    return true;
}

template <int HD, int G, int NW, bool PAGED, int DT>
__global__ __launch_bounds__(NW * kWave) void k_attn_mfma16(AttnArgs a) {
    __shared__ SmemM<HD, G, NW> sm;
    attn_item_mfma16<HD, G, NW, PAGED, DT, true>(a, blockIdx.x, blockIdx.y, sm);
}

template <int HD, int G, int NW>
void launch_nw(const AttnArgs &a, dim3 grid, bool paged, hipStream_t st) {
    const dim3 blk(NW * kWave);
    const int dt = a.c.dtype;
    if constexpr (HD == 128 && NW == 8) {  // never paged (launch_hd_g)
        if (dt == CK_KV_BF16) hipLaunchKernelGGL((k_attn_mfma16<HD, G, NW, false, CK_KV_BF16>), grid, blk, 0, st, a);
        else hipLaunchKernelGGL((k_attn_mfma16<HD, G, NW, false, CK_KV_FP8_E4M3>), grid, blk, 0, st, a);
    } else if (paged) {
        if (dt == CK_KV_BF16) hipLaunchKernelGGL((k_attn_mfma16<HD, G, NW, true, CK_KV_BF16>), grid, blk, 0, st, a);
        else hipLaunchKernelGGL((k_attn_mfma16<HD, G, NW, true, CK_KV_FP8_E4M3>), grid, blk, 0, st, a);
    } else {
        if (dt == CK_KV_BF16) hipLaunchKernelGGL((k_attn_mfma16<HD, G, NW, false, CK_KV_BF16>), grid, blk, 0, st, a);
        else hipLaunchKernelGGL((k_attn_mfma16<HD, G, NW, false, CK_KV_FP8_E4M3>), grid, blk, 0, st, a);
    }
}

// one wave per 32-token step of a chunk, rounded up to 2, 4 or 8 waves; a
// paged 128-wide kernel stops at 4 (at 8 waves, two a SIMD, its page-table
// addressing beside the two step buffers would not fit 256 registers)
template <int HD, int G>
void launch_hd_g(const AttnArgs &a, dim3 grid, bool paged, hipStream_t st) {
    const int steps = (a.chunk + 31) / 32;
    if (steps <= 2) launch_nw<HD, G, 2>(a, grid, paged, st);
    else if (steps <= 4 || (paged && HD == 128)) launch_nw<HD, G, 4>(a, grid, paged, st);
    else launch_nw<HD, G, 8>(a, grid, paged, st);
}

template <int HD>
void launch_hd(const AttnArgs &a, int G, dim3 grid, bool paged, hipStream_t st) {
    switch (G) {
        case 1: launch_hd_g<HD, 1>(a, grid, paged, st); break;
        case 2: launch_hd_g<HD, 2>(a, grid, paged, st); break;
        case 3: launch_hd_g<HD, 3>(a, grid, paged, st); break;
        case 4: launch_hd_g<HD, 4>(a, grid, paged, st); break;
        case 5: launch_hd_g<HD, 5>(a, grid, paged, st); break;
        case 6: launch_hd_g<HD, 6>(a, grid, paged, st); break;
        case 7: launch_hd_g<HD, 7>(a, grid, paged, st); break;
        default: launch_hd_g<HD, 8>(a, grid, paged, st); break;
    }
}

}  // namespace

hipError_t launch_attn_mfma16(const attn::AttnArgs &a, int G, int hd, dim3 grid, bool paged,
                              hipStream_t st) {
    if (hd == 64) launch_hd<64>(a, G, grid, paged, st);
    else launch_hd<128>(a, G, grid, paged, st);
    return hipGetLastError();
}

}  // namespace ck
