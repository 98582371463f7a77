// ck_attn_common.hpp — the split-K grouped-query decode attention item,
// shared by the attention kernel (k_attn.hip) and the attention + merge + O
// projection kernel (k_ato.hip): argument block, workgroup shape, per-lane
// K/V row slices, the LDS state and the body that computes one chunk's
// online-softmax partial for every query head of a KV head.
//
// What it computes (C-Kernel-Engine "mega_fused_attention_decode_q5_0.c",
// MAIN KERNEL STEP 7): for query head h, KV head g = h*KV/H, tokens t <= pos,
//   out_h = sum_t softmax_t(scale * q_h . K_g[t]) V_g[t],
// split into chunks of tokens whose partials (running max in log2 units, sum
// of exponentials, unnormalized output) a log-sum-exp pass merges.
#pragma once

#include <type_traits>

#include "ck_device.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace attn {

constexpr int kMaxG = 8;
constexpr int kMaxChunks = 4096;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const float *q;       // [m][H][HD]
    CacheView c;
    Positions pos;
    float scale;
    int chunk;            // tokens per chunk (rows past a chunk are masked)
    int nchunks;
    int H;
    float *po;            // [m][KV][nchunks][G][HD]  unnormalized outputs
    float *pml;           // [m][KV][nchunks][G][2]   (max in log2 units, sum)
    int m;
    int first[kMaxSeqs + 1];  // first work item of each sequence; first[m] = items
    // sparse attention (sel not null): sequence s attends the token positions
    // sel[s*topk .. s*topk + topk) (-1 = absent) instead of its tokens; chunks
    // then split the selection entries
    const int32_t *sel;
    int topk;
};

constexpr int kPagesLds = 512;   // page ids of a chunk staged in LDS
constexpr int kSelLds = 1024;    // selection entries of a chunk staged in LDS
// Workgroup shape: 4 waves; per step a wave loads 4 rows per round, 4 rounds
// (a 64-token step), or 3 rounds (48 tokens) for large query groups, whose
// per-lane accumulators leave fewer registers for loads. Two workgroups fit
// a compute unit either way. The attention plan sizes chunks in whole steps.
template <int G>
struct AttnShape {
    static constexpr int waves = 4;
    static constexpr int rounds = G > 4 ? 3 : 4;
    static constexpr int sub = rounds;              // rows per online-softmax batch
    static constexpr int threads = waves * 64;
    static constexpr int step = waves * 4 * rounds;
};

// How one wave holds K/V rows: a row is read by LPR lanes, F = HD/LPR
// elements each, so one load round covers 64/LPR rows. fp32 rows of 128 are
// read as two 16-byte pieces per lane (columns 4i.. and 64+4i..), so that one
// load instruction covers 256 contiguous bytes of each of its rows; otherwise
// a lane's F elements are contiguous (columns F*i..). fp8 rows use 8 lanes
// where the query group is small (16 codes, one 16-byte load a lane), so that
// a step holds twice the rows for the same load instructions: with a quarter
// of fp32's bytes per row, the rows per step set the bytes in flight (bf16
// would need 32 bytes a lane, more registers than two workgroups per CU
// leave). WORDS: raw words per lane per row.
template <int DT, int HD, int G>
struct RowGeo {
    static constexpr int EB = DT == CK_KV_F32 ? 4 : (DT == CK_KV_BF16 ? 2 : 1);
    static constexpr int LPR = (DT == CK_KV_FP8_E4M3 && G <= 4) ? 8 : 16;
    static constexpr int F = HD / LPR;
    static constexpr int RPR = kWave / LPR;            // rows per load round
    static constexpr int WORDS = F * EB / 4;
    static constexpr bool SPLIT = DT == CK_KV_F32 && F == 8;
};


// One lane's slice of a K or V row.
template <int DT, int HD, int G>
struct Slice {
    typedef RowGeo<DT, HD, G> Geo;
    static constexpr int F = Geo::F;
    static constexpr int EB = Geo::EB;
    static constexpr int WORDS = Geo::WORDS;
    uint32_t w[WORDS];

    __device__ static __forceinline__ int col(int li, int e) {
        if constexpr (Geo::SPLIT) return e < 4 ? 4 * li + e : 64 + 4 * li + (e - 4);
        else return F * li + e;
    }
    // NT: non-temporal loads (the rows are read once; measured faster where
    // the chunks are long and the kernel streams). The plain path keeps its
    // own code: the vector-typed loads of the streaming path change the
    // register allocation of the short-chunk kernels.
    template <bool NT>
    __device__ __forceinline__ void load(const void *base, long long off, int li) {
        if constexpr (NT) {
            typedef unsigned int u4 __attribute__((ext_vector_type(4)));
            typedef unsigned int u2 __attribute__((ext_vector_type(2)));
            auto ld4 = [](const void *q) { return __builtin_nontemporal_load(static_cast<const u4 *>(q)); };
            if constexpr (Geo::SPLIT) {
                const float *p = static_cast<const float *>(base) + off + 4 * li;
                const u4 a = ld4(p);
                const u4 b = ld4(p + 64);
                w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
            } else {
                const uint8_t *p = static_cast<const uint8_t *>(base) + (off + (long long)F * li) * EB;
                if constexpr (WORDS == 8) {
                    const u4 a = ld4(p);
                    const u4 b = ld4(p + 16);
                    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
                } else if constexpr (WORDS == 4) {
                    const u4 a = ld4(p);
                    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                } else if constexpr (WORDS == 2) {
                    const u2 a = __builtin_nontemporal_load(reinterpret_cast<const u2 *>(p));
                    w[0] = a.x; w[1] = a.y;
                } else {
                    static_assert(WORDS == 1, "slice size");
                    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
                }
            }
        } else if constexpr (Geo::SPLIT) {
            const float *p = static_cast<const float *>(base) + off + 4 * li;
            const uint4 a = *reinterpret_cast<const uint4 *>(p);
            const uint4 b = *reinterpret_cast<const uint4 *>(p + 64);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        } else {
            const uint8_t *p = static_cast<const uint8_t *>(base) + (off + (long long)F * li) * EB;
            if constexpr (WORDS == 8) {
                const uint4 a = *reinterpret_cast<const uint4 *>(p);
                const uint4 b = *reinterpret_cast<const uint4 *>(p + 16);
                w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
            } else if constexpr (WORDS == 4) {
                const uint4 a = *reinterpret_cast<const uint4 *>(p);
                w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            } else if constexpr (WORDS == 2) {
                const uint2 a = *reinterpret_cast<const uint2 *>(p);
                w[0] = a.x; w[1] = a.y;
            } else {
                static_assert(WORDS == 1, "slice size");
                w[0] = *reinterpret_cast<const uint32_t *>(p);
            }
        }
    }
    // fp32 values (fp8: the code values; the tensor's scale is applied by
    // the caller, to q for K and to the output for V)
    __device__ __forceinline__ void to_f32(float (&f)[F]) const {
        if constexpr (DT == CK_KV_F32) {
#pragma unroll
            for (int e = 0; e < F; e++) f[e] = __uint_as_float(w[e]);
        } else if constexpr (DT == CK_KV_BF16) {
#pragma unroll
            for (int i = 0; i < WORDS; i++) {
                f[2 * i] = __uint_as_float(w[i] << 16);
                f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        } else {
            // v_cvt_pk_f32_fp8 decodes OCP E4M3 on gfx950 (checked against the
            // format's definition over all 256 codes, NaN included)
#pragma unroll
            for (int i = 0; i < WORDS; i++) {
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
                f[4 * i] = lo[0];
                f[4 * i + 1] = lo[1];
                f[4 * i + 2] = hi[0];
                f[4 * i + 3] = hi[1];
            }
        }
    }
};

template <int HD, int G, int NS>
struct Smem {
    // the online-softmax state of every row group (NS of them): unnormalized
    // outputs, running max (log2 units), sum of exponentials; then the
    // weight of each state in the combination
    // rows padded by 4 floats, so that the states of a wave's row groups do
    // not start on the same bank (measured neutral: the conflict counter
    // reads about 48% of the LDS cycles either way, the four row groups of
    // a store instruction writing a full set of banks each; the combination
    // is a small part of the kernel)
    float ro[NS][G][HD + 4];
    float rm[NS][G];
    float rl[NS][G];
    float rw[NS][G];
    int pages[kPagesLds];                   // paged caches: the chunk's page ids
    int sel[kSelLds];                       // sparse: the chunk's selection entries
    int bad;
};

// Row groups of a workgroup (the states combined at the end of an item).
template <int DT, int HD, int G>
constexpr int kAttnNS = AttnShape<G>::waves * RowGeo<DT, HD, G>::RPR;

// A partial's store: plain, or device-coherent (a relaxed agent-scope store:
// written through to where workgroups of other XCDs read it in the same
// launch).
template <bool COH>
__device__ __forceinline__ void part_store(float *p, float v) {
    if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// One work item: the chunk `item` (counted over every sequence's chunks, back
// to back) of KV head g. Each K/V row is held by a group of LPR lanes
// (RowGeo), so a wave covers 64/LPR rows per load round and keeps its rows
// in registers: no LDS staging and no barrier inside the token loop. Scores:
// per lane the partial dot products of its slice with every query head of
// the group (q slice in registers), summed over the row group with DPP.
// Every row group keeps its own online softmax (running max, sum,
// unnormalized output of its slice) over the rows it sees; at the end the
// row groups' states are combined by log-sum-exp through LDS and the chunk's
// partial is stored (COH: with device-coherent stores). Returns false, having
// stored nothing, for an item past its sequence's chunks (device positions).
template <int HD, int G, bool PAGED, int DT, bool STREAM, bool COH>
__device__ __forceinline__ bool attn_item(const AttnArgs &a, int item, int g,
                                          Smem<HD, G, kAttnNS<DT, HD, G>> &sm) {
    static_assert(HD % 64 == 0 && G >= 1 && G <= kMaxG, "shape");
    typedef Slice<DT, HD, G> SL;
    typedef RowGeo<DT, HD, G> GEO;
    constexpr int F = SL::F;
    constexpr int LPR = GEO::LPR;
    constexpr int RPR = GEO::RPR;
    constexpr int NW = AttnShape<G>::waves;
    constexpr int NT = AttnShape<G>::threads;
    constexpr int NR = AttnShape<G>::rounds;
    constexpr int WROWS = NR * RPR;                  // rows per wave per step
    constexpr int STEP = WROWS * NW;                 // tokens per workgroup step
    constexpr int NS = NW * RPR;                     // row groups of the workgroup
    static_assert(NS == kAttnNS<DT, HD, G>, "state groups");

    int s = 0;
    while (s + 1 < a.m && item >= a.first[s + 1]) s++;
    const int cidx = item - a.first[s];
    const int L = a.pos.get(s) + 1;
    const bool sparse = a.sel != nullptr;
    // The chunk's rows [t0, t1): tokens, counted from the window's first token
    // (0 without a window); sparse, the selection entries.
    int t0, t1;
    if (sparse) {
        t0 = cidx * a.chunk;
        if (t0 >= a.topk || L <= 0) return false;
        t1 = min(a.topk, t0 + a.chunk);
    } else {
        t0 = window_start(L, a.c.window) + cidx * a.chunk;
        if (t0 >= L) return false;   // device positions: items past this sequence's chunks
        t1 = min(L, t0 + a.chunk);
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & (LPR - 1), rg = lane / LPR;
    const int KV = a.c.kv_heads;

    if (tid == 0) sm.bad = 0;
    // paged: the chunk's page ids in one batch of loads, so that row
    // addresses do not wait on table reads (chunks with more pages than the
    // LDS slots read the table per row)
    int pg0 = 0;
    bool pages_in_lds = false;
    if (PAGED && !sparse) {
        const int ps = a.c.page_size;
        pg0 = t0 / ps;
        const int npg = (t1 - 1) / ps - pg0 + 1;
        pages_in_lds = npg <= kPagesLds;
        if (pages_in_lds)
            for (int i = tid; i < npg; i += NT)
                sm.pages[i] = a.c.table[(long long)s * a.c.max_pages + pg0 + i];
    }
    // sparse: the chunk's selection entries, read once
    const int32_t *sel_s = sparse ? a.sel + (size_t)s * a.topk : nullptr;
    const bool sel_in_lds = sparse && t1 - t0 <= kSelLds;
    if (sel_in_lds)
        for (int i = tid; i < t1 - t0; i += NT) sm.sel[i] = sel_s[t0 + i];
    __syncthreads();

    const size_t seq_base = PAGED ? 0 : ((size_t)s * KV + g) * a.c.capacity * HD;
    bool bad = false;
    // element offset of token t's row (t < t1); an unmapped page reads page 0
    // of the pool and marks the chunk bad
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
            if (off < 0) bad = true;      // unmapped page: the sum becomes NaN
            return off < 0 ? 0 : off;
        } else {
            // ring: slot t % capacity (t < L, so t is never negative)
            const int slot = a.c.ring ? t % a.c.capacity : t;
            return (long long)(seq_base + (size_t)slot * HD);
        }
    };
    // Rows past the chunk re-read its last row (their scores are masked), so
    // that every load is issued unconditionally: no branch around the loads
    // and no wait on the loads still in flight. okbits: bit r set where row r
    // is attended. Sparse: an absent entry (-1) reads the first row of the
    // buffer and is masked; an entry past the sequence or no longer held by
    // a ring marks the chunk bad.
    uint32_t okbits = 0;
    auto fetch = [&](SL (&k)[NR], SL (&v)[NR], int st) {
        okbits = 0;
#pragma unroll
        for (int r = 0; r < NR; r++) {
            const int row = st + wave * WROWS + r * RPR + rg;
            const int e = min(row, t1 - 1);
            bool ok = row < t1;
            long long off;
            if (sparse) {
                const int t = sel_in_lds ? sm.sel[e - t0] : sel_s[e];
                bool held = t >= 0 && t < L;
                if (!PAGED && a.c.ring) held = held && t >= L - a.c.capacity;
                if (t >= 0 && !held) bad = true;
                ok = ok && held;
                off = held ? row_off(t) : (long long)seq_base;
            } else {
                off = row_off(e);
            }
            okbits |= (ok ? 1u : 0u) << r;
            k[r].template load<STREAM>(a.c.k, off, li);
            v[r].template load<STREAM>(a.c.v, off, li);
        }
    };

    SL ka[NR], va[NR];
    fetch(ka, va, t0);                               // first rows in flight before q

    // the q slice of every head of the group, pre-scaled so that scores are
    // in log2 units
    float qr[G][F];
    {
        // fp8: the K scale folded in here (scores = q . (code * k_scale))
        const float qs = a.scale * kLog2e * (DT == CK_KV_FP8_E4M3 ? a.c.k_scale : 1.0f);
        const float *qg = a.q + ((size_t)s * a.H + (size_t)g * G) * HD;
#pragma unroll
        for (int j = 0; j < G; j++) {
#pragma unroll
            for (int e = 0; e < F; e += 4) {
                const float4 v4 = *reinterpret_cast<const float4 *>(qg + j * HD + SL::col(li, e));
                qr[j][e] = v4.x * qs;
                qr[j][e + 1] = v4.y * qs;
                qr[j][e + 2] = v4.z * qs;
                qr[j][e + 3] = v4.w * qs;
            }
        }
    }

    float m[G], l[G], o[G][F];
#pragma unroll
    for (int j = 0; j < G; j++) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
#pragma unroll
        for (int e = 0; e < F; e++) o[j][e] = 0.0f;
    }

    // The online softmax advances over the step's rows in batches of SUB
    // rows (scores, running max and sum, then P.V), which bounds the score
    // registers whatever the rows per step.
    constexpr int SUB = AttnShape<G>::sub;
    // MASKED: some row of the step lies outside the chunk (or is an absent
    // selection entry) somewhere in the wave; steps where every row is
    // attended skip the masking selects.
    auto compute = [&](const SL (&k)[NR], const SL (&v)[NR], auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
        for (int r0 = 0; r0 < NR; r0 += SUB) {
            float sc[SUB][G];
            bool ok[SUB];                            // row inside the chunk
#pragma unroll
            for (int r = 0; r < SUB; r++) {
                ok[r] = (okbits >> (r0 + r)) & 1u;
                float kf[F];
                k[r0 + r].to_f32(kf);
#pragma unroll
                for (int j = 0; j < G; j++) {
                    float acc = 0.0f;
#pragma unroll
                    for (int e = 0; e < F; e++) acc = fmaf(qr[j][e], kf[e], acc);
                    sc[r][j] = group_sum<LPR>(acc);
                    if constexpr (MASKED) sc[r][j] = ok[r] ? sc[r][j] : -INFINITY;
                }
            }
            float p[SUB][G];
#pragma unroll
            for (int j = 0; j < G; j++) {
                float mx = sc[0][j];
#pragma unroll
                for (int r = 1; r < SUB; r++) mx = fmaxf(mx, sc[r][j]);
                const float mn = fmaxf(m[j], mx);
                const float mr = mn == -INFINITY ? 0.0f : mn;
                const float alpha = exp2f(m[j] - mr);
                float ps = 0.0f;
#pragma unroll
                for (int r = 0; r < SUB; r++) {
                    p[r][j] = exp2f(sc[r][j] - mr);
                    ps += p[r][j];
                }
                l[j] = l[j] * alpha + ps;
                m[j] = mn;
#pragma unroll
                for (int e = 0; e < F; e++) o[j][e] *= alpha;
            }
#pragma unroll
            for (int r = 0; r < SUB; r++) {
                float vf[F];
                v[r0 + r].to_f32(vf);
                // a row past the chunk (a re-read of its last row) adds
                // nothing, also where that row holds an infinity
                if constexpr (MASKED) {
#pragma unroll
                    for (int e = 0; e < F; e++) vf[e] = ok[r] ? vf[e] : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < G; j++) {
#pragma unroll
                    for (int e = 0; e < F; e++) o[j][e] = fmaf(p[r][j], vf[e], o[j][e]);
                }
            }
        }
    };

    // One register set per step: a step's loads are all issued, then waited
    // for and computed on. (A second set for the next step's loads does not
    // stay in flight across the loop: the compiler waits for every load at
    // the loop head.)
    // The unmasked copy of the step costs registers; it is kept where two
    // workgroups per CU still fit (small query groups, fp32 and bf16 rows).
    constexpr bool kTwoBodies = G <= 4 && DT != CK_KV_FP8_E4M3;
    constexpr uint32_t kAllRows = (1u << NR) - 1u;
    for (int st = t0;;) {
        if (kTwoBodies && __builtin_amdgcn_ballot_w64(okbits != kAllRows) == 0)
            compute(ka, va, std::integral_constant<bool, !kTwoBodies>{});
        else
            compute(ka, va, std::true_type{});
        st += STEP;
        if (st >= t1) break;
        fetch(ka, va, st);
    }

    // Every row group's state goes to LDS as it is (no cross-lane exchange),
    // then the chunk's state is their log-sum-exp combination: per head the
    // largest max M, each state's weight 2^(m - M), the weighted sums.
    const int sid = wave * RPR + rg;
    if (bad) sm.bad = 1;
#pragma unroll
    for (int j = 0; j < G; j++) {
#pragma unroll
        for (int e = 0; e < F; e += 4)
            *reinterpret_cast<float4 *>(&sm.ro[sid][j][SL::col(li, e)]) =
                make_float4(o[j][e], o[j][e + 1], o[j][e + 2], o[j][e + 3]);
        if (li == 0) {
            sm.rm[sid][j] = m[j];
            sm.rl[sid][j] = l[j];
        }
    }
    __syncthreads();
    const size_t part = ((size_t)s * KV + g) * a.nchunks + cidx;
    // one lane per (head, state), the NS states of a head in one aligned lane
    // group: the max and the weighted sum are group reductions
    static_assert(NS <= kWave && (NS & (NS - 1)) == 0 && G * NS <= NT, "state groups");
    if (tid < G * NS) {
        const int j = tid / NS, i = tid % NS;
        const float mi = sm.rm[i][j];
        const float M = group_max<NS>(mi);
        const float Mr = M == -INFINITY ? 0.0f : M;
        const float w = exp2f(mi - Mr);
        sm.rw[i][j] = w;
        const float ls = group_sum<NS>(sm.rl[i][j] * w);
        if (i == 0) {
            part_store<COH>(&a.pml[(part * G + j) * 2 + 0], M);
            part_store<COH>(&a.pml[(part * G + j) * 2 + 1], sm.bad ? NAN : ls);
        }
    }
    __syncthreads();
    // fp8: the V scale applied once to the weighted sum of code values
    const float vsc = DT == CK_KV_FP8_E4M3 ? a.c.v_scale : 1.0f;
    for (int idx = tid; idx < G * HD; idx += NT) {
        const int j = idx / HD, c = idx % HD;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NS; i++) acc = fmaf(sm.ro[i][j][c], sm.rw[i][j], acc);
        part_store<COH>(&a.po[part * G * HD + idx], acc * vsc);
    }
    return true;
}

// --------------------------------------------------------------------------
// The item on the fp32 matrix cores, for query groups of 5..8 heads over an
// fp32 cache (no selection). There the group makes the scores Q K^T and the
// weighted sum P V small dense contractions, and the vector path above is
// bound by instruction issue: every score needs a 16-lane reduction, and
// with one wave per SIMD nothing hides the dependent chains. Here a wave
// takes 16 tokens per tile, and v_mfma_f32_16x16x4f32 computes
//   S^T[token][head] = sum_d K[token][d] q[head][d]     (HD/4 instructions)
//   O^T[dim][head]  += sum_t V[t][dim] P[t][head]        (HD/4 instructions)
// with the group's heads in the 16 columns (heads >= G are zero). Lane l
// (hl = l % 16, kq = l / 16) holds, by the operand layout of the
// instruction (checked on the device): for the scores, at step 4j + e, K
// of token hl and q of head hl at dim 16j + 4kq + e (a contraction may
// visit its index in any order: this one lets the four lanes of a token
// read 64 adjacent bytes of its row per load); it receives the scores of
// tokens 4*kq + r (r < 4) for head hl. For P V, step s (< 4) contracts
// tokens 4*kq + s, so the lane's own probability p[s] is its B operand, and
// its A operand is V of that token at dims 64b + 4hl + e for the VD output
// tiles T = 4b + e (tile T covers dims 64b + 4m + e, m < 16; the 16 lanes
// of a token read 256 adjacent bytes of its row per load): the lane ends
// holding, for head hl, dims 64b + 16kq + 4r + e. The softmax statistics of
// a head are reduced over r in the lane and over kq with two cross-lane
// exchanges. Each wave keeps one online softmax per head; the NW waves'
// states are combined through LDS as above. A workgroup has one wave per
// 16-token tile of its chunk (at most 8; longer chunks give a wave every
// NW-th tile).
template <int HD, int G, int NW, int HF = 1>
struct alignas(16) SmemM {
    // wave states: one per tile wave, or per wave where the two waves of a
    // tile split its tokens (HF = 2 with 64-wide heads)
    static constexpr int NST = (HF == 2 && HD == 64) ? 2 * NW : NW;
    float ro[NST][G][HD + 4];
    float rm[NST][G];
    float rl[NST][G];
    alignas(16) float sx[HF == 2 ? NW : 1][HF][kWave][4];   // HF = 2: the halves' partial scores
    int pages[kPagesLds];
    int bad;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

//
// HF = 2 (chunks of at most NW tiles): two waves per tile, wave hf
// contracting head dims [hf HD/2, (hf + 1) HD/2) for the scores (the two
// partial score tiles are added through LDS, in the same order in both
// waves), so each wave issues half the score MFMAs after its loads land.
// P V: with 128-wide heads wave hf produces those output dims; with 64-wide
// heads (a single 64-dim output tile group, which 16-byte V loads cannot
// split) it contracts half of the tile's tokens (steps 2hf, 2hf + 1) and the
// two waves' sums are added as two states with the same max. Every wave
// takes exactly one tile (a tile past the chunk is fully masked), so the
// exchange's barrier is reached by all.
template <int HD, int G, int NW, bool PAGED, bool STREAM, bool COH, int HF = 1>
__device__ __forceinline__ bool attn_item_mfma(const AttnArgs &a, int item, int g,
                                               SmemM<HD, G, NW, HF> &sm) {
    static_assert(HD == 64 || HD == 128, "head size");
    static_assert(G >= 1 && G <= 16 && NW >= 1 && NW <= 8, "query group, waves");
    static_assert(HF == 1 || HF == 2, "dim halves");
    constexpr bool TSPLIT = HF == 2 && HD == 64;   // P V split over tokens
    constexpr int NT = NW * HF * kWave;
    constexpr int KD = HD / 4 / HF;   // dims of a K row per lane (one per MFMA step)
    constexpr int VD = TSPLIT ? HD / 16 : HD / 16 / HF;   // V dims per lane; output tiles
    constexpr int NVR = TSPLIT ? 2 : 4;                   // V rows per lane (P V steps)
    int s = 0;
    while (s + 1 < a.m && item >= a.first[s + 1]) s++;
    const int cidx = item - a.first[s];
    const int L = a.pos.get(s) + 1;
    const int t0 = window_start(L, a.c.window) + cidx * a.chunk;
    if (t0 >= L) return false;       // device positions: items past this sequence's chunks
    const int t1 = min(L, t0 + a.chunk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wid % NW, hf = wid / NW;    // tile wave, dim half
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
    const int d0 = hf * (HD / HF);               // the half's first head dim
    const int dv0 = TSPLIT ? 0 : d0;             // its first output dim
    const int sv0 = TSPLIT ? 2 * hf : 0;         // its first P V step
    const int slot0 = (!PAGED && a.c.ring) ? t0 % a.c.capacity : t0;
    bool bad = false;
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
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    auto ld4 = [](const float *p) -> float4 {
        if constexpr (STREAM) {
            const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(p));
            return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                               __uint_as_float(v.w));
        } else {
            return *reinterpret_cast<const float4 *>(p);
        }
    };
    const float *Kc = static_cast<const float *>(a.c.k);
    const float *Vc = static_cast<const float *>(a.c.v);

    // q of head hl at the dims of the lane's K pieces: 16j + 4kq + e for
    // step 4j + e. The padding heads (hl >= G) repeat head G - 1: their
    // columns are never read, and stay finite. The scale (with log2 e) is
    // applied to the scores, so that nothing waits for q before the K/V
    // loads go out.
    float qr[KD];
    {
        const float *qh = a.q + ((size_t)s * a.H + (size_t)g * G + min(hl, G - 1)) * HD + d0 + 4 * kq;
#pragma unroll
        for (int i = 0; i < KD; i += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(qh + 4 * i);
            qr[i] = v.x;
            qr[i + 1] = v.y;
            qr[i + 2] = v.z;
            qr[i + 3] = v.w;
        }
    }
    const float qs = a.scale * kLog2e;

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 o[VD];
#pragma unroll
    for (int T = 0; T < VD; T++) o[T] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ntile = (t1 - t0 + 15) / 16;
    // HF = 2: one pass for every wave (the launcher keeps a chunk within NW
    // tiles; a tile past the chunk reads its last row, fully masked)
    for (int tile = wave; HF == 2 ? tile == wave : tile < ntile; tile += NW) {
        const int tb = t0 + 16 * tile;
        // every load first, unconditional (tokens past the chunk re-read its
        // last row and are masked). K of token tb + hl: the four lanes of a
        // row read 64 adjacent bytes per instruction (dims 16j + 4kq..), 16
        // rows per instruction. V of tokens tb + 4kq + sidx: the 16 lanes of
        // a row read 256 adjacent bytes per instruction (dims 64b + 4hl..),
        // 4 rows per instruction.
        float kr[KD];
        {
            const float *kp = Kc + row_off(min(tb + hl, t1 - 1)) + d0 + 4 * kq;
#pragma unroll
            for (int i = 0; i < KD; i += 4) {
                const float4 v = ld4(kp + 4 * i);
                kr[i] = v.x;
                kr[i + 1] = v.y;
                kr[i + 2] = v.z;
                kr[i + 3] = v.w;
            }
        }
        float vr[NVR][VD];
#pragma unroll
        for (int sv = 0; sv < NVR; sv++) {
            const int sidx = sv0 + sv;
            const float *vp = Vc + row_off(min(tb + 4 * kq + sidx, t1 - 1)) + dv0 + 4 * hl;
#pragma unroll
            for (int T = 0; T < VD; T += 4) {
                const float4 v = ld4(vp + 16 * T);
                vr[sv][T] = v.x;
                vr[sv][T + 1] = v.y;
                vr[sv][T + 2] = v.z;
                vr[sv][T + 3] = v.w;
            }
        }
        // keep the loads together ahead of the arithmetic (left alone, the
        // scheduler spreads them among the MFMAs and waits for each)
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KD; i++) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i], qr[i], sc, 0, 0, 0);
        if constexpr (HF == 2) {
            // the whole dot: half 0's partial plus half 1's, in both waves
            *reinterpret_cast<f32x4 *>(sm.sx[wave][hf][lane]) = sc;
            __syncthreads();
            const f32x4 p0 = *reinterpret_cast<const f32x4 *>(sm.sx[wave][0][lane]);
            const f32x4 p1 = *reinterpret_cast<const f32x4 *>(sm.sx[wave][1][lane]);
            sc = p0 + p1;
        }
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; r++) sv[r] = (tb + 4 * kq + r < t1) ? sc[r] * qs : -INFINITY;
        float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m_run, mt);
        const float mr = mn == -INFINITY ? 0.0f : mn;
        const float alpha = exp2f(m_run - mr);
        float p[4], ps = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            p[r] = exp2f(sv[r] - mr);
            ps += p[r];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        m_run = mn;
        // V of a token past the chunk adds nothing (it re-reads a row that
        // may hold anything, an infinity included)
#pragma unroll
        for (int sv = 0; sv < NVR; sv++) {
            const bool ok = tb + 4 * kq + sv0 + sv < t1;
#pragma unroll
            for (int T = 0; T < VD; T++) vr[sv][T] = ok ? vr[sv][T] : 0.0f;
        }
#pragma unroll
        for (int T = 0; T < VD; T++) {
            o[T] *= alpha;
#pragma unroll
            for (int sv = 0; sv < NVR; sv++)
                o[T] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[sv][T], p[sv0 + sv], o[T], 0, 0, 0);
        }
    }

    // the waves' states through LDS: o[4b + e][r] is dim 64b + 16kq + 4r + e
    // (token halves: each wave its own state, the same max, the sum once)
    constexpr int NST = SmemM<HD, G, NW, HF>::NST;
    const int st = TSPLIT ? 2 * wave + hf : wave;
    if (bad) sm.bad = 1;
    if (hl < G) {
#pragma unroll
        for (int r = 0; r < 4; r++)
#pragma unroll
            for (int T = 0; T < VD; T += 4)
                *reinterpret_cast<float4 *>(&sm.ro[st][hl][dv0 + 16 * T + 16 * kq + 4 * r]) =
                    make_float4(o[T][r], o[T + 1][r], o[T + 2][r], o[T + 3][r]);
        if (kq == 0 && (TSPLIT || hf == 0)) {
            sm.rm[st][hl] = m_run;
            sm.rl[st][hl] = hf == 0 ? l_run : 0.0f;
        }
    }
    __syncthreads();
    // every thread weighs the waves' states of its own output slice (the
    // same arithmetic for every slice of a head, so no second barrier):
    // partials of the chunk, and the chunk's (max, sum) from each head's
    // first slice
    const size_t part = ((size_t)s * KV + g) * a.nchunks + cidx;
    const bool any_bad = sm.bad != 0;
    for (int i4 = tid; i4 < G * HD / 4; i4 += NT) {
        const int j = i4 / (HD / 4), c = 4 * (i4 % (HD / 4));
        float M = sm.rm[0][j];
#pragma unroll
        for (int w = 1; w < NST; w++) M = fmaxf(M, sm.rm[w][j]);
        const float Mr = M == -INFINITY ? 0.0f : M;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float ls = 0.0f;
#pragma unroll
        for (int w = 0; w < NST; w++) {
            const float wt = exp2f(sm.rm[w][j] - Mr);
            ls = fmaf(sm.rl[w][j], wt, ls);
            const float4 v = *reinterpret_cast<const float4 *>(&sm.ro[w][j][c]);
            acc = make_float4(fmaf(v.x, wt, acc.x), fmaf(v.y, wt, acc.y), fmaf(v.z, wt, acc.z),
                              fmaf(v.w, wt, acc.w));
        }
        float *po = &a.po[part * G * HD + (size_t)j * HD + c];
        part_store<COH>(po + 0, acc.x);
        part_store<COH>(po + 1, acc.y);
        part_store<COH>(po + 2, acc.z);
        part_store<COH>(po + 3, acc.w);
        if (c == 0) {
            part_store<COH>(&a.pml[(part * G + j) * 2 + 0], M);
            part_store<COH>(&a.pml[(part * G + j) * 2 + 1], any_bad ? NAN : ls);
        }
    }
    return true;
}

}  // namespace attn

// The attention over a bf16 or fp8 cache on the bf16 matrix cores (no
// selection): grid and partials as the vector kernel's (k_attn16.hip).
hipError_t launch_attn_mfma16(const attn::AttnArgs &a, int G, int hd, dim3 grid, bool paged,
                              hipStream_t st);

}  // namespace ck
