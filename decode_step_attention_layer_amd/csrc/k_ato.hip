// k_ato.hip — the second half of the layer in one launch: split-K grouped-query
// attention, the log-sum-exp merge with the Q8_0 quantization of the
// attention output, and the O projection + bias + residual (C-Kernel-Engine
// "mega_fused_attention_decode_q5_0.c", MAIN KERNEL steps 7-8).
//
// The grid holds three kinds of workgroups, in this order of ids:
//   attention  one (chunk, KV head) item each, exactly as the attention kernel
//              computes it (ck_attn_common.hpp), its partial stored with
//              device-coherent stores, then counted done for its (sequence,
//              KV head);
//   merge      one (sequence, query head): waits until every chunk of its KV
//              head is counted, merges the partials (coherent loads), writes
//              the attention output, its Q8_0 blocks and a dword-aligned
//              staged copy of them (codes, fp32 scale, code sum; coherent
//              stores) for the O projection, then counts itself done;
//   O          a group of output rows: loads its Wo rows, bias and residual
//              first (they depend on nothing), waits until every merge is
//              counted, then stages each token's quantized attention output
//              into LDS and computes its rows.
// A workgroup waits only for workgroups with smaller ids. Each XCD starts its
// workgroups in id order, so the smallest unfinished workgroup is always
// resident and never waits on an unfinished one: the launch cannot deadlock,
// however few of its workgroups fit at once. Every wait is a bounded spin; on
// time-out the status word is set and the workgroup goes on (its outputs are
// then undefined), so the launch always ends.
//
// Data crosses workgroups (and XCDs) only through relaxed agent-scope loads
// and stores, which gfx950 issues as plain vector accesses coherent at device
// level (no L2 write-back or invalidate): a producer waits for its stores to
// complete, passes a barrier, then increments the counter; a consumer reads
// the counter before it issues the loads. The counters are cleared by the
// launch before this one (the Q/K/V projection), so nothing has to be zero
// when the layer starts.
#include "ck_attn_common.hpp"
#include "ck_gemv_common.hpp"

namespace ck {

namespace {

using namespace attn;

constexpr int kAtoThreads = 256;
constexpr int kAtoWaves = kAtoThreads / kWave;
constexpr int kOR = 4;              // O rows per wave
constexpr int kOUPL = 2;            // O block pairs per lane: rows of up to 8192 inputs
constexpr int kAtoMaxChunks = 1024; // chunks per (sequence, KV head) the merge phase holds
constexpr unsigned kAtoSpins = 1u << 22;
// Words from one counter to the next: each on a cache line of its own. With
// every counter on one line, the line that ~250 workgroups poll and
// increment became a hot spot: measured, waits then ended 5-7 us after
// their count was reached (1.3-1.8 us with a line each).
constexpr int kCS = 64;

struct AtoArgs {
    AttnArgs at;              // attention items; partials in at.po / at.pml
    int n_att, n_mrg;         // first merge workgroup = n_att, first O one = n_att + n_mrg
    int window;               // the cache's window (0 = none): chunks count from its start
    float *attn;              // [m][H][HD] attention output
    uint8_t *aq;              // [m][H*HD/32] its Q8_0 blocks
    XBlock *aqx;              // [m][H*HD/32] the same, staged (codes, fp32 scale, code sum)
    const uint8_t *wo;        // Q5_0 [D][H*HD]
    const float *bo;          // nullable
    const float *residual;    // nullable, [m][D]
    float *out;               // [m][D]
    int D;
    unsigned *cnt;            // counters kCS words apart: chunks done per (sequence, KV
                              // head) [m*KV], merges done, status
};

template <int HD, int NS>
struct MrgSmem {
    float w[kAtoMaxChunks];   // chunk weights 2^(m_c - M)
    float l[kAtoMaxChunks];   // chunk sums
    float red[kAtoWaves];
    alignas(16) float part[kAtoThreads / (HD / 4)][HD];   // float4 per (chunk group, 4 dims)
};

template <int HD, int G, int DT>
union AtoSmem {
    Smem<HD, G, kAttnNS<DT, HD, G>> att;
    MrgSmem<HD, kAttnNS<DT, HD, G>> mrg;
    XBlock xs[2 * kOUPL * kWave];   // one token's quantized attention output (O phase)
};

// Waits (thread 0 spinning, the workgroup at a barrier) until *c >= target.
// SLEEP: s_sleep units (64 clocks) between polls; the O workgroups, which
// wait through the whole attention, poll less often.
template <int SLEEP>
__device__ __forceinline__ void wait_count(const unsigned *c, unsigned target, unsigned *status) {
    if (threadIdx.x == 0) {
        unsigned n = 0;
        while (ld_cu(c) < target) {
            if (++n > kAtoSpins) {
                st_cu(status, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(SLEEP);
        }
    }
    __syncthreads();
}

// Completes this workgroup's coherent stores, then counts it done.
__device__ __forceinline__ void signal_done(unsigned *c) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void st_cf(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ci(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of query head h of sequence s: the chunks' (max, sum) pairs give the
// global max M and the denominator; thread (4 dims, chunk group) accumulates
// its chunks' weighted outputs; the groups are summed through LDS; the HD/4
// threads of the result write it, its Q8_0 blocks and their staged copy.
template <int HD, int NS>
__device__ void merge_item(const AtoArgs &a, int s, int h, MrgSmem<HD, NS> &sm) {
    constexpr int C4 = HD / 4;
    constexpr int CG = kAtoThreads / C4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.at.H, KV = a.at.c.kv_heads, G = H / KV, g = h / G, j = h % G;
    const int L = a.at.pos.get(s) + 1;
    const int n = L - window_start(L, a.window);
    const int nc = n > 0 ? (n + a.at.chunk - 1) / a.at.chunk : 0;
    const size_t base = ((size_t)s * KV + g) * a.at.nchunks;
    unsigned *status = a.cnt + (a.at.m * KV + 1) * kCS;
    wait_count<1>(a.cnt + (s * KV + g) * kCS, (unsigned)nc, status);

    // Every load that does not depend on another goes out at once, none of
    // them conditional (slots past the last chunk re-read it and are not
    // used): this thread's first (max, sum) pair, then its first kPre
    // chunks' output slices.
    constexpr int kPre = 8;
    const int d4 = tid % C4, cg = tid / C4;
    const int ncl = nc > 0 ? nc - 1 : 0;
    const float2 ml0 = ld_c2(&a.at.pml[((base + min(tid, ncl)) * G + j) * 2]);
    float4 pre[kPre];
#pragma unroll
    for (int i = 0; i < kPre; i++)
        pre[i] = ld_c4(&a.at.po[((base + min(cg + i * CG, ncl)) * G + j) * HD + 4 * d4]);
    __builtin_amdgcn_sched_barrier(0);

    float mx = -INFINITY;
    if (tid < nc) {
        sm.w[tid] = ml0.x;
        sm.l[tid] = ml0.y;
        mx = ml0.x;
    }
    for (int c = tid + kAtoThreads; c < nc; c += kAtoThreads) {
        const float2 ml = ld_c2(&a.at.pml[((base + c) * G + j) * 2]);
        sm.w[c] = ml.x;
        sm.l[c] = ml.y;
        mx = fmaxf(mx, ml.x);
    }
    mx = wave_max(mx);
    if (lane == 0) sm.red[wave] = mx;
    __syncthreads();
    float M = sm.red[0];
#pragma unroll
    for (int i = 1; i < kAtoWaves; i++) M = fmaxf(M, sm.red[i]);
    const float Mr = M == -INFINITY ? 0.0f : M;
    __syncthreads();
    float den = 0.0f;
    for (int c = tid; c < nc; c += kAtoThreads) {
        const float w = exp2f(sm.w[c] - Mr);
        sm.w[c] = w;
        den = fmaf(w, sm.l[c], den);
    }
    den = wave_sum(den);
    if (lane == 0) sm.red[wave] = den;
    __syncthreads();
    float D = 0.0f;
#pragma unroll
    for (int i = 0; i < kAtoWaves; i++) D += sm.red[i];

    auto fma4 = [](float w, float4 v, float4 acc) {
        return make_float4(fmaf(w, v.x, acc.x), fmaf(w, v.y, acc.y), fmaf(w, v.z, acc.z),
                           fmaf(w, v.w, acc.w));
    };
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kPre; i++) {
        const int c = cg + i * CG;
        if (c < nc) acc = fma4(sm.w[c], pre[i], acc);
    }
    for (int c = cg + kPre * CG; c < nc; c += CG)
        acc = fma4(sm.w[c], ld_c4(&a.at.po[((base + c) * G + j) * HD + 4 * d4]), acc);
    *reinterpret_cast<float4 *>(&sm.part[cg][4 * d4]) = acc;
    __syncthreads();
    if (tid < C4) {
        float4 t = *reinterpret_cast<const float4 *>(&sm.part[0][4 * tid]);
#pragma unroll
        for (int i = 1; i < CG; i++) {
            const float4 u = *reinterpret_cast<const float4 *>(&sm.part[i][4 * tid]);
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        // D == 0: nothing attended, the output is zero; a NaN D (a chunk that
        // read an unmapped page) stays NaN
        const float inv = D == 0.0f ? 0.0f : 1.0f / D;
        const float4 v = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
        const size_t oi = ((size_t)s * H + h) * HD + 4 * tid;
        *reinterpret_cast<float4 *>(&a.attn[oi]) = v;
        uint32_t packed;
        uint16_t dbits;
        quantize_q8_0_x4_codes(v, packed, dbits);
        float csum = (float)(int8_t)(packed & 0xFF) + (float)(int8_t)((packed >> 8) & 0xFF) +
                     (float)(int8_t)((packed >> 16) & 0xFF) + (float)(int8_t)(packed >> 24);
        csum = group_sum<8>(csum);
        const size_t b = oi / kQK;
        const int sub = tid & 7;
        uint8_t *blk = a.aq + b * kQ8Bytes;
        uint16_t *dst = reinterpret_cast<uint16_t *>(blk + 2 + 4 * sub);
        dst[0] = (uint16_t)(packed & 0xFFFF);
        dst[1] = (uint16_t)(packed >> 16);
        if (sub == 0) *reinterpret_cast<uint16_t *>(blk) = dbits;
        XBlock *xb = a.aqx + b;
        st_ci(&xb->c[sub], (int)packed);
        if (sub == 0) {
            st_cf(&xb->d, half_bits_to_float(dbits));
            st_ci(&xb->sum, (int)csum);
        }
    }
    signal_done(a.cnt + a.at.m * KV * kCS);
}

// O rows of workgroup o: wave w owns rows (o * waves + w) * kOR + r; a row
// is owned by the whole wave, lane l holding block pairs l and l + 64.
// Weights, bias and the first token's residual load before the wait.
__device__ void o_item(const AtoArgs &a, int o, XBlock *xs) {
    using F = Fmt<true, true>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = a.at.H * a.at.c.head_dim, nb = K / kQK, nunits = nb / 2;
    const size_t row_bytes = (size_t)nb * kQ5Bytes;
    const int row0 = (o * kAtoWaves + wave) * kOR;
    const int m = a.at.m;
    uint32_t wr[kOR][kOUPL][F::words];
#pragma unroll
    for (int r = 0; r < kOR; r++) {
        const int row = min(row0 + r, a.D - 1);
        const uint8_t *rp = a.wo + (size_t)row * row_bytes;
#pragma unroll
        for (int u = 0; u < kOUPL; u++) {
            const int unit = min(lane + u * kWave, nunits - 1);
            load_unit<true, true>(rp + (size_t)unit * F::bytes, wr[r][u]);
        }
    }
    float bias_v[kOR], res0[kOR];
#pragma unroll
    for (int r = 0; r < kOR; r++) {
        const int row = min(row0 + r, a.D - 1);
        bias_v[r] = a.bo ? a.bo[row] : 0.0f;
        res0[r] = a.residual ? a.residual[row] : 0.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_count<8>(a.cnt + m * a.at.c.kv_heads * kCS, (unsigned)a.n_mrg,
                  a.cnt + (m * a.at.c.kv_heads + 1) * kCS);

    for (int s = 0; s < m; s++) {
        // this token's staged blocks into LDS (coherent loads, 8 bytes each)
        const int nw = nb * (int)(sizeof(XBlock) / 8);
        const unsigned long long *src =
            reinterpret_cast<const unsigned long long *>(a.aqx + (size_t)s * nb);
        unsigned long long *dst = reinterpret_cast<unsigned long long *>(xs);
        for (int i = threadIdx.x; i < nw; i += kAtoThreads)
            dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        XBlock xb[kOUPL][2];
#pragma unroll
        for (int u = 0; u < kOUPL; u++) {
            const int unit = lane + u * kWave;
#pragma unroll
            for (int b = 0; b < 2; b++) {
                if (unit < nunits)
                    xb[u][b] = xs[2 * unit + b];
                else
                    xb[u][b] = XBlock{{0, 0, 0, 0, 0, 0, 0, 0}, 0.0f, 0, {0, 0}};
            }
        }
#pragma unroll
        for (int r = 0; r < kOR; r++) {
            float acc = 0.0f;
#pragma unroll
            for (int u = 0; u < kOUPL; u++) acc = unit_dot<true, true>(wr[r][u], xb[u], acc);
            acc = row_reduce<kWave>(acc);
            const int row = row0 + r;
            if (lane == 0 && row < a.D) {
                float v = acc + bias_v[r];
                if (a.residual) v = v + (s == 0 ? res0[r] : a.residual[(size_t)s * a.D + row]);
                a.out[(size_t)s * a.D + row] = v;
            }
        }
        __syncthreads();   // xs is rewritten for the next token
    }
}

template <int HD, int G, bool PAGED, int DT, bool STREAM>
__global__ __launch_bounds__(kAtoThreads) void k_ato(AtoArgs a) {
    static_assert(AttnShape<G>::threads == kAtoThreads, "one workgroup shape for every phase");
    __shared__ AtoSmem<HD, G, DT> sm;
    const int wg = blockIdx.x;
    if (wg < a.n_att) {
        const int items = a.at.first[a.at.m];
        const int item = wg % items, g = wg / items;
        int s = 0;
        while (s + 1 < a.at.m && item >= a.at.first[s + 1]) s++;
        if (attn_item<HD, G, PAGED, DT, STREAM, true>(a.at, item, g, sm.att))
            signal_done(a.cnt + (s * a.at.c.kv_heads + g) * kCS);
    } else if (wg < a.n_att + a.n_mrg) {
        const int i = wg - a.n_att;
        merge_item<HD, kAttnNS<DT, HD, G>>(a, i / a.at.H, i % a.at.H, sm.mrg);
    } else {
        o_item(a, wg - a.n_att - a.n_mrg, sm.xs);
    }
}

template <int HD, int G>
hipError_t launch_t(const AtoArgs &a, int nblocks, bool paged, hipStream_t st) {
    const int dt = a.at.c.dtype;
    // the attention kernel's streaming rule (non-temporal K/V loads except
    // in short chunks of large query groups with 128-wide heads)
    const bool nt = a.at.chunk >= 256 || !(HD == 128 && G > 4);
#define CK_ATO_LAUNCH(P, D)                                                                      \
    do {                                                                                         \
        if (nt) hipLaunchKernelGGL((k_ato<HD, G, P, D, true>), dim3(nblocks), dim3(kAtoThreads), \
                                   0, st, a);                                                    \
        else hipLaunchKernelGGL((k_ato<HD, G, P, D, false>), dim3(nblocks), dim3(kAtoThreads),   \
                                0, st, a);                                                       \
    } while (0)
    if (paged) {
        if (dt == CK_KV_BF16) CK_ATO_LAUNCH(true, CK_KV_BF16);
        else if (dt == CK_KV_FP8_E4M3) CK_ATO_LAUNCH(true, CK_KV_FP8_E4M3);
        else CK_ATO_LAUNCH(true, CK_KV_F32);
    } else {
        if (dt == CK_KV_BF16) CK_ATO_LAUNCH(false, CK_KV_BF16);
        else if (dt == CK_KV_FP8_E4M3) CK_ATO_LAUNCH(false, CK_KV_FP8_E4M3);
        else CK_ATO_LAUNCH(false, CK_KV_F32);
    }
#undef CK_ATO_LAUNCH
    return hipGetLastError();
}

template <int HD>
hipError_t launch_g(const AtoArgs &a, int nblocks, int G, bool paged, hipStream_t st) {
    switch (G) {
        case 1: return launch_t<HD, 1>(a, nblocks, paged, st);
        case 2: return launch_t<HD, 2>(a, nblocks, paged, st);
        case 3: return launch_t<HD, 3>(a, nblocks, paged, st);
        case 4: return launch_t<HD, 4>(a, nblocks, paged, st);
        case 5: return launch_t<HD, 5>(a, nblocks, paged, st);
        case 6: return launch_t<HD, 6>(a, nblocks, paged, st);
        case 7: return launch_t<HD, 7>(a, nblocks, paged, st);
        case 8: return launch_t<HD, 8>(a, nblocks, paged, st);
    }
    return hipErrorInvalidValue;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Counters, kCS words apart: chunks done per (sequence, KV head), merges
// done, the status word.
size_t ato_counter_words(int m, int KV) { return ((size_t)m * KV + 2) * kCS; }
size_t ato_status_word(int m, int KV) { return ((size_t)m * KV + 1) * kCS; }
int ato_counters(int m, int KV) { return m * KV + 2; }
int ato_counter_stride() { return kCS; }

bool ato_supported(int H, int hd, int nchunks) {
    const int nb = H * hd / kQK;
    return nb % 2 == 0 && nb / 2 <= kOUPL * kWave && nchunks <= kAtoMaxChunks;
}

hipError_t launch_ato(const float *q, const CacheView &c, const Positions &pos, int m, int H,
                      float scale, const AttnPlan &plan, void *partials, float *attn_out,
                      uint8_t *aq, void *aqx, const uint8_t *wo, const float *bo,
                      const float *residual, float *out, int D, unsigned *cnt, hipStream_t st) {
    AtoArgs a;
    AttnArgs &t = a.at;
    t.q = q;
    t.c = c;
    t.pos = pos;
    t.scale = scale;
    t.chunk = plan.chunk;
    t.nchunks = plan.nchunks;
    t.H = H;
    uint8_t *base = static_cast<uint8_t *>(partials);
    t.po = reinterpret_cast<float *>(base);
    t.pml = reinterpret_cast<float *>(base + up256(sizeof(float) * (size_t)m * H * plan.nchunks *
                                                   c.head_dim));
    t.m = m;
    t.sel = nullptr;
    t.topk = 0;
    const int items = attn_first(pos, c.window, plan, m, false, t.first);
    if (items < 1) return hipErrorInvalidValue;
    a.n_att = items * c.kv_heads;
    a.n_mrg = m * H;
    const int n_o = (D + kAtoWaves * kOR - 1) / (kAtoWaves * kOR);
    a.window = c.window;
    a.attn = attn_out;
    a.aq = aq;
    a.aqx = static_cast<XBlock *>(aqx);
    a.wo = wo;
    a.bo = bo;
    a.residual = residual;
    a.out = out;
    a.D = D;
    a.cnt = cnt;
    const int G = H / c.kv_heads;
    const int nblocks = a.n_att + a.n_mrg + n_o;
    return c.head_dim == 64 ? launch_g<64>(a, nblocks, G, c.page_size != 0, st)
                            : launch_g<128>(a, nblocks, G, c.page_size != 0, st);
}

}  // namespace ck
