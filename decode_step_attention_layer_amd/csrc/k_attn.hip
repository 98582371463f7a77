// k_attn.hip — split-K grouped-query decode attention for gfx950.
//
// What it computes (C-Kernel-Engine "mega_fused_attention_decode_q5_0.c",
// MAIN KERNEL STEP 7): for query head h, KV head g = h*KV/H, tokens t <= pos,
//   out_h = sum_t softmax_t(scale * q_h . K_g[t]) V_g[t].
// Paged caches are addressed through the block table of the metrale
// "prefill_attn_a.rs" paged decode launchers; the GQA packing (one workgroup
// serves all query heads of a KV head) follows its paged_decode_attn_*_gqa.
// A sliding window (that page's sliding_window) restricts t to the last W
// positions: chunks then count from the window's first token, so the grid
// covers only attended tokens. A ring cache (the spark_model page's window
// ring) keeps token t in slot t % capacity.
//
// One kernel, grid (chunk, KV head, sequence). A workgroup walks its chunk of
// tokens in tiles of 64: the K and V tiles are staged through LDS with
// coalesced 16-byte loads (the next tile's loads are in flight while the
// current one is computed), so each K/V byte is read from HBM once for the
// whole query group. Scores: wave j owns query head j of the group, lane =
// token, q (pre-scaled by scale * log2 e) broadcast from LDS; the online
// softmax keeps a running max per head (wave-uniform) and per-lane sums.
// P.V: thread = (4 output dims, token subset), p broadcast from LDS. The
// chunk's (max, sum, unnormalized output) per head goes to the partials.
// A second kernel, one workgroup per (head, sequence), merges the chunks by
// log-sum-exp with all chunks' loads in flight at once, writes the attention
// output and, optionally, its Q8_0 blocks. (Merging inside the first kernel
// by the last workgroup to finish needs an agent-scope release per
// workgroup, an L2 write-back on this GPU; measured, it cost more than the
// kernel boundary.)
#include "ck_device.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

constexpr int kTile = 64;   // tokens per tile
constexpr int kMaxG = 8;
constexpr int kMaxChunks = 4096;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const float *q;       // [m][H][HD]
    CacheView c;
    Positions pos;
    float scale;
    int chunk;            // tokens per chunk, multiple of kTile
    int nchunks;
    int H;
    float *po;            // [m][KV][nchunks][G][HD]  unnormalized outputs
    float *pml;           // [m][KV][nchunks][G][2]   (max in log2 units, sum)
    int m;
    int first[kMaxSeqs + 1];  // first work item of each sequence; first[m] = items
};

constexpr int kPagesLds = 512;   // page ids of a chunk staged in LDS

template <int HD>
struct Smem {
    static constexpr int stride = HD + 4;  // padded row: conflict-free b128 reads
    float kv[2 * kTile * stride];           // K tile, then V tile; reused by reductions
    float q[kMaxG * HD];
    float p[kTile * kMaxG];
    float alpha[kMaxG];
    int pages[kPagesLds];                   // paged caches: the chunk's page ids
    int bad;
};

template <int HD, int G, bool PAGED, int DT>
__global__ __launch_bounds__(G > 4 ? 512 : 256) void k_attn(AttnArgs a) {
    static_assert(HD % 64 == 0 && G >= 1 && G <= kMaxG, "shape");
    constexpr int NT = G > 4 ? 512 : 256;            // threads
    constexpr int C4 = HD / 4;                       // float4 columns per row
    constexpr int NLD = kTile * C4 / NT;             // float4 loads per thread per tile (K or V)
    constexpr int ROWS_PER_LD = NT / C4;             // rows covered by one load round
    constexpr int NTG = NT / C4;                     // token groups in the P.V phase
    constexpr int TPG = kTile / NTG;                 // tokens per group per tile
    constexpr int S = Smem<HD>::stride;
    __shared__ Smem<HD> sm;

    // grid: (work item, KV head); the items are the chunks of every sequence
    // back to back, so a batch of unequal lengths launches no idle workgroups
    const int item = blockIdx.x, g = blockIdx.y;
    int s = 0;
    while (s + 1 < a.m && item >= a.first[s + 1]) s++;
    const int cidx = item - a.first[s];
    const int L = a.pos.get(s) + 1;
    // chunks count from the window's first token (0 without a window)
    const int t0 = window_start(L, a.c.window) + cidx * a.chunk;
    if (t0 >= L) return;             // device positions: items past this sequence's chunks
    const int t1 = min(L, t0 + a.chunk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, KV = a.c.kv_heads;
    const float *qg = a.q + ((size_t)s * H + (size_t)g * G) * HD;

    float *sk = sm.kv;
    float *sv = sm.kv + kTile * S;
    if (tid == 0) sm.bad = 0;
    // paged: the chunk's page ids in one batch of loads, so that a tile's K/V
    // addresses do not wait on table reads (chunks with more pages than the
    // LDS slots read the table per row)
    int pg0 = 0;
    bool pages_in_lds = false;
    if constexpr (PAGED) {
        const int ps = a.c.page_size;
        pg0 = t0 / ps;
        const int npg = (t1 - 1) / ps - pg0 + 1;
        pages_in_lds = npg <= kPagesLds;
        if (pages_in_lds)
            for (int i = tid; i < npg; i += NT)
                sm.pages[i] = a.c.table[(long long)s * a.c.max_pages + pg0 + i];
        __syncthreads();
    }

    // loader geometry: this thread loads column ld_col of rows ld_row + i*ROWS_PER_LD
    const int ld_col = tid % C4, ld_row = tid / C4;
    const size_t seq_base = PAGED ? 0 : ((size_t)s * KV + g) * a.c.capacity * HD;
    typedef typename CacheRaw4<DT>::type Raw;
    Raw kreg[NLD], vreg[NLD];   // raw elements (fp32, bf16 or fp8), converted at the LDS store
    auto fetch = [&](int st) {
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int t = st + ld_row + i * ROWS_PER_LD;
            long long off = -1;
            if (t < t1) {
                if constexpr (PAGED) {
                    if (pages_in_lds) {
                        const int ps = a.c.page_size;
                        const int page = sm.pages[t / ps - pg0];
                        if (page >= 0 && page < a.c.num_pages)
                            off = (((long long)page * KV + g) * ps + t % ps) * (long long)HD;
                    } else {
                        off = cache_row(a.c, s, g, t);
                    }
                    if (off < 0) sm.bad = 1;
                } else {
                    // ring: slot t % capacity (t < L, so t is never negative)
                    const int slot = a.c.ring ? t % a.c.capacity : t;
                    off = (long long)(seq_base + (size_t)slot * HD);
                }
            }
            if (off >= 0) {
                kreg[i] = cache_raw4<DT>(a.c, true, off + 4 * ld_col);
                vreg[i] = cache_raw4<DT>(a.c, false, off + 4 * ld_col);
            } else {
                kreg[i] = vreg[i] = cache_raw4_zero<DT>();
            }
        }
    };

    float m_run = -INFINITY, l_lane = 0.0f;          // this wave's head (wave < G)
    const int pv_col = tid % C4, pv_tg = tid / C4;
    float4 o[G];
#pragma unroll
    for (int j = 0; j < G; j++) o[j] = make_float4(0.f, 0.f, 0.f, 0.f);

    // the first tile's K/V loads, then q's, in flight together
    fetch(t0);
    // q of the group into LDS, pre-scaled so that scores are in log2 units
    const float qs = a.scale * kLog2e;
    for (int i = tid; i < G * HD; i += NT) sm.q[i] = qg[i] * qs;
    for (int st = t0; st < t1; st += kTile) {
        __syncthreads();                             // previous tile fully consumed
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int r = ld_row + i * ROWS_PER_LD;
            *reinterpret_cast<float4 *>(&sk[r * S + 4 * ld_col]) = cache_cvt4<DT>(a.c, true, kreg[i]);
            *reinterpret_cast<float4 *>(&sv[r * S + 4 * ld_col]) = cache_cvt4<DT>(a.c, false, vreg[i]);
        }
        __syncthreads();
        if (st + kTile < t1) fetch(st + kTile);      // next tile's loads in flight

        // ---- scores: wave j = head j, lane = token
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
            const float p = exp2f(sv2 - m_new);
            l_lane = l_lane * alpha + p;
            m_run = m_new;
            sm.p[lane * kMaxG + wave] = p;
            if (lane == 0) sm.alpha[wave] = alpha;
        }
        __syncthreads();

        // ---- P.V
#pragma unroll
        for (int j = 0; j < G; j++) {
            const float al = sm.alpha[j];
            o[j].x *= al; o[j].y *= al; o[j].z *= al; o[j].w *= al;
        }
#pragma unroll
        for (int i = 0; i < TPG; i++) {
            const int r = pv_tg + i * NTG;
            const float4 vv = *reinterpret_cast<const float4 *>(&sv[r * S + 4 * pv_col]);
            const float4 p0 = *reinterpret_cast<const float4 *>(&sm.p[r * kMaxG]);
            const float4 p1 = *reinterpret_cast<const float4 *>(&sm.p[r * kMaxG + 4]);
            const float pj[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int j = 0; j < G; j++) {
                o[j].x = fmaf(pj[j], vv.x, o[j].x);
                o[j].y = fmaf(pj[j], vv.y, o[j].y);
                o[j].z = fmaf(pj[j], vv.z, o[j].z);
                o[j].w = fmaf(pj[j], vv.w, o[j].w);
            }
        }
    }
    __syncthreads();

    // ---- reduce the P.V token groups: first the groups inside a wave (xor
    // shuffles over the C4-lane groups), then one group per wave through LDS
    // (reusing the K/V tiles)
    constexpr int NW = NT / kWave;
    float *red = sm.kv;   // [NW][G][HD]
    static_assert(NW * G * HD <= 2 * kTile * (HD + 4), "reduction buffer");
#pragma unroll
    for (int j = 0; j < G; j++) {
#pragma unroll
        for (int sh = C4; sh < kWave; sh <<= 1) {
            o[j].x += __shfl_xor(o[j].x, sh);
            o[j].y += __shfl_xor(o[j].y, sh);
            o[j].z += __shfl_xor(o[j].z, sh);
            o[j].w += __shfl_xor(o[j].w, sh);
        }
        if (lane < C4) *reinterpret_cast<float4 *>(&red[(wave * G + j) * HD + 4 * lane]) = o[j];
    }
    const float lsum = wave_sum(l_lane);
    __syncthreads();

    const size_t grp = (size_t)s * KV + g;
    const size_t part = grp * a.nchunks + cidx;
    for (int e = tid; e < G * HD; e += NT) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; w++) acc += red[w * G * HD + e];
        a.po[part * G * HD + e] = acc;
    }
    if (wave < G && lane == 0) {
        a.pml[(part * G + wave) * 2 + 0] = m_run;
        a.pml[(part * G + wave) * 2 + 1] = sm.bad ? NAN : lsum;
    }
}

struct MergeArgs {
    const float *po;
    const float *pml;
    Positions pos;
    int chunk, nchunks, H, KV;
    int window;          // 0 = none: the chunks cover the last `window` tokens
    float *out;          // [m][H][HD]
    uint8_t *out_q8;     // nullable: [m][H*HD/32] Q8_0 blocks
};

constexpr int kMergeThreads = 256;

// One workgroup per (head, sequence). Phase 1: one chunk per thread reads
// (max, sum), the block reduces the global max M and the denominator, and
// the weights 2^(m_c - M) go to LDS. Phase 2: thread (4 dims, chunk group)
// accumulates its chunks' outputs with independent loads in flight; the
// chunk groups are summed with a shuffle inside the wave and through LDS.
template <int HD>
__global__ __launch_bounds__(kMergeThreads) void k_attn_merge(MergeArgs a) {
    constexpr int C4 = HD / 4;
    constexpr int CG = kMergeThreads / C4;        // chunk groups
    constexpr int NW = kMergeThreads / kWave;
    __shared__ float w_s[kMaxChunks];
    __shared__ float l_s[kMaxChunks];
    __shared__ float red[NW];
    __shared__ float4 part[NW][C4];
    const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int G = a.H / a.KV, g = h / G, j = h % G;
    const int L = a.pos.get(s) + 1;
    const int nc = (L - window_start(L, a.window) + a.chunk - 1) / a.chunk;
    const size_t base = ((size_t)s * a.KV + g) * a.nchunks;

    // Every load that does not depend on another goes out first: the (max,
    // sum) pairs of this thread's chunks and the outputs of its first kPre
    // chunk slots, so that the merge costs one memory round trip.
    constexpr int kPre = 8;
    const int d4 = tid % C4, cg = tid / C4;
    auto ld = [&](int c) {
        return *reinterpret_cast<const float4 *>(&a.po[((base + c) * G + j) * HD + 4 * d4]);
    };
    float4 pre[kPre];
#pragma unroll
    for (int i = 0; i < kPre; i++) {
        const int c = cg + i * CG;
        pre[i] = c < nc ? ld(c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mx = -INFINITY;
    for (int c = tid; c < nc; c += kMergeThreads) {
        const float2 ml = *reinterpret_cast<const float2 *>(&a.pml[((base + c) * G + j) * 2]);
        w_s[c] = ml.x;
        l_s[c] = ml.y;
        mx = fmaxf(mx, ml.x);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++) M = fmaxf(M, red[i]);
    __syncthreads();
    float den = 0.0f;
    for (int c = tid; c < nc; c += kMergeThreads) {
        const float w = exp2f(w_s[c] - M);
        w_s[c] = w;
        den = fmaf(w, l_s[c], den);
    }
    den = wave_sum(den);
    if (lane == 0) red[wave] = den;
    __syncthreads();
    float D = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; i++) D += red[i];

    float4 n0 = make_float4(0.f, 0.f, 0.f, 0.f), n1 = n0;
    auto fma4 = [](float w, float4 v, float4 acc) {
        return make_float4(fmaf(w, v.x, acc.x), fmaf(w, v.y, acc.y), fmaf(w, v.z, acc.z),
                           fmaf(w, v.w, acc.w));
    };
#pragma unroll
    for (int i = 0; i < kPre; i++) {
        const int c = cg + i * CG;
        if (c < nc) {
            if (i & 1) n1 = fma4(w_s[c], pre[i], n1);
            else n0 = fma4(w_s[c], pre[i], n0);
        }
    }
    int c = cg + kPre * CG;
    for (; c + CG < nc; c += 2 * CG) {
        const float4 v0 = ld(c), v1 = ld(c + CG);
        n0 = fma4(w_s[c], v0, n0);
        n1 = fma4(w_s[c + CG], v1, n1);
    }
    if (c < nc) n0 = fma4(w_s[c], ld(c), n0);
    float4 acc = make_float4(n0.x + n1.x, n0.y + n1.y, n0.z + n1.z, n0.w + n1.w);
#pragma unroll
    for (int sh = C4; sh < kWave; sh <<= 1) {
        acc.x += __shfl_xor(acc.x, sh);
        acc.y += __shfl_xor(acc.y, sh);
        acc.z += __shfl_xor(acc.z, sh);
        acc.w += __shfl_xor(acc.w, sh);
    }
    if (lane < C4) part[wave][lane] = acc;
    __syncthreads();
    if (tid < C4) {
        float4 t = part[0][tid];
#pragma unroll
        for (int w = 1; w < NW; w++) {
            const float4 u = part[w][tid];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        const float inv = 1.0f / D;
        const float4 v = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
        const size_t oi = ((size_t)s * a.H + h) * HD + 4 * tid;
        *reinterpret_cast<float4 *>(&a.out[oi]) = v;
        if (a.out_q8) quantize_q8_0_x4(v, a.out_q8 + (oi / kQK) * kQ8Bytes, tid & 7);
    }
}

template <int HD, int G>
hipError_t launch_t(const AttnArgs &a, int m, bool paged, hipStream_t st) {
    constexpr int NT = G > 4 ? 512 : 256;
    const dim3 grid(a.first[m], a.c.kv_heads);
    const int dt = a.c.dtype;
#define CK_ATTN_LAUNCH(P, D) hipLaunchKernelGGL((k_attn<HD, G, P, D>), grid, dim3(NT), 0, st, a)
    if (paged) {
        if (dt == CK_KV_BF16) CK_ATTN_LAUNCH(true, CK_KV_BF16);
        else if (dt == CK_KV_FP8_E4M3) CK_ATTN_LAUNCH(true, CK_KV_FP8_E4M3);
        else CK_ATTN_LAUNCH(true, CK_KV_F32);
    } else {
        if (dt == CK_KV_BF16) CK_ATTN_LAUNCH(false, CK_KV_BF16);
        else if (dt == CK_KV_FP8_E4M3) CK_ATTN_LAUNCH(false, CK_KV_FP8_E4M3);
        else CK_ATTN_LAUNCH(false, CK_KV_F32);
    }
#undef CK_ATTN_LAUNCH
    return hipGetLastError();
}

template <int HD>
hipError_t launch_g(const AttnArgs &a, int G, int m, bool paged, hipStream_t st) {
    switch (G) {
        case 1: return launch_t<HD, 1>(a, m, paged, st);
        case 2: return launch_t<HD, 2>(a, m, paged, st);
        case 3: return launch_t<HD, 3>(a, m, paged, st);
        case 4: return launch_t<HD, 4>(a, m, paged, st);
        case 5: return launch_t<HD, 5>(a, m, paged, st);
        case 6: return launch_t<HD, 6>(a, m, paged, st);
        case 7: return launch_t<HD, 7>(a, m, paged, st);
        case 8: return launch_t<HD, 8>(a, m, paged, st);
    }
    return hipErrorInvalidValue;
}

// Compute units of the current device, queried once per device (the value
// cannot change; a racing first query writes the same number).
int cus_of_current_device() {
    static int cached[64];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    if (dev < 64) cached[dev] = n;
    return n;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int num_cus() { return cus_of_current_device(); }

bool attn_shape_supported(int G, int hd) {
    return G >= 1 && G <= kMaxG && (hd == 64 || hd == 128);
}

bool attn_chunks_supported(int nchunks) { return nchunks >= 1 && nchunks <= kMaxChunks; }

AttnPlan attn_plan(int KV, int max_tokens, long long total_tokens, int chunk_req) {
    AttnPlan p;
    if (chunk_req > 0) {
        p.chunk = (chunk_req + kTile - 1) / kTile * kTile;
    } else {
        // about two workgroups per compute unit over all (sequence, KV head,
        // chunk) items: chunks are sized from the tokens of every sequence,
        // so that a batch of unequal lengths still fills the GPU
        const long long target = 2LL * cus_of_current_device();
        if (total_tokens < max_tokens) total_tokens = max_tokens;
        const long long c = (total_tokens * KV + target - 1) / target;
        p.chunk = (int)((c + kTile - 1) / kTile * kTile);
    }
    if (p.chunk < kTile) p.chunk = kTile;
    p.nchunks = (max_tokens + p.chunk - 1) / p.chunk;
    if (p.nchunks < 1) p.nchunks = 1;
    return p;
}

int attn_max_chunks(int KV, int max_tokens, int chunk_req) {
    // the largest nchunks attn_plan returns for any positions with at most
    // max_tokens tokens per sequence: the chunk is at least
    // max_tokens * KV / (2 CUs), so nchunks <= ceil(2 CUs / KV)
    if (chunk_req > 0) return attn_plan(KV, max_tokens, max_tokens, chunk_req).nchunks;
    const int target = 2 * cus_of_current_device();
    const int by_items = (target + KV - 1) / KV;
    const int by_tile = (max_tokens + kTile - 1) / kTile;
    return by_tile < by_items ? by_tile : by_items;
}

// Workspace of the attention: unnormalized outputs, then (max, sum) per chunk
// and head; each region 256-byte aligned.
size_t attn_partials_bytes(int m, int H, int hd, int nchunks) {
    return up256(sizeof(float) * (size_t)m * H * nchunks * hd) +
           up256(sizeof(float) * (size_t)m * H * nchunks * 2);
}

hipError_t launch_attn_partial(const float *q, const CacheView &c, const Positions &pos, int m,
                               int H, float scale, const AttnPlan &plan, void *partials,
                               hipStream_t st) {
    const int G = H / c.kv_heads;
    AttnArgs a;
    a.q = q;
    a.c = c;
    a.pos = pos;
    a.scale = scale;
    a.chunk = plan.chunk;
    a.nchunks = plan.nchunks;
    a.H = H;
    uint8_t *base = static_cast<uint8_t *>(partials);
    a.po = reinterpret_cast<float *>(base);
    a.pml = reinterpret_cast<float *>(base + up256(sizeof(float) * (size_t)m * H * plan.nchunks *
                                                   c.head_dim));
    a.m = m;
    // work items: host positions give each sequence exactly its chunks; with
    // device positions every sequence gets plan.nchunks items and the ones
    // past its length return at once
    a.first[0] = 0;
    for (int s = 0; s < m; s++) {
        const int n = pos.p[s] + 1 - window_start(pos.p[s] + 1, c.window);
        a.first[s + 1] = a.first[s] + (pos.dev ? plan.nchunks : (n + plan.chunk - 1) / plan.chunk);
    }
    for (int s = m + 1; s <= kMaxSeqs; s++) a.first[s] = a.first[m];
    const bool paged = c.page_size != 0;
    return c.head_dim == 64 ? launch_g<64>(a, G, m, paged, st) : launch_g<128>(a, G, m, paged, st);
}

hipError_t launch_attn_merge(const void *partials, const Positions &pos, int window, int m,
                             int H, int KV, int hd, const AttnPlan &plan, float *out,
                             uint8_t *out_q8, hipStream_t st) {
    const uint8_t *base = static_cast<const uint8_t *>(partials);
    MergeArgs b;
    b.po = reinterpret_cast<const float *>(base);
    b.pml = reinterpret_cast<const float *>(base + up256(sizeof(float) * (size_t)m * H *
                                                         plan.nchunks * hd));
    b.pos = pos;
    b.chunk = plan.chunk;
    b.nchunks = plan.nchunks;
    b.H = H;
    b.KV = KV;
    b.window = window;
    b.out = out;
    b.out_q8 = out_q8;
    if (hd == 64)
        hipLaunchKernelGGL(k_attn_merge<64>, dim3(H, m), dim3(kMergeThreads), 0, st, b);
    else
        hipLaunchKernelGGL(k_attn_merge<128>, dim3(H, m), dim3(kMergeThreads), 0, st, b);
    return hipGetLastError();
}

hipError_t launch_attention(const float *q, const CacheView &c, const Positions &pos, float *out,
                            uint8_t *out_q8, int m, int H, float scale, const AttnPlan &plan,
                            void *partials, hipStream_t st) {
    hipError_t e = launch_attn_partial(q, c, pos, m, H, scale, plan, partials, st);
    if (e != hipSuccess) return e;
    return launch_attn_merge(partials, pos, c.window, m, H, c.kv_heads, c.head_dim, plan, out,
                             out_q8, st);
}

}  // namespace ck
