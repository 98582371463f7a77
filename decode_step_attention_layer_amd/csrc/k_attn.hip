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
// A sparse mode (the spark_model page's sparse_attn) attends, per sequence,
// the token positions of a selection (-1 = absent) with per-head sink
// logits that join the denominator: the chunks then split the selection.
//
// One kernel, grid (chunk, KV head): the chunks of every sequence back to
// back. A workgroup serves all query heads of its KV head over its chunk, so
// each K/V byte is read from HBM once for the whole query group. Its waves
// hold K/V rows in registers, a row spread over a group of 16 lanes (8 for
// fp8), and walk the chunk in steps of 16 (fp8: 32) rows per wave: every
// load of a step is issued, then the rows are scored against the q slices
// the lanes hold (pre-scaled by scale * log2 e), the partial dots summed over
// the row group with DPP, and each row group keeps its own online softmax
// (running max, sum, unnormalized output slice). No LDS staging and no
// barrier inside the token loop. At the end the row groups' states are
// combined by log-sum-exp through LDS into the chunk's (max, sum,
// unnormalized output) per head, the partials. K/V rows stream with
// non-temporal loads (each row is read once), except in short chunks of
// large query groups with 128-wide heads. Query groups of 5 to 8 heads over
// an fp32 cache (no selection) take the same grid and partials on the fp32
// matrix cores (k_attn_mfma): per 16-token tile, the scores of the whole
// group and the value sums are 16x16x4 MFMA contractions, one wave per tile
// of the chunk (at most eight; two per tile, each taking half of the work,
// where the chunk has at most eight tiles). A second kernel, one workgroup
// per (head, sequence) (one wavefront per 32 chunks where a sequence has at
// most 128, and then a workgroup per 32 output dims while the grid leaves
// compute units free), merges the chunks by log-sum-exp with all chunks'
// loads in flight at once (the sink joins here), writes the attention
// output and, optionally, its Q8_0 blocks. (Merging inside the first kernel
// by the last workgroup to finish needs an agent-scope release per
// workgroup, an L2 write-back on this GPU; measured, it cost more than the
// kernel boundary.)

#include "ck_attn_common.hpp"

namespace ck {

namespace {

using namespace attn;

// Grid: (work item, KV head); the items are the chunks of every sequence back
// to back, so a batch of unequal lengths launches no idle workgroups.
template <int HD, int G, bool PAGED, int DT, bool STREAM>
__global__ __launch_bounds__(AttnShape<G>::threads) void k_attn(AttnArgs a) {
    __shared__ Smem<HD, G, kAttnNS<DT, HD, G>> sm;
    attn_item<HD, G, PAGED, DT, STREAM, false>(a, blockIdx.x, blockIdx.y, sm);
}

// The same on the fp32 matrix cores (query groups of 5 to 8 heads, fp32
// cache, no selection): same grid, same partials.
template <int HD, int G, int NW, bool PAGED, bool STREAM, int HF>
__global__ __launch_bounds__(NW * HF * kWave) void k_attn_mfma(AttnArgs a) {
    __shared__ SmemM<HD, G, NW, HF> sm;
    attn_item_mfma<HD, G, NW, PAGED, STREAM, false, HF>(a, blockIdx.x, blockIdx.y, sm);
}

constexpr int kMfmaMaxWaves = 8;

// One wave per 16-token tile of a chunk, at most eight (longer chunks give a
// wave every eighth tile); chunks of at most eight tiles take two waves per
// tile, one per half of the head dims for the scores. 128-wide heads
// stream their rows only from chunks of kNtChunk tokens (see launch_t),
// which take eight waves.
template <int HD, int G, int NW, int HF = 2>
void launch_mfma_nw(const AttnArgs &a, dim3 grid, bool paged, hipStream_t st) {
    constexpr bool NT = HD == 64;
    const dim3 blk(NW * HF * kWave);
    if (paged) hipLaunchKernelGGL((k_attn_mfma<HD, G, NW, true, NT, HF>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_attn_mfma<HD, G, NW, false, NT, HF>), grid, blk, 0, st, a);
}

template <int HD, int G>
void launch_mfma(const AttnArgs &a, dim3 grid, bool paged, bool nt, hipStream_t st) {
    const int tiles = (a.chunk + 15) / 16;
    if (HD == 128 && nt) {
        const dim3 blk(kMfmaMaxWaves * kWave);
        if (paged)
            hipLaunchKernelGGL((k_attn_mfma<HD, G, kMfmaMaxWaves, true, true, 1>), grid, blk, 0, st,
                               a);
        else
            hipLaunchKernelGGL((k_attn_mfma<HD, G, kMfmaMaxWaves, false, true, 1>), grid, blk, 0,
                               st, a);
        return;
    }
    switch (tiles < kMfmaMaxWaves ? tiles : kMfmaMaxWaves) {
        case 1: launch_mfma_nw<HD, G, 1>(a, grid, paged, st); break;
        case 2: launch_mfma_nw<HD, G, 2>(a, grid, paged, st); break;
        case 3: launch_mfma_nw<HD, G, 3>(a, grid, paged, st); break;
        case 4: launch_mfma_nw<HD, G, 4>(a, grid, paged, st); break;
        case 5: launch_mfma_nw<HD, G, 5>(a, grid, paged, st); break;
        case 6: launch_mfma_nw<HD, G, 6>(a, grid, paged, st); break;
        case 7: launch_mfma_nw<HD, G, 7>(a, grid, paged, st); break;
        default:
            // over eight tiles a wave takes several: one wave per tile
            if (tiles > kMfmaMaxWaves) launch_mfma_nw<HD, G, 8, 1>(a, grid, paged, st);
            else launch_mfma_nw<HD, G, 8>(a, grid, paged, st);
            break;
    }
}

struct MergeArgs {
    const float *po;
    const float *pml;
    Positions pos;
    int chunk, nchunks, H, KV;
    int window;          // 0 = none: the chunks cover the last `window` tokens
    int topk;            // > 0: sparse, the chunks split topk selection entries
    const float *sink;   // nullable: [H] logits joining the denominator only
    float *out;          // [m][H][HD]
    uint8_t *out_q8;     // nullable: [m][H*HD/32] Q8_0 blocks
    XImage xi;           // with out_q8: the blocks also as an activation image
};

// The Q8_0 of output elements 4*e4.. of (sequence s, head h) (every lane of
// the block's group of 8 calling), into out_q8 and the image; the image's
// zero scales of blocks [pb0, pb1) written by the sequence-0 workgroup's
// lanes (lane ptid of pn).
template <int HD>
__device__ __forceinline__ void merge_q8_out(const MergeArgs &a, float4 v, int s, int h, int e4,
                                             int pb0, int pb1, int ptid, int pn) {
    const size_t oi = ((size_t)s * a.H + h) * HD + 4 * e4;
    uint32_t packed;
    uint16_t dbits;
    quantize_q8_0_x4_codes(v, packed, dbits);
    uint8_t *blk = a.out_q8 + (oi / kQK) * kQ8Bytes;
    uint16_t *dst = reinterpret_cast<uint16_t *>(blk + 2 + 4 * (e4 & 7));
    dst[0] = (uint16_t)(packed & 0xFFFF);
    dst[1] = (uint16_t)(packed >> 16);
    if ((e4 & 7) == 0) *reinterpret_cast<uint16_t *>(blk) = dbits;
    if (a.xi.base) {
        ximage_put(a.xi, s, (h * HD + 4 * e4) / kQK, e4 & 7, packed, dbits);
        if (s == 0) ximage_zero_pads(a.xi, pb0, pb1, ptid, pn);
    }
}

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
    const int n = a.topk > 0 ? (L > 0 ? a.topk : 0) : L - window_start(L, a.window);
    const int nc = (n + a.chunk - 1) / a.chunk;
    const size_t base = ((size_t)s * a.KV + g) * a.nchunks;
    // the sink, in the partials' log2 units
    const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;

    // Every load that does not depend on another goes out first, none of
    // them conditional (a slot past the last chunk re-reads the last one and
    // is not used; a load under a branch makes the compiler wait early for
    // it and for everything issued before it): this thread's first (max,
    // sum) pair, then the outputs of its first kPre chunk slots, so that the
    // merge costs one memory round trip.
    constexpr int kPre = 16;
    const int d4 = tid % C4, cg = tid / C4;
    const int ncl = nc > 0 ? nc - 1 : 0;
    auto ld = [&](int c) {
        return *reinterpret_cast<const float4 *>(&a.po[((base + c) * G + j) * HD + 4 * d4]);
    };
    const float2 ml0 =
        *reinterpret_cast<const float2 *>(&a.pml[((base + min(tid, ncl)) * G + j) * 2]);
    float4 pre[kPre];
#pragma unroll
    for (int i = 0; i < kPre; i++) pre[i] = ld(min(cg + i * CG, ncl));
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
    if (tid < nc) {
        w_s[tid] = ml0.x;
        l_s[tid] = ml0.y;
        mx = ml0.x;
    }
    for (int c = tid + kMergeThreads; c < nc; c += kMergeThreads) {
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
    M = fmaxf(M, sk);
    // no attended row and no sink (a selection of absent entries): the
    // weights are zero and so is the output
    const float Mr = M == -INFINITY ? 0.0f : M;
    __syncthreads();
    float den = 0.0f;
    for (int c = tid; c < nc; c += kMergeThreads) {
        const float w = exp2f(w_s[c] - Mr);
        w_s[c] = w;
        den = fmaf(w, l_s[c], den);
    }
    den = wave_sum(den);
    if (lane == 0) red[wave] = den;
    __syncthreads();
    float D = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; i++) D += red[i];
    if (a.sink) D += exp2f(sk - Mr);

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
        // D == 0: nothing attended and no sink, the output is zero; a NaN D
        // (a chunk that read an unmapped or unheld row) stays NaN
        const float inv = D == 0.0f ? 0.0f : 1.0f / D;
        const float4 v = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
        const size_t oi = ((size_t)s * a.H + h) * HD + 4 * tid;
        *reinterpret_cast<float4 *>(&a.out[oi]) = v;
        if (a.out_q8)
            merge_q8_out<HD>(a, v, s, h, tid, h * HD / kQK, (h + 1) * HD / kQK, tid, HD / 4);
    }
}

// The merge for sequences of at most kMerge1Chunks chunks per wavefront: a
// workgroup per (head, sequence, DQ output dims), no barrier with one
// wavefront. A chunk's DQ dims are held by DQ/4 lanes (4 values each); the
// chunks are dealt round-robin to the 64 / (DQ/4) lane groups. Every load
// goes out at once and none is conditional (a slot past the last chunk
// re-reads the last one and is not used): lane c's chunk (max, sum) pair,
// then (DQ = 32) the pairs of the lane's own slots, then the lane's output
// slices. The global max and the denominator are wave reductions; with DQ
// = 32 each lane weighs its own 4 slots, with whole heads (DQ = HD, where
// the grid already fills the GPU) each chunk's weight is computed by lane c
// and read from it into scalar registers; the lane groups' sums are
// combined with cross-lane exchanges.
constexpr int kMerge1Chunks = 32;   // chunks per wavefront

// NWV wavefronts: wave w merges chunks [32w, 32w + 32) as above into its own
// (max, denominator, weighted sum); with two waves the states are combined by
// log-sum-exp through LDS after one barrier.
template <int HD, int NWV, int DQ>
__global__ __launch_bounds__(kWave * NWV) void k_attn_merge1(MergeArgs a) {
    static_assert(DQ == 32 || DQ == HD, "output dims per workgroup");
    constexpr bool SPLIT = DQ < HD;            // each lane weighs its own slots
    constexpr int LG = DQ / 4;                 // lanes per chunk group
    constexpr int NGRP = kWave / LG;           // chunk groups
    constexpr int PER = kMerge1Chunks / NGRP;  // chunk slots per lane
    const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x & (kWave - 1);
    const int dq = blockIdx.z * DQ;            // this workgroup's first output dim
    const int wave = NWV > 1 ? (int)(threadIdx.x >> 6) : 0;
    const int G = a.H / a.KV, g = h / G, j = h % G;
    const int L = a.pos.get(s) + 1;
    const int n = a.topk > 0 ? (L > 0 ? a.topk : 0) : L - window_start(L, a.window);
    const int nc_all = (n + a.chunk - 1) / a.chunk;
    const int c0 = wave * kMerge1Chunks;                       // this wave's first chunk
    const int nc = min(max(nc_all - c0, 0), kMerge1Chunks);    // and its count
    const int ncl = nc_all > 0 ? nc_all - 1 : 0;               // last valid chunk
    const size_t base = ((size_t)s * a.KV + g) * a.nchunks;
    const float sk = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const int d4 = lane % LG, grp = lane / LG;

    const float2 ml =
        *reinterpret_cast<const float2 *>(&a.pml[((base + min(c0 + lane, ncl)) * G + j) * 2]);
    float2 mls[SPLIT ? PER : 1];
    float4 ov[PER];
    if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int c = min(c0 + grp + NGRP * i, ncl);
            mls[i] = *reinterpret_cast<const float2 *>(&a.pml[((base + c) * G + j) * 2]);
        }
    }
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int c = min(c0 + grp + NGRP * i, ncl);
        ov[i] = *reinterpret_cast<const float4 *>(&a.po[((base + c) * G + j) * HD + dq + 4 * d4]);
    }
    __builtin_amdgcn_sched_barrier(0);

    const bool mine = lane < nc;
    // one wave: the sink joins the max here; two: after the combination
    const float Mw = fmaxf(wave_max(mine ? ml.x : -INFINITY), NWV == 1 ? sk : -INFINITY);
    // no attended row and no sink (a selection of absent entries): the
    // weights are zero and so is the output
    const float Mr = Mw == -INFINITY ? 0.0f : Mw;
    const float w = mine ? exp2f(ml.x - Mr) : 0.0f;
    float D = wave_sum(mine ? w * ml.y : 0.0f);

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int c = grp + NGRP * i;
        float wc;
        if constexpr (SPLIT) {
            // the slot's weight, as lane c computed it for the denominator
            wc = exp2f(mls[i].x - Mr);
        } else {
            // chunk c's weight: read from lane c into a scalar register (the
            // lane index is a constant per group), no wait on a permute
            wc = readlane_f(w, NGRP * i);
#pragma unroll
            for (int q = 1; q < NGRP; q++) {
                const float t = readlane_f(w, NGRP * i + q);
                wc = grp == q ? t : wc;
            }
        }
        if (c < nc)
            acc = make_float4(fmaf(wc, ov[i].x, acc.x), fmaf(wc, ov[i].y, acc.y),
                              fmaf(wc, ov[i].z, acc.z), fmaf(wc, ov[i].w, acc.w));
    }
#pragma unroll
    for (int sh = LG; sh < kWave; sh <<= 1) {
        acc.x += __shfl_xor(acc.x, sh);
        acc.y += __shfl_xor(acc.y, sh);
        acc.z += __shfl_xor(acc.z, sh);
        acc.w += __shfl_xor(acc.w, sh);
    }
    if constexpr (NWV == 1) {
        if (a.sink) D += exp2f(sk - Mr);
    } else {
        // the waves' states: (max, denominator, weighted sum) relative to
        // their own max, combined by log-sum-exp with the sink
        __shared__ float4 sacc[NWV][LG];
        __shared__ float smd[NWV][2];
        if (grp == 0) sacc[wave][d4] = acc;
        if (lane == 0) {
            smd[wave][0] = Mw;
            smd[wave][1] = D;
        }
        __syncthreads();
        if (wave != 0) return;
        float M = sk;
#pragma unroll
        for (int v = 0; v < NWV; v++) M = fmaxf(M, smd[v][0]);
        const float Mt = M == -INFINITY ? 0.0f : M;
        D = a.sink ? exp2f(sk - Mt) : 0.0f;
        acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int v = 0; v < NWV; v++) {
            const float sc = smd[v][0] == -INFINITY ? 0.0f : exp2f(smd[v][0] - Mt);
            D = fmaf(sc, smd[v][1], D);
            const float4 t = sacc[v][d4];
            acc = make_float4(fmaf(sc, t.x, acc.x), fmaf(sc, t.y, acc.y), fmaf(sc, t.z, acc.z),
                              fmaf(sc, t.w, acc.w));
        }
    }
    if (grp == 0) {
        // D == 0: nothing attended and no sink, the output is zero; a NaN D
        // (a chunk that read an unmapped or unheld row) stays NaN
        const float inv = D == 0.0f ? 0.0f : 1.0f / D;
        const float4 v = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        const size_t oi = ((size_t)s * a.H + h) * HD + dq + 4 * d4;
        *reinterpret_cast<float4 *>(&a.out[oi]) = v;
        if (a.out_q8)
            merge_q8_out<HD>(a, v, s, h, dq / 4 + d4, (h * HD + dq) / kQK,
                             (h * HD + dq + DQ) / kQK, d4, LG);
    }
}

constexpr int kNtChunk = 256;   // chunks this long always stream (see launch_t)

template <int HD, int G>
hipError_t launch_t(const AttnArgs &a, int m, bool paged, hipStream_t st) {
    constexpr int NT = AttnShape<G>::threads;
    const dim3 grid(a.first[m], a.c.kv_heads);
    const int dt = a.c.dtype;
    // K/V rows stream with non-temporal loads (measured: 47.9 against 55.5
    // us for 32,769 tokens x 8 KV heads; 9.7 against 10.6 us for a 4096-token
    // window). The exception is short chunks of large query groups with
    // 128-wide heads, where the streaming variant takes 11 more registers
    // and measured slower per step (the 7B shape, 96-token chunks).
    const bool nt = a.chunk >= kNtChunk || !(HD == 128 && G > 4);
    // bf16 and fp8 caches: the bf16 matrix cores
    if (attn_matrix_path(G, dt, m, a.sel != nullptr) && dt != CK_KV_F32)
        return launch_attn_mfma16(a, G, HD, grid, paged, st);
    if constexpr (G >= 5) {
        // query groups of 5 to 8 heads over an fp32 cache: the matrix cores
        if (attn_matrix_path(G, dt, m, a.sel != nullptr)) {
            launch_mfma<HD, G>(a, grid, paged, nt, st);
            return hipGetLastError();
        }
    }
#define CK_ATTN_LAUNCH(P, D)                                                                   \
    do {                                                                                       \
        if (nt) hipLaunchKernelGGL((k_attn<HD, G, P, D, true>), grid, dim3(NT), 0, st, a);     \
        else hipLaunchKernelGGL((k_attn<HD, G, P, D, false>), grid, dim3(NT), 0, st, a);       \
    } while (0)
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

// The vector kernel's step: 4 waves x load rounds (3 for groups over 4
// heads) x rows per round (8 for fp8 rows of groups up to 4 heads, held by
// 8 lanes each; otherwise 4). The matrix-core kernels': 16-token tiles
// (fp32 caches), 32-token steps (bf16 and fp8 caches).
int attn_step(int G, int dtype, bool matrix) {
    if (dtype < 0) return G > 4 ? 96 : 128;   // a multiple of every kernel's
    if (matrix) return dtype == CK_KV_F32 ? 16 : 32;
    const int waves = 4, rounds = G > 4 ? 3 : 4;
    return waves * rounds * ((dtype == CK_KV_FP8_E4M3 && G <= 4) ? 8 : 4);
}

// The matrix cores take fp32 caches for groups over 4 heads (fp32 MFMA) and
// the bf16 and fp8 caches of one sequence for every group size (bf16 MFMA,
// the exact cache values against two-term q and P); selections keep the
// vector kernel. A batch of unequal sequences over a bf16 or fp8 cache keeps
// it too: the matrix plan's one workgroup per unit leaves the short
// sequences' units idle, and the vector kernel measured faster there (32.9
// against 42.3 us, 8 sequences of 512 to 8192 tokens, 8 KV heads, bf16).
bool attn_matrix_path(int G, int dtype, int m, bool selection) {
    if (selection) return false;
    if (dtype == CK_KV_F32) return G > 4;
    return (dtype == CK_KV_BF16 || dtype == CK_KV_FP8_E4M3) && m == 1;
}

AttnPlan attn_plan(int KV, int G, int max_tokens, long long total_tokens, int chunk_req, int step,
                   bool matrix) {
    AttnPlan p;
    if (chunk_req > 0) {
        p.chunk = chunk_req;
    } else if (matrix) {
        // the matrix-core kernel: about one workgroup per compute unit over
        // all (sequence, KV head, chunk) items, a wave per 16-token tile. Its
        // waves hold one tile each and compute only once their loads have
        // landed, so a unit holding two workgroups sets the time (measured
        // at 4097 tokens x 4 KV heads, 128-wide heads: 9.2 us at 80-token
        // chunks, 208 workgroups, against 10.0 at 48, 344 workgroups)
        if (total_tokens < max_tokens) total_tokens = max_tokens;
        const long long cus = cus_of_current_device();
        const long long c = (total_tokens * KV + cus - 1) / cus;
        p.chunk = (int)((c + step - 1) / step * step);
    } else {
        // about two workgroups per compute unit over all (sequence, KV head,
        // chunk) items: chunks are sized from the tokens of every sequence,
        // so that a batch of unequal lengths still fills the GPU
        const long long target = 2LL * cus_of_current_device();
        if (total_tokens < max_tokens) total_tokens = max_tokens;
        const long long c = (total_tokens * KV + target - 1) / target;
        p.chunk = (int)((c + step - 1) / step * step);
        // between one and one and a half workgroups per compute unit, the
        // units holding two set the time: twice the chunk gives every busy
        // unit the same work in half the workgroups (and half the partials
        // to merge)
        const long long items = (total_tokens + p.chunk - 1) / p.chunk * KV;
        const long long cus = cus_of_current_device();
        if (items > cus && 2 * items <= 3 * cus) p.chunk *= 2;
    }
    if (chunk_req <= 0 && p.chunk < step) p.chunk = step;
    p.nchunks = (max_tokens + p.chunk - 1) / p.chunk;
    if (p.nchunks < 1) p.nchunks = 1;
    return p;
}

int attn_max_chunks(int KV, int G, int max_tokens, int chunk_req) {
    // the largest nchunks attn_plan returns for any positions with at most
    // max_tokens tokens per sequence: an explicit chunk is used as given;
    // the automatic chunk is at least max_tokens * KV / (2 CUs) (the matrix
    // kernel's twice that) and at least the smallest step of a kernel for
    // this group size, so nchunks <= ceil(2 CUs / KV)
    if (chunk_req > 0) return (max_tokens + chunk_req - 1) / chunk_req;
    const int target = 2 * cus_of_current_device();
    const int by_items = (target + KV - 1) / KV;
    const int step = G > 4 ? 16 : 32;
    const int by_tile = (max_tokens + step - 1) / step;
    return by_tile < by_items ? by_tile : by_items;
}

// Workspace of the attention: unnormalized outputs, then (max, sum) per chunk
// and head; each region 256-byte aligned.
size_t attn_partials_bytes(int m, int H, int hd, int nchunks) {
    return up256(sizeof(float) * (size_t)m * H * nchunks * hd) +
           up256(sizeof(float) * (size_t)m * H * nchunks * 2);
}

int attn_first(const Positions &pos, int window, const AttnPlan &plan, int m, bool uniform,
               int *first) {
    first[0] = 0;
    for (int s = 0; s < m; s++) {
        const int n = pos.p[s] + 1 - window_start(pos.p[s] + 1, window);
        first[s + 1] = first[s] + ((pos.dev || uniform) ? plan.nchunks
                                                        : (n + plan.chunk - 1) / plan.chunk);
    }
    for (int s = m + 1; s <= kMaxSeqs; s++) first[s] = first[m];
    return first[m];
}

hipError_t launch_attn_partial(const float *q, const CacheView &c, const Positions &pos, int m,
                               int H, float scale, const AttnPlan &plan, void *partials,
                               hipStream_t st, const SparseSel *sp) {
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
    a.sel = sp ? sp->sel : nullptr;
    a.topk = sp ? sp->topk : 0;
    // work items (a selection: the same topk entries for every sequence)
    attn_first(pos, c.window, plan, m, sp != nullptr, a.first);
    const bool paged = c.page_size != 0;
    return c.head_dim == 64 ? launch_g<64>(a, G, m, paged, st) : launch_g<128>(a, G, m, paged, st);
}

hipError_t launch_attn_merge(const void *partials, const Positions &pos, int window, int m,
                             int H, int KV, int hd, const AttnPlan &plan, float *out,
                             uint8_t *out_q8, hipStream_t st, const SparseSel *sp,
                             uint32_t *ximg) {
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
    b.topk = sp ? sp->topk : 0;
    b.sink = sp ? sp->sink : nullptr;
    b.out = out;
    b.out_q8 = out_q8;
    b.xi = XImage{out_q8 ? ximg : nullptr, m, H * hd / kQK};
    // up to 128 chunks per sequence: one wavefront per 32 chunks (measured
    // faster than the workgroup merge at 22 and 43 chunks with one and two
    // wavefronts, neutral at 57, and faster at 86 with three: 4.4 against
    // 4.9 us at the 7B shape; one wavefront for 43 or 57 chunks measured
    // slower: its serial loads cost more than the barriers save); beyond,
    // the workgroup merge
    const int nwv = (plan.nchunks + kMerge1Chunks - 1) / kMerge1Chunks;
    // a workgroup per 32 output dims while that keeps within one per CU (7B
    // shape: 24.87 against 25.29 us per layer; a batch of 8, whose heads
    // already fill the GPU, measured slower split)
    const bool split = (long long)H * m * (hd / 32) <= cus_of_current_device();
#define CK_MERGE1(HD_, NWV_) \
    do {                                                                                        \
        if (split)                                                                              \
            hipLaunchKernelGGL((k_attn_merge1<HD_, NWV_, 32>), dim3(H, m, HD_ / 32),            \
                               dim3(NWV_ * kWave), 0, st, b);                                   \
        else                                                                                    \
            hipLaunchKernelGGL((k_attn_merge1<HD_, NWV_, HD_>), dim3(H, m), dim3(NWV_ * kWave), \
                               0, st, b);                                                       \
    } while (0)
    if (nwv <= 4) {
        if (hd == 64) {
            if (nwv <= 1) CK_MERGE1(64, 1);
            else if (nwv == 2) CK_MERGE1(64, 2);
            else if (nwv == 3) CK_MERGE1(64, 3);
            else CK_MERGE1(64, 4);
        } else {
            if (nwv <= 1) CK_MERGE1(128, 1);
            else if (nwv == 2) CK_MERGE1(128, 2);
            else if (nwv == 3) CK_MERGE1(128, 3);
            else CK_MERGE1(128, 4);
        }
    } else if (hd == 64) {
        hipLaunchKernelGGL(k_attn_merge<64>, dim3(H, m), dim3(kMergeThreads), 0, st, b);
    } else {
        hipLaunchKernelGGL(k_attn_merge<128>, dim3(H, m), dim3(kMergeThreads), 0, st, b);
    }
#undef CK_MERGE1
    return hipGetLastError();
}

hipError_t launch_attention(const float *q, const CacheView &c, const Positions &pos, float *out,
                            uint8_t *out_q8, int m, int H, float scale, const AttnPlan &plan,
                            void *partials, hipStream_t st, const SparseSel *sp,
                            uint32_t *ximg) {
    hipError_t e = launch_attn_partial(q, c, pos, m, H, scale, plan, partials, st, sp);
    if (e != hipSuccess) return e;
    return launch_attn_merge(partials, pos, c.window, m, H, c.kv_heads, c.head_dim, plan, out,
                             out_q8, st, sp, ximg);
}

}  // namespace ck
