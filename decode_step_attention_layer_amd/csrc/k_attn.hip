// k_attn.hip — split-K grouped-query decode attention for gfx950.
//
// What it computes (C-Kernel-Engine "mega_fused_attention_decode_q5_0.c",
// MAIN KERNEL STEP 7): for query head h, KV head g = h*KV/H, tokens t <= pos,
//   out_h = sum_t softmax_t(scale * q_h . K_g[t]) V_g[t].
// Paged caches are addressed through the block table of the metrale
// "prefill_attn_a.rs" paged decode launchers; the GQA packing (one workgroup
// serves all query heads of a KV head) follows its paged_decode_attn_*_gqa.
//
// Pass 1 (k_attn_partial), grid (chunk, KV head, sequence): a workgroup walks
// its chunk in tiles of 64 tokens. K and V tiles are staged through LDS with
// coalesced 16-byte loads (prefetched into registers one tile ahead), so every
// K/V byte is read from HBM once for the whole query group. Scores: wave w
// owns heads w and w+4, lane = token, q read through the scalar unit; online
// softmax keeps a running max per head and per-lane partial sums. P.V: thread
// = (4 output dims, token subset), p broadcast from LDS. The chunk's
// (max, sum, unnormalized output) per head goes to the partials buffer.
// Pass 2 (k_attn_merge), grid (head, sequence): log-sum-exp merge of the
// chunks, optionally followed by Q8_0 quantization of the head's output.
#include "ck_device.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kTile = 64;  // tokens per tile
constexpr int kMaxG = 8;

struct AttnArgs {
    const float *q;       // [m][H][HD]
    CacheView c;
    Positions pos;
    float scale;
    int chunk;            // tokens per chunk, multiple of kTile
    int nchunks;
    int H;
    float *po;            // [m][KV][nchunks][G][HD]
    float *pml;           // [m][KV][nchunks][G][2]  (max, sum)
};

template <int HD>
struct Smem {
    static constexpr int stride = HD + 4;  // padded row: conflict-free b128 reads
    float kv[2 * kTile * stride];           // K tile, then V tile
    float p[kTile * kMaxG];
    float alpha[kMaxG];
    int bad;
};

template <int HD, int G>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(AttnArgs a) {
    static_assert(HD % 64 == 0 && G >= 1 && G <= kMaxG, "shape");
    constexpr int C4 = HD / 4;                       // float4 columns per row
    constexpr int NLD = kTile * C4 / kAttnThreads;   // float4 loads per thread per tile (K or V)
    constexpr int ROWS_PER_LD = kAttnThreads / C4;   // rows covered by one load round
    constexpr int NTG = kAttnThreads / C4;           // token groups in the P.V phase
    constexpr int TPG = kTile / NTG;                 // tokens per group per tile
    constexpr int S = Smem<HD>::stride;
    __shared__ Smem<HD> sm;

    const int cidx = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    const int L = a.pos.p[s] + 1;
    const int t0 = cidx * a.chunk;
    if (t0 >= L) return;                             // the merge skips this chunk
    const int t1 = min(L, t0 + a.chunk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, KV = a.c.kv_heads;
    const float *qg = a.q + ((size_t)s * H + (size_t)g * G) * HD;

    float *sk = sm.kv;
    float *sv_ = sm.kv + kTile * S;
    if (tid == 0) sm.bad = 0;
    __syncthreads();

    // loader geometry: this thread loads column ld_col of rows ld_row + i*ROWS_PER_LD
    const int ld_col = tid % C4, ld_row = tid / C4;
    float4 kreg[NLD], vreg[NLD];
    auto fetch = [&](int st) {
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int t = st + ld_row + i * ROWS_PER_LD;
            long long off = -1;
            if (t < t1) {
                off = cache_row(a.c, s, g, t);
                if (off < 0) sm.bad = 1;
            }
            if (off >= 0) {
                kreg[i] = *reinterpret_cast<const float4 *>(a.c.k + off + 4 * ld_col);
                vreg[i] = *reinterpret_cast<const float4 *>(a.c.v + off + 4 * ld_col);
            } else {
                kreg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                vreg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int r = ld_row + i * ROWS_PER_LD;
            *reinterpret_cast<float4 *>(&sk[r * S + 4 * ld_col]) = kreg[i];
            *reinterpret_cast<float4 *>(&sv_[r * S + 4 * ld_col]) = vreg[i];
        }
    };

    // score-phase state: this wave's heads (w, w+4), running max and per-lane sums
    constexpr int HPW = (G + 3) / 4;
    float m_run[HPW], l_lane[HPW];
#pragma unroll
    for (int k = 0; k < HPW; k++) { m_run[k] = -INFINITY; l_lane[k] = 0.0f; }

    // P.V state: dims 4*pv_col.., tokens pv_tg + j*NTG of each tile
    const int pv_col = tid % C4, pv_tg = tid / C4;
    float4 o[G];
#pragma unroll
    for (int j = 0; j < G; j++) o[j] = make_float4(0.f, 0.f, 0.f, 0.f);

    fetch(t0);
    for (int st = t0; st < t1; st += kTile) {
        __syncthreads();                 // previous tile fully consumed
        stash();
        __syncthreads();
        if (st + kTile < t1) fetch(st + kTile);   // next tile's loads in flight

        // ---- scores, one token per lane, heads w and w+4
        const int tok = st + lane;
        float sc[HPW];
#pragma unroll
        for (int k = 0; k < HPW; k++) sc[k] = 0.0f;
        const float *krow = &sk[lane * S];
#pragma unroll 4
        for (int d = 0; d < HD; d += 4) {
            const float4 kk = *reinterpret_cast<const float4 *>(krow + d);
#pragma unroll
            for (int k = 0; k < HPW; k++) {
                const int j = wave + 4 * k;
                if (j < G) {
                    const float *qj = qg + (size_t)j * HD + d;
                    sc[k] = fmaf(kk.x, qj[0], sc[k]);
                    sc[k] = fmaf(kk.y, qj[1], sc[k]);
                    sc[k] = fmaf(kk.z, qj[2], sc[k]);
                    sc[k] = fmaf(kk.w, qj[3], sc[k]);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < HPW; k++) {
            const int j = wave + 4 * k;
            if (j < G) {
                const float sv = tok < t1 ? sc[k] * a.scale : -INFINITY;
                const float m_new = fmaxf(m_run[k], wave_max(sv));
                const float alpha = __expf(m_run[k] - m_new);
                const float p = __expf(sv - m_new);
                l_lane[k] = l_lane[k] * alpha + p;
                m_run[k] = m_new;
                sm.p[lane * kMaxG + j] = p;
                if (lane == 0) sm.alpha[j] = alpha;
            }
        }
        __syncthreads();

        // ---- P.V
#pragma unroll
        for (int j = 0; j < G; j++) {
            const float al = sm.alpha[j];
            o[j].x *= al; o[j].y *= al; o[j].z *= al; o[j].w *= al;
        }
#pragma unroll 2
        for (int i = 0; i < TPG; i++) {
            const int r = pv_tg + i * NTG;
            const float4 vv = *reinterpret_cast<const float4 *>(&sv_[r * S + 4 * pv_col]);
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

    // ---- reduce the P.V token groups through LDS (reusing the K/V tiles)
    float *red = sm.kv;   // [NTG][G][HD] floats
    static_assert(NTG * G * HD <= 2 * kTile * (HD + 4), "reduction buffer");
#pragma unroll
    for (int j = 0; j < G; j++)
        *reinterpret_cast<float4 *>(&red[(pv_tg * G + j) * HD + 4 * pv_col]) = o[j];
    float lsum[HPW];
#pragma unroll
    for (int k = 0; k < HPW; k++) lsum[k] = wave_sum(l_lane[k]);
    __syncthreads();

    const size_t part = ((size_t)s * KV + g) * a.nchunks + cidx;
    const bool bad = sm.bad != 0;
    for (int e = tid; e < G * HD; e += kAttnThreads) {
        float acc = 0.0f;
#pragma unroll
        for (int tg = 0; tg < NTG; tg++) acc += red[tg * G * HD + e];
        a.po[part * G * HD + e] = acc;
    }
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < HPW; k++) {
            const int j = wave + 4 * k;
            if (j < G) {
                a.pml[(part * G + j) * 2 + 0] = m_run[k];
                a.pml[(part * G + j) * 2 + 1] = bad ? NAN : lsum[k];
            }
        }
    }
}

struct MergeArgs {
    const float *po;
    const float *pml;
    Positions pos;
    int chunk, nchunks, H, KV;
    float *out;          // [m][H][HD]
    uint8_t *out_q8;     // nullable: [m][H*HD/32] Q8_0 blocks
};

template <int HD>
__global__ __launch_bounds__(HD) void k_attn_merge(MergeArgs a) {
    const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
    const int G = a.H / a.KV, g = h / G, j = h % G;
    const int L = a.pos.p[s] + 1;
    const int nc = (L + a.chunk - 1) / a.chunk;
    const size_t base = ((size_t)s * a.KV + g) * a.nchunks;
    float M = -INFINITY;
    for (int c = 0; c < nc; c++) M = fmaxf(M, a.pml[((base + c) * G + j) * 2]);
    float num = 0.0f, den = 0.0f;
    for (int c = 0; c < nc; c++) {
        const size_t pj = (base + c) * G + j;
        const float w = __expf(a.pml[pj * 2] - M);
        den = fmaf(w, a.pml[pj * 2 + 1], den);
        num = fmaf(w, a.po[pj * HD + d], num);
    }
    const float v = num / den;
    const size_t oi = ((size_t)s * a.H + h) * HD + d;
    a.out[oi] = v;
    if (a.out_q8) {
        int code;
        uint16_t dbits;
        quantize_q8_0_half(v, code, dbits);
        uint8_t *blk = a.out_q8 + (oi / kQK) * kQ8Bytes;
        blk[2 + (d & 31)] = (uint8_t)(int8_t)code;
        if ((d & 31) == 0) {
            blk[0] = (uint8_t)(dbits & 0xFF);
            blk[1] = (uint8_t)(dbits >> 8);
        }
    }
}

template <int HD, int G>
hipError_t launch_partial(const AttnArgs &a, int m, hipStream_t st) {
    hipLaunchKernelGGL((k_attn_partial<HD, G>), dim3(a.nchunks, a.c.kv_heads, m),
                       dim3(kAttnThreads), 0, st, a);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_partial_g(const AttnArgs &a, int G, int m, hipStream_t st) {
    switch (G) {
        case 1: return launch_partial<HD, 1>(a, m, st);
        case 2: return launch_partial<HD, 2>(a, m, st);
        case 3: return launch_partial<HD, 3>(a, m, st);
        case 4: return launch_partial<HD, 4>(a, m, st);
        case 5: return launch_partial<HD, 5>(a, m, st);
        case 6: return launch_partial<HD, 6>(a, m, st);
        case 7: return launch_partial<HD, 7>(a, m, st);
        case 8: return launch_partial<HD, 8>(a, m, st);
    }
    return hipErrorInvalidValue;
}

// Compute units of the current device, queried once per device (the value
// cannot change; a racing first query writes the same number).
int num_cus() {
    static int cached[64];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    if (dev < 64) cached[dev] = n;
    return n;
}

}  // namespace

bool attn_shape_supported(int G, int hd) {
    return G >= 1 && G <= kMaxG && (hd == 64 || hd == 128);
}

AttnPlan attn_plan(int m, int KV, int max_tokens, int chunk_req) {
    AttnPlan p;
    if (chunk_req > 0) {
        p.chunk = (chunk_req + kTile - 1) / kTile * kTile;
    } else {
        // about two workgroups per compute unit over all (sequence, KV head) pairs
        int target = 2 * num_cus() / (m * KV);
        if (target < 1) target = 1;
        int c = (max_tokens + target - 1) / target;
        p.chunk = (c + kTile - 1) / kTile * kTile;
    }
    if (p.chunk < kTile) p.chunk = kTile;
    p.nchunks = (max_tokens + p.chunk - 1) / p.chunk;
    if (p.nchunks < 1) p.nchunks = 1;
    return p;
}

int attn_max_chunks(int m, int KV, int max_tokens, int chunk_req) {
    // the largest nchunks attn_plan returns for any token count <= max_tokens
    if (chunk_req > 0) return attn_plan(m, KV, max_tokens, chunk_req).nchunks;
    int target = 2 * num_cus() / (m * KV);
    if (target < 1) target = 1;
    int by_tile = (max_tokens + kTile - 1) / kTile;
    return by_tile < target ? by_tile : target;
}

size_t attn_partials_bytes(int m, int H, int hd, int nchunks) {
    // o: m*H*nchunks*hd floats, (max, sum): m*H*nchunks*2 floats
    return sizeof(float) * (size_t)m * H * nchunks * (hd + 2);
}

hipError_t launch_attention(const float *q, const CacheView &c, const Positions &pos, float *out,
                            uint8_t *out_q8, int m, int H, float scale, const AttnPlan &plan,
                            void *partials, hipStream_t st) {
    const int G = H / c.kv_heads;
    AttnArgs a;
    a.q = q;
    a.c = c;
    a.pos = pos;
    a.scale = scale;
    a.chunk = plan.chunk;
    a.nchunks = plan.nchunks;
    a.H = H;
    a.po = reinterpret_cast<float *>(partials);
    a.pml = a.po + (size_t)m * H * plan.nchunks * c.head_dim;
    hipError_t e = c.head_dim == 64 ? launch_partial_g<64>(a, G, m, st)
                                    : launch_partial_g<128>(a, G, m, st);
    if (e != hipSuccess) return e;
    MergeArgs b;
    b.po = a.po;
    b.pml = a.pml;
    b.pos = pos;
    b.chunk = plan.chunk;
    b.nchunks = plan.nchunks;
    b.H = H;
    b.KV = c.kv_heads;
    b.out = out;
    b.out_q8 = out_q8;
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_attn_merge<64>, dim3(H, m), dim3(64), 0, st, b);
    else
        hipLaunchKernelGGL(k_attn_merge<128>, dim3(H, m), dim3(128), 0, st, b);
    return hipGetLastError();
}

}  // namespace ck
