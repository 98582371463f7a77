// k_qkv.hip — fused RMSNorm + Q8_0 + Q/K/V projections + RoPE + KV append.
//
// The first half of the layer of the C-Kernel-Engine page
// "mega_fused_attention_decode_q5_0.c" (MAIN KERNEL steps 1-6) in one launch:
//   xn = RMSNorm(x); xq = Q8_0(xn); q = Wq xq + bq; k = Wk xq + bk; v = Wv xq + bv
//   RoPE(q, k, pos); cache[pos] = (k, v)
// One token per launch. Every workgroup issues the loads of x and gamma and
// then those of its weight rows (they do not depend on x), recomputes the
// normalization and quantization of x into LDS while the weight loads are in
// flight (x and gamma come from L2; every workgroup computes bit-identical
// values), then the block dots.
// Logical rows are ordered so that the two rows a RoPE rotation pairs (head
// element i and i + hd/2) sit in the same wavefront: consecutive iterations
// of a wave when a row spans the wave, neighbouring lane groups otherwise.
// The epilogue adds the bias, rotates q and k and writes k and v into the
// cache at the token's position. Workgroup 0 also writes xn and xq to the
// workspace, so the intermediates can be inspected.
#include "ck_device.hpp"
#include "ck_gemv_common.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

struct QkvArgs {
    const float *x;         // [m][D]
    const float *gamma;     // [D]
    float eps;
    int D, H, KV, hd, m;
    const uint8_t *wq, *wk, *wv;
    const float *bq, *bk, *bv;
    const float *cos_tab, *sin_tab;   // [rows][hd/2]
    Positions pos;
    CacheView c;
    float *q, *k, *v;       // [m][H*hd], [m][KV*hd], [m][KV*hd]
    float *xn;              // [m][D]   written by workgroup 0
    uint8_t *xq;            // [m][D/32] Q8_0 blocks, written by workgroup 0
    int wg_k, wg_v;         // first workgroups of the K and V segments
    unsigned *zero;         // nullable: nzero words, zstride apart, that workgroup 0
    int nzero, zstride;     // clears (the counters of the launch that follows)
};

// Physical row of logical row r of a rotated segment: consecutive logical
// rows (2p, 2p+1) are elements i and i + hd/2 of the same head.
__device__ __forceinline__ int rope_row(int r, int hd) {
    const int half = hd >> 1, p = r >> 1;
    return (p / half) * hd + (p % half) + (r & 1) * half;
}

// RMSNorm + Q8_0 of the token into LDS (codes, fp16-rounded scale, code
// sum); workgroup 0 also writes xn and the xq bytes to the workspace. x and
// gamma arrive preloaded in `in`.
template <bool TAIL>
__device__ __forceinline__ void stage_normalized(const QkvArgs &a, const NormIn &in, XBlock *xs,
                                                 float *red, bool write_trace) {
    const int D = a.D;
    norm_quant_finish<TAIL>(in, a.x, a.gamma, D, a.eps, red,
                            [&](int c, float4 v, uint32_t packed, uint16_t dbits, int csum) {
                                const int b = c >> 3, sub = c & 7;
                                XBlock &xb = xs[b];
                                xb.c[sub] = (int)packed;
                                if (sub == 0) {
                                    xb.d = half_bits_to_float(dbits);
                                    xb.sum = csum;
                                }
                                if (write_trace) {
                                    reinterpret_cast<float4 *>(a.xn)[c] = v;
                                    uint8_t *blk = a.xq + (size_t)b * kQ8Bytes;
                                    uint16_t *dst = reinterpret_cast<uint16_t *>(blk + 2 + 4 * sub);
                                    dst[0] = (uint16_t)(packed & 0xFFFF);
                                    dst[1] = (uint16_t)(packed >> 16);
                                    if (sub == 0) *reinterpret_cast<uint16_t *>(blk) = dbits;
                                }
                            });
}

// One token (the kernel serves m = 1). The loads go out in the order their
// values are needed and none is conditional (rows and units past the end
// re-read the last one; what they contribute is discarded), so that every
// wait covers only what it needs: the memory counter retires loads in issue
// order, and a load under a branch makes the compiler wait early for it and
// for everything before it. Order: the position (device positions), x and
// gamma, bias and RoPE factors, then the weights; the normalization and
// quantization of x run while the weights are in flight.
template <bool Q5, int LPR, int UPL, int R, bool PAIRED, bool TAIL>
__device__ __forceinline__ void qkv_body(const QkvArgs &a, int seg, int wg_in_seg, XBlock *xs,
                                         float *red) {
    using F = Fmt<Q5, PAIRED>;
    constexpr int RPW = kWave / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPR, rsel = lane / LPR;
    const int D = a.D, nb = D / kQK, hd = a.hd, half = hd >> 1;
    const int nunits = nb / F::blocks;
    const size_t row_bytes = (size_t)nb * (Q5 ? kQ5Bytes : kQ8Bytes);
    const uint8_t *W = seg == 0 ? a.wq : (seg == 1 ? a.wk : a.wv);
    const float *bias = seg == 0 ? a.bq : (seg == 1 ? a.bk : a.bv);
    const int rows = (seg == 0 ? a.H : a.KV) * hd;
    const bool rotate = seg < 2;
    const int row0 = (wg_in_seg * kGemvWaves + wave) * (RPW * R);

    // an invalid device position reads table row 0 and appends nothing
    const int pv = a.pos.get(0);
    const int p = max(pv, 0);
    NormIn xin;
    norm_load(a.x, a.gamma, D, xin);

    int pr[R];
    float bias_v[R], cs[R], sn[R];
#pragma unroll
    for (int it = 0; it < R; it++) {
        const int lr = min(row0 + it * RPW + rsel, rows - 1);
        pr[it] = rotate ? rope_row(lr, hd) : lr;
        bias_v[it] = bias ? bias[pr[it]] : 0.0f;
        const int i = (lr >> 1) % half;
        cs[it] = a.cos_tab[(size_t)p * half + i];
        sn[it] = a.sin_tab[(size_t)p * half + i];
    }
    uint32_t wr[R][UPL][F::words];
#pragma unroll
    for (int it = 0; it < R; it++) {
        const uint8_t *rp = W + (size_t)pr[it] * row_bytes;
#pragma unroll
        for (int u = 0; u < UPL; u++) {
            const int unit = min(sub + u * LPR, nunits - 1);
            load_unit<Q5, PAIRED>(rp + (size_t)unit * F::bytes, wr[it][u]);
        }
    }
    // keep the scheduler from moving the normalization's arithmetic above
    // the weight loads
    __builtin_amdgcn_sched_barrier(0);

    // normalized, quantized activations into LDS (overlaps the weight loads)
    stage_normalized<TAIL>(a, xin, xs, red, blockIdx.x == 0);

    // dots, bias, RoPE, stores; units past the row take a zero activation
    // block, so the re-read unit adds exactly zero
    XBlock xb[UPL][F::blocks];
#pragma unroll
    for (int u = 0; u < UPL; u++) {
        const int unit = sub + u * LPR;
#pragma unroll
        for (int b = 0; b < F::blocks; b++) {
            if (unit < nunits)
                xb[u][b] = xs[unit * F::blocks + b];
            else
                xb[u][b] = XBlock{{0, 0, 0, 0, 0, 0, 0, 0}, 0.0f, 0, {0, 0}};
        }
    }
    float val[R];
#pragma unroll
    for (int it = 0; it < R; it++) {
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < UPL; u++) acc = unit_dot<Q5, PAIRED>(wr[it][u], xb[u], acc);
        acc = row_reduce<LPR>(acc);
        val[it] = acc + bias_v[it];
    }
#pragma unroll
    for (int it = 0; it < R; it++) {
        const int lr = row0 + it * RPW + rsel;
        float out = val[it];
        if (rotate) {
            // the partner of this row: the next/previous iteration when a
            // row spans the wave, the neighbouring lane group otherwise
            float other;
            if constexpr (LPR == kWave) {
                other = val[it ^ 1];
            } else {
                other = __shfl_xor(val[it], LPR);
            }
            out = (lr & 1) ? other * sn[it] + val[it] * cs[it] : val[it] * cs[it] - other * sn[it];
        }
        if (sub == 0 && lr < rows) {
            const int g = pr[it] / hd, d = pr[it] % hd;
            if (seg == 0) {
                a.q[pr[it]] = out;
            } else {
                (seg == 1 ? a.k : a.v)[pr[it]] = out;
                const long long off = pv >= 0 ? cache_row(a.c, 0, g, p) : -1;
                if (off >= 0) cache_put(a.c, seg == 1, off + d, out);
            }
        }
    }
}

template <int LPR, int UPL, int R, bool PAIRED, bool TAIL>
__global__ __launch_bounds__(kGemvThreads) void k_qkv(QkvArgs a) {
    extern __shared__ XBlock xs[];
    __shared__ float red[2 * kGemvWaves];
    const int wg = blockIdx.x;
    if (wg == 0)
        for (int i = threadIdx.x; i < a.nzero; i += kGemvThreads)
            __hip_atomic_store(a.zero + (size_t)i * a.zstride, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
    const int seg = wg >= a.wg_v ? 2 : (wg >= a.wg_k ? 1 : 0);
    const int wg_in_seg = wg - (seg == 2 ? a.wg_v : (seg == 1 ? a.wg_k : 0));
    if (seg == 2)
        qkv_body<false, LPR, UPL, R, PAIRED, TAIL>(a, seg, wg_in_seg, xs, red);
    else
        qkv_body<true, LPR, UPL, R, PAIRED, TAIL>(a, seg, wg_in_seg, xs, red);
}

template <int LPR, int UPL, int R, bool PAIRED>
hipError_t launch_t(QkvArgs a, hipStream_t st) {
    const int rows_per_wg = kGemvWaves * (kWave / LPR) * R;
    const int nq = (a.H * a.hd + rows_per_wg - 1) / rows_per_wg;
    const int nk = (a.KV * a.hd + rows_per_wg - 1) / rows_per_wg;
    a.wg_k = nq;
    a.wg_v = nq + nk;
    const size_t lds = sizeof(XBlock) * (size_t)(a.D / kQK);
    if (a.D <= NormIn::KEEP * kGemvThreads * 4)
        hipLaunchKernelGGL((k_qkv<LPR, UPL, R, PAIRED, false>), dim3(nq + 2 * nk),
                           dim3(kGemvThreads), lds, st, a);
    else
        hipLaunchKernelGGL((k_qkv<LPR, UPL, R, PAIRED, true>), dim3(nq + 2 * nk),
                           dim3(kGemvThreads), lds, st, a);
    return hipGetLastError();
}

template <int LPR, bool PAIRED, int R>
hipError_t launch_upl_r(const QkvArgs &a, int upl, hipStream_t st) {
    if (upl <= 1) return launch_t<LPR, 1, R, PAIRED>(a, st);
    if (upl <= 2) return launch_t<LPR, 2, R, PAIRED>(a, st);
    return launch_t<LPR, 4, R, PAIRED>(a, st);
}

template <int LPR, bool PAIRED>
hipError_t launch_upl(const QkvArgs &a, int upl, hipStream_t st) {
    // rows per wave and iteration: 2 (a RoPE pair when a row spans the
    // wave), so that the workgroups are small and many, each CU's share of
    // the weights, not the total, setting the time (four rows measured
    // slower at the 7B shape); 1 where rows narrower than the wave pair up
    // across lane groups and 2 would leave compute units without a
    // workgroup
    if constexpr (LPR < kWave) {
        const int per2 = kGemvWaves * (kWave / LPR) * 2;
        const int total2 = (a.H * a.hd + per2 - 1) / per2 + 2 * ((a.KV * a.hd + per2 - 1) / per2);
        if (total2 < num_cus()) return launch_upl_r<LPR, PAIRED, 1>(a, upl, st);
    }
    return launch_upl_r<LPR, PAIRED, 2>(a, upl, st);
}

template <bool PAIRED>
hipError_t launch_lpr(const QkvArgs &a, int nunits, hipStream_t st) {
    if (nunits <= 4) return launch_upl<4, PAIRED>(a, 1, st);
    if (nunits <= 8) return launch_upl<8, PAIRED>(a, 1, st);
    if (nunits <= 16) return launch_upl<16, PAIRED>(a, 1, st);
    if (nunits <= 32) return launch_upl<32, PAIRED>(a, 1, st);
    return launch_upl<64, PAIRED>(a, (nunits + 63) / 64, st);
}

}  // namespace

// One token per call only: every workgroup recomputes the normalization of
// the input, which is one row's latency for one token but serializes m rows
// for a batch (measured on the 8-token paged workload: the separate
// normalization kernel, parallel over tokens, then the projections saved
// about 20 us per layer).
bool qkv_shape_supported(int D, int m) {
    const int nb = D / kQK;
    const int nunits = (nb % 2 == 0) ? nb / 2 : nb;
    return m == 1 && nunits <= 64 * 4 && sizeof(XBlock) * (size_t)m * nb <= 64 * 1024;
}

hipError_t launch_qkv(const float *x, const float *gamma, float eps, int D, int H, int KV, int hd,
                      int m, const uint8_t *wq, const uint8_t *wk, const uint8_t *wv,
                      const float *bq, const float *bk, const float *bv, const float *cos_tab,
                      const float *sin_tab, const Positions &pos, const CacheView &c, float *q,
                      float *k, float *v, float *xn, uint8_t *xq, hipStream_t st,
                      unsigned *zero, int nzero, int zstride) {
    QkvArgs a;
    a.x = x;
    a.gamma = gamma;
    a.eps = eps;
    a.D = D;
    a.H = H;
    a.KV = KV;
    a.hd = hd;
    a.m = m;
    a.wq = wq;
    a.wk = wk;
    a.wv = wv;
    a.bq = bq;
    a.bk = bk;
    a.bv = bv;
    a.cos_tab = cos_tab;
    a.sin_tab = sin_tab;
    a.pos = pos;
    a.c = c;
    a.q = q;
    a.k = k;
    a.v = v;
    a.xn = xn;
    a.xq = xq;
    a.wg_k = a.wg_v = 0;
    a.zero = zero;
    a.nzero = zero ? nzero : 0;
    a.zstride = zstride;
    const int nb = D / kQK;
    return (nb % 2 == 0) ? launch_lpr<true>(a, nb / 2, st) : launch_lpr<false>(a, nb, st);
}

}  // namespace ck
