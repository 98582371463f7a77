// k_gemv.hip — Q5_0 / Q8_0 weight x Q8_0 activation GEMV for gfx950.
//
// Computes, for every token s and output row r of up to three weight
// segments in one launch (Q, K and V share one quantized input, as the page's
// helper "Q5_0 GEMV with inline processing" feeds each projection the same
// quantized row):
//   y[s][r] = sum_b d_w(r,b) * d_x(s,b) * S(r,s,b) + bias[r] (+ residual[s][r])
// with S the exact integer dot of block b (v_dot4_i32_i8 over int8 lanes).
//
// Mapping: a row is owned by LPR lanes of one wavefront (LPR = 64 for long
// rows: one row per wavefront; fewer for short rows, several rows per wave).
// A lane owns "units" of the row: pairs of consecutive blocks (44 B of Q5_0
// or 68 B of Q8_0, dword aligned whenever K/32 is even) read with dwordx4
// loads straight from the canonical block layout, or single blocks read with
// 16-bit loads when K/32 is odd. Each wavefront loads the weights of its R
// rows before any arithmetic, keeps them in registers and reuses them for all
// m tokens. The quantized activations are staged once per workgroup into LDS
// in a dword-aligned form (codes, scale as fp32, code sum for the Q5_0 offset)
// while the weight loads are in flight (for one token, their loads are issued
// before the weights').
// Partial sums are reduced across the LPR lanes with DPP / ds_swizzle.
#include "ck_device.hpp"
#include "ck_gemv_common.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

// Stages the quantized activations (m * nb Q8_0 blocks) into LDS in a
// dword-aligned form: codes, fp32 scale, code sum. Ends with a barrier.
__device__ __forceinline__ void stage_xq(const uint8_t *xq, int nxb, XBlock *xs) {
    for (int b = threadIdx.x; b < nxb; b += kGemvThreads) {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(xq + (size_t)b * kQ8Bytes);
        XBlock xb;
        xb.d = half_bits_to_float(src[0]);
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t c = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
            xb.c[i] = (int)c;
            sum = __builtin_amdgcn_sdot4((int)c, 0x01010101, sum, false);
        }
        xb.sum = sum;
        xb.pad[0] = xb.pad[1] = 0;
        xs[b] = xb;
    }
    __syncthreads();
}

template <bool Q5, int LPR, int UPL, int R, bool PAIRED>
__device__ __forceinline__ void gemv_body(const GemvSeg &sg, int wg_in_seg, XBlock *xs,
                                          const uint8_t *xq, int nb, int m) {
    using F = Fmt<Q5, PAIRED>;
    constexpr int RPW = kWave / LPR;  // rows per wave per iteration
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPR, rsel = lane / LPR;
    const int nunits = nb / F::blocks;
    const size_t row_bytes = (size_t)nb * (Q5 ? kQ5Bytes : kQ8Bytes);
    const int row0 = (wg_in_seg * kGemvWaves + wave) * (RPW * R);

    // 1. weights of all R rows into registers (all loads issued up front)
    uint32_t wr[R][UPL][F::words];
#pragma unroll
    for (int it = 0; it < R; it++) {
        const int row = row0 + it * RPW + rsel;
        const uint8_t *rp = sg.W + (size_t)row * row_bytes;
#pragma unroll
        for (int u = 0; u < UPL; u++) {
            const int unit = sub + u * LPR;
            if (row < sg.rows && unit < nunits) {
                load_unit<Q5, PAIRED>(rp + (size_t)unit * F::bytes, wr[it][u]);
            } else {
#pragma unroll
                for (int i = 0; i < F::words; i++) wr[it][u][i] = 0;
            }
        }
    }

    // bias and the first token's residual do not depend on anything either:
    // their loads go out with the weights' (one round trip less at the end)
    float bias_v[R], res0[R];
#pragma unroll
    for (int it = 0; it < R; it++) {
        const int row = row0 + it * RPW + rsel;
        const bool mine = sub == 0 && row < sg.rows;
        bias_v[it] = (mine && sg.bias) ? sg.bias[row] : 0.0f;
        res0[it] = (mine && sg.residual) ? sg.residual[row] : 0.0f;
    }

    // 2. the activations into LDS while the weight loads are in flight
    stage_xq(xq, m * nb, xs);

    // 3. per token: activation blocks of this lane's units, dots, reduction
    for (int s = 0; s < m; s++) {
        XBlock xb[UPL][F::blocks];
#pragma unroll
        for (int u = 0; u < UPL; u++) {
            const int unit = sub + u * LPR;
#pragma unroll
            for (int b = 0; b < F::blocks; b++) {
                if (unit < nunits) {
                    xb[u][b] = xs[(size_t)s * nb + unit * F::blocks + b];
                } else {
                    xb[u][b] = XBlock{{0, 0, 0, 0, 0, 0, 0, 0}, 0.0f, 0, {0, 0}};
                }
            }
        }
#pragma unroll
        for (int it = 0; it < R; it++) {
            float acc = 0.0f;
#pragma unroll
            for (int u = 0; u < UPL; u++) acc = unit_dot<Q5, PAIRED>(wr[it][u], xb[u], acc);
            acc = row_reduce<LPR>(acc);
            const int row = row0 + it * RPW + rsel;
            if (sub == 0 && row < sg.rows) {
                float o = acc + bias_v[it];
                if (sg.residual) o = o + (s == 0 ? res0[it] : sg.residual[(size_t)s * sg.rows + row]);
                sg.y[(size_t)s * sg.rows + row] = o;
            }
        }
    }
}

// One token with at most 256 activation blocks (m = 1, K <= 8192). The
// loads go out in the order their values are needed and none is
// conditional (rows and units past the end re-read the last one; what they
// contribute is discarded), because the memory counter retires loads in
// issue order and a load under a branch makes the compiler wait early for
// it and for everything before it: this thread's activation block, bias and
// residual, then the weights. The activation block is staged into LDS while
// the weights are in flight.
template <bool Q5, int LPR, int UPL, int R, bool PAIRED>
__device__ __forceinline__ void gemv_body1(const GemvSeg &sg, int wg_in_seg, XBlock *xs,
                                           const uint8_t *xq, int nb) {
    using F = Fmt<Q5, PAIRED>;
    constexpr int RPW = kWave / LPR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPR, rsel = lane / LPR;
    const int nunits = nb / F::blocks;
    const size_t row_bytes = (size_t)nb * (Q5 ? kQ5Bytes : kQ8Bytes);
    const int row0 = (wg_in_seg * kGemvWaves + wave) * (RPW * R);

    const uint16_t *src = reinterpret_cast<const uint16_t *>(xq + (size_t)min(tid, nb - 1) * kQ8Bytes);
    uint32_t xr[9];
    xr[0] = src[0];
#pragma unroll
    for (int i = 0; i < 8; i++) xr[1 + i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);

    int row[R];
    float bias_v[R], res_v[R];
#pragma unroll
    for (int it = 0; it < R; it++) {
        row[it] = min(row0 + it * RPW + rsel, sg.rows - 1);
        bias_v[it] = sg.bias ? sg.bias[row[it]] : 0.0f;
        res_v[it] = sg.residual ? sg.residual[row[it]] : 0.0f;
    }
    uint32_t wr[R][UPL][F::words];
#pragma unroll
    for (int it = 0; it < R; it++) {
        const uint8_t *rp = sg.W + (size_t)row[it] * row_bytes;
#pragma unroll
        for (int u = 0; u < UPL; u++) {
            const int unit = min(sub + u * LPR, nunits - 1);
            load_unit<Q5, PAIRED>(rp + (size_t)unit * F::bytes, wr[it][u]);
        }
    }
    // keep the scheduler from moving the staging above the weight loads
    __builtin_amdgcn_sched_barrier(0);

    if (tid < nb) {
        XBlock xb;
        xb.d = half_bits_to_float(xr[0]);
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            xb.c[i] = (int)xr[1 + i];
            sum = __builtin_amdgcn_sdot4((int)xr[1 + i], 0x01010101, sum, false);
        }
        xb.sum = sum;
        xb.pad[0] = xb.pad[1] = 0;
        xs[tid] = xb;
    }
    __syncthreads();

    // units past the row take a zero activation block: the re-read unit adds
    // exactly zero
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
#pragma unroll
    for (int it = 0; it < R; it++) {
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < UPL; u++) acc = unit_dot<Q5, PAIRED>(wr[it][u], xb[u], acc);
        acc = row_reduce<LPR>(acc);
        const int r = row0 + it * RPW + rsel;
        if (sub == 0 && r < sg.rows) {
            float o = acc + bias_v[it];
            if (sg.residual) o = o + res_v[it];
            sg.y[r] = o;
        }
    }
}

template <int LPR, int UPL, int R, bool PAIRED, bool ONE>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(GemvArgs a) {
    extern __shared__ XBlock xs[];
    const int wg = blockIdx.x;
    const int si = (a.nseg > 2 && wg >= a.seg[2].wg_begin) ? 2
                   : (a.nseg > 1 && wg >= a.seg[1].wg_begin) ? 1 : 0;
    const GemvSeg sg = si == 0 ? a.seg[0] : (si == 1 ? a.seg[1] : a.seg[2]);
    const int nb = a.K / kQK;

    const int wg_in_seg = wg - sg.wg_begin;
    if constexpr (ONE) {
        if (sg.is_q5)
            gemv_body1<true, LPR, UPL, R, PAIRED>(sg, wg_in_seg, xs, a.xq, nb);
        else
            gemv_body1<false, LPR, UPL, R, PAIRED>(sg, wg_in_seg, xs, a.xq, nb);
    } else {
        if (sg.is_q5)
            gemv_body<true, LPR, UPL, R, PAIRED>(sg, wg_in_seg, xs, a.xq, nb, a.m);
        else
            gemv_body<false, LPR, UPL, R, PAIRED>(sg, wg_in_seg, xs, a.xq, nb, a.m);
    }
}

// Rows per wave and iteration: 2, or 1 where 2 would leave compute units
// without a workgroup (the Qwen2-0.5B-shaped O projection, 28 workgroups
// against 56: 15.6 against 16.1 us per layer; at the 7B and long-context
// shapes, 448 and 512 workgroups, one row measured the same or slower).
template <int LPR, int UPL, bool PAIRED, int R>
hipError_t launch_t(GemvArgs a, hipStream_t st) {
    const int rows_per_wg = kGemvWaves * (kWave / LPR) * R;
    int total = 0;
    for (int i = 0; i < a.nseg; i++) {
        a.seg[i].wg_begin = total;
        total += (a.seg[i].rows + rows_per_wg - 1) / rows_per_wg;
    }
    for (int i = a.nseg; i < 3; i++) a.seg[i] = a.seg[0], a.seg[i].wg_begin = 1 << 30;
    const size_t lds = sizeof(XBlock) * (size_t)a.m * (a.K / kQK);
    if (a.m == 1 && a.K / kQK <= kGemvThreads)
        hipLaunchKernelGGL((k_gemv<LPR, UPL, R, PAIRED, true>), dim3(total),
                           dim3(kGemvThreads), lds, st, a);
    else
        hipLaunchKernelGGL((k_gemv<LPR, UPL, R, PAIRED, false>), dim3(total),
                           dim3(kGemvThreads), lds, st, a);
    return hipGetLastError();
}

template <int LPR, bool PAIRED, int R>
hipError_t launch_upl_r(const GemvArgs &a, int upl, hipStream_t st) {
    if (upl <= 1) return launch_t<LPR, 1, PAIRED, R>(a, st);
    if (upl <= 2) return launch_t<LPR, 2, PAIRED, R>(a, st);
    return launch_t<LPR, 4, PAIRED, R>(a, st);
}

template <int LPR, bool PAIRED>
hipError_t launch_upl(const GemvArgs &a, int upl, hipStream_t st) {
    const int rows_per_wg2 = kGemvWaves * (kWave / LPR) * 2;
    int total2 = 0;
    for (int i = 0; i < a.nseg; i++) total2 += (a.seg[i].rows + rows_per_wg2 - 1) / rows_per_wg2;
    if (total2 < num_cus()) return launch_upl_r<LPR, PAIRED, 1>(a, upl, st);
    return launch_upl_r<LPR, PAIRED, 2>(a, upl, st);
}

template <bool PAIRED>
hipError_t launch_lpr(const GemvArgs &a, int nunits, hipStream_t st) {
    if (nunits <= 4) return launch_upl<4, PAIRED>(a, 1, st);
    if (nunits <= 8) return launch_upl<8, PAIRED>(a, 1, st);
    if (nunits <= 16) return launch_upl<16, PAIRED>(a, 1, st);
    if (nunits <= 32) return launch_upl<32, PAIRED>(a, 1, st);
    return launch_upl<64, PAIRED>(a, (nunits + 63) / 64, st);
}

constexpr size_t kGemvLds = 64 * 1024;

}  // namespace

bool gemv_shape_supported(int K) {
    const int nb = K / kQK;
    const int nunits = (nb % 2 == 0) ? nb / 2 : nb;
    return nunits <= 64 * 4 && sizeof(XBlock) * (size_t)nb <= kGemvLds;
}

// Tokens are processed in slices whose staged activations fit the LDS budget;
// each slice re-reads the weights, so a slice holds as many tokens as fit.
hipError_t launch_gemv(const GemvArgs &a, hipStream_t st) {
    const int nb = a.K / kQK;
    const int per = (int)(kGemvLds / (sizeof(XBlock) * (size_t)nb));
    for (int s0 = 0; s0 < a.m; s0 += per) {
        GemvArgs b = a;
        b.m = a.m - s0 < per ? a.m - s0 : per;
        b.xq = a.xq + (size_t)s0 * nb * kQ8Bytes;
        for (int i = 0; i < a.nseg; i++) {
            b.seg[i].y = a.seg[i].y + (size_t)s0 * a.seg[i].rows;
            if (a.seg[i].residual) b.seg[i].residual = a.seg[i].residual + (size_t)s0 * a.seg[i].rows;
        }
        hipError_t e = (nb % 2 == 0) ? launch_lpr<true>(b, nb / 2, st) : launch_lpr<false>(b, nb, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ck
