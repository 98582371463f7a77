// ck_gemv_common.hpp — the block-GEMV building blocks shared by the plain
// GEMV kernel (k_gemv.hip) and the fused QKV kernel (k_qkv.hip): weight-unit
// formats and loads, the staged activation block, the unit dot product and
// the reduction of a row's partial sums across its lanes.
#pragma once

#include "ck_device.hpp"

namespace ck {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// Words of register storage for one unit of each format.
template <bool Q5, bool PAIRED>
struct Fmt {
    static constexpr int blocks = PAIRED ? 2 : 1;
    static constexpr int bytes = (Q5 ? kQ5Bytes : kQ8Bytes) * blocks;
    static constexpr int words = PAIRED ? (Q5 ? 11 : 17) : (Q5 ? 6 : 9);
};

template <bool Q5, bool PAIRED>
__device__ __forceinline__ void load_unit(const uint8_t *p, uint32_t *w) {
    if constexpr (PAIRED) {
        const uint32_t *p32 = reinterpret_cast<const uint32_t *>(p);
        if constexpr (Q5) {
            u32x4a4 a = *reinterpret_cast<const u32x4a4 *>(p32);
            u32x4a4 b = *reinterpret_cast<const u32x4a4 *>(p32 + 4);
            u32x3a4 c = *reinterpret_cast<const u32x3a4 *>(p32 + 8);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
            w[8] = c.x; w[9] = c.y; w[10] = c.z;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                u32x4a4 a = *reinterpret_cast<const u32x4a4 *>(p32 + 4 * i);
                w[4 * i] = a.x; w[4 * i + 1] = a.y; w[4 * i + 2] = a.z; w[4 * i + 3] = a.w;
            }
            w[16] = p32[16];
        }
    } else {
        const uint16_t *p16 = reinterpret_cast<const uint16_t *>(p);
        w[0] = p16[0];
        if constexpr (Q5) {
            w[1] = (uint32_t)p16[1] | ((uint32_t)p16[2] << 16);
#pragma unroll
            for (int i = 0; i < 4; i++) w[2 + i] = (uint32_t)p16[3 + 2 * i] | ((uint32_t)p16[4 + 2 * i] << 16);
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) w[1 + i] = (uint32_t)p16[1 + 2 * i] | ((uint32_t)p16[2 + 2 * i] << 16);
        }
    }
}

// Activation block staged in LDS / registers.
struct alignas(16) XBlock {
    int c[8];     // 32 int8 codes, 4 per dword
    float d;      // scale
    int sum;      // sum of the 32 codes
    int pad[2];
};

// Dot of one weight unit with its activation blocks.
template <bool Q5, bool PAIRED>
__device__ __forceinline__ float unit_dot(const uint32_t *w, const XBlock *x, float acc) {
    if constexpr (PAIRED && Q5) {
        int s0 = q5_codes_dot(align2(w[1], w[0]), align2(w[2], w[1]), align2(w[3], w[2]),
                              align2(w[4], w[3]), align2(w[5], w[4]), x[0].c) - 16 * x[0].sum;
        acc = fmaf((float)s0, half_bits_to_float(w[0]) * x[0].d, acc);
        int s1 = q5_codes_dot(w[6], w[7], w[8], w[9], w[10], x[1].c) - 16 * x[1].sum;
        acc = fmaf((float)s1, half_bits_to_float(w[5] >> 16) * x[1].d, acc);
    } else if constexpr (PAIRED) {
        uint32_t c0[8];
#pragma unroll
        for (int i = 0; i < 8; i++) c0[i] = align2(w[i + 1], w[i]);
        int s0 = q8_codes_dot(c0, x[0].c);
        acc = fmaf((float)s0, half_bits_to_float(w[0]) * x[0].d, acc);
        int s1 = q8_codes_dot(w + 9, x[1].c);
        acc = fmaf((float)s1, half_bits_to_float(w[8] >> 16) * x[1].d, acc);
    } else if constexpr (Q5) {
        int s0 = q5_codes_dot(w[1], w[2], w[3], w[4], w[5], x[0].c) - 16 * x[0].sum;
        acc = fmaf((float)s0, half_bits_to_float(w[0]) * x[0].d, acc);
    } else {
        int s0 = q8_codes_dot(w + 1, x[0].c);
        acc = fmaf((float)s0, half_bits_to_float(w[0]) * x[0].d, acc);
    }
    return acc;
}

template <int LPR>
__device__ __forceinline__ float row_reduce(float v) {
    if constexpr (LPR == 64) {
        v = group_sum<32>(v);
        return readlane_f(v, 0) + readlane_f(v, 32);
    } else {
        return group_sum<LPR>(v);
    }
}


// RMSNorm of one token row and its Q8_0 quantization by a 256-thread
// workgroup, latency-lean: thread t holds float4 chunks t, t+256, t+512,
// t+768 of x and gamma, loaded in one batch (rows up to 4096 wide stay in
// registers; wider rows are re-read in a second pass), one block reduction
// of sum(x^2), then every aligned group of 8 lanes quantizes one 32-element
// block (quantize_q8_0_x4_codes). For each chunk c the sink receives
// (c, normalized float4, packed codes of the chunk, scale bits, code sum of
// the chunk's block, valid on the block's first lane). red: 8 floats of LDS.
// The first KEEP float4 chunks of x and gamma per thread, loaded by
// norm_load so that a caller can issue them before other loads.
struct NormIn {
    static constexpr int KEEP = 4;
    float4 xv[KEEP], gv[KEEP];
};

__device__ __forceinline__ void norm_load(const float *x, const float *gamma, int D, NormIn &in) {
    constexpr int NT = kGemvThreads;
    const int tid = threadIdx.x, n4 = D / 4;
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const float4 *g4 = reinterpret_cast<const float4 *>(gamma);
    // unconditional loads (chunks past the row re-read its last chunk, and
    // norm_quant_finish ignores them): a conditional load would make the
    // compiler wait for it, and for every load issued before it, early
#pragma unroll
    for (int i = 0; i < NormIn::KEEP; i++) {
        const int c = min(tid + i * NT, n4 - 1);
        in.xv[i] = x4[c];
        in.gv[i] = g4[c];
    }
}

// TAIL = false: the row has at most KEEP * 256 float4 chunks (D <= 4096),
// so the second-pass loops over wider rows are compiled out.
template <bool TAIL = true, class Sink>
__device__ __forceinline__ void norm_quant_finish(const NormIn &in, const float *x,
                                                  const float *gamma, int D, float eps, float *red,
                                                  Sink sink) {
    constexpr int NT = kGemvThreads, KEEP = NormIn::KEEP;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n4 = D / 4;
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const float4 *g4 = reinterpret_cast<const float4 *>(gamma);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < KEEP; i++) {
        const float t = (in.xv[i].x * in.xv[i].x + in.xv[i].y * in.xv[i].y) +
                        (in.xv[i].z * in.xv[i].z + in.xv[i].w * in.xv[i].w);
        ss += tid + i * NT < n4 ? t : 0.0f;
    }
    if constexpr (TAIL) {
        for (int c = tid + KEEP * NT; c < n4; c += NT) {
            const float4 t = x4[c];
            ss += (t.x * t.x + t.y * t.y) + (t.z * t.z + t.w * t.w);
        }
    }
    ss = group_sum<32>(ss);
    if (lane == 0) red[2 * wave] = ss;
    if (lane == 32) red[2 * wave + 1] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < 2 * (NT / kWave); i++) tot += red[i];
    const float r = 1.0f / sqrtf(tot / (float)D + eps);
    auto emit = [&](int c, float4 xx, float4 gg) {
        const float4 v = make_float4(xx.x * r * gg.x, xx.y * r * gg.y, xx.z * r * gg.z,
                                     xx.w * r * gg.w);
        uint32_t packed;
        uint16_t dbits;
        quantize_q8_0_x4_codes(v, packed, dbits);
        float cs = (float)(int8_t)(packed & 0xFF) + (float)(int8_t)((packed >> 8) & 0xFF) +
                   (float)(int8_t)((packed >> 16) & 0xFF) + (float)(int8_t)(packed >> 24);
        cs = group_sum<8>(cs);
        sink(c, v, packed, dbits, (int)cs);
    };
#pragma unroll
    for (int i = 0; i < KEEP; i++) {
        const int c = tid + i * NT;
        if (c < n4) emit(c, in.xv[i], in.gv[i]);
    }
    if constexpr (TAIL)
        for (int c = tid + KEEP * NT; c < n4; c += NT) emit(c, x4[c], g4[c]);
    __syncthreads();   // red is free again
}

template <class Sink>
__device__ __forceinline__ void norm_quant_row(const float *x, const float *gamma, int D,
                                               float eps, float *red, Sink sink) {
    NormIn in;
    norm_load(x, gamma, D, in);
    norm_quant_finish(in, x, gamma, D, eps, red, sink);
}

}  // namespace ck
