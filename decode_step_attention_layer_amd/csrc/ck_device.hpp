// ck_device.hpp — device helpers shared by the gfx950 kernels of libck.so:
// wave64 cross-lane reductions (DPP within 16-lane rows, ds_swizzle across
// rows of a 32-lane half, readlane across halves), the bit-exact Q8_0
// quantizer of one 32-element block held by 32 lanes, and Q5_0/Q8_0 block
// decoding into int8 lanes for v_dot4_i32_i8.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace ck {

constexpr int kWave = 64;
constexpr int kQK = 32;
constexpr int kQ8Bytes = 34;
constexpr int kQ5Bytes = 22;

// ---------------------------------------------------------------- DPP -----
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
// DPP controls (GFX9): quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;
constexpr int kHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float swz_xor16_f(float v) {
    // ds_swizzle bit-mask mode inside 32-lane groups: and 0x1f, or 0, xor 0x10
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ int swz_xor16_i(int v) {
    return __builtin_amdgcn_ds_swizzle(v, 0x401F);
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8, 16, 32); every lane of a
// group receives the group's sum. The butterfly pairs lanes symmetrically, so
// all lanes of a group hold bit-identical values.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp_f<kQuadXor1>(v);
    if constexpr (N >= 4) v += dpp_f<kQuadXor2>(v);
    if constexpr (N >= 8) v += dpp_f<kHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_f<kRowMirror>(v);
    if constexpr (N >= 32) v += swz_xor16_f(v);
    return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp_f<kQuadXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_f<kQuadXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_f<kHalfMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_f<kRowMirror>(v));
    if constexpr (N >= 32) v = fmaxf(v, swz_xor16_f(v));
    return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Whole-wave sum / max, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<32>(v);
    return readlane_f(v, 0) + readlane_f(v, 32);
}
__device__ __forceinline__ float wave_max(float v) {
    v = group_max<32>(v);
    return fmaxf(readlane_f(v, 0), readlane_f(v, 32));
}

// ------------------------------------------------------ Q8_0 quantizer -----
// One block per 32 lanes: lane j of the half-wave holds x_j. Every lane gets
// its code and the half-wave's binary16 scale bits. In fp32 operations:
// amax = max |x|, d = amax / 127, id = (d != 0 ? 1 / d : 0), code =
// round-half-away-from-zero(x * id); the stored scale is binary16(d), ties to
// even. Division is IEEE-correct (built with correctly rounded divide), and
// contraction is off here so x * id is one rounded product.
__device__ __forceinline__ void quantize_q8_0_half(float x, int &code, uint16_t &dbits) {
#pragma clang fp contract(off)
    float amax = group_max<32>(fabsf(x));
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    float v = x * id;
    float t = truncf(v);
    if (fabsf(v - t) >= 0.5f) t += copysignf(1.0f, v);
    code = (int)t;
    dbits = __half_as_ushort(__float2half_rn(d));
}

// Q8_0 of one 32-element block held as 4 consecutive values by each of 8
// lanes (an aligned 8-lane group); the same arithmetic as quantize_q8_0_half.
// Returns this lane's 4 codes packed in a dword and the block's scale bits.
__device__ __forceinline__ void quantize_q8_0_x4_codes(float4 v, uint32_t &packed,
                                                       uint16_t &dbits) {
#pragma clang fp contract(off)
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = group_max<8>(a);
    const float d = a / 127.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    const float xs[4] = {v.x, v.y, v.z, v.w};
    packed = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float s = xs[i] * id;
        float t = truncf(s);
        if (fabsf(s - t) >= 0.5f) t += copysignf(1.0f, s);
        packed |= ((uint32_t)(uint8_t)(int8_t)(int)t) << (8 * i);
    }
    dbits = __half_as_ushort(__float2half_rn(d));
}

// The same, stored into the Q8_0 block `blk` (lane `sub` of the 8 writes
// codes 4*sub..4*sub+3; lane 0 also writes the scale).
__device__ __forceinline__ void quantize_q8_0_x4(float4 v, uint8_t *blk, int sub) {
    uint32_t packed;
    uint16_t dbits;
    quantize_q8_0_x4_codes(v, packed, dbits);
    uint16_t *dst = reinterpret_cast<uint16_t *>(blk + 2 + 4 * sub);
    dst[0] = (uint16_t)(packed & 0xFFFF);
    dst[1] = (uint16_t)(packed >> 16);
    if (sub == 0) *reinterpret_cast<uint16_t *>(blk) = dbits;
}

// -------------------------------------------------------- block fields -----
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xFFFFu)));
}

// Bits 0..3 of t become bit 0 of bytes 0..3 (t < 16; a 24-bit multiply lays
// the four bits 7 positions apart, the mask keeps one per byte).
__device__ __forceinline__ uint32_t spread4(uint32_t t) {
    return __umul24(t, 0x00204081u) & 0x01010101u;
}

// Sum over the 32 elements of a Q5_0 block of code_j * x_j (codes 0..31,
// unsigned), given qh, the 16 qs bytes as 4 dwords and the activation codes as
// 8 dwords of int8 (dword i of xa = elements 4i..4i+3). The caller subtracts
// 16 * sum(x) to get sum (code_j - 16) * x_j.
__device__ __forceinline__ int q5_codes_dot(uint32_t qh, uint32_t qs0, uint32_t qs1,
                                            uint32_t qs2, uint32_t qs3, const int *xa) {
    const uint32_t qs[4] = {qs0, qs1, qs2, qs3};
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t lo = qs[i] & 0x0F0F0F0Fu;
        uint32_t hi = (qs[i] >> 4) & 0x0F0F0F0Fu;
        lo |= spread4(__builtin_amdgcn_ubfe(qh, 4 * i, 4)) << 4;
        hi |= spread4(__builtin_amdgcn_ubfe(qh, 16 + 4 * i, 4)) << 4;
        acc = __builtin_amdgcn_sdot4((int)lo, xa[i], acc, false);
        acc = __builtin_amdgcn_sdot4((int)hi, xa[4 + i], acc, false);
    }
    return acc;
}

__device__ __forceinline__ int q8_codes_dot(const uint32_t *w, const int *xa) {
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) acc = __builtin_amdgcn_sdot4((int)w[i], xa[i], acc, false);
    return acc;
}

// v_alignbyte: the 4 bytes starting `shift` bytes into the 8-byte (hi:lo).
__device__ __forceinline__ uint32_t align2(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// 16-byte and 12-byte vector types that only require 4-byte alignment, so a
// lane can read any dword-aligned run of a weight row with dwordx4/x3 loads.
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3a4 __attribute__((ext_vector_type(3), aligned(4)));

// ----------------------------------------------- cache element codecs -----
// bf16: the top half of binary32; stores round to nearest, ties to even.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; no
// infinities; S.1111.111 is NaN; largest finite 448; subnormals m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t sgn = (c & 0x80u) << 24, e = (c >> 3) & 0xFu, m = c & 7u;
    if (e == 0xFu && m == 7u) return __uint_as_float(sgn | 0x7FC00000u);
    if (e == 0u) return __uint_as_float(sgn | __float_as_uint((float)m * 0x1p-9f));
    return __uint_as_float(sgn | ((e + 120u) << 23) | (m << 20));
}

// Nearest code, ties to even, saturating at +-448; NaN -> 0x7F.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7F;
    const uint32_t sgn = (u >> 24) & 0x80u;
    const float a = __uint_as_float(u & 0x7FFFFFFFu);
    if (a >= 448.0f) return (uint8_t)(sgn | 0x7Eu);
    if (a < 0x1p-6f) {
        // subnormal codes m * 2^-9 (m = 8 is the smallest normal, code 0x08)
        return (uint8_t)(sgn | (uint32_t)rintf(a * 512.0f));
    }
    int E = (int)((u >> 23) & 0xFFu) - 127;                // a in [2^E, 2^(E+1)), E in [-6, 8]
    uint32_t mant = u & 0x7FFFFFu;
    mant += 0x7FFFFu + ((mant >> 20) & 1u);                // round the 23-bit mantissa to 3 bits
    if (mant & 0x800000u) {                                // carried into the next binade
        E += 1;
        mant = 0;
    }
    return (uint8_t)(sgn | ((uint32_t)(E + 7) << 3) | ((mant >> 20) & 7u));
}

// Device-coherent accesses between workgroups of one launch: relaxed
// agent-scope atomic loads and stores, which gfx950 issues as ordinary vector
// loads/stores with device-scope coherence (no L2 write-back or invalidate).
// A producer completes its stores (s_waitcnt) before it signals; a consumer
// reads the signal before it issues these loads.
__device__ __forceinline__ float ld_c(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_cu(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_c(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_cu(unsigned *p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// two floats (8-byte aligned) in one coherent 64-bit load
__device__ __forceinline__ float2 ld_c2(const float *p) {
    const unsigned long long u = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((unsigned)u), __uint_as_float((unsigned)(u >> 32)));
}
// four floats (8-byte aligned) in two coherent 64-bit loads
__device__ __forceinline__ float4 ld_c4(const float *p) {
    const float2 a = ld_c2(p), b = ld_c2(p + 2);
    return make_float4(a.x, a.y, b.x, b.y);
}

}  // namespace ck
