// k_gemv_mfma.hip — small-M block GEMV on the int8 matrix cores (gfx950).
//
// For a batch of m tokens sharing the weights (the batched decode layer, all
// of its projections), y[s][r] = sum_b d_w(r,b) d_x(s,b) S(r,s,b) + bias[r]
// (+ residual[s][r]) with S the exact integer dot of block b. The per-block
// scales forbid accumulating across blocks in int32, so every
// v_mfma_i32_16x16x32_i8 covers exactly one 32-element block: A = the
// activation codes of 16 token slots (m used), B = the weight codes of 16
// rows, D[token][row] = S. Lane l supplies token slot l%16 and row l%16 for
// the k-slice 8*(l/16)..+7 and receives D[4*(l/16)+t][l%16], t < 4, so every
// output a lane scales belongs to the weight row whose block scale it loaded.
// Q5_0 codes are unpacked straight to signed bytes (code - 16), so the
// integer dot is the block's S itself.
//
// Workgroup: 8 waves on one tile of 16 rows; wave w takes an eighth of the
// rows' block pairs, loads them with coalesced dword loads (all before any
// arithmetic, after the activation blocks) and redistributes them to the MFMA
// lane layout through its own LDS region, in phases of 4 Q5_0 (2 Q8_0) block
// pairs; the activations are staged in LDS once per workgroup (codes, scale,
// code sum; block-major, so one block's token slots sit on distinct banks)
// while the weights are in flight (codes block-major, the m tokens of a block
// consecutive; scales in a separate array padded to 16 token slots, so a
// lane's four token scales of a block are one 16-byte read), and the 8
// partial sums of each (token, row) are added through LDS in wave order
// (deterministic).
// The Q/K/V launch of the batched layer can end in RoPE and the KV append
// (C-Kernel-Engine MAIN KERNEL steps 5-6): its q and k tiles then take their
// rows in rotation order (tile rows 2p and 2p + 1 are elements i and
// i + hd/2 of one head), so a row's partner is the neighbouring lane, and
// each output thread rotates its value and stores it, and k and v into the
// cache; the positions, table entries and cache rows load before the
// weights.
#include "ck_device.hpp"
#include "ck_gemv_common.hpp"
#include "ck_internal.hpp"

namespace ck {

namespace {

constexpr int kMT = 512;             // threads
constexpr int kMW = kMT / kWave;     // waves
constexpr int kTileRows = 16;
constexpr int kMaxUnitsPerWave = 8;  // block pairs per wave: K <= 8 * 8 * 64 = 4096

typedef int v4i __attribute__((ext_vector_type(4)));

// The dwords of one block pair a lane needs for its k-slice ks (Q5_0: 9,
// Q8_0: 7), read from the wave's LDS copy of the pair.
template <bool Q5>
struct SliceWords {
    static constexpr int n = Q5 ? 9 : 7;
};

template <bool Q5>
__device__ __forceinline__ void load_slice(const uint32_t *u, int ks, uint32_t *w) {
    if constexpr (Q5) {
        const int k2 = 2 * (ks & 1);
        w[0] = u[0];            // d0 | qh0 bytes 0-1
        w[1] = u[1];            // qh0 bytes 2-3 | qs0 bytes 0-1
        w[2] = u[1 + k2];       // qs0 slice, shifted by 2 bytes
        w[3] = u[2 + k2];
        w[4] = u[3 + k2];
        w[5] = u[5];            // ... | d1
        w[6] = u[6];            // qh1
        w[7] = u[7 + k2];       // qs1 slice
        w[8] = u[8 + k2];
    } else {
        const int k2 = 2 * ks;
        w[0] = u[0];            // d0 | codes 0-1
        w[1] = u[k2];           // block-0 codes of the slice, shifted by 2 bytes
        w[2] = u[k2 + 1];
        w[3] = u[k2 + 2];
        w[4] = u[8];            // ... | d1
        w[5] = u[9 + k2];       // block-1 codes of the slice
        w[6] = u[10 + k2];
    }
}

// The 8 codes of block bb (0, 1) in the lane's k-slice as a 64-bit operand,
// and the block's weight scale.
template <bool Q5>
__device__ __forceinline__ long slice_codes(const uint32_t *w, int bb, int ks, float &dw) {
    uint32_t c0, c1;
    if constexpr (Q5) {
        uint32_t qh, q0, q1;
        if (bb == 0) {
            dw = half_bits_to_float(w[0]);
            qh = align2(w[1], w[0]);
            q0 = align2(w[3], w[2]);
            q1 = align2(w[4], w[3]);
        } else {
            dw = half_bits_to_float(w[5] >> 16);
            qh = w[6];
            q0 = w[7];
            q1 = w[8];
        }
        // code - 16 as a signed byte: the low nibble, with 0xF0 above it
        // where the fifth bit is clear
        const int sh = ks < 2 ? 0 : 4;
        c0 = (q0 >> sh) & 0x0F0F0F0Fu;
        c1 = (q1 >> sh) & 0x0F0F0F0Fu;
        c0 |= spread4(__builtin_amdgcn_ubfe(~qh, 8 * ks, 4)) * 0xF0u;
        c1 |= spread4(__builtin_amdgcn_ubfe(~qh, 8 * ks + 4, 4)) * 0xF0u;
    } else {
        if (bb == 0) {
            dw = half_bits_to_float(w[0]);
            c0 = align2(w[2], w[1]);
            c1 = align2(w[3], w[2]);
        } else {
            dw = half_bits_to_float(w[4] >> 16);
            c0 = w[5];
            c1 = w[6];
        }
    }
    return (long)((unsigned long)c0 | ((unsigned long)c1 << 32));
}

// Weight staging: a wave loads its 16 rows' block pairs with coalesced dword
// loads (consecutive lanes, consecutive dwords of a row segment), all phases
// before any arithmetic, then per phase writes them to its own LDS region
// and every lane reads back the dwords of its (row, k-slice).
template <bool Q5>
struct Stage {
    static constexpr int words = Q5 ? 11 : 17;        // dwords per block pair
    static constexpr int pu = Q5 ? 4 : 2;             // block pairs per phase
    static constexpr int nph = kMaxUnitsPerWave / pu; // phases (at most)
    static constexpr int stride = pu * words + 1;     // LDS row stride (dwords)
    static constexpr int per_lane = (kTileRows * pu * words + kWave - 1) / kWave;
    static constexpr int region = kTileRows * stride; // dwords per wave
};

constexpr int kStageRegion = Stage<true>::region > Stage<false>::region ? Stage<true>::region
                                                                        : Stage<false>::region;

constexpr int kSlots = 16;   // token slots of an MFMA tile

// Physical row of tile row r of a rotated segment: consecutive rows (2p,
// 2p+1) are elements i and i + hd/2 of the same head.
__device__ __forceinline__ int rope_row(int r, int hd) {
    const int half = hd >> 1, p = r >> 1;
    return (p / half) * hd + (p % half) + (r & 1) * half;
}

constexpr int kImgPer = 5;   // 16-byte image pieces a thread loads (ximage_fits)

template <bool Q5, bool EPI, bool IMG>
__device__ void mfma_body(const GemvSeg &sg, int si, int tile, const uint8_t *xq,
                          const uint32_t *ximg, int nb, int m, uint32_t *xc, float *xd,
                          uint32_t *wst, float *red, const QkvEpi &e) {
    using St = Stage<Q5>;
    constexpr int NSW = SliceWords<Q5>::n;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, ks = lane >> 4;
    const int nunits = nb / 2;
    const int upw = (nunits + kMW - 1) / kMW;
    const int u0 = wave * upw;
    const int uend = min(u0 + upw, nunits);                // this wave's block pairs [u0, uend)
    const size_t row_bytes = (size_t)nb * (Q5 ? kQ5Bytes : kQ8Bytes);
    const int row0 = tile * kTileRows;

    // The loads go out in the order their values are needed, the weights
    // unconditionally (the memory counter retires loads in issue order, and a
    // load under a branch makes the compiler wait early for it and for every
    // load issued before it): the activation blocks of this thread (up to
    // two, when the batch has at most 2 * kMT blocks), the output thread's
    // bias and residual, then every phase's weight dwords.
    // An activation image goes straight into LDS, no registers: wave w's
    // i-th load fills pieces [i*512 + 64w, +64) of the LDS image from 64
    // consecutive 16-byte global pieces; lanes past the image re-read its
    // last piece and land in the slack after it (mfma_lds).
    const int nxb = m * nb;
    const bool xpre = nxb <= 2 * kMT;
    const int n16 = nb * (2 * m + 4);
    uint32_t xr[IMG ? 1 : 2][9];
    if constexpr (IMG) {
        const uint8_t *src = reinterpret_cast<const uint8_t *>(ximg);
#pragma unroll
        for (int i = 0; i < kImgPer; i++) {
            const int p0 = i * kMT + wave * kWave;
            __builtin_amdgcn_global_load_lds(src + (size_t)min(p0 + lane, n16 - 1) * 16,
                                             xc + (size_t)p0 * 4, 16, 0, 0);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int b = min(tid + q * kMT, nxb - 1);
            const uint16_t *src = reinterpret_cast<const uint16_t *>(xq + (size_t)b * kQ8Bytes);
            xr[q][0] = src[0];
#pragma unroll
            for (int i = 0; i < 8; i++)
                xr[q][1 + i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
        }
    }
    // with the epilogue the Q5_0 segments are q and k (rows in rotation
    // order) and the Q8_0 one is v (the launcher checks)
    constexpr bool rot = EPI && Q5;
    auto phys = [&](int r) { return rot ? rope_row(r, e.hd) : r; };
    const int otok = tid / kTileRows, orow = row0 + tid % kTileRows;
    const bool writer = tid < m * kTileRows && orow < sg.rows;
    const int prow = phys(min(orow, sg.rows - 1));
    const float bias_o = (writer && sg.bias) ? sg.bias[prow] : 0.0f;
    const float res_o = (!EPI && writer && sg.residual)
                            ? sg.residual[(size_t)otok * sg.rows + orow] : 0.0f;
    // the epilogue's position, RoPE factors and cache row (an invalid
    // position reads table row 0 and rotates and appends nothing)
    int pv = -1;
    float cs = 1.0f, sn = 0.0f;
    long long coff = -1;
    if constexpr (EPI) {
        const int tk = min(otok, m - 1);
        pv = e.pos.get(tk);
        if constexpr (rot) {
            const int half = e.hd >> 1, pp = max(pv, 0);
            const int i = (min(orow, sg.rows - 1) >> 1) % half;
            cs = e.cos_tab[(size_t)pp * half + i];
            sn = e.sin_tab[(size_t)pp * half + i];
        }
        if (si >= 1 && pv >= 0 && writer) coff = cache_row(e.c, tk, prow / e.hd, pv);
    }

    // every phase's weight dwords, coalesced: flat index f over [16 rows]
    // [St::pu block pairs][words] of the phase; rows past the matrix re-read
    // its last row and dwords past the row its last dword (neither reaches
    // LDS or an output)
    constexpr int kPh = St::pu * St::words;
    const size_t pair_bytes = 2 * (Q5 ? kQ5Bytes : kQ8Bytes);
    uint32_t raw[St::nph][St::per_lane];
#pragma unroll
    for (int p = 0; p < St::nph; p++) {
        const int pb = u0 + p * St::pu;
#pragma unroll
        for (int i = 0; i < St::per_lane; i++) {
            const int f = min(lane + kWave * i, kTileRows * kPh - 1);
            const int r = f / kPh, d = f - r * kPh;
            const int row = phys(min(row0 + r, sg.rows - 1));
            const size_t off = min((size_t)pb * pair_bytes + 4 * (size_t)d, row_bytes - 4);
            raw[p][i] = *reinterpret_cast<const uint32_t *>(sg.W + (size_t)row * row_bytes + off);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. the activations of all m tokens into LDS: codes block-major (the m
    // tokens of a block are consecutive 32-byte rows, so the lanes reading
    // one block's token slots spread over the banks), scales [block][16
    // slots] with the slots past the batch zero (their MFMA rows are zero
    // codes; a zero scale keeps stale LDS bits out of the sums)
    auto put_x = [&](int bf, const uint32_t *w) {
        const int b = bf % nb, tok = bf / nb;     // bf: flat index of the xq block
        xd[b * kSlots + tok] = half_bits_to_float(w[0]);
        uint4 *dst = reinterpret_cast<uint4 *>(xc + (b * m + tok) * 8);
        dst[0] = make_uint4(w[1], w[2], w[3], w[4]);
        dst[1] = make_uint4(w[5], w[6], w[7], w[8]);
    };
    if constexpr (IMG) {
        // the image is this LDS layout (codes, then the scales with their
        // zero slots): every load of this thread has landed, its image
        // pieces among them, and the barrier below publishes them
        __builtin_amdgcn_s_waitcnt(0);
    } else {
    for (int i = tid; i < nb * kSlots; i += kMT)
        if ((i & (kSlots - 1)) >= m) xd[i] = 0.0f;
    if (xpre) {
#pragma unroll
        for (int q = 0; q < 2; q++)
            if (tid + q * kMT < nxb) put_x(tid + q * kMT, xr[q]);
    } else {
        for (int b = tid; b < nxb; b += kMT) {
            const uint16_t *src = reinterpret_cast<const uint16_t *>(xq + (size_t)b * kQ8Bytes);
            uint32_t w[9];
            w[0] = src[0];
#pragma unroll
            for (int i = 0; i < 8; i++)
                w[1 + i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
            put_x(b, w);
        }
    }
    }
    __syncthreads();

    // 3. per phase: weights into this wave's LDS region, then one MFMA per
    // block: A = token slot j's codes, B = row j's codes
    uint32_t *reg = wst + wave * kStageRegion;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool a_valid = j < m;
    const int jr = min(j, m - 1);
#pragma unroll
    for (int p = 0; p < St::nph; p++) {
        const int pb = u0 + p * St::pu;
        const int np = max(0, min(St::pu, uend - pb));
        if (np == 0) break;
#pragma unroll
        for (int i = 0; i < St::per_lane; i++) {
            const int f = lane + kWave * i;
            const int r = f / kPh, d = f - r * kPh;
            if (f < kTileRows * kPh && d < np * St::words) reg[r * St::stride + d] = raw[p][i];
        }
        __builtin_amdgcn_wave_barrier();
        // every block's MFMA of the phase first (independent, so they
        // pipeline), then the scaling: a block at a time, each MFMA result
        // was consumed at once and the chain LDS read -> MFMA -> LDS read ->
        // FMA ran serially
        v4i dd[St::pu][2];
        float dws[St::pu][2];
#pragma unroll
        for (int k = 0; k < St::pu; k++) {
            if (k < np) {
                uint32_t w[NSW];
                load_slice<Q5>(reg + j * St::stride + k * St::words, ks, w);
#pragma unroll
                for (int bb = 0; bb < 2; bb++) {
                    const int b = 2 * (pb + k) + bb;
                    const long bop = slice_codes<Q5>(w, bb, ks, dws[k][bb]);
                    const uint2 c = *reinterpret_cast<const uint2 *>(&xc[(b * m + jr) * 8 + 2 * ks]);
                    const long aop = a_valid ? (long)((unsigned long)c.x |
                                                      ((unsigned long)c.y << 32))
                                             : 0;
                    v4i z = {0, 0, 0, 0};
                    dd[k][bb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, z, 0, 0, 0);
                }
            }
        }
        // the lane's token slots 4ks..4ks+3: their scales in one read (zero
        // past the batch)
#pragma unroll
        for (int k = 0; k < St::pu; k++) {
            if (k < np) {
#pragma unroll
                for (int bb = 0; bb < 2; bb++) {
                    const int b = 2 * (pb + k) + bb;
                    const float4 dx = *reinterpret_cast<const float4 *>(&xd[b * kSlots + 4 * ks]);
                    acc[0] = fmaf((float)dd[k][bb][0], dws[k][bb] * dx.x, acc[0]);
                    acc[1] = fmaf((float)dd[k][bb][1], dws[k][bb] * dx.y, acc[1]);
                    acc[2] = fmaf((float)dd[k][bb][2], dws[k][bb] * dx.z, acc[2]);
                    acc[3] = fmaf((float)dd[k][bb][3], dws[k][bb] * dx.w, acc[3]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();   // the region is rewritten by the next phase
    }

    // 4. the waves' partial sums, added in wave order; thread (token, row)
    // writes the output
    __syncthreads();   // the staged activations are no longer read; red aliases them
#pragma unroll
    for (int t = 0; t < 4; t++) red[(wave * kWave + lane) * 4 + t] = acc[t];
    __syncthreads();
    float o = 0.0f;
    if (writer) {
        const int src_lane = tid % kTileRows + 16 * (otok / 4), t = otok % 4;
        float v = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kMW; wv++) v += red[(wv * kWave + src_lane) * 4 + t];
        o = v + bias_o;
        if (!EPI && sg.residual) o = o + res_o;
    }
    if constexpr (EPI) {
        // the partner row (element i + hd/2 for an even tile row, i for an
        // odd one) is the neighbouring lane's
        const float other = __shfl_xor(o, 1);
        if (writer) {
            float out = o;
            if (rot && pv >= 0) out = (orow & 1) ? other * sn + o * cs : o * cs - other * sn;
            sg.y[(size_t)otok * sg.rows + prow] = out;
            if (coff >= 0) cache_put(e.c, si == 1, coff + prow % e.hd, out);
        }
    } else if (writer) {
        sg.y[(size_t)otok * sg.rows + orow] = o;
    }
}

// four waves per SIMD, two workgroups per compute unit (at most 128
// registers): a Q/K/V launch
// has more tiles than compute units
template <bool EPI, bool IMG>
__global__ __launch_bounds__(kMT, 4) void k_gemv_mfma(GemvArgs a, QkvEpi e) {
    extern __shared__ __align__(16) uint32_t lds[];   // staged weights, then activations
    const int wg = blockIdx.x;
    const int si = (a.nseg > 2 && wg >= a.seg[2].wg_begin) ? 2
                   : (a.nseg > 1 && wg >= a.seg[1].wg_begin) ? 1 : 0;
    const GemvSeg sg = si == 0 ? a.seg[0] : (si == 1 ? a.seg[1] : a.seg[2]);
    const int nb = a.K / kQK;
    // LDS: the staged weights of the 8 waves, then the activation codes and
    // scales (the final reduction reuses their space)
    uint32_t *wst = lds;
    uint32_t *xc = wst + kMW * kStageRegion;
    float *xd = reinterpret_cast<float *>(xc + (size_t)a.m * nb * 8);
    float *red = reinterpret_cast<float *>(xc);
    if (sg.is_q5)
        mfma_body<true, EPI, IMG>(sg, si, wg - sg.wg_begin, a.xq, a.ximg, nb, a.m, xc, xd, wst,
                                  red, e);
    else
        mfma_body<false, EPI, IMG>(sg, si, wg - sg.wg_begin, a.xq, a.ximg, nb, a.m, xc, xd, wst,
                                   red, e);
}

// img: room for every piece the image loads write (kImgPer per thread)
size_t mfma_lds(int m, int nb, bool img = false) {
    size_t xs = sizeof(uint32_t) * 8 * (size_t)m * nb + sizeof(float) * kSlots * (size_t)nb;
    const size_t red = sizeof(float) * kMT * 4;
    if (img && xs < (size_t)16 * kImgPer * kMT) xs = (size_t)16 * kImgPer * kMT;
    return sizeof(uint32_t) * kMW * kStageRegion + (xs > red ? xs : red);
}

}  // namespace

// Batches of 4..16 tokens, K a multiple of 64 up to 4096, the workgroup's LDS
// (staged weights, activation bytes and scales) within 80 KB, two workgroups
// per compute unit.
bool gemv_mfma_supported(int K, int m) {
    const int nb = K / kQK;
    return m >= 4 && m <= 16 && K % 64 == 0 && nb / 2 <= kMW * kMaxUnitsPerWave &&
           mfma_lds(m, nb) <= 80 * 1024;
}

namespace {

int plan_tiles(GemvArgs &a) {
    int total = 0;
    for (int i = 0; i < a.nseg; i++) {
        a.seg[i].wg_begin = total;
        total += (a.seg[i].rows + kTileRows - 1) / kTileRows;
    }
    for (int i = a.nseg; i < 3; i++) a.seg[i] = a.seg[0], a.seg[i].wg_begin = 1 << 30;
    return total;
}

}  // namespace

hipError_t launch_gemv_mfma(GemvArgs a, hipStream_t st) {
    const int total = plan_tiles(a);
    const QkvEpi none{};
    const int nb = a.K / kQK;
    if (a.ximg && ximage_fits(a.m, nb))
        hipLaunchKernelGGL((k_gemv_mfma<false, true>), dim3(total), dim3(kMT),
                           mfma_lds(a.m, nb, true), st, a, none);
    else
        hipLaunchKernelGGL((k_gemv_mfma<false, false>), dim3(total), dim3(kMT), mfma_lds(a.m, nb),
                           st, a, none);
    return hipGetLastError();
}

// Segments q and k (Q5_0) and v (Q8_0), no residual, row counts multiples of
// the head size (the caller checks the sizes; the weight formats are checked
// here).
hipError_t launch_gemv_mfma_qkv(GemvArgs a, const QkvEpi &e, hipStream_t st) {
    if (a.nseg != 3 || !a.seg[0].is_q5 || !a.seg[1].is_q5 || a.seg[2].is_q5 || a.seg[0].residual ||
        a.seg[1].residual || a.seg[2].residual || !a.ximg || !ximage_fits(a.m, a.K / kQK))
        return hipErrorInvalidValue;
    const int total = plan_tiles(a);
    hipLaunchKernelGGL((k_gemv_mfma<true, true>), dim3(total), dim3(kMT),
                       mfma_lds(a.m, a.K / kQK, true), st, a, e);
    return hipGetLastError();
}

}  // namespace ck
