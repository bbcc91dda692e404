// Decode step specialised for 128 x 128 heads: the serving shapes, with a
// compile-time 4/8-bit row split (n8 a multiple of 16) or, in one more
// instance, the split read at run time (any n8).  Same arithmetic contract as
// decode.hip (STEPQuant paper, Sec. 2.1 Eq. (1) with D_t = a I or, in the KDA
// form, D_t = diag(d) over the key rows; Sec. 2.2 quantizer; Sec. 4.3
// representation; App. C.3 Table C2 step order), arranged to keep the vector
// ALU count per state entry low:
//
//  * a row gate d_i enters only through the row's factor: the gated state row
//    is d_i r_i z_i, so every per-row coefficient below uses d_i r_i in place
//    of r_i and the scalar gate is 1 (a scalar gate a keeps d_i = 1 and
//    applies a to the column sums, as before);
//
//  * one workgroup of 256 lanes per (slot, head); lane (g, c), g = lane / 16,
//    c = lane % 16, owns columns 8c..8c+7 of physical rows g + 16 m, m = 0..7;
//    with n8 a multiple of 16, row m of every lane is 8-bit iff m < n8 / 16,
//    so the row width is a compile-time property of m and no lane diverges
//    (the runtime-split instance branches per slot on a wave-uniform test);
//  * the packed state is streamed with non-temporal loads and stores; the
//    per-unit vectors (perm, r, k, q, v, c, gate) are loaded before the codes
//    (loads complete in issue order) at addresses that depend on no other
//    load: k and q are read in logical order, two entries per lane, and
//    brought into physical row order by lane permutes instead of a gather
//    through perm;
//  * per-row factors are formed once per row by the staging lanes and read
//    from LDS: r k and r q (with 1/16 folded in for 4-bit rows, whose codes are
//    widened as 16 z), and the update in the form
//        x_ij = X_ij / c_j = s_i (P_i z_ij + E_ij)
//    with s_i = b k_i, P_i = a r_i / (b k_i), E_ij = e_j for a row whose b k_i
//    is not negligible next to a r_i, and s_i = 1, P_i = a r_i, E_ij = 0 for a
//    row where |b k_i| <= 2^-64 |a r_i| (then b k_i e_j is below fp32
//    resolution against any non-zero code).  Either way one FMA per entry;
//    the lane picks e or a zero vector per row by its LDS address;
//  * the row absmax over the 16 lanes of a row is a DPP reduce-scatter that
//    leaves row c / 2 in lane c, so each lane derives one row factor and its
//    reciprocal, and the 8 multipliers are exchanged through LDS inside the
//    wave (a wave-level fence, no workgroup barrier);
//  * codes: one FMA adds 1.5 * 2^23 (round-half-even to an integer in the low
//    mantissa bits), then bytes are gathered with v_perm and nibbles with one
//    shift and one bit-field insert per 8 codes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "stq_internal.h"

namespace stq {
namespace {

constexpr int D = 128;
constexpr float kRoundMagic = 12582912.0f;               // 1.5 * 2^23
constexpr float kRowFloor = 1.17549435082228750797e-38f; // 2^-126
constexpr float kMulMax = 1.70141183460469231732e38f;    // 2^127
constexpr float kFormTiny = 5.42101086242752217004e-20f; // 2^-64

template <typename T> struct In;
template <> struct In<float> {
    static __device__ __forceinline__ float get(const void *p, unsigned i) {
        return static_cast<const float *>(p)[i];
    }
    static __device__ __forceinline__ uint32_t raw(const void *p, unsigned i) {
        return static_cast<const uint32_t *>(p)[i];
    }
    static __device__ __forceinline__ float cvt(uint32_t bits) { return __uint_as_float(bits); }
};
template <> struct In<uint16_t> {
    static __device__ __forceinline__ float get(const void *p, unsigned i) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
    }
    // the element's bits, widened later (a load whose result is only moved
    // does not wait for it)
    static __device__ __forceinline__ uint32_t raw(const void *p, unsigned i) {
        return static_cast<const uint16_t *>(p)[i];
    }
    static __device__ __forceinline__ float cvt(uint32_t bits) { return __uint_as_float(bits << 16); }
};

__device__ __forceinline__ float sbyte(uint32_t w, int k) {
    return static_cast<float>(static_cast<int8_t>(w >> (8 * k)));
}

// DPP lane exchange inside 16-lane rows (controls from the GFX9 DPP encoding).
template <int CTRL> __device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
constexpr int kRowRor8 = 0x128;       // lane l <- lane l^8 within the row
constexpr int kRowHalfMirror = 0x141; // lane l <- lane 7-l within each half row
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kRowMirror = 0x140;     // lane l <- lane 15-l within the row

template <int CTRL> __device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes of a wave (valid in every lane): DPP within 16-lane
// rows, then the four row sums through v_readlane.
__device__ __forceinline__ float wave_sum(float v) {
    v += dppf<kQuadXor1>(v);
    v += dppf<kQuadXor2>(v);
    v += dppf<kRowHalfMirror>(v);
    v += dppf<kRowMirror>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// MFMA operand A for the column sums: per wave w and lane group gl, seven
// 8-entry bf16 rows: r k (hi, mid, lo), r q (hi, mid, lo) of the lane group's
// 8 state rows, then a zero row for the unused outputs.
struct Smem {
    uint16_t coef[4][4][7][8];
    float4 row[D];          // {P, s, w2, offset of E in ez} per physical row
    float v[D], c[D];
    float ez[2 * D];        // e, then a zero vector; each as [e/4][c][e%4]
    float4 red[4][8][2][16]; // per wave, column offset e, lane group, chunk c
    float kq[2];
    float mul[16][8];       // per row group: code multipliers of its 8 rows
    float ra[16][8], rb[16][8]; // column refit: w2 r' s and w2 r'^2 per row
};

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

// x = hi + mid + lo exactly (each step removes the leading 8 significant bits
// and the remainders are exact fp32 differences).
__device__ __forceinline__ void split3(float x, uint32_t &h0, uint32_t &h1, uint32_t &h2) {
    h0 = bf16_bits(x);
    const float r1 = x - bf16_val(h0);
    h1 = bf16_bits(r1);
    const float r2 = r1 - bf16_val(h1);
    h2 = bf16_bits(r2);
}

// n / d for a wave-uniform n < 2^31, with m = ceil(2^32 / d) (d >= 2) or
// m = 0 (d = 1): hi(n m) is the quotient or one more (scalar unit only).
__device__ __forceinline__ unsigned udiv(unsigned n, unsigned d, unsigned m) {
    if (m == 0) return n;
    unsigned q = __umulhi(n, m);
    if (q * d > n) --q;
    return q;
}

// N8 = kRuntimeN8 selects the instance whose 4/8-bit split is read at run
// time (any n8): slot m of wave w holds rows 16 m + 4 w .. 16 m + 4 w + 3, so
// a slot is all 8-bit, all 4-bit, or (at most one per wave) straddles n8;
// the first two take a scalar branch, the last a per-lane one.
constexpr int kRuntimeN8 = -1;

struct Lane {
    int t, c, g;
    int n8, wv;        // the split (runtime instance) and the wave, wave-uniform
    unsigned unit;
    float alpha, beta;
    const int8_t *p8;  // packed rows read ...
    const uint8_t *p4;
    int8_t *q8;        // ... and written (the same unless decoding out of place)
    uint8_t *q4;
    const float *rr;   // row factors read ...
    float *rw;         // ... and written
    float *cw;         // refit column factors written (REFIT format)
};

// Fetch this lane's packed rows (Table C2 step 1).  The packed state is read
// once and written once per step and nothing reuses it within the step, so
// its loads and stores carry the non-temporal hint (measured 5 % faster than
// cached accesses at B = 1024).
// Class of slot m for this wave in the runtime instance: 1 all 8-bit, 0 all
// 4-bit, -1 straddling n8 (wave-uniform).
__device__ __forceinline__ int slot_class(const Lane &L, int m) {
    const int p0 = 16 * m + 4 * L.wv;
    return p0 + 3 < L.n8 ? 1 : (p0 >= L.n8 ? 0 : -1);
}

template <int N8>
__device__ __forceinline__ void load_codes(const Lane &L, uint32_t (&w0)[8], uint32_t (&w1)[8]) {
    if constexpr (N8 == kRuntimeN8) {
        // one 8-byte load per slot whatever its width (4-bit rows: the aligned
        // 8 bytes holding the lane's 4), so no register is written by
        // different loads on different paths; only the address depends on it
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int p = L.g + 16 * m;
            const int k = slot_class(L, m);
            const uint8_t *addr;
            if (k == 1) {
                addr = reinterpret_cast<const uint8_t *>(L.p8) + (16 * m * D) +
                       static_cast<unsigned>(L.g * D + 8 * L.c);
            } else if (k == 0) {
                addr = L.p4 + ((16 * m - L.n8) * (D / 2)) +
                       static_cast<unsigned>(L.g * (D / 2) + ((4 * L.c) & ~7));
            } else {
                addr = p < L.n8 ? reinterpret_cast<const uint8_t *>(L.p8) + (p * D + 8 * L.c)
                                : L.p4 + ((p - L.n8) * (D / 2) + ((4 * L.c) & ~7));
            }
            const u32x2 v2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(addr));
            w0[m] = v2[0];
            w1[m] = v2[1];
        }
    } else {
    constexpr int M8 = N8 / 16;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const unsigned p = static_cast<unsigned>(L.g + 16 * m);
        if (m < M8) {
            const u32x2 v2 =
                __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(L.p8 + (p * D + 8 * L.c)));
            w0[m] = v2[0];
            w1[m] = v2[1];
        } else {
            w0[m] = __builtin_nontemporal_load(
                reinterpret_cast<const uint32_t *>(L.p4 + ((p - N8) * (D / 2) + 4 * L.c)));
            w1[m] = 0u;
        }
    }
    }
}

// Everything after the barrier that follows the per-row factors.
template <int N8, bool REFIT>
__device__ __forceinline__ void finish_unit(const DecodeArgs &a, Smem &sh, const Lane &L,
                                            const uint32_t (&w0)[8], const uint32_t (&w1)[8]) {
    constexpr int M8 = N8 < 0 ? 0 : N8 / 16;
    const int t = L.t, c = L.c, g = L.g;

    // ---- widen the codes; column sums u~ = S~^T (r k), w~ = S~^T (r q) on the
    // matrix cores: per column offset e, one 16x16x32 bf16 MFMA multiplies the
    // 6 x 32 coefficient splits of the wave's 32 rows with the 32 x 16 codes of
    // column 8c + e (codes are small integers, exact in bf16; the splits are
    // exact, so only the fp32 accumulation rounds)
    const int w = t >> 6;
    const int gl = (t >> 4) & 3;
    float z[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        if constexpr (N8 == kRuntimeN8) {
            // the slot's class is wave-uniform (a scalar branch) except in
            // the one slot that straddles n8; there each lane selects, with
            // no branch, the two words whose bytes are its eight codes
            const int k = slot_class(L, m);
            const uint32_t w4 = (c & 1) ? w1[m] : w0[m]; // a 4-bit row's 4 bytes
            const uint32_t hi = w4 & 0xF0F0F0F0u;          // odd columns, x16
            const uint32_t lo = (w4 << 4) & 0xF0F0F0F0u;   // even columns, x16
            if (k == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[m][e] = sbyte(w0[m], e);
                    z[m][4 + e] = sbyte(w1[m], e);
                }
            } else if (k == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[m][2 * e] = sbyte(lo, e);
                    z[m][2 * e + 1] = sbyte(hi, e);
                }
            } else {
                // bytes in column order: lo0 hi0 lo1 hi1 | lo2 hi2 lo3 hi3
                const bool own8 = g + 16 * m < L.n8;
                const uint32_t x0 = own8 ? w0[m] : __builtin_amdgcn_perm(hi, lo, 0x05010400u);
                const uint32_t x1 = own8 ? w1[m] : __builtin_amdgcn_perm(hi, lo, 0x07030602u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[m][e] = sbyte(x0, e);
                    z[m][4 + e] = sbyte(x1, e);
                }
            }
            continue;
        }
        const bool is8 = m < M8;
        if (is8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[m][e] = sbyte(w0[m], e);
                z[m][4 + e] = sbyte(w1[m], e);
            }
        } else {
            const uint32_t hi = w0[m] & 0xF0F0F0F0u;         // odd columns, x16
            const uint32_t lo = (w0[m] << 4) & 0xF0F0F0F0u;  // even columns, x16
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[m][2 * e] = sbyte(lo, e);
                z[m][2 * e + 1] = sbyte(hi, e);
            }
        }
    }
    {
        const u32x4 araw = *reinterpret_cast<const u32x4 *>(&sh.coef[w][gl][c < 6 ? c : 6][0]);
        const bf16x8 A = __builtin_bit_cast(bf16x8, araw);
        // lanes of group 0 receive (u hi, u mid, u lo, w hi), group 1 (w mid, w lo);
        // two accumulators alternate so a result is stored while the next
        // product is in flight
        auto product = [&](int e) {
            u32x4 braw;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                braw[v] = __builtin_amdgcn_perm(__float_as_uint(z[2 * v + 1][e]),
                                                __float_as_uint(z[2 * v][e]), 0x07060302u);
            const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, braw), zero,
                                                           0, 0, 0);
        };
        float4 *red = &sh.red[w][0][gl][c]; // column offset e at red[32 e]
        auto store = [&](int e, const f32x4 &acc) {
            if (gl < 2) red[32 * e] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        };
        f32x4 acc0 = product(0);
        f32x4 acc1 = product(1);
#pragma unroll
        for (int e = 2; e < 8; e += 2) {
            store(e - 2, acc0);
            acc0 = product(e);
            store(e - 1, acc1);
            acc1 = product(e + 1);
        }
        store(6, acc0);
        store(7, acc1);
    }
    __syncthreads();

    // ---- column sums over the 4 waves: u~ (lanes 0..127) -> e; w~ (128..255)
    // kept for o.  Lane t handles column 8 (t % 16) + (t / 16) % 8.
    float wsum = 0.0f;
    const int cc = t & 15;
    const int ce = (t >> 4) & 7;
    const int jcol = 8 * cc + ce;
    const int ezi = (ce >> 2) * 64 + cc * 4 + (ce & 3);
    if (t < D) {
        float u = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float4 f = sh.red[ww][ce][0][cc];
            u += (f.x + f.y) + f.z;
        }
        sh.ez[ezi] = __builtin_fmaf(-L.alpha, u, sh.v[jcol] * __builtin_amdgcn_rcpf(sh.c[jcol]));
    } else {
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float4 f0 = sh.red[ww][ce][0][cc];
            const float4 f1 = sh.red[ww][ce][1][cc];
            wsum += (f0.w + f1.x) + f1.y;
        }
    }
    __syncthreads();

    // ---- Table C2 step 3: readout of the updated state, before requantizing
    if (t >= D) {
        const float kq = sh.kq[0] + sh.kq[1];
        store_o(a, static_cast<size_t>(L.unit) * D + jcol, sh.c[jcol] * __builtin_fmaf(L.alpha, wsum, (L.beta * kq) * sh.ez[ezi]));
    }

    // ---- Table C2 steps 2 and 4: updated entries and row absmax
    uint32_t amax[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 rp = sh.row[g + 16 * m];
        const float *E = &sh.ez[__float_as_int(rp.w) + 4 * c];
        const float4 e0 = *reinterpret_cast<const float4 *>(E);
        const float4 e1 = *reinterpret_cast<const float4 *>(E + 64);
        const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            z[m][e] = __builtin_fmaf(rp.x, z[m][e], ev[e]); // x / s
            mx = fmaxf(mx, fabsf(z[m][e]));
        }
        amax[m] = __float_as_uint(mx);
    }
    // reduce-scatter over the 16 lanes of the row group: lane c ends with row
    // c / 2 (non-negative floats order like their bit patterns: integer max)
    const bool hiHalf = (c & 8) != 0;
    const bool upper = (c & 4) != 0;
    const bool q2 = (c & 2) != 0;
    uint32_t r1[4], r2[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t keep = hiHalf ? amax[k + 4] : amax[k];
        const uint32_t send = hiHalf ? amax[k] : amax[k + 4];
        r1[k] = max(keep, dpp<kRowRor8>(send));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t keep = upper ? r1[k + 2] : r1[k];
        const uint32_t send = upper ? r1[k] : r1[k + 2];
        r2[k] = max(keep, dpp<kRowHalfMirror>(send));
    }
    float rmax;
    {
        const uint32_t keep = q2 ? r2[1] : r2[0];
        const uint32_t send = q2 ? r2[0] : r2[1];
        uint32_t v = max(keep, dpp<kQuadXor2>(send));
        v = max(v, dpp<kQuadXor1>(v));
        rmax = __uint_as_float(v);
    }
    {
        const int mm = c >> 1;
        const int p = g + 16 * mm;
        const float sc = sh.row[p].y;
        const float mrow = fabsf(sc) * rmax;
        const bool row8 = N8 == kRuntimeN8 ? p < L.n8 : mm < M8;
        const float qinv = row8 ? (1.0f / 127.0f) : (1.0f / 7.0f);
        const float rn = fmaxf(mrow * qinv, kRowFloor);
        const float inv = __builtin_amdgcn_rcpf(rn);
        float mul = sc * inv;
        mul = fminf(fmaxf(mul, -kMulMax), kMulMax);
        if ((c & 1) == 0) {
            L.rw[p] = rn;
            sh.mul[g][mm] = mul;
            if (REFIT) {
                const float w2 = sh.row[p].z;
                sh.ra[g][mm] = (w2 * rn) * sc;
                sh.rb[g][mm] = (w2 * rn) * rn;
            }
        }
    }
    // the multipliers of a row group are written and read by the 16 lanes of
    // that group, inside one wave: a wave-level fence suffices
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- Table C2 step 6: codes against the stored factors, pack, write back
    float mulv[8];
    {
        const float4 m0 = *reinterpret_cast<const float4 *>(&sh.mul[g][0]);
        const float4 m1 = *reinterpret_cast<const float4 *>(&sh.mul[g][4]);
        mulv[0] = m0.x; mulv[1] = m0.y; mulv[2] = m0.z; mulv[3] = m0.w;
        mulv[4] = m1.x; mulv[5] = m1.y; mulv[6] = m1.z; mulv[7] = m1.w;
    }
    // column refit partial sums over this lane's 8 rows (REFIT): with
    // x = s y, X = c x and v = r' z', sum_i w2 v X = c sum_i (w2 r' s) z' y
    // and sum_i w2 v^2 = sum_i (w2 r'^2) z'^2
    float num[8], den[8], rav[8], rbv[8];
    if (REFIT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            num[e] = 0.0f;
            den[e] = 0.0f;
            rav[e] = sh.ra[g][e];
            rbv[e] = sh.rb[g][e];
        }
    }
    if constexpr (N8 == kRuntimeN8) {
        const int n8 = L.n8;
    #pragma unroll
        for (int m = 0; m < 8; ++m) {
            const unsigned p = static_cast<unsigned>(g + 16 * m);
            // codes, refit sums and the packed store of slot m; the whole body sits
            // inside the width branch (in the runtime instance this keeps the
            // codes of one slot live at a time)
            auto emit = [&](auto W8) __attribute__((always_inline)) {
                constexpr bool IS8 = decltype(W8)::value;
                uint32_t bt[8];
    #pragma unroll
                for (int e = 0; e < 8; ++e)
                    bt[e] = __float_as_uint(__builtin_fmaf(z[m][e], mulv[m], kRoundMagic));
                if (REFIT) {
    #pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float zq = __uint_as_float(bt[e]) - kRoundMagic; // the code, exactly
                        num[e] = __builtin_fmaf(rav[m] * zq, z[m][e], num[e]);
                        den[e] = __builtin_fmaf(rbv[m] * zq, zq, den[e]);
                    }
                }
                if constexpr (IS8) {
                    const uint32_t a01 = __builtin_amdgcn_perm(bt[1], bt[0], 0x0C0C0400u);
                    const uint32_t a23 = __builtin_amdgcn_perm(bt[3], bt[2], 0x04000C0Cu);
                    const uint32_t a45 = __builtin_amdgcn_perm(bt[5], bt[4], 0x0C0C0400u);
                    const uint32_t a67 = __builtin_amdgcn_perm(bt[7], bt[6], 0x04000C0Cu);
                    __builtin_nontemporal_store(u32x2{a01 | a23, a45 | a67},
                                                reinterpret_cast<u32x2 *>(L.q8 + (p * D + 8 * c)));
                } else {
                    // even columns -> low nibbles, odd columns -> high nibbles
                    const uint32_t ev02 = __builtin_amdgcn_perm(bt[2], bt[0], 0x0C0C0400u);
                    const uint32_t ev46 = __builtin_amdgcn_perm(bt[6], bt[4], 0x04000C0Cu);
                    const uint32_t od13 = __builtin_amdgcn_perm(bt[3], bt[1], 0x0C0C0400u);
                    const uint32_t od57 = __builtin_amdgcn_perm(bt[7], bt[5], 0x04000C0Cu);
                    const uint32_t evn = ev02 | ev46;
                    const uint32_t odd = (od13 | od57) << 4;
                    const uint32_t word = (evn & 0x0F0F0F0Fu) | (odd & 0xF0F0F0F0u);
                    __builtin_nontemporal_store(
                        word,
                        reinterpret_cast<uint32_t *>(L.q4 + ((static_cast<int>(p) - n8) * (D / 2) + 4 * c)));
                }
            };
            const int k = slot_class(L, m);
            if (k == 1) emit(std::true_type{});
            else if (k == 0) emit(std::false_type{});
            else if (static_cast<int>(p) < n8) emit(std::true_type{});
            else emit(std::false_type{});
        }
    } else {
    #pragma unroll
        for (int m = 0; m < 8; ++m) {
            const unsigned p = static_cast<unsigned>(g + 16 * m);
            uint32_t bt[8];
    #pragma unroll
            for (int e = 0; e < 8; ++e) bt[e] = __float_as_uint(__builtin_fmaf(z[m][e], mulv[m], kRoundMagic));
            if (REFIT) {
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float zq = __uint_as_float(bt[e]) - kRoundMagic; // the code, exactly
                    num[e] = __builtin_fmaf(rav[m] * zq, z[m][e], num[e]);
                    den[e] = __builtin_fmaf(rbv[m] * zq, zq, den[e]);
                }
            }
            if (m < M8) {
                const uint32_t a01 = __builtin_amdgcn_perm(bt[1], bt[0], 0x0C0C0400u);
                const uint32_t a23 = __builtin_amdgcn_perm(bt[3], bt[2], 0x04000C0Cu);
                const uint32_t a45 = __builtin_amdgcn_perm(bt[5], bt[4], 0x0C0C0400u);
                const uint32_t a67 = __builtin_amdgcn_perm(bt[7], bt[6], 0x04000C0Cu);
                __builtin_nontemporal_store(u32x2{a01 | a23, a45 | a67},
                                            reinterpret_cast<u32x2 *>(L.q8 + (p * D + 8 * c)));
            } else {
                // even columns -> low nibbles, odd columns -> high nibbles
                const uint32_t ev02 = __builtin_amdgcn_perm(bt[2], bt[0], 0x0C0C0400u);
                const uint32_t ev46 = __builtin_amdgcn_perm(bt[6], bt[4], 0x04000C0Cu);
                const uint32_t od13 = __builtin_amdgcn_perm(bt[3], bt[1], 0x0C0C0400u);
                const uint32_t od57 = __builtin_amdgcn_perm(bt[7], bt[5], 0x04000C0Cu);
                const uint32_t evn = ev02 | ev46;
                const uint32_t odd = (od13 | od57) << 4;
                const uint32_t word = (evn & 0x0F0F0F0Fu) | (odd & 0xF0F0F0F0u);
                __builtin_nontemporal_store(word,
                                            reinterpret_cast<uint32_t *>(L.q4 + ((p - N8) * (D / 2) + 4 * c)));
            }
        }
    }
    if (REFIT) {
        // ---- Table C2 step 5: the column factors refit to the new codes
        // (App. C.1 fixed-code update).  Partials per (wave, lane group,
        // chunk c, column offset e) go through the MFMA reduction buffer,
        // free since the column sums were read.
        float2 *red2 = reinterpret_cast<float2 *>(&sh.red[0][0][0][0]); // [4][4][16][8]
        float4 *mine = reinterpret_cast<float4 *>(red2 + ((w * 4 + gl) * 16 + c) * 8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) mine[e / 2] = make_float4(num[e], den[e], num[e + 1], den[e + 1]);
        __syncthreads();
        if (t < D) {
            const int cc = t & 15;
            const int ce = (t >> 4) & 7;
            const int jcol = 8 * cc + ce;
            float nsum = 0.0f, dsum = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float2 f = red2[(q * 16 + cc) * 8 + ce];
                nsum += f.x;
                dsum += f.y;
            }
            const float cold = sh.c[jcol];
            L.cw[jcol] = dsum > 0.0f ? fmaxf(cold * (nsum / dsum), kRowFloor) : cold;
        }
    }
}

template <int N8, typename TIn, bool REFIT, bool GATED>
__global__ __launch_bounds__(256) void decode128_kernel(DecodeArgs a, int xcd_remap, unsigned hv_m,
                                                        unsigned g_m) {
    static_assert(N8 == kRuntimeN8 || (N8 % 16 == 0 && N8 >= 0 && N8 <= D),
                  "n8 must be a multiple of 16 (or read at run time)");
    __shared__ Smem sh;

    Lane L;
    L.t = threadIdx.x;
    L.c = L.t & 15;
    L.g = L.t >> 4;
    const int t = L.t;
    unsigned unit = blockIdx.x;
    if (xcd_remap) {
        // workgroups are dealt round-robin to the 8 XCDs; give each XCD a
        // contiguous range of units so value heads sharing a key head (and
        // their q, k) meet in the same L2
        const unsigned per = gridDim.x >> 3;
        unit = (blockIdx.x & 7u) * per + (blockIdx.x >> 3);
    }
    L.unit = unit;
    const int Hv = a.Hv;
    const int b = static_cast<int>(udiv(unit, static_cast<unsigned>(Hv), hv_m));
    const int h = static_cast<int>(unit - static_cast<unsigned>(b) * static_cast<unsigned>(Hv));
    const int hk = static_cast<int>(udiv(static_cast<unsigned>(h), static_cast<unsigned>(Hv / a.Hk), g_m));
    const int slot = a.slots ? a.slots[b] : b;
    if (slot < 0 || slot >= a.n_slots) { // whole workgroup leaves together
        if (t < D) store_o(a, static_cast<size_t>(unit) * D + t, __int_as_float(0x7fc00000));
        return;
    }
    L.alpha = GATED ? 1.0f : a.alpha[unit];
    L.beta = a.beta[unit];
    const size_t ub = static_cast<size_t>(slot) * Hv + h;
    const int n8 = N8 == kRuntimeN8 ? a.n8 : N8;
    L.n8 = n8;
    L.wv = 0;
    if constexpr (N8 == kRuntimeN8) L.wv = __builtin_amdgcn_readfirstlane(t >> 6);
    L.p8 = a.pool8 + ub * (n8 * D);
    L.p4 = a.pool4 + ub * ((D - n8) * (D / 2));
    L.rr = a.r + ub * D;
    L.q8 = a.pool8_out + ub * (n8 * D);
    L.q4 = a.pool4_out + ub * ((D - n8) * (D / 2));
    L.rw = a.r_out + ub * D;
    L.cw = REFIT ? a.cs_out + ub * D : nullptr;

    // ---- the per-unit vectors, loaded at logical indices so that no load
    // waits for another one (the gathers through perm are lane permutes
    // below); they are issued before the codes, because loads complete in
    // the order they are issued.  Waves 0 and 1 (lanes below D) each load
    // all 128 entries of k and q (two per lane), the others v and c.
    const int tl = t & (D - 1);
    const int l64 = t & 63;
    const bool lowhalf = __builtin_amdgcn_readfirstlane(t) < D; // wave-uniform
    const unsigned kb = static_cast<unsigned>((b * a.Hk + hk) * D);
    const int praw = a.perm[h * D + tl];
    const float rpv = L.rr[tl];
    // raw bits only: widening here would make the branch wait for the loads
    uint32_t x0, x1, x2 = 0u, x3 = 0u, g0 = 0u, g1 = 0u, u0 = 0u, u1 = 0u;
    if (lowhalf) {
        x0 = In<TIn>::raw(a.k, kb + l64);
        x1 = In<TIn>::raw(a.k, kb + 64 + l64);
        x2 = In<TIn>::raw(a.q, kb + l64);
        x3 = In<TIn>::raw(a.q, kb + 64 + l64);
        if (GATED) {
            const uint32_t *gp = reinterpret_cast<const uint32_t *>(a.gate) + static_cast<size_t>(unit) * D;
            g0 = gp[l64];
            g1 = gp[64 + l64];
        }
        if (REFIT) {
            const uint32_t *wp = reinterpret_cast<const uint32_t *>(a.w2) + h * D;
            u0 = wp[l64];
            u1 = wp[64 + l64];
        }
    } else {
        x0 = In<TIn>::raw(a.v, static_cast<unsigned>((b * Hv + h) * D + tl));
        x1 = REFIT ? reinterpret_cast<const uint32_t *>(a.cs)[ub * D + tl]
                   : reinterpret_cast<const uint32_t *>(a.c)[h * D + tl];
    }
    // ---- Table C2 step 1: issue the loads of this lane's packed rows
    uint32_t w0[8], w1[8];
    load_codes<N8>(L, w0, w1);
    if (lowhalf) {
        // ---- per-row and per-column factors, once per unit
        const int p = t;
        const int i = praw & (D - 1);
        const int src = (i & 63) << 2;
        const bool up = (i & 64) != 0;
        auto pick = [&](uint32_t lo, uint32_t hi) {
            const uint32_t a0 = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(lo));
            const uint32_t a1 = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(hi));
            return up ? a1 : a0;
        };
        const float kp = In<TIn>::cvt(pick(x0, x1));
        const float qp = In<TIn>::cvt(pick(x2, x3));
        const float rp = rpv;
        // 4-bit codes are widened as 16 z; a row gate scales the whole row
        float scale = p < n8 ? rp : rp * 0.0625f;
        if (GATED) scale *= __uint_as_float(pick(g0, g1));
        {
            // row p = 4 w + gl + 16 m of wave w, lane group gl, slot m
            uint16_t(&cf)[7][8] = sh.coef[(p & 15) >> 2][p & 3];
            const int mm = p >> 4;
            uint32_t h0, h1, h2;
            split3(scale * kp, h0, h1, h2);
            cf[0][mm] = static_cast<uint16_t>(h0);
            cf[1][mm] = static_cast<uint16_t>(h1);
            cf[2][mm] = static_cast<uint16_t>(h2);
            split3(scale * qp, h0, h1, h2);
            cf[3][mm] = static_cast<uint16_t>(h0);
            cf[4][mm] = static_cast<uint16_t>(h1);
            cf[5][mm] = static_cast<uint16_t>(h2);
        }
        const float ar = L.alpha * scale;
        const float bk = L.beta * kp;
        // |b k| > 2^-64 |a r| (false when both vanish: then x = 0 * z = 0)
        const bool scaled = fabsf(bk) > fabsf(ar) * kFormTiny;
        const float w2 = REFIT ? __uint_as_float(pick(u0, u1)) : 0.0f;
        sh.row[p] = make_float4(scaled ? ar * __builtin_amdgcn_rcpf(bk) : ar, scaled ? bk : 1.0f, w2,
                                __int_as_float(scaled ? 0 : D));
        const float kq = wave_sum(kp * qp);
        if ((t & 63) == 0) sh.kq[t >> 6] = kq;
    } else {
        // (a use on this side too, so the compiler keeps the two loads ahead
        // of the code loads instead of sinking them into the branch above)
        asm volatile("" ::"v"(praw), "v"(rpv));
        const int j = tl;
        sh.v[j] = In<TIn>::cvt(x0);
        sh.c[j] = __uint_as_float(x1);
        sh.ez[D + j] = 0.0f;
        if (j < 16) *reinterpret_cast<uint4 *>(&sh.coef[j >> 2][j & 3][6][0]) = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    finish_unit<N8, REFIT>(a, sh, L, w0, w1);
}

// ceil(2^32 / d) for d >= 2, 0 for d = 1 (see udiv)
unsigned div_magic(unsigned d) {
    return d <= 1 ? 0u : static_cast<unsigned>(((1ull << 32) + d - 1) / d);
}

template <int N8, typename TIn, bool REFIT, bool GATED>
void launch_one(const DecodeArgs &a, unsigned units, int remap, unsigned hv_m, unsigned g_m,
                hipStream_t s) {
    hipLaunchKernelGGL((decode128_kernel<N8, TIn, REFIT, GATED>), dim3(units), dim3(256), 0, s, a,
                       remap, hv_m, g_m);
}

template <int N8, typename TIn>
void launch_in(const DecodeArgs &a, unsigned units, int remap, unsigned hv_m, unsigned g_m,
               hipStream_t s) {
    const bool refit = a.cs != nullptr;
    const bool gated = a.gate != nullptr;
    if (refit && gated) launch_one<N8, TIn, true, true>(a, units, remap, hv_m, g_m, s);
    else if (refit) launch_one<N8, TIn, true, false>(a, units, remap, hv_m, g_m, s);
    else if (gated) launch_one<N8, TIn, false, true>(a, units, remap, hv_m, g_m, s);
    else launch_one<N8, TIn, false, false>(a, units, remap, hv_m, g_m, s);
}

template <int N8>
hipError_t launch_n8(bool bf16, const DecodeArgs &a, hipStream_t s) {
    const unsigned units = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    const int remap = (units % 8u) == 0u ? 1 : 0;
    const unsigned hv_m = div_magic(static_cast<unsigned>(a.Hv));
    const unsigned g_m = div_magic(static_cast<unsigned>(a.Hv / a.Hk));
    if (bf16)
        launch_in<N8, uint16_t>(a, units, remap, hv_m, g_m, s);
    else
        launch_in<N8, float>(a, units, remap, hv_m, g_m, s);
    return hipGetLastError();
}

} // namespace

bool decode128_supported(int n8) { return n8 >= 0 && n8 <= D; }

hipError_t launch_decode128(int n8, bool bf16, const DecodeArgs &a, hipStream_t s) {
    switch (n8) {
    case 0: return launch_n8<0>(bf16, a, s);
    case 16: return launch_n8<16>(bf16, a, s);
    case 32: return launch_n8<32>(bf16, a, s);
    case 48: return launch_n8<48>(bf16, a, s);
    case 64: return launch_n8<64>(bf16, a, s);
    case 80: return launch_n8<80>(bf16, a, s);
    case 96: return launch_n8<96>(bf16, a, s);
    case 112: return launch_n8<112>(bf16, a, s);
    case 128: return launch_n8<128>(bf16, a, s);
    default: return launch_n8<kRuntimeN8>(bf16, a, s);
    }
}

} // namespace stq
