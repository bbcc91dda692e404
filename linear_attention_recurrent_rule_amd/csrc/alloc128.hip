// Decode step of the ragged row-class formats (ALLOC, ALLOC_REFIT) for
// 128 x 128 heads: FP16 pivot rows and 8-, 6-, 4-, 2-bit rows per head
// (STEPQuant paper, arXiv 2609.38169: App. C.2 Table C1 for the classes,
// App. C.3 Table C2 for the step with pivots; Sec. 2.1 Eq. (1) with either
// gate; Sec. 2.2 quantizer; Sec. 4.3 representation).  Same arithmetic
// contract as decode_alloc_kernel in alloc_kernels.hip, arranged like the
// fixed-split 128 x 128 kernel:
//
//  * lane (g, c), g = lane / 16, c = lane % 16, owns columns 8c..8c+7 of
//    physical rows g + 16 m, m = 0..7; wave w therefore holds rows
//    16 m + 4 w .. 16 m + 4 w + 3 in slot m.  A head's rows are sorted by
//    class, so those four rows almost always share one class: the wave then
//    branches on a scalar class and runs the code of that class; only a slot
//    that straddles a class boundary takes a per-lane branch;
//  * the per-unit vectors (perm, r, k, q, v, c, gate) are loaded before the
//    codes at addresses that depend on no other load: k and q are read in
//    logical order, two entries per lane, and brought into physical row order
//    by lane permutes instead of a gather through perm;
//  * integer codes are widened so that every class fits a signed byte: 8-bit
//    codes as z, 6-bit as 4 z, 4-bit as 16 z, 2-bit as 64 z (the row
//    coefficients carry the inverse power of two);
//  * column sums u~ = S~^T (r k), w~ = S~^T (r q) on the matrix cores as bf16
//    products with exact three-way splits of the row coefficients; a pivot
//    row enters with its binary16 value h split exactly into two bf16 parts
//    (hi: the top 8 significant bits, lo: the remaining 3) and its
//    coefficients in separate output rows, whose sums are divided by c_j
//    afterwards (a pivot row has no column factor: its contribution to the
//    column-normalised sums is k_i h_ij / c_j);
//  * the update x_ij = X_ij / c_j = s_i (P_i z_ij + E_ij), the DPP row-max
//    reduce-scatter, the row factors and the code FMA against 1.5 * 2^23 are
//    those of the fixed-split kernel; a pivot row uses z_ij = h_ij / c_j and a
//    row factor of 1 and stores X = c_j s_i y_ij in binary16 (round to nearest
//    even, saturated at +-65504), with r = 0 and no part in the column refit.
#include <hip/hip_runtime.h>

#include "stq_internal.h"

namespace stq {
namespace {

constexpr int D = 128;
constexpr float kRoundMagic = 12582912.0f;               // 1.5 * 2^23
constexpr float kRowFloor = 1.17549435082228750797e-38f; // 2^-126
constexpr float kMulMax = 1.70141183460469231732e38f;    // 2^127
constexpr float kFormTiny = 5.42101086242752217004e-20f; // 2^-64
constexpr float kHalfMax = 65504.0f;

// Input elements as raw bits (a load whose result is only moved does not
// wait for it) and their fp32 value.
template <typename T> struct In;
template <> struct In<float> {
    static __device__ __forceinline__ uint32_t raw(const void *p, unsigned i) {
        return static_cast<const uint32_t *>(p)[i];
    }
    static __device__ __forceinline__ float cvt(uint32_t bits) { return __uint_as_float(bits); }
};
template <> struct In<uint16_t> {
    static __device__ __forceinline__ uint32_t raw(const void *p, unsigned i) {
        return static_cast<const uint16_t *>(p)[i];
    }
    static __device__ __forceinline__ float cvt(uint32_t bits) { return __uint_as_float(bits << 16); }
};

// Bytes per row of each class (pivot, 8, 6, 4, 2 bits).
template <int K> struct Cls;
template <> struct Cls<0> { static constexpr int row = 2 * D; };
template <> struct Cls<1> { static constexpr int row = D; };
template <> struct Cls<2> { static constexpr int row = 3 * D / 4; };
template <> struct Cls<3> { static constexpr int row = D / 2; };
template <> struct Cls<4> { static constexpr int row = D / 4; };

template <int K> struct IC { static constexpr int value = K; };

// Class boundaries of one head (wave-uniform): first physical row and first
// segment byte of classes 1..4 (class 0 starts at row 0, byte 0).
struct Bounds {
    int s1, s2, s3, s4;
    int b1, b2, b3, b4;
};

__device__ __forceinline__ int class_of(const Bounds &L, int p) {
    return (p >= L.s1) + (p >= L.s2) + (p >= L.s3) + (p >= L.s4);
}

// Rows of class K lie at b_K + (p - s_K) RB_K.  For slot m (rows g + 16 m)
// that splits into a wave-uniform part, b_K + (16 m - s_K) RB_K, and the lane
// part g RB_K.
template <int K> __device__ __forceinline__ int slot_base(const Bounds &L, int m) {
    if constexpr (K == 0) return 16 * m * Cls<0>::row;
    else if constexpr (K == 1) return L.b1 + (16 * m - L.s1) * Cls<1>::row;
    else if constexpr (K == 2) return L.b2 + (16 * m - L.s2) * Cls<2>::row;
    else if constexpr (K == 3) return L.b3 + (16 * m - L.s3) * Cls<3>::row;
    else return L.b4 + (16 * m - L.s4) * Cls<4>::row;
}

template <typename F> __device__ __forceinline__ void with_class(int k, F &&f) {
    switch (k) {
    case 0: f(IC<0>{}); break;
    case 1: f(IC<1>{}); break;
    case 2: f(IC<2>{}); break;
    case 3: f(IC<3>{}); break;
    default: f(IC<4>{}); break;
    }
}

// Per wave, once per unit: the class of each slot's four rows (4 bits per
// slot), or 7 where they straddle a class boundary.  Lane m computes slot m
// and the eight results are read back into a scalar.
__device__ __forceinline__ unsigned slot_table(const Bounds &L, int wv, int lane) {
    const int m = lane & 7;
    const int p0 = 16 * m + 4 * wv;
    const int ka = class_of(L, p0);
    const int kb = class_of(L, p0 + 3);
    const int v = ka == kb ? ka : 7;
    unsigned tab = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        tab |= static_cast<unsigned>(__builtin_amdgcn_readlane(v, q)) << (4 * q);
    return tab;
}

// Run f with the class of this lane's row in slot m: a scalar branch when the
// wave's four rows of the slot share a class, a per-lane branch otherwise.
// f must not exchange data between lanes.
template <typename F>
__device__ __forceinline__ void per_slot(const Bounds &L, unsigned tab, int g, int m, F &&f) {
    const int k = static_cast<int>((tab >> (4 * m)) & 15u);
    if (k != 7) with_class(k, f);
    else with_class(class_of(L, g + 16 * m), f);
}

// Every slot issues the same two 8-byte loads, A and B, whatever its class
// (so no register is written by different instructions on different paths
// and the loads of all slots stay in flight together); the class only
// chooses the addresses.  row = byte offset of the lane's row in the
// segment.  Pivot: A, B = bytes 16c..16c+15.  8-bit: A = bytes 8c..8c+7.
// 6-bit: A = the 8-byte word holding the lane's 4 bytes of low nibbles, B the
// 8-byte word holding its 2 bytes of high fields.  4-bit: A as for 6-bit.
// 2-bit: A = the 8-byte word holding its 2 bytes.  Unused B repeats A.
template <int K>
__device__ __forceinline__ void chunk_offsets(unsigned row, int c, unsigned &offA, unsigned &offB) {
    const unsigned uc = static_cast<unsigned>(c);
    if constexpr (K == 0) {
        offA = row + 16u * uc;
        offB = offA + 8u;
    } else if constexpr (K == 1) {
        offA = row + 8u * uc;
        offB = offA;
    } else if constexpr (K == 2) {
        offA = row + ((4u * uc) & ~7u);
        offB = row + D / 2 + ((2u * uc) & ~7u);
    } else if constexpr (K == 3) {
        offA = row + ((4u * uc) & ~7u);
        offB = offA;
    } else {
        offA = row + ((2u * uc) & ~7u);
        offB = offA;
    }
}

// The raw words of the lane's chunk from the two loads.
template <int K>
__device__ __forceinline__ void chunk_words(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                            int c, uint32_t (&w)[4]) {
    if constexpr (K == 0) {
        w[0] = a0; w[1] = a1; w[2] = b0; w[3] = b1;
    } else if constexpr (K == 1) {
        w[0] = a0; w[1] = a1;
    } else if constexpr (K == 2) {
        w[0] = (c & 1) ? a1 : a0;
        w[1] = (((c & 2) ? b1 : b0) >> (16 * (c & 1))) & 0xFFFFu;
    } else if constexpr (K == 3) {
        w[0] = (c & 1) ? a1 : a0;
    } else {
        w[0] = (((c & 2) ? a1 : a0) >> (16 * (c & 1))) & 0xFFFFu;
    }
}

__device__ __forceinline__ float sbyte(uint32_t w, int k) {
    return static_cast<float>(static_cast<int8_t>(w >> (8 * k)));
}

// Byte e' of the result holds nibble e' of the 16-bit value x (e' = 0..3).
__device__ __forceinline__ uint32_t nibbles_to_bytes(uint32_t x) {
    const uint32_t t = __builtin_amdgcn_perm(x, x, 0x01010000u); // bytes [x0, x0, x1, x1]
    return (t & 0x000F000Fu) | ((t >> 4) & 0x0F000F00u);
}

// Widen a chunk: z = W code as fp32 for integer rows (W = 1, 4, 16, 64 for
// 8, 6, 4, 2 bits); the binary16 value for pivot rows.
template <int K> __device__ __forceinline__ void widen(const uint32_t (&w)[4], float (&z)[8]) {
    if constexpr (K == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            z[e] = static_cast<float>(
                __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)))));
    } else if constexpr (K == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = sbyte(w[0], e);
            z[4 + e] = sbyte(w[1], e);
        }
    } else if constexpr (K == 2) {
        // code bits 0..3 from the nibble word, bits 4..5 from the 2-bit
        // fields; byte e' of ev (od) = code of column 2e' (2e'+1) << 2
        const uint32_t s = nibbles_to_bytes(w[1]);
        const uint32_t ev = ((w[0] << 2) & 0x3C3C3C3Cu) | ((s << 6) & 0xC0C0C0C0u);
        const uint32_t od = ((w[0] >> 2) & 0x3C3C3C3Cu) | ((s << 4) & 0xC0C0C0C0u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[2 * e] = sbyte(ev, e);
            z[2 * e + 1] = sbyte(od, e);
        }
    } else if constexpr (K == 3) {
        const uint32_t hi = w[0] & 0xF0F0F0F0u;        // odd columns, x16
        const uint32_t lo = (w[0] << 4) & 0xF0F0F0F0u; // even columns, x16
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[2 * e] = sbyte(lo, e);
            z[2 * e + 1] = sbyte(hi, e);
        }
    } else {
        const uint32_t s = nibbles_to_bytes(w[0]);
        const uint32_t ev = (s << 6) & 0xC0C0C0C0u;
        const uint32_t od = (s << 4) & 0xC0C0C0C0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[2 * e] = sbyte(ev, e);
            z[2 * e + 1] = sbyte(od, e);
        }
    }
}

// Compact the low nibbles of bytes 0..3 of n into a 16-bit value (nibble e'
// from byte e').
__device__ __forceinline__ uint32_t bytes_to_nibbles(uint32_t n) {
    const uint32_t m = n | (n >> 4);
    return __builtin_amdgcn_perm(m, m, 0x0C0C0200u);
}

// Store the codes of an integer chunk: bt[e] holds fl32(y mul + 1.5 * 2^23),
// whose low byte is the code in two's complement.
template <int K>
__device__ __forceinline__ void store_codes(uint8_t *base, unsigned off, int c,
                                            const uint32_t (&bt)[8]) {
    if constexpr (K == 1) {
        const uint32_t a01 = __builtin_amdgcn_perm(bt[1], bt[0], 0x0C0C0400u);
        const uint32_t a23 = __builtin_amdgcn_perm(bt[3], bt[2], 0x04000C0Cu);
        const uint32_t a45 = __builtin_amdgcn_perm(bt[5], bt[4], 0x0C0C0400u);
        const uint32_t a67 = __builtin_amdgcn_perm(bt[7], bt[6], 0x04000C0Cu);
        *reinterpret_cast<uint2 *>(base + (off + 8u * c)) = make_uint2(a01 | a23, a45 | a67);
    } else {
        // bytes of the even columns 0, 2, 4, 6 and of the odd columns
        const uint32_t evn = __builtin_amdgcn_perm(bt[2], bt[0], 0x0C0C0400u) |
                             __builtin_amdgcn_perm(bt[6], bt[4], 0x04000C0Cu);
        const uint32_t odd = __builtin_amdgcn_perm(bt[3], bt[1], 0x0C0C0400u) |
                             __builtin_amdgcn_perm(bt[7], bt[5], 0x04000C0Cu);
        if constexpr (K == 2 || K == 3) {
            const uint32_t word = (evn & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
            *reinterpret_cast<uint32_t *>(base + (off + 4u * c)) = word;
        }
        if constexpr (K == 2) {
            // bits 4..5 of each code: column e in bits 2e of a 16-bit field
            const uint32_t n = ((evn >> 4) & 0x03030303u) | ((odd >> 2) & 0x0C0C0C0Cu);
            *reinterpret_cast<uint16_t *>(base + (off + D / 2 + 2u * c)) =
                static_cast<uint16_t>(bytes_to_nibbles(n));
        }
        if constexpr (K == 4) {
            const uint32_t n = (evn & 0x03030303u) | ((odd << 2) & 0x0C0C0C0Cu);
            *reinterpret_cast<uint16_t *>(base + (off + 2u * c)) =
                static_cast<uint16_t>(bytes_to_nibbles(n));
        }
    }
}

__device__ __forceinline__ uint32_t half_bits(float x) {
    x = fminf(fmaxf(x, -kHalfMax), kHalfMax);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

template <int CTRL> __device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kRowRor8 = 0x128;
constexpr int kRowHalfMirror = 0x141;
constexpr int kQuadXor2 = 0x4E;
constexpr int kQuadXor1 = 0xB1;
constexpr int kRowMirror = 0x140;

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

// Matrix-core operand A: per wave and lane group, 13 rows of 8 bf16 (one per
// slot): 0..2 r k (hi, mid, lo) and 3..5 r q of integer rows; 6..8 d k and
// 9..11 d q of pivot rows (d the row gate, 1 for the scalar gate); 12 zero.
constexpr int kCoefRows = 13;
struct Smem {
    uint16_t coef[4][4][kCoefRows][8];
    float4 row[D];          // {P, s, w2, offset of E in ez} per physical row
    float qinv[D];          // 1 / q_b per physical row, 0 for pivot rows
    float v[D], c[D];
    float ez[2 * D];        // e, then a zero vector; each as [e/4][c][e%4]
    float4 red[4][8][3][16]; // per wave, column offset e, lane group, chunk c
    float kq[2];
    float mul[16][8];
    float ra[16][8], rb[16][8];
};

__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ void split3(float x, uint32_t &h0, uint32_t &h1, uint32_t &h2) {
    h0 = bf16_bits(x);
    const float r1 = x - bf16_val(h0);
    h1 = bf16_bits(r1);
    const float r2 = r1 - bf16_val(h1);
    h2 = bf16_bits(r2);
}

__device__ __forceinline__ unsigned udiv(unsigned n, unsigned d, unsigned m) {
    if (m == 0) return n;
    unsigned q = __umulhi(n, m);
    if (q * d > n) --q;
    return q;
}

template <typename TIn, bool REFIT, bool GATED>
__global__ __launch_bounds__(256) void decode_alloc128_kernel(DecodeArgs a, int xcd_remap,
                                                              unsigned hv_m, unsigned g_m) {
    __shared__ Smem sh;
    const int t = threadIdx.x;
    const int c = t & 15;
    const int g = t >> 4;
    const int w = t >> 6;
    const int gl = (t >> 4) & 3;
    const int wv = __builtin_amdgcn_readfirstlane(w);

    unsigned unit = blockIdx.x;
    if (xcd_remap) {
        const unsigned per = gridDim.x >> 3;
        unit = (blockIdx.x & 7u) * per + (blockIdx.x >> 3);
    }
    const int Hv = a.Hv;
    const int b = static_cast<int>(udiv(unit, static_cast<unsigned>(Hv), hv_m));
    const int h = static_cast<int>(unit - static_cast<unsigned>(b) * static_cast<unsigned>(Hv));
    const int hk = static_cast<int>(udiv(static_cast<unsigned>(h), static_cast<unsigned>(Hv / a.Hk), g_m));
    const int slot = a.slots ? a.slots[b] : b;
    if (slot < 0 || slot >= a.n_slots) { // whole workgroup leaves together
        if (t < D) store_o(a, static_cast<size_t>(unit) * D + t, __int_as_float(0x7fc00000));
        return;
    }
    const float alpha = GATED ? 1.0f : a.alpha[unit];
    const float beta = a.beta[unit];
    const size_t ub = static_cast<size_t>(slot) * Hv + h;

    const int32_t *lay = a.layout + static_cast<size_t>(h) * kLayoutStride;
    Bounds L;
    {
        const int n0 = lay[0], n1 = lay[1], n2 = lay[2], n3 = lay[3];
        L.s1 = n0;
        L.s2 = L.s1 + n1;
        L.s3 = L.s2 + n2;
        L.s4 = L.s3 + n3;
        L.b1 = n0 * Cls<0>::row;
        L.b2 = L.b1 + n1 * Cls<1>::row;
        L.b3 = L.b2 + n2 * Cls<2>::row;
        L.b4 = L.b3 + n3 * Cls<3>::row;
    }
    const size_t seg = static_cast<size_t>(slot) * static_cast<size_t>(a.slot_bytes) +
                       static_cast<size_t>(lay[kLayoutSegOff]);
    const uint8_t *seg_in = reinterpret_cast<const uint8_t *>(a.pool8) + seg;
    uint8_t *seg_out = reinterpret_cast<uint8_t *>(a.pool8_out) + seg;
    const float *rr = a.r + ub * D;
    float *rw = a.r_out + ub * D;

    const unsigned tab = slot_table(L, wv, t);
    // ---- the per-unit vectors, loaded at logical indices so that no load
    // waits for another one (the gathers through perm are lane permutes
    // below); they are issued before the codes, because loads complete in
    // the order they are issued.  Waves 0 and 1 (lanes below D) each load
    // all 128 entries of k and q (two per lane), the others v and c.
    const int tl = t & (D - 1);
    const int l64 = t & 63;
    const bool lowhalf = wv < 2;
    const unsigned kb = static_cast<unsigned>((b * a.Hk + hk) * D);
    const int praw = a.perm[h * D + tl];
    const float rpv = rr[tl];
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

    // ---- Table C2 step 1: issue the loads of this lane's row chunks
    uint32_t ld[8][4]; // per slot: A.x, A.y, B.x, B.y
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        unsigned offA = 0u, offB = 0u;
        per_slot(L, tab, g, m, [&](auto KC) __attribute__((always_inline)) {
            constexpr int K = decltype(KC)::value;
            chunk_offsets<K>(static_cast<unsigned>(slot_base<K>(L, m) + g * Cls<K>::row), c, offA,
                             offB);
        });
        const uint2 A = *reinterpret_cast<const uint2 *>(seg_in + offA);
        const uint2 Bw = *reinterpret_cast<const uint2 *>(seg_in + offB);
        ld[m][0] = A.x;
        ld[m][1] = A.y;
        ld[m][2] = Bw.x;
        ld[m][3] = Bw.y;
    }

    // ---- per-row and per-column factors, once per unit
    if (lowhalf) {
        const int p = t;
        const int k = class_of(L, p);
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
        // integer rows: r / W (codes are widened as W z); pivot rows: 1
        const float winv = k == 1 ? 1.0f : (k == 2 ? 0.25f : (k == 3 ? 0.0625f : 0.015625f));
        float scale = k == 0 ? 1.0f : rpv * winv;
        if (GATED) scale *= __uint_as_float(pick(g0, g1));
        {
            uint16_t(&cf)[kCoefRows][8] = sh.coef[(p & 15) >> 2][p & 3];
            const int mm = p >> 4;
            const int on = k == 0 ? 6 : 0; // this row's coefficient rows
            const int off = 6 - on;        // the other class's rows stay zero
            uint32_t h0, h1, h2;
            split3(scale * kp, h0, h1, h2);
            cf[on + 0][mm] = static_cast<uint16_t>(h0);
            cf[on + 1][mm] = static_cast<uint16_t>(h1);
            cf[on + 2][mm] = static_cast<uint16_t>(h2);
            split3(scale * qp, h0, h1, h2);
            cf[on + 3][mm] = static_cast<uint16_t>(h0);
            cf[on + 4][mm] = static_cast<uint16_t>(h1);
            cf[on + 5][mm] = static_cast<uint16_t>(h2);
#pragma unroll
            for (int q = 0; q < 6; ++q) cf[off + q][mm] = 0;
        }
        const float ar = alpha * scale;
        const float bk = beta * kp;
        const bool scaled = fabsf(bk) > fabsf(ar) * kFormTiny;
        const float w2v = REFIT ? __uint_as_float(pick(u0, u1)) : 0.0f;
        const float w2 = k != 0 ? w2v : 0.0f;
        sh.row[p] = make_float4(scaled ? ar * __builtin_amdgcn_rcpf(bk) : ar, scaled ? bk : 1.0f, w2,
                                __int_as_float(scaled ? 0 : D));
        sh.qinv[p] = k == 0 ? 0.0f
                            : (k == 1 ? (1.0f / 127.0f)
                                      : (k == 2 ? (1.0f / 31.0f) : (k == 3 ? (1.0f / 7.0f) : 1.0f)));
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
        if (j < 16)
            *reinterpret_cast<uint4 *>(&sh.coef[j >> 2][j & 3][kCoefRows - 1][0]) =
                make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();

    // ---- widen the codes
    float z[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        per_slot(L, tab, g, m, [&](auto KC) __attribute__((always_inline)) {
            constexpr int K = decltype(KC)::value;
            uint32_t w[4];
            chunk_words<K>(ld[m][0], ld[m][1], ld[m][2], ld[m][3], c, w);
            widen<K>(w, z[m]);
        });
    }

    // ---- column sums on the matrix cores: per column offset e, one
    // 16x16x32 bf16 product of the 12 coefficient rows of the wave's 32 rows
    // with the 32 x 16 widened entries of column 8c + e (integer codes and
    // the hi part of pivot values are exact in bf16); waves holding pivot
    // rows add a second product with the lo parts of the pivot values
    const bool wave_pivots = 4 * wv < L.s1;
    {
        const u32x4 araw =
            *reinterpret_cast<const u32x4 *>(&sh.coef[w][gl][c < 12 ? c : 12][0]);
        const bf16x8 A = __builtin_bit_cast(bf16x8, araw);
        auto product = [&](int e) {
            u32x4 braw;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                braw[v] = __builtin_amdgcn_perm(__float_as_uint(z[2 * v + 1][e]),
                                                __float_as_uint(z[2 * v][e]), 0x07060302u);
            const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, braw),
                                                               zero, 0, 0, 0);
            if (wave_pivots) {
                // lo = h - hi (exact, at most 3 significant bits) on pivot rows
                float lo[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    lo[m] = 0.0f;
                    if (16 * m + 4 * wv < L.s1 && g + 16 * m < L.s1) {
                        const float x = z[m][e];
                        lo[m] = x - __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
                    }
                }
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    braw[v] = __builtin_amdgcn_perm(__float_as_uint(lo[2 * v + 1]),
                                                    __float_as_uint(lo[2 * v]), 0x07060302u);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, braw),
                                                             acc, 0, 0, 0);
            }
            return acc;
        };
        float4 *red = &sh.red[w][0][gl][c]; // column offset e at red[48 e]
        auto store = [&](int e, const f32x4 &acc) {
            if (gl < 3) red[48 * e] = make_float4(acc[0], acc[1], acc[2], acc[3]);
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
    // pivot rows enter the update as h / c
    if (wave_pivots) {
        float cinv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cinv[e] = __builtin_amdgcn_rcpf(sh.c[8 * c + e]);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            if (16 * m + 4 * wv < L.s1 && g + 16 * m < L.s1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) z[m][e] *= cinv[e];
            }
    }
    __syncthreads();

    // ---- column sums over the 4 waves: u~ (lanes 0..127) -> e; w~ (128..255)
    // kept for o.  Lane t handles column 8 (t % 16) + (t / 16) % 8.  Output
    // rows per lane group: 0: u hi, mid, lo, w hi; 1: w mid, lo, pivot u hi,
    // mid; 2: pivot u lo, pivot w hi, mid, lo.
    const bool head_pivots = L.s1 > 0;
    float wsum = 0.0f;
    const int cc = t & 15;
    const int ce = (t >> 4) & 7;
    const int jcol = 8 * cc + ce;
    const int ezi = (ce >> 2) * 64 + cc * 4 + (ce & 3);
    const float cinv_j = __builtin_amdgcn_rcpf(sh.c[jcol]);
    if (t < D) {
        float u = 0.0f, up = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float4 f = sh.red[ww][ce][0][cc];
            u += (f.x + f.y) + f.z;
        }
        if (head_pivots) {
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float4 f1 = sh.red[ww][ce][1][cc];
                const float4 f2 = sh.red[ww][ce][2][cc];
                up += (f1.z + f1.w) + f2.x;
            }
            u = __builtin_fmaf(up, cinv_j, u);
        }
        sh.ez[ezi] = __builtin_fmaf(-alpha, u, sh.v[jcol] * cinv_j);
    } else {
        float wp = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float4 f0 = sh.red[ww][ce][0][cc];
            const float4 f1 = sh.red[ww][ce][1][cc];
            wsum += (f0.w + f1.x) + f1.y;
        }
        if (head_pivots) {
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float4 f2 = sh.red[ww][ce][2][cc];
                wp += (f2.y + f2.z) + f2.w;
            }
            wsum = __builtin_fmaf(wp, cinv_j, wsum);
        }
    }
    __syncthreads();

    // ---- Table C2 step 3: readout of the updated state, before requantizing
    if (t >= D) {
        const float kq = sh.kq[0] + sh.kq[1];
        store_o(a, static_cast<size_t>(unit) * D + jcol, sh.c[jcol] * __builtin_fmaf(alpha, wsum, (beta * kq) * sh.ez[ezi]));
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
    // reduce-scatter over the 16 lanes of the row group: lane c ends with row c / 2
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
        const float qinv = sh.qinv[p];
        float rn = 0.0f, mul = 0.0f;
        if (qinv != 0.0f) {
            rn = fmaxf((fabsf(sc) * rmax) * qinv, kRowFloor);
            mul = fminf(fmaxf(sc * __builtin_amdgcn_rcpf(rn), -kMulMax), kMulMax);
        }
        if ((c & 1) == 0) {
            rw[p] = rn;
            sh.mul[g][mm] = mul;
            if (REFIT) {
                const float w2 = sh.row[p].z; // 0 on pivot rows
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

    // ---- Table C2 steps 5-6: codes against the stored factors, pack, write back
    float mulv[8];
    {
        const float4 m0 = *reinterpret_cast<const float4 *>(&sh.mul[g][0]);
        const float4 m1 = *reinterpret_cast<const float4 *>(&sh.mul[g][4]);
        mulv[0] = m0.x; mulv[1] = m0.y; mulv[2] = m0.z; mulv[3] = m0.w;
        mulv[4] = m1.x; mulv[5] = m1.y; mulv[6] = m1.z; mulv[7] = m1.w;
    }
    float num[8], den[8];
    if (REFIT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            num[e] = 0.0f;
            den[e] = 0.0f;
        }
    }
    // fresh copies of the lane coordinates: keeps the compiler from carrying
    // the row addresses of the loads through the whole kernel
    int gs = g, cs_ = c;
    asm volatile("" : "+v"(gs), "+v"(cs_));
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        // one slot at a time: keeps the codes of later slots from being
        // formed early (they would hold registers through the stores)
        per_slot(L, tab, gs, m, [&](auto KC) __attribute__((always_inline)) {
            constexpr int K = decltype(KC)::value;
            const int p = gs + 16 * m;
            uint8_t *base = seg_out + slot_base<K>(L, m);
            const unsigned off = static_cast<unsigned>(gs * Cls<K>::row);
            if constexpr (K == 0) {
                // X = c_j s y, stored in binary16, four columns at a time
                const float sc = sh.row[p].y;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float4 cq = *reinterpret_cast<const float4 *>(&sh.c[8 * cs_ + 4 * hf]);
                    const float *y = &z[m][4 * hf];
                    const uint32_t lo = half_bits(cq.x * (sc * y[0])) | (half_bits(cq.y * (sc * y[1])) << 16);
                    const uint32_t hi = half_bits(cq.z * (sc * y[2])) | (half_bits(cq.w * (sc * y[3])) << 16);
                    *reinterpret_cast<uint2 *>(base + (off + 16u * cs_ + 8u * hf)) = make_uint2(lo, hi);
                }
            } else {
                uint32_t bt[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) bt[e] = __float_as_uint(__builtin_fmaf(z[m][e], mulv[m], kRoundMagic));
                if (REFIT) {
                    const float ram = sh.ra[g][m], rbm = sh.rb[g][m];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float zq = __uint_as_float(bt[e]) - kRoundMagic; // the code, exactly
                        num[e] = __builtin_fmaf(ram * zq, z[m][e], num[e]);
                        den[e] = __builtin_fmaf(rbm * zq, zq, den[e]);
                    }
                }
                store_codes<K>(base, off, cs_, bt);
            }
        });
    }
    if (REFIT) {
        // ---- Table C2 step 5: the column factors refit over the integer rows
        float2 *red2 = reinterpret_cast<float2 *>(&sh.red[0][0][0][0]); // [4][4][16][8]
        float4 *mine = reinterpret_cast<float4 *>(red2 + ((w * 4 + gl) * 16 + c) * 8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) mine[e / 2] = make_float4(num[e], den[e], num[e + 1], den[e + 1]);
        __syncthreads();
        if (t < D) {
            float nsum = 0.0f, dsum = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float2 f = red2[(q * 16 + cc) * 8 + ce];
                nsum += f.x;
                dsum += f.y;
            }
            const float cold = sh.c[jcol];
            a.cs_out[ub * D + jcol] = dsum > 0.0f ? fmaxf(cold * (nsum / dsum), kRowFloor) : cold;
        }
    }
}

unsigned div_magic(unsigned d) {
    return d <= 1 ? 0u : static_cast<unsigned>(((1ull << 32) + d - 1) / d);
}

template <typename TIn, bool REFIT, bool GATED>
void launch_one(const DecodeArgs &a, unsigned units, int remap, unsigned hv_m, unsigned g_m,
                hipStream_t s) {
    hipLaunchKernelGGL((decode_alloc128_kernel<TIn, REFIT, GATED>), dim3(units), dim3(256), 0, s, a,
                       remap, hv_m, g_m);
}

template <typename TIn>
void launch_in(const DecodeArgs &a, unsigned units, int remap, unsigned hv_m, unsigned g_m,
               hipStream_t s) {
    const bool refit = a.cs != nullptr;
    const bool gated = a.gate != nullptr;
    if (refit && gated) launch_one<TIn, true, true>(a, units, remap, hv_m, g_m, s);
    else if (refit) launch_one<TIn, true, false>(a, units, remap, hv_m, g_m, s);
    else if (gated) launch_one<TIn, false, true>(a, units, remap, hv_m, g_m, s);
    else launch_one<TIn, false, false>(a, units, remap, hv_m, g_m, s);
}

} // namespace

hipError_t launch_decode_alloc128(bool bf16, const DecodeArgs &a, hipStream_t s) {
    const unsigned units = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    const int remap = (units % 8u) == 0u ? 1 : 0;
    const unsigned hv_m = div_magic(static_cast<unsigned>(a.Hv));
    const unsigned g_m = div_magic(static_cast<unsigned>(a.Hv / a.Hk));
    if (bf16)
        launch_in<uint16_t>(a, units, remap, hv_m, g_m, s);
    else
        launch_in<float>(a, units, remap, hv_m, g_m, s);
    return hipGetLastError();
}

} // namespace stq
