// Decode step of the ragged row-class formats (ALLOC, ALLOC_REFIT) for
// 128 x 128 heads: FP16 pivot rows and 8-, 6-, 4-, 2-bit rows per head
// (STEPQuant paper, arXiv 2609.38169: App. C.2 Table C1 for the classes,
// App. C.3 Table C2 for the step with pivots; Sec. 2.1 Eq. (1) with either
// gate; Sec. 2.2 quantizer; Sec. 4.3 representation).  Same arithmetic
// contract as decode_alloc_kernel in alloc_kernels.hip, on the tile and the
// helpers of the fixed-split 128 x 128 kernel (tile128.h):
//
//  * lane (g, c) owns columns 8c..8c+7 of physical rows g + 16 m; wave w
//    holds rows 16 m + 4 w .. 16 m + 4 w + 3 in slot m.  A head's rows are
//    sorted by class, so those four rows almost always share one class: the
//    wave then branches on a scalar class and runs the code of that class;
//    only a slot that straddles a class boundary takes a per-lane branch;
//  * the per-unit vectors (perm, r, k, q, v, c, gate) are loaded before the
//    codes at addresses that depend on no other load; k and q are brought
//    into physical row order by lane permutes;
//  * integer codes are widened so that every class fits a signed byte: 8-bit
//    codes as z, 6-bit as 4 z, 4-bit as 16 z, 2-bit as 64 z (the row
//    coefficients carry the inverse power of two).  A widened code is an fp32
//    register whose low 16 bits are zero, fed to the matrix cores as the
//    bf16 pair (0, z) with the coefficient words at the odd K positions;
//  * a pivot row holds its binary16 value h in that register: the matrix
//    core reads its high half, h truncated to 8 significant bits, and a
//    second product adds the remainder h - hi (at most 3 significant bits,
//    exact in bf16) where the wave holds pivot rows.  Pivot coefficients sit
//    in separate output rows, whose sums are divided by c_j afterwards (a
//    pivot row has no column factor: its contribution to the
//    column-normalised sums is k_i h_ij / c_j);
//  * the update x_ij = X_ij / c_j = s_i (P_i z_ij + E_ij), the DPP row-max
//    reduce-scatter, the row factors and the code FMA against 1.5 * 2^23 are
//    those of the fixed-split kernel; a pivot row uses z_ij = h_ij / c_j and a
//    row factor of 1 and stores X = c_j s_i y_ij in binary16 (round to nearest
//    even, saturated at +-65504), with r = 0 and no part in the column refit.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tile128.h"

namespace stq {
namespace {

using namespace t128;

constexpr float kHalfMax = 65504.0f;

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
    case 2: f(IC<2>{}); break; // the commonest classes first
    case 1: f(IC<1>{}); break;
    case 3: f(IC<3>{}); break;
    case 0: f(IC<0>{}); break;
    default: f(IC<4>{}); break;
    }
}

// Per wave, once per unit: the class of each slot's four rows (4 bits per
// slot), or 7 where they straddle a class boundary.  Lane m computes slot m
// and the eight results are read back into a scalar (so the per-slot class
// branches below are scalar branches).
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

// Lane constants of the chunk layouts: the mask of c & 1 (which 32-bit half
// of an 8-byte word holds the lane's 4 bytes of nibbles), and the byte
// selector that picks the lane's 2 bytes of 2-bit fields (bytes b, b + 1 of
// an 8-byte word, b = 2 (c % 4)) as [b, b, b + 1, b + 1].
struct ChunkLane {
    uint32_t odd;  // lane mask of c & 1
    uint32_t fsel; // v_perm selector of the lane's 16-bit field, doubled
};

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

// Byte e' of the result holds nibble e' of the lane's 16-bit field in the
// 8-byte word (hi, lo), which one byte permute brings out as [f0, f0, f1, f1].
__device__ __forceinline__ uint32_t field_nibbles(uint32_t hi, uint32_t lo, const ChunkLane &cl) {
    const uint32_t t = __builtin_amdgcn_perm(hi, lo, cl.fsel);
    return (t & 0x000F000Fu) | ((t >> 4) & 0x0F000F00u);
}

// The codes of one integer slot as two words of left-aligned bytes: byte j
// of ev (od) is the code of column 8c + 2j (2j + 1) times W = 1, 4, 16, 64
// for 8, 6, 4, 2 bits.  Only these two words depend on the class, so the
// class branch defines two registers and the conversions to fp32 follow it.
// ld = the slot's two loads (A.x, A.y, B.x, B.y).
template <int K>
__device__ __forceinline__ void code_words(const uint32_t (&ld)[4], const ChunkLane &cl, uint32_t &ev,
                                           uint32_t &od) {
    if constexpr (K == 0) {
        ev = 0u; // a pivot slot: its values are converted separately
        od = 0u;
    } else if constexpr (K == 1) {
        ev = __builtin_amdgcn_perm(ld[1], ld[0], 0x06040200u);
        od = __builtin_amdgcn_perm(ld[1], ld[0], 0x07050301u);
    } else if constexpr (K == 3) {
        const uint32_t w = sel(cl.odd, ld[1], ld[0]);
        ev = (w << 4) & 0xF0F0F0F0u;
        od = w & 0xF0F0F0F0u;
    } else if constexpr (K == 2) {
        // code bits 0..3 from the nibble word, bits 4..5 from the 2-bit fields
        const uint32_t w = sel(cl.odd, ld[1], ld[0]);
        const uint32_t n = field_nibbles(ld[3], ld[2], cl);
        ev = ((w << 2) & 0x3C3C3C3Cu) | ((n << 6) & 0xC0C0C0C0u);
        od = ((w >> 2) & 0x3C3C3C3Cu) | ((n << 4) & 0xC0C0C0C0u);
    } else {
        const uint32_t n = field_nibbles(ld[1], ld[0], cl);
        ev = (n << 6) & 0xC0C0C0C0u;
        od = (n << 4) & 0xC0C0C0C0u;
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
                                            const uint32_t (&bt)[8], uint32_t lo4) {
    if constexpr (K == 1) {
        *reinterpret_cast<u32x2 *>(base + (off + 8u * c)) = pack_bytes(bt);
    } else {
        uint32_t evn, odd;
        even_odd_bytes(bt, evn, odd);
        if constexpr (K == 2 || K == 3) {
            *reinterpret_cast<uint32_t *>(base + (off + 4u * c)) = sel(lo4, evn, odd << 4);
        }
        if constexpr (K == 2) {
            // bits 4..5 of each code: column e in bits 2e of a 16-bit field
            const uint32_t n = ((evn >> 4) & 0x03030303u) | ((odd >> 2) & 0x0C0C0C0Cu);
            *reinterpret_cast<uint16_t *>(base + (off + D / 2 + 2u * c)) = static_cast<uint16_t>(bytes_to_nibbles(n));
        }
        if constexpr (K == 4) {
            const uint32_t n = (evn & 0x03030303u) | ((odd << 2) & 0x0C0C0C0Cu);
            *reinterpret_cast<uint16_t *>(base + (off + 2u * c)) = static_cast<uint16_t>(bytes_to_nibbles(n));
        }
    }
}

__device__ __forceinline__ uint32_t half_bits(float x) {
    x = fminf(fmaxf(x, -kHalfMax), kHalfMax);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

// Matrix-core operand A: per wave and lane group, 12 rows of 8 words (one
// per slot), each a bf16 part in its high half, in the order of the
// product's output rows: 0..2 r k (hi, mid, lo) of integer rows, 3..5 d k of
// pivot rows, 6..7 d q (hi, mid) of pivot rows, 8..10 r q of integer rows,
// 11 d q (lo) of pivot rows (d the row gate, 1 for the scalar gate).  A
// row's words of the other kind are zero.  The product's lane groups 0, 1
// and 2 then hold (u hi, mid, lo, pivot u hi), (pivot u mid, lo, pivot w hi,
// mid) and (w hi, mid, lo, pivot w lo): each reader takes whole 16-byte
// entries.
constexpr int kCoefRows = 12;
// Words of lane group G: slot m of row r at 24 (m / 2) + 2 r + m % 2 (slot
// pairs 8-byte aligned for ds_read2_b64), groups 98 words apart, so that
// the staging lanes (16 groups, two slots per half wave) and the operand
// reads (two groups per 32 lanes) both spread over all banks.
constexpr int kCoefStride = 98;
struct Smem {
    uint32_t coef[16 * kCoefStride];
    float2 row[D];          // {P, byte offset of E in ez} per physical row
    float srow[D];          // s per row, at srow_index(g, m)
    float qbrow[D];         // q_b per row, 0 for pivot rows, at srow_index(g, m)
    float w2row[D];         // column refit: w2 per row, at srow_index(g, m)
    float v[D], c[D];
    float ez[2 * D];        // e, then a zero vector; each as [e/4][c][e%4]
    float4 red[4][8][3][16]; // per wave, column offset e, lane group, chunk c
    float kq[2];
    float mul[16][8];       // per row group: code multipliers of its 8 rows
    float ra[16][8], rb[16][8]; // column refit: w2 r' s and w2 r'^2 per row
};

// Three workgroups per CU cap the registers at 168. The instances without the
// column refit sit well below that; the refit ones would otherwise take 172
// and drop to two waves per SIMD, which costs about a third more time than the
// few values the cap spills.
template <typename TIn, bool REFIT, bool GATED>
__global__ __launch_bounds__(256, 3) void decode_alloc128_kernel(DecodeArgs a, UnitGeom ug) {
    __shared__ Smem sh;
    const int t = threadIdx.x;
    const int c = t & 15;
    const int g = t >> 4;
    const int w = t >> 6;
    const int gl = (t >> 4) & 3;
    const int wv = __builtin_amdgcn_readfirstlane(w);

    const unsigned unit = unit_of_block(ug);
    const int Hv = a.Hv;
    const int b = static_cast<int>(udiv(unit, static_cast<unsigned>(Hv), ug.hv_m));
    const int h = static_cast<int>(unit - static_cast<unsigned>(b) * static_cast<unsigned>(Hv));
    const int hk = static_cast<int>(udiv(static_cast<unsigned>(h), static_cast<unsigned>(ug.G), ug.g_m));
    // the head's layout, read through the constant address space: nothing
    // writes it during the step, and so it comes through the scalar cache,
    // where the workgroups of a head find it, instead of a vector load whose
    // latency would delay every row address
    // (the whole row in one scalar load: the class counts and the segment
    // offset, both needed before the first row address, in one round trip,
    // issued with the slot's load, on which it does not depend)
    static_assert(kLayoutStride == 8 && kLayoutSegOff < 8, "one layout row is eight words");
    typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(4))) const i32x8 ci32x8;
    const i32x8 lay = *(ci32x8 *)(reinterpret_cast<uintptr_t>(a.layout) + static_cast<size_t>(h) * kLayoutStride * 4);
    // and this wave's eight slot descriptors (row base, row bytes, class and
    // the lane's chunk offsets of each slot), written with the layout
    static_assert(kSlotDescWords == 4 * 16, "16 descriptor words per wave");
    typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
    typedef __attribute__((address_space(4))) const i32x16 ci32x16;
    i32x16 sd = {};
    if constexpr (!REFIT)
        sd = *(ci32x16 *)(reinterpret_cast<uintptr_t>(a.layout) +
                          (static_cast<size_t>(Hv) * kLayoutStride + static_cast<size_t>(h) * kSlotDescWords +
                           16u * static_cast<unsigned>(wv)) * 4);
    const int slot = slot_of(a, b);
    prefetch_args(a);
    asm volatile("" ::"s"(a.slot_bytes), "s"(a.pool8)); // (as above)
    if (slot < 0 || slot >= a.n_slots) { // whole workgroup leaves together
        if (t < D) store_o(a, static_cast<size_t>(unit) * D + t, __int_as_float(0x7fc00000));
        return;
    }
    const float alpha = GATED ? 1.0f : a.alpha[unit];
    const float beta = a.beta[unit];
    const size_t ub = static_cast<size_t>(slot) * Hv + h;

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

    // ---- the per-unit vectors, loaded at logical indices so that no load
    // waits for another one (the gathers through perm are lane permutes
    // below); they are issued before the codes, because loads complete in
    // the order they are issued.  Waves 0 and 1 (lanes below D) each load
    // all 128 entries of k and q (two per lane), the others v and c.
    const int tl = t & (D - 1);
    const int l64 = t & 63;
    const bool lowhalf = wv < 2;
    // (each vector's unit-wide offset goes into its base pointer, so that the
    // loads take a scalar base and a small per-lane offset)
    const size_t kb = static_cast<size_t>(b * a.Hk + hk) * D;
    const TIn *kp0 = static_cast<const TIn *>(a.k) + kb;
    const TIn *qp0 = static_cast<const TIn *>(a.q) + kb;
    const int praw = (a.perm + h * D)[tl];
    const float rpv = rr[tl];
    // raw bits only: widening here would make the branch wait for the loads
    uint32_t x0, x1, x2 = 0u, x3 = 0u, g0 = 0u, g1 = 0u, u0 = 0u, u1 = 0u;
    constexpr bool kPairs = std::is_same<TIn, uint16_t>::value; // bf16 k, q: two per 4-byte load
    if (lowhalf) {
        if constexpr (kPairs) {
            // lane l holds entries 2l and 2l + 1 of k and of q
            x0 = reinterpret_cast<const uint32_t *>(kp0)[l64];
            x2 = reinterpret_cast<const uint32_t *>(qp0)[l64];
        } else {
            x0 = In<TIn>::raw(kp0, l64);
            x1 = In<TIn>::raw(kp0, 64 + l64);
            x2 = In<TIn>::raw(qp0, l64);
            x3 = In<TIn>::raw(qp0, 64 + l64);
        }
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
        x0 = In<TIn>::raw(static_cast<const TIn *>(a.v) + static_cast<size_t>(b * Hv + h) * D, tl);
        const uint32_t *cp0 = REFIT ? reinterpret_cast<const uint32_t *>(a.cs) + ub * D
                                    : reinterpret_cast<const uint32_t *>(a.c) + h * D;
        x1 = cp0[tl];
    }

    // ---- Table C2 step 1: issue the loads of this lane's row chunks.  A slot
    // whose rows share a class (almost all) takes its addresses from its
    // descriptor with no branch on the class; a slot straddling a class
    // boundary takes the per-lane path
    // (the refit instances keep the per-slot class dispatch: their register
    // budget is spent, and the descriptors' scalar registers cost them spills)
    const unsigned c2 = 2u * static_cast<unsigned>(c);
    uint32_t ld[8][4]; // per slot: A.x, A.y, B.x, B.y
    unsigned tab = 0u;
    if constexpr (REFIT) {
        tab = slot_table(L, wv, t);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            unsigned offA = 0u, offB = 0u;
            per_slot(L, tab, g, m, [&](auto KC) __attribute__((always_inline)) {
                constexpr int K = decltype(KC)::value;
                chunk_offsets<K>(static_cast<unsigned>(slot_base<K>(L, m) + g * Cls<K>::row), c, offA,
                                 offB);
            });
            const u32x2 A = *reinterpret_cast<const u32x2 *>(seg_in + offA);
            const u32x2 Bw = *reinterpret_cast<const u32x2 *>(seg_in + offB);
            ld[m][0] = A[0];
            ld[m][1] = A[1];
            ld[m][2] = Bw[0];
            ld[m][3] = Bw[1];
        }
    } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int P = sd[2 * m + 1];
        unsigned offA = 0u, offB = 0u;
        if (__builtin_expect(P >= 0, 1)) {
            const unsigned rb = static_cast<unsigned>(P) & 0x1FFu;
            const unsigned shA = (static_cast<unsigned>(P) >> 16) & 15u;
            const unsigned shB = (static_cast<unsigned>(P) >> 20) & 15u;
            const unsigned ob = (static_cast<unsigned>(P) >> 24) & 0x7Fu;
            const unsigned row = static_cast<unsigned>(sd[2 * m]) + static_cast<unsigned>(g) * rb;
            offA = row + ((c2 >> shA) << 3);
            offB = row + ob + ((c2 >> shB) << 3);
        } else {
            with_class(class_of(L, g + 16 * m), [&](auto KC) __attribute__((always_inline)) {
                constexpr int K = decltype(KC)::value;
                chunk_offsets<K>(static_cast<unsigned>(slot_base<K>(L, m) + g * Cls<K>::row), c, offA,
                                 offB);
            });
        }
        const u32x2 A = *reinterpret_cast<const u32x2 *>(seg_in + offA);
        const u32x2 Bw = *reinterpret_cast<const u32x2 *>(seg_in + offB);
        ld[m][0] = A[0];
        ld[m][1] = A[1];
        ld[m][2] = Bw[0];
        ld[m][3] = Bw[1];
    }
    // the class of each slot's four rows (4 bits per slot, 7 where they
    // straddle a class boundary), for the class branches below
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int P = sd[2 * m + 1];
        tab |= (P < 0 ? 7u : (static_cast<unsigned>(P) >> 9) & 7u) << (4 * m);
    }
    }

    // ---- per-row and per-column factors, once per unit
    if (lowhalf) {
        const int p = t;
        const int k = class_of(L, p);
        const int i = praw & (D - 1);
        const int src = (i & 63) << 2;
        const uint32_t up = lane_mask(i & 64);
        auto pick = [&](uint32_t lo, uint32_t hi) {
            const uint32_t a0 = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(lo));
            const uint32_t a1 = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(hi));
            return sel(up, a1, a0);
        };
        float kp, qp;
        if constexpr (kPairs) {
            // entry i in half i & 1 of lane i >> 1: one permute per vector
            const int src2 = (i >> 1) << 2;
            const uint32_t odd = lane_mask(i & 1);
            auto pick2 = [&](uint32_t w) {
                const uint32_t v2 = __builtin_amdgcn_ds_bpermute(src2, static_cast<int>(w));
                return __uint_as_float(sel(odd, v2 & 0xFFFF0000u, v2 << 16));
            };
            kp = pick2(x0);
            qp = pick2(x2);
        } else {
            kp = In<TIn>::cvt(pick(x0, x1));
            qp = In<TIn>::cvt(pick(x2, x3));
        }
        // integer rows: r / W (codes are widened as W z); pivot rows: 1
        const uint32_t piv = lane_mask(k == 0);
        const float winv = __uint_as_float((127u - 2u * static_cast<unsigned>(k - 1)) << 23); // 2^(2 - 2k)
        float scale = self(piv, 1.0f, rpv * winv);
        if (GATED) scale *= __uint_as_float(pick(g0, g1));
        {
            const int mm = p >> 4;
            uint32_t *cf = &sh.coef[(p & 15) * kCoefStride + 24 * (mm >> 1) + (mm & 1)]; // row r at 2 r
            uint32_t wk[3], wq[3];
            split3w(scale * kp, wk[0], wk[1], wk[2]);
            split3w(scale * qp, wq[0], wq[1], wq[2]);
            // this row's coefficient words in its kind's rows, zero in the other's
            constexpr int kInt[2][3] = {{0, 1, 2}, {8, 9, 10}};
            constexpr int kPiv[2][3] = {{3, 4, 5}, {6, 7, 11}};
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                cf[2 * kInt[0][q]] = sel(piv, 0u, wk[q]);
                cf[2 * kInt[1][q]] = sel(piv, 0u, wq[q]);
                cf[2 * kPiv[0][q]] = sel(piv, wk[q], 0u);
                cf[2 * kPiv[1][q]] = sel(piv, wq[q], 0u);
            }
        }
        const float ar = alpha * scale;
        const float bk = beta * kp;
        // |b k| > 2^-64 |a r| (false when both vanish: then x = 0 * z = 0)
        const uint32_t scaled = lane_mask(fabsf(bk) > fabsf(ar) * kFormTiny);
        sh.row[p] = make_float2(self(scaled, div_refined(ar, bk), ar), __uint_as_float(sel(scaled, 0u, 4u * D)));
        const int si = srow_index(p & 15, p >> 4);
        sh.srow[si] = self(scaled, bk, 1.0f);
        if (REFIT) sh.w2row[si] = __uint_as_float(sel(piv, 0u, pick(u0, u1)));
        // q_b = 2^(b-1) - 1 for b = 8, 6, 4, 2; 0 marks a pivot row
        const float qbk = static_cast<float>((1 << (9 - 2 * k)) - 1);
        sh.qbrow[si] = self(piv, 0.0f, qbk);
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
    }
    __syncthreads();

    // ---- widen the codes: z[m][e] = code (or pivot value) of slot m in
    // column 8c + e
    ChunkLane cl;
    cl.odd = lane_mask(c & 1);
    {
        const uint32_t b = 2u * static_cast<uint32_t>(c & 3);
        cl.fsel = b * 0x00000101u + (b + 1u) * 0x01010000u;
    }
    uint32_t lo4 = 0x0F0F0F0Fu;
    asm volatile("" : "+v"(lo4));
    float z[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        uint32_t ev = 0u, od = 0u;
        per_slot(L, tab, g, m, [&](auto KC) __attribute__((always_inline)) {
            constexpr int K = decltype(KC)::value;
            code_words<K>(ld[m], cl, ev, od);
        });
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            z[m][2 * j] = sbyte(ev, j);
            z[m][2 * j + 1] = sbyte(od, j);
        }
        // pivot rows (the first s1 rows of the head): their binary16 values
        if (16 * m + 4 * wv < L.s1) {
            const uint32_t pm = lane_mask(g + 16 * m < L.s1);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                z[m][e] = self(pm,
                               static_cast<float>(__builtin_bit_cast(
                                   _Float16, static_cast<uint16_t>(ld[m][e >> 1] >> (16 * (e & 1))))),
                               z[m][e]);
        }
    }

    // ---- column sums on the matrix cores: per column offset e, two
    // 16x16x32 bf16 products of the 12 coefficient rows of the wave's 32
    // rows with their widened entries of column 8c + e; waves holding pivot
    // rows add the products with the low parts of the pivot values
    const bool wave_pivots = 4 * wv < L.s1;
    {
        const int crow = c < kCoefRows ? c : kCoefRows - 1;
        const u32x2 *cw = reinterpret_cast<const u32x2 *>(&sh.coef[(4 * w + gl) * kCoefStride + 2 * crow]);
        const u32x2 a0 = cw[0], a1 = cw[12], a2 = cw[24], a3 = cw[36]; // slot pairs
        const u32x4 A[2] = {u32x4{a0[0], a0[1], a1[0], a1[1]}, u32x4{a2[0], a2[1], a3[0], a3[1]}};
        float4 *red = &sh.red[w][0][gl][c]; // column offset e at red[48 e]
        auto store = [&](int e, const f32x4 &acc) {
            if (gl < 3) red[48 * e] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        };
        // the eight products as one straight run, with or without the pivot
        // low parts (two copies, so that the waves without pivot rows do not
        // issue those products)
        auto run = [&](auto PIV) __attribute__((always_inline)) {
            constexpr bool WITH = decltype(PIV)::value;
            auto product = [&](int e) {
                const f32x4 zz[2] = {f32x4{z[0][e], z[1][e], z[2][e], z[3][e]},
                                     f32x4{z[4][e], z[5][e], z[6][e], z[7][e]}};
                f32x4 acc = column_sums(A, zz);
                if constexpr (WITH) {
                    // h - hi, where hi = h with its low 16 bits cleared (what
                    // the matrix core read), in the slots holding pivot rows
                    f32x4 lo[2];
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const float x = z[m][e];
                        lo[m >> 2][m & 3] = 16 * m + 4 * wv < L.s1
                                                ? x - __uint_as_float(__float_as_uint(x) & 0xFFFF0000u)
                                                : 0.0f;
                    }
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, A[0]), __builtin_bit_cast(bf16x8, lo[0]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, A[1]), __builtin_bit_cast(bf16x8, lo[1]), acc, 0, 0, 0);
                }
                return acc;
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
        };
        if (wave_pivots) {
            asm volatile(""); // keeps this copy behind its branch
            run(std::true_type{});
        } else {
            run(std::false_type{});
        }
    }
    // pivot rows enter the update as h / c
    if (wave_pivots) {
        float cinv[8];
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
            const float4 cq = *reinterpret_cast<const float4 *>(&sh.c[8 * c + 4 * h4]);
            cinv[4 * h4] = __builtin_amdgcn_rcpf(cq.x);
            cinv[4 * h4 + 1] = __builtin_amdgcn_rcpf(cq.y);
            cinv[4 * h4 + 2] = __builtin_amdgcn_rcpf(cq.z);
            cinv[4 * h4 + 3] = __builtin_amdgcn_rcpf(cq.w);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m)
            if (16 * m + 4 * wv < L.s1 && g + 16 * m < L.s1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) z[m][e] *= cinv[e];
            }
    }
    __syncthreads();

    // ---- column sums over the 4 waves: u~ (lanes 0..127) -> e; w~ (128..255)
    // kept for o.  Lane t takes column 8 cc + ce, cc = t % 16, with ce =
    // (t / 16) % 8 rotated by 2 (cc / 4): the 16 lanes of a row group still
    // read 16 different chunks of the sums, and the 32 lanes of a half wave
    // read v and c from 32 different banks.  Output rows per lane group: 0: u hi, mid,
    // lo, pivot u hi; 1: pivot u mid, lo, pivot w hi, mid; 2: w hi, mid, lo,
    // pivot w lo.  Each entry is read whole (16 bytes, or the first 12):
    // narrower reads of 16-byte entries collide in the LDS banks.
    const bool head_pivots = L.s1 > 0;
    float wsum;
    const int cc = t & 15;
    const int ce = ((t >> 4) + ((t >> 1) & 6)) & 7;
    const int jcol = 8 * cc + ce;
    const int ezi = (ce >> 2) * 64 + cc * 4 + (ce & 3);
    auto whole = [](const float4 &f) __attribute__((always_inline)) {
        asm volatile("" ::"v"(f.x), "v"(f.y), "v"(f.z), "v"(f.w));
    };
    if (t < D) {
        const float4 u0 = sh.red[0][ce][0][cc];
        float u = (u0.x + u0.y) + u0.z;
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            const float4 f = sh.red[ww][ce][0][cc];
            u += (f.x + f.y) + f.z;
        }
        float vp = sh.v[jcol];
        if (head_pivots) {
            float up = 0.0f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float4 f0 = sh.red[ww][ce][0][cc];
                const float4 f1 = sh.red[ww][ce][1][cc];
                whole(f0);
                whole(f1);
                up += (f0.w + f1.x) + f1.y;
            }
            vp = __builtin_fmaf(-alpha, up, vp); // v - a u_pivots, divided by c below
        }
        // e = (v - a u_pivots) / c - a u, the quotient to within a hair of
        // correct rounding (see the fixed-split kernel)
        sh.ez[ezi] = __builtin_fmaf(-alpha, u, div_refined(vp, sh.c[jcol]));
    } else {
        const float4 w0 = sh.red[0][ce][2][cc];
        wsum = (w0.x + w0.y) + w0.z;
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            const float4 f2 = sh.red[ww][ce][2][cc];
            wsum += (f2.x + f2.y) + f2.z;
        }
        if (head_pivots) {
            float wp = 0.0f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float4 f1 = sh.red[ww][ce][1][cc];
                const float4 f2 = sh.red[ww][ce][2][cc];
                whole(f1);
                whole(f2);
                wp += (f1.z + f1.w) + f2.w;
            }
            wsum += div_refined(wp, sh.c[jcol]);
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
    const char *ezc = reinterpret_cast<const char *>(&sh.ez[4 * c]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float2 rp = sh.row[g + 16 * m];
        const float *E = reinterpret_cast<const float *>(ezc + __float_as_int(rp.y));
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
    const uint32_t mk[3] = {lane_mask(c & 8), lane_mask(c & 4), lane_mask(c & 2)};
    const float rmax = row_max_scatter(amax, mk);
    {
        const int mm = c >> 1;
        const int p = g + 16 * mm;
        const int si = srow_index(g, mm);
        const float sc = sh.srow[si];
        const float qb = sh.qbrow[si];
        float rn = 0.0f, mul = 0.0f;
        if (qb != 0.0f) {
            rn = fmaxf(div_refined(fabsf(sc) * rmax, qb), kRowFloor);
            mul = fminf(fmaxf(sc * __builtin_amdgcn_rcpf(rn), -kMulMax), kMulMax);
        }
        if ((c & 1) == 0) {
            rw[p] = rn;
            sh.mul[g][mm] = mul;
            if (REFIT) {
                const float w2 = sh.w2row[si]; // 0 on pivot rows
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
        // formed early (they would hold registers through the stores).  The
        // codes and the refit sums are formed for every row (a pivot row has
        // multiplier 0 and weight 0, so its codes are 0 and add nothing);
        // only the packing depends on the class
        uint32_t bt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bt[e] = __float_as_uint(__builtin_fmaf(z[m][e], mulv[m], kRoundMagic));
        if (REFIT) {
            const float ram = sh.ra[gs][m], rbm = sh.rb[gs][m];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float zq = __uint_as_float(bt[e]) - kRoundMagic; // the code, exactly
                num[e] = __builtin_fmaf(ram * zq, z[m][e], num[e]);
                den[e] = __builtin_fmaf(rbm * zq, zq, den[e]);
            }
        }
        per_slot(L, tab, gs, m, [&](auto KC) __attribute__((always_inline)) {
            constexpr int K = decltype(KC)::value;
            const int p = gs + 16 * m;
            uint8_t *base = seg_out + slot_base<K>(L, m);
            const unsigned off = static_cast<unsigned>(gs * Cls<K>::row);
            if constexpr (K == 0) {
                // X = c_j s y, stored in binary16, four columns at a time
                (void)p;
                const float sc = sh.srow[srow_index(gs, m)];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float4 cq = *reinterpret_cast<const float4 *>(&sh.c[8 * cs_ + 4 * hf]);
                    const int e0 = 4 * hf;
                    const uint32_t lo = half_bits(cq.x * (sc * z[m][e0])) |
                                        (half_bits(cq.y * (sc * z[m][e0 + 1])) << 16);
                    const uint32_t hi = half_bits(cq.z * (sc * z[m][e0 + 2])) |
                                        (half_bits(cq.w * (sc * z[m][e0 + 3])) << 16);
                    *reinterpret_cast<u32x2 *>(base + (off + 16u * cs_ + 8u * hf)) = u32x2{lo, hi};
                }
            } else {
                store_codes<K>(base, off, cs_, bt, lo4);
            }
        });
    }
    if (REFIT) {
        // ---- Table C2 step 5: the column factors refit over the integer rows.
        // Partials per (wave and lane group q, column-offset pair e / 2,
        // chunk c), written 16 bytes and read 8 bytes per lane without bank
        // conflicts
        // (the lane's coordinates formed afresh from its index: keeps the
        // compiler from holding them in registers through the codes)
        int tt = t;
        asm volatile("" : "+v"(tt));
        float4 *red4 = &sh.red[0][0][0][0]; // [16 q][4 e/2][16 c]
        const int q0 = tt >> 4, cq = tt & 15;
#pragma unroll
        for (int e = 0; e < 8; e += 2)
            red4[(q0 * 4 + e / 2) * 16 + cq] = make_float4(num[e], den[e], num[e + 1], den[e + 1]);
        __syncthreads();
        if (tt < D) {
            const int c2 = tt & 15, e2 = ((tt >> 4) + ((tt >> 1) & 6)) & 7; // as in the reduction
            const float2 *red2 = reinterpret_cast<const float2 *>(red4);
            float nsum = 0.0f, dsum = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float2 f = red2[((q * 4 + (e2 >> 1)) * 16 + c2) * 2 + (e2 & 1)];
                nsum += f.x;
                dsum += f.y;
            }
            const int j = 8 * c2 + e2;
            const float cold = sh.c[j];
            a.cs_out[ub * D + j] = dsum > 0.0f ? fmaxf(cold * (nsum / dsum), kRowFloor) : cold;
        }
    }
}

template <typename TIn, bool REFIT, bool GATED>
void launch_one(const DecodeArgs &a, unsigned units, const UnitGeom &ug, hipStream_t s) {
    hipLaunchKernelGGL((decode_alloc128_kernel<TIn, REFIT, GATED>), dim3(units), dim3(256), 0, s, a, ug);
}

template <typename TIn>
void launch_in(const DecodeArgs &a, unsigned units, const UnitGeom &ug, hipStream_t s) {
    const bool refit = a.cs != nullptr;
    const bool gated = a.gate != nullptr;
    if (refit && gated) launch_one<TIn, true, true>(a, units, ug, s);
    else if (refit) launch_one<TIn, true, false>(a, units, ug, s);
    else if (gated) launch_one<TIn, false, true>(a, units, ug, s);
    else launch_one<TIn, false, false>(a, units, ug, s);
}

} // namespace

hipError_t launch_decode_alloc128(bool bf16, const DecodeArgs &a, hipStream_t s) {
    const unsigned units = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    const UnitGeom ug = unit_geom(a);
    if (bf16)
        launch_in<uint16_t>(a, units, ug, s);
    else
        launch_in<float>(a, units, ug, s);
    return hipGetLastError();
}

} // namespace stq
