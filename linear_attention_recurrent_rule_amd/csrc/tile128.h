// Device helpers shared by the two 128 x 128 decode kernels (decode128.hip:
// the fixed 4/8-bit row split; alloc128.hip: the ragged row classes).  Both
// follow the STEPQuant paper (arXiv 2609.38169): Sec. 2.1 Eq. (1) for the
// update, Sec. 2.2 for the symmetric quantizer, Sec. 4.3 for the
// representation S = r_i c_j z_ij, App. C.3 Table C2 for the step order.
//
// Tile: one workgroup of 256 lanes per (slot, head).  Lane (g, c), g = lane
// / 16, c = lane % 16, owns columns 8c..8c+7 of physical rows g + 16 m,
// m = 0..7; wave w = lane / 64 holds rows 4w + gl + 16m (gl = g % 4), and
// every row lies in one 16-lane row group.
//
// Choices made for the vector ALU of gfx950, where fp32 FMA / add / mul and
// the plain bitwise and right-shift operations issue in about half the time
// of conversions, byte permutes, max, left shifts and lane exchanges, and a
// run of VOP2 selects reading one VCC costs several times a select with an
// explicit lane-mask operand:
//  * a widened code is an fp32 register holding a small integer, whose low
//    16 bits are zero: read as two bf16 it is the pair (0, z).  The column
//    sums feed those registers to the matrix cores unchanged, four slots per
//    product, with the row coefficients at the odd K positions and zeros at
//    the even ones, so no code is repacked into bf16;
//  * the exact three-way bf16 splits of the row coefficients are formed with
//    v_cvt_pk_bf16_f32 (round to nearest even) straight into the high half of
//    a 32-bit word, which is the operand word itself;
//  * per-lane selects use a lane mask held in a vector register and a
//    three-input bitwise operation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stq_internal.h"

namespace stq {
namespace t128 {

constexpr int D = 128;
constexpr float kRoundMagic = 12582912.0f;               // 1.5 * 2^23
constexpr float kRowFloor = 1.17549435082228750797e-38f; // 2^-126
constexpr float kMulMax = 1.70141183460469231732e38f;    // 2^127
constexpr float kFormTiny = 5.42101086242752217004e-20f; // 2^-64

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Inputs as raw bits (a load whose result is only moved does not wait for
// it) and their fp32 value.
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

__device__ __forceinline__ float sbyte(uint32_t w, int k) {
    return static_cast<float>(static_cast<int8_t>(w >> (8 * k)));
}
// the signed 4-bit field in bits 8k..8k+3 of w, widened exactly as z / 16:
// one conversion, the byte select folded into it
__device__ __forceinline__ float snib(uint32_t w, int k) {
    return __builtin_amdgcn_cvt_off_f32_i4((w >> (8 * k)) & 0xFFu);
}

// ---- per-lane selects: m is all ones or all zeros in each lane
__device__ __forceinline__ uint32_t lane_mask(bool b) {
    uint32_t m = b ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(m)); // an opaque mask: keeps the select bitwise
    return m;
}
// m ? a : b bit by bit, as one three-input bitwise operation (truth table
// 0xE4 of (S0, S1, S2) = (a, b, m)); written out because the compiler would
// otherwise choose a bit-field insert, which issues at half the rate.
__device__ __forceinline__ uint32_t sel(uint32_t m, uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0xe4" : "=v"(d) : "v"(a), "v"(b), "v"(m));
    return d;
}
__device__ __forceinline__ float self(uint32_t m, float a, float b) {
    return __uint_as_float(sel(m, __float_as_uint(a), __float_as_uint(b)));
}

// n / d to within a hair of correct rounding: the hardware reciprocal r of d
// (about 1 ulp), the quotient q = n r, and one Newton correction of q by its
// exactly computed residual n - d q (Markstein's scheme).  Where a row factor
// or a scaled coefficient ends in a near-cancellation, an ulp more in a
// quotient shows up amplified in the result.
__device__ __forceinline__ float div_refined(float n, float d) {
    const float r = __builtin_amdgcn_rcpf(d);
    const float q = n * r;
    return __builtin_fmaf(__builtin_fmaf(-d, q, n), r, q);
}
// The same with the reciprocal of d supplied (r ~ 1/d to about 1 ulp).
__device__ __forceinline__ float div_refined(float n, float d, float r) {
    const float q = n * r;
    return __builtin_fmaf(__builtin_fmaf(-d, q, n), r, q);
}

// ---- LDS layout.  Measured on gfx950 with the bank-conflict counter: a
// 4-byte access is served a half wave at a time over 32 banks (lanes of one
// half hitting one bank at different addresses serialise); reading whole
// 16-byte entries (or their first 12 bytes) of 16 consecutive entries is
// free of conflicts, while reading one 4- or 8-byte field of such entries
// collides, and any number of lanes may share an address.
//
// Per-row values read by the lane pairs of a row group (row g + 16 mm in
// lanes 2 mm and 2 mm + 1 of group g) and written by one lane per row
// (lane p for row p, so half a wave covers 16 groups and two slots):
// rotating the 8 slots of group g by 2 (g / 4) spreads both over the banks.
__device__ __forceinline__ int srow_index(int g, int mm) {
    return 8 * g + ((mm + 2 * (g >> 2)) & 7);
}

// ---- lane exchange inside 16-lane rows (GFX9 DPP controls)
template <int CTRL> __device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kRowRor8 = 0x128;       // lane l <- lane l^8 within the row
constexpr int kRowHalfMirror = 0x141; // lane l <- lane 7-l within each half row
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kRowMirror = 0x140;     // lane l <- lane 15-l within the row

// The value held by lane N of this lane's 16-lane row (DPP row_newbcast).
template <int N> __device__ __forceinline__ float row_bcast(float v) {
    static_assert(N >= 0 && N < 16, "a row has 16 lanes");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave (valid in every lane).
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

// Row absmax, reduce-scatter over the 16 lanes of a row group: amax[m] is
// the lane's maximum over its 8 entries of slot m (non-negative floats, which
// order like their bit patterns); lane c ends with the maximum of slot c / 2
// over the whole row.  mk[0..2]: lane masks of c & 8, c & 4, c & 2.
__device__ __forceinline__ float row_max_scatter(const uint32_t (&amax)[8], const uint32_t (&mk)[3]) {
    uint32_t r1[4], r2[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t keep = sel(mk[0], amax[k + 4], amax[k]);
        const uint32_t send = sel(mk[0], amax[k], amax[k + 4]);
        r1[k] = max(keep, dpp<kRowRor8>(send));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t keep = sel(mk[1], r1[k + 2], r1[k]);
        const uint32_t send = sel(mk[1], r1[k], r1[k + 2]);
        r2[k] = max(keep, dpp<kRowHalfMirror>(send));
    }
    const uint32_t keep = sel(mk[2], r2[1], r2[0]);
    const uint32_t send = sel(mk[2], r2[0], r2[1]);
    uint32_t v = max(keep, dpp<kQuadXor2>(send));
    v = max(v, dpp<kQuadXor1>(v));
    return __uint_as_float(v);
}

// x rounded to nearest even bf16, placed in the high half of a word whose low
// half is zero (read as two bf16: the pair (0, bf16(x))).
__device__ __forceinline__ uint32_t bf16_word(float x) {
    uint32_t d;
    asm("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(d) : "v"(x));
    return d;
}

// x = hi + mid + lo exactly, each part a bf16 in the high half of its word
// (each step removes the leading 8 significant bits, and the remainders are
// exact fp32 differences).
__device__ __forceinline__ void split3w(float x, uint32_t &w0, uint32_t &w1, uint32_t &w2) {
    w0 = bf16_word(x);
    const float r1 = x - __uint_as_float(w0);
    w1 = bf16_word(r1);
    const float r2 = r1 - __uint_as_float(w1);
    w2 = bf16_word(r2);
}

// Column sums of the wave's 32 rows for one column offset: a holds the lane
// group's coefficient words of slots 0..3 (a[0]) and 4..7 (a[1]) for output
// row c; z[h] the widened codes of slots 4h..4h+3 in this column.
__device__ __forceinline__ f32x4 column_sums(const u32x4 (&a)[2], const f32x4 (&z)[2]) {
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, a[0]), __builtin_bit_cast(bf16x8, z[0]), zero, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, a[1]), __builtin_bit_cast(bf16x8, z[1]), acc, 0, 0, 0);
}

// n / d for a wave-uniform n < 2^31, with m = ceil(2^32 / d) (d >= 2) or
// m = 0 (d = 1): hi(n m) is the quotient or one more.
__device__ __forceinline__ unsigned udiv(unsigned n, unsigned d, unsigned m) {
    // (selects, not branches: the unit's first scalar loads then stay in one
    // block and issue together)
    const unsigned q = m == 0 ? n : __umulhi(n, m);
    return q * d > n ? q - 1 : q;
}

inline unsigned div_magic(unsigned d) {
    return d <= 1 ? 0u : static_cast<unsigned>(((1ull << 32) + d - 1) / d);
}

// Unit geometry computed once on the host: the divisors of the unit index
// and the XCD remap.
struct UnitGeom {
    unsigned hv_m; // div_magic(Hv)
    int G;         // value heads per key head
    unsigned g_m;  // div_magic(G)
    int remap;     // xcd remap on
    unsigned per;  // units per XCD under the remap (units / 8)
};

inline UnitGeom unit_geom(const DecodeArgs &a) {
    const unsigned units = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    UnitGeom u;
    u.hv_m = div_magic(static_cast<unsigned>(a.Hv));
    u.G = a.Hv / a.Hk;
    u.g_m = div_magic(static_cast<unsigned>(u.G));
    u.remap = (units % 8u) == 0u ? 1 : 0;
    u.per = units >> 3;
    return u;
}

// Workgroups are dealt round-robin to the 8 XCDs; with remap each XCD gets a
// contiguous range of units, so value heads sharing a key head (and their
// q, k) meet in the same L2.  (The grid size comes from the host, so no
// scalar load of the launch's dimensions precedes the first address.)
__device__ __forceinline__ unsigned unit_of_block(const UnitGeom &ug) {
    const unsigned x = blockIdx.x;
    return ug.remap ? (x & 7u) * ug.per + (x >> 3) : x;
}

// The state slot of sequence b: slots[b], or b when slots is null.  The load
// is made in either case (from the first word of q, which every decode
// reads, when slots is null), so that it issues with the unit's other scalar
// loads instead of behind a branch.
__device__ __forceinline__ int slot_of(const DecodeArgs &a, int b) {
    const int32_t *sp = a.slots ? a.slots + b : static_cast<const int32_t *>(a.q);
    const int v = *sp;
    return a.slots ? v : b;
}

// The decode arguments that the first addresses of a unit need, read into
// scalar registers together with the slot index: otherwise some are loaded
// only after the test of the slot, one more scalar round trip before the
// first row address.  (Placed after the slot's load: a volatile statement
// ahead of it would make that load a vector-memory one.)
__device__ __forceinline__ void prefetch_args(const DecodeArgs &a) {
    asm volatile("" ::"s"(a.pool8), "s"(a.pool4), "s"(a.r), "s"(a.perm), "s"(a.c), "s"(a.q), "s"(a.k),
                 "s"(a.v), "s"(a.beta), "s"(a.n_slots));
}

// ---- packing of requantized codes.  bt[e] holds fl32(y_e mul + 1.5 * 2^23),
// whose low byte is the code of column e in two's complement.
__device__ __forceinline__ u32x2 pack_bytes(const uint32_t (&bt)[8]) {
    const uint32_t a01 = __builtin_amdgcn_perm(bt[1], bt[0], 0x0C0C0400u);
    const uint32_t a23 = __builtin_amdgcn_perm(bt[3], bt[2], 0x04000C0Cu);
    const uint32_t a45 = __builtin_amdgcn_perm(bt[5], bt[4], 0x0C0C0400u);
    const uint32_t a67 = __builtin_amdgcn_perm(bt[7], bt[6], 0x04000C0Cu);
    return u32x2{a01 | a23, a45 | a67};
}
// Bytes of the even columns (0, 2, 4, 6) and of the odd ones.
__device__ __forceinline__ void even_odd_bytes(const uint32_t (&bt)[8], uint32_t &evn, uint32_t &odd) {
    evn = __builtin_amdgcn_perm(bt[2], bt[0], 0x0C0C0400u) | __builtin_amdgcn_perm(bt[6], bt[4], 0x04000C0Cu);
    odd = __builtin_amdgcn_perm(bt[3], bt[1], 0x0C0C0400u) | __builtin_amdgcn_perm(bt[7], bt[5], 0x04000C0Cu);
}
// Eight 4-bit codes as one word, column e in nibble e (even column low):
// the low nibbles of the even bytes, the high nibbles of the odd bytes moved
// up by four.  lo4 is a register holding 0x0F0F0F0F.
__device__ __forceinline__ uint32_t pack_nibbles(const uint32_t (&bt)[8], uint32_t lo4) {
    uint32_t evn, odd;
    even_odd_bytes(bt, evn, odd);
    return sel(lo4, evn, odd << 4);
}

} // namespace t128
} // namespace stq
