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
//    from LDS: r k and r q (with 16 folded in for 4-bit rows, whose signed
//    nibbles are converted directly to z / 16), and the update in the form
//        x_ij = X_ij / c_j = s_i (P_i z_ij + E_ij)
//    with s_i = b k_i, P_i = a r_i / (b k_i), E_ij = e_j for a row whose b k_i
//    is not negligible next to a r_i, and s_i = 1, P_i = a r_i, E_ij = 0 for a
//    row where |b k_i| <= 2^-64 |a r_i| (then b k_i e_j is below fp32
//    resolution against any non-zero code).  Either way one FMA per entry;
//    the lane picks e or a zero vector per row by its LDS address;
//  * the row absmax over the 16 lanes of a row is a DPP reduce-scatter that
//    leaves row c / 2 in lane c, so each lane derives one row factor and its
//    reciprocal, and each lane takes the 8 multipliers of its rows from the
//    lanes that formed them by DPP row broadcasts (no LDS, no barrier);
//  * codes: one FMA adds 1.5 * 2^23 (round-half-even to an integer in the low
//    mantissa bits), then bytes are gathered with v_perm and nibbles with one
//    shift and one bit-field insert per 8 codes;
//  * the widened codes feed the matrix cores as they are (tile128.h), so the
//    column sums take two products per column offset and no repacking.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tile128.h"

namespace stq {
namespace {

using namespace t128;

// Matrix-core operand A for the column sums: per wave and lane group, six
// rows of 8 words (one per slot), each a bf16 part in its high half: r k
// (hi, mid, lo), r q (hi, mid, lo).  The r k parts are output rows 0-2 of
// the product and the r q parts rows 4-6, so each lane group of the result
// holds one sum's three parts; lanes of the other output rows read one of
// these rows too and their products are not used.
// Every array below is laid out for the LDS banks (tile128.h) as seen by
// the lanes that write it and the lanes that read it.
constexpr int kCoefStride = 52; // words per lane group (6 x 8 used)
struct Smem {
    // coefficient words, group G = 4 w + gl at G * kCoefStride, row r at 8 r,
    // slot m at m: the operand reads (16 bytes per lane) are free of
    // conflicts; the staging writes (16 groups, two slots per half wave)
    // meet two to a bank, which no 16-byte aligned stride avoids
    uint32_t coef[16 * kCoefStride];
    float2 row[D];          // {P, byte offset of E in ez} per physical row
    float srow[D + 8];      // s of row p at p + p / 16
    float w2row[D + 8];     // column refit: w2 of row p at p + p / 16
    float vc[D], c[D];      // v / c and c per column
    float ez[2 * D];        // e, then a zero vector; each as [e/4][c][e%4]
    float4 red[4][8][2][16]; // per wave, column offset e, lane group, chunk c
    float kq[2];
    float ra[16][8], rb[16][8]; // column refit: w2 r' s and w2 r'^2 per row
};

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

    // ---- widen the codes into fp32 registers zb[h][e][s] = code of slot
    // 4h + s in column 8c + e (4-bit codes as z / 16, or as 16 z in a slot
    // that mixes the two widths); column sums
    // u~ = S~^T (r k), w~ = S~^T (r q) on the matrix cores, two 16x16x32 bf16
    // products per column offset e reading those registers as (0, z) pairs
    // (codes are small integers, exact in bf16; the coefficient splits are
    // exact, so only the fp32 accumulation rounds)
    const int w = t >> 6;
    const int gl = (t >> 4) & 3;
    f32x4 zb[2][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int hh = m >> 2, s = m & 3;
        if constexpr (N8 == kRuntimeN8) {
            // the slot's class is wave-uniform (a scalar branch) except in
            // the one slot that straddles n8; there each lane selects, with
            // no branch, the two words whose bytes are its eight codes
            const int k = slot_class(L, m);
            const uint32_t w4 = (c & 1) ? w1[m] : w0[m]; // a 4-bit row's 4 bytes
            if (k == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zb[hh][e][s] = sbyte(w0[m], e);
                    zb[hh][4 + e][s] = sbyte(w1[m], e);
                }
            } else if (k == 0) {
                uint32_t w4h = w4 >> 4;
                asm volatile("" : "+v"(w4h)); // one shift, then byte selects
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zb[hh][2 * e][s] = snib(w4, e);
                    zb[hh][2 * e + 1][s] = snib(w4h, e);
                }
            } else {
                // a 4-bit lane's codes as 16 z, so that one sign-extending
                // byte conversion serves both widths; bytes in column order:
                // lo0 hi0 lo1 hi1 | lo2 hi2 lo3 hi3
                const uint32_t hi = w4 & 0xF0F0F0F0u;        // odd columns
                const uint32_t lo = (w4 << 4) & 0xF0F0F0F0u; // even columns
                const uint32_t own8 = lane_mask(g + 16 * m < L.n8);
                const uint32_t x0 = sel(own8, w0[m], __builtin_amdgcn_perm(hi, lo, 0x05010400u));
                const uint32_t x1 = sel(own8, w1[m], __builtin_amdgcn_perm(hi, lo, 0x07030602u));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zb[hh][e][s] = sbyte(x0, e);
                    zb[hh][4 + e][s] = sbyte(x1, e);
                }
            }
            continue;
        }
        if (m < M8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                zb[hh][e][s] = sbyte(w0[m], e);
                zb[hh][4 + e][s] = sbyte(w1[m], e);
            }
        } else {
            // even columns in the low nibbles, odd columns in the high ones
            // (an opaque copy of the shifted word: otherwise the compiler
            // merges the shift into a bit-field extract per column)
            uint32_t wh = w0[m] >> 4;
            asm volatile("" : "+v"(wh));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                zb[hh][2 * e][s] = snib(w0[m], e);
                zb[hh][2 * e + 1][s] = snib(wh, e);
            }
        }
    }
    {
        // output row c of the product: rows 0-2 the r k parts, 3 and 4 the
        // r q high part, 5 and 6 its other parts, 7-15 the last one (unused)
        const int crow = c < 4 ? c : (c < 7 ? c - 1 : 5);
        const u32x4 *cw = reinterpret_cast<const u32x4 *>(&sh.coef[(4 * w + gl) * kCoefStride + 8 * crow]);
        const u32x4 A[2] = {cw[0], cw[1]};
        // lanes of group 0 receive (u hi, u mid, u lo, -), group 1 (w hi,
        // w mid, w lo, -); two accumulators alternate so a result is stored
        // while the next product is in flight
        auto product = [&](int e) {
            const f32x4 zz[2] = {zb[0][e], zb[1][e]};
            return column_sums(A, zz);
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
    // kept for o.  Lane t takes column 8 cc + ce, cc = t % 16, with ce =
    // (t / 16) % 8 rotated by 2 (cc / 4): the 16 lanes of a row group still
    // read 16 different chunks of the sums, and the 32 lanes of a half wave
    // read v / c and c from 32 different banks
    const int cc = t & 15;
    const int ce = ((t >> 4) + ((t >> 1) & 6)) & 7;
    const int jcol = 8 * cc + ce;
    const int ezi = (ce >> 2) * 64 + cc * 4 + (ce & 3);
    // the three parts of the column's sum in each wave, then the four waves
    float wsum = 0.0f;
    if (t < D) {
        const float4 f0 = sh.red[0][ce][0][cc];
        float u = (f0.x + f0.y) + f0.z;
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            const float4 f = sh.red[ww][ce][0][cc];
            u += (f.x + f.y) + f.z;
        }
        sh.ez[ezi] = __builtin_fmaf(-L.alpha, u, sh.vc[jcol]);
    } else {
        const float4 f0 = sh.red[0][ce][1][cc];
        wsum = (f0.x + f0.y) + f0.z;
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            const float4 f = sh.red[ww][ce][1][cc];
            wsum += (f.x + f.y) + f.z;
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
    const char *ezc = reinterpret_cast<const char *>(&sh.ez[4 * c]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int hh = m >> 2, s = m & 3;
        const float2 rp = sh.row[g + 16 * m];
        const float *E = reinterpret_cast<const float *>(ezc + __float_as_int(rp.y));
        const float4 e0 = *reinterpret_cast<const float4 *>(E);
        const float4 e1 = *reinterpret_cast<const float4 *>(E + 64);
        const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            zb[hh][e][s] = __builtin_fmaf(rp.x, zb[hh][e][s], ev[e]); // x / s
            mx = fmaxf(mx, fabsf(zb[hh][e][s]));
        }
        amax[m] = __float_as_uint(mx);
    }
    const uint32_t mk[3] = {lane_mask(c & 8), lane_mask(c & 4), lane_mask(c & 2)};
    const float rmax = row_max_scatter(amax, mk);
    float mulv[8];
    {
        const int mm = c >> 1;
        const int p = g + 16 * mm;
        const int si = p + mm;
        const float sc = sh.srow[si];
        const float mrow = fabsf(sc) * rmax;
        const bool row8 = N8 == kRuntimeN8 ? p < L.n8 : mm < M8;
        const uint32_t m8 = lane_mask(row8);
        const float rn = fmaxf(div_refined(mrow, self(m8, 127.0f, 7.0f), self(m8, 1.0f / 127.0f, 1.0f / 7.0f)),
                               kRowFloor);
        const float inv = __builtin_amdgcn_rcpf(rn);
        float mul = sc * inv;
        mul = fminf(fmaxf(mul, -kMulMax), kMulMax);
        if ((c & 1) == 0) {
            L.rw[p] = rn;
            if (REFIT) {
                const float w2 = sh.w2row[si];
                sh.ra[g][mm] = (w2 * rn) * sc;
                sh.rb[g][mm] = (w2 * rn) * rn;
            }
        }
        // every lane of the row group takes the 8 multipliers of its rows
        // from the lanes that formed them (row m in lanes 2m and 2m + 1)
        mulv[0] = row_bcast<0>(mul);
        mulv[1] = row_bcast<2>(mul);
        mulv[2] = row_bcast<4>(mul);
        mulv[3] = row_bcast<6>(mul);
        mulv[4] = row_bcast<8>(mul);
        mulv[5] = row_bcast<10>(mul);
        mulv[6] = row_bcast<12>(mul);
        mulv[7] = row_bcast<14>(mul);
    }
    if (REFIT) {
        // the refit factors of a row group are written and read by the 16
        // lanes of that group, inside one wave: a wave-level fence suffices
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- Table C2 step 6: codes against the stored factors, pack, write back
    // column refit partial sums over this lane's 8 rows (REFIT): with
    // x = s y, X = c x and v = r' z', sum_i w2 v X = c sum_i (w2 r' s) z' y
    // and sum_i w2 v^2 = sum_i (w2 r'^2) z'^2
    float num[8], den[8];
    if (REFIT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            num[e] = 0.0f;
            den[e] = 0.0f;
        }
    }
    uint32_t lo4 = 0x0F0F0F0Fu;
    asm volatile("" : "+v"(lo4));
    // codes, refit sums and the packed store of slot m; in the runtime
    // instance the whole body sits inside the width branch (keeps the codes
    // of one slot live at a time)
    // In the run-time split instance the lane's coordinates are formed
    // afresh here (an opaque copy), so that the compiler does not hold the
    // row addresses of the loads through the whole kernel: that instance
    // needs the registers.  The fixed-split instances reuse them.
    int gs = g, cs = c;
    if constexpr (N8 == kRuntimeN8) asm volatile("" : "+v"(gs), "+v"(cs));
    // this lane's first byte in row g of each pool (slot m adds a
    // compile-time offset in the fixed-split instances)
    int8_t *const q8l = L.q8 + (static_cast<unsigned>(gs) * D + 8u * cs);
    uint8_t *const q4l = L.q4 + (static_cast<unsigned>(gs) * (D / 2) + 4u * cs);
    auto emit = [&](int m, auto W8) __attribute__((always_inline)) {
        constexpr bool IS8 = decltype(W8)::value;
        const int hh = m >> 2, s = m & 3;
        uint32_t bt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            bt[e] = __float_as_uint(__builtin_fmaf(zb[hh][e][s], mulv[m], kRoundMagic));
        if (REFIT) {
            // the row's refit factors from LDS slot by slot (holding all eight
            // in registers would cost the kernel a wave of occupancy)
            const float ram = sh.ra[gs][m], rbm = sh.rb[gs][m];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float zq = __uint_as_float(bt[e]) - kRoundMagic; // the code, exactly
                num[e] = __builtin_fmaf(ram * zq, zb[hh][e][s], num[e]);
                den[e] = __builtin_fmaf(rbm * zq, zq, den[e]);
            }
        }
        if constexpr (IS8) {
            __builtin_nontemporal_store(pack_bytes(bt), reinterpret_cast<u32x2 *>(q8l + 16 * m * D));
        } else {
            __builtin_nontemporal_store(pack_nibbles(bt, lo4),
                                        reinterpret_cast<uint32_t *>(q4l + (16 * m - L.n8) * (D / 2)));
        }
    };
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        if constexpr (N8 == kRuntimeN8) {
            const int k = slot_class(L, m);
            if (k == 1) emit(m, std::true_type{});
            else if (k == 0) emit(m, std::false_type{});
            else if (gs + 16 * m < L.n8) emit(m, std::true_type{});
            else emit(m, std::false_type{});
        } else {
            if (m < M8) emit(m, std::true_type{});
            else emit(m, std::false_type{});
        }
    }
    if (REFIT) {
        // ---- Table C2 step 5: the column factors refit to the new codes
        // (App. C.1 fixed-code update).  Partials per (wave and lane group
        // q, column-offset pair e / 2, chunk c) go through the matrix-core
        // reduction buffer, free since the column sums were read: written 16
        // bytes per lane, read 8 bytes per lane, both without bank conflicts.
        // (the lane's coordinates formed afresh from its index: keeps the
        // compiler from holding them in registers through the codes)
        int tt = L.t;
        asm volatile("" : "+v"(tt));
        float4 *red4 = &sh.red[0][0][0][0]; // [16 q][4 e/2][16 c]
        const int q0 = tt >> 4, cq = tt & 15;
#pragma unroll
        for (int e = 0; e < 8; e += 2)
            red4[(q0 * 4 + e / 2) * 16 + cq] = make_float4(num[e], den[e], num[e + 1], den[e + 1]);
        __syncthreads();
        if (tt < D) {
            const int c2 = tt & 15, e2 = ((tt >> 4) + ((tt >> 1) & 6)) & 7; // as above
            const float2 *red2 = reinterpret_cast<const float2 *>(red4);
            float nsum = 0.0f, dsum = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float2 f = red2[((q * 4 + (e2 >> 1)) * 16 + c2) * 2 + (e2 & 1)];
                nsum += f.x;
                dsum += f.y;
            }
            const float cold = sh.c[8 * c2 + e2];
            L.cw[8 * c2 + e2] = dsum > 0.0f ? fmaxf(cold * (nsum / dsum), kRowFloor) : cold;
        }
    }
}

template <int N8, typename TIn, bool REFIT, bool GATED>
__global__ __launch_bounds__(256) void decode128_kernel(DecodeArgs a, UnitGeom ug) {
    static_assert(N8 == kRuntimeN8 || (N8 % 16 == 0 && N8 >= 0 && N8 <= D),
                  "n8 must be a multiple of 16 (or read at run time)");
    __shared__ Smem sh;

    Lane L;
    L.t = threadIdx.x;
    L.c = L.t & 15;
    L.g = L.t >> 4;
    const int t = L.t;
    const unsigned unit = unit_of_block(ug);
    L.unit = unit;
    const int Hv = a.Hv;
    const int b = static_cast<int>(udiv(unit, static_cast<unsigned>(Hv), ug.hv_m));
    const int h = static_cast<int>(unit - static_cast<unsigned>(b) * static_cast<unsigned>(Hv));
    const int hk = static_cast<int>(udiv(static_cast<unsigned>(h), static_cast<unsigned>(ug.G), ug.g_m));
    const int slot = slot_of(a, b);
    prefetch_args(a);
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
    // (each vector's unit-wide offset goes into its base pointer, so that the
    // loads take a scalar base and a small per-lane offset)
    const size_t kb = static_cast<size_t>(b * a.Hk + hk) * D;
    const TIn *kp0 = static_cast<const TIn *>(a.k) + kb;
    const TIn *qp0 = static_cast<const TIn *>(a.q) + kb;
    const int praw = (a.perm + h * D)[tl];
    const float rpv = L.rr[tl];
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
    // ---- Table C2 step 1: issue the loads of this lane's packed rows
    uint32_t w0[8], w1[8];
    load_codes<N8>(L, w0, w1);
    if (lowhalf) {
        // ---- per-row and per-column factors, once per unit
        const int p = t;
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
        const float rp = rpv;
        // 4-bit codes are widened as z / 16, except in the group of four rows
        // that straddles a split which is not a multiple of 4 (16 z there);
        // a row gate scales the whole row
        float f4 = 16.0f;
        if constexpr (N8 == kRuntimeN8)
            if ((n8 & 3) != 0 && (p >> 2) == (n8 >> 2)) f4 = 0.0625f;
        float scale = rp * self(lane_mask(p < n8), 1.0f, f4);
        if (GATED) scale *= __uint_as_float(pick(g0, g1));
        {
            // row p = 4 w + gl + 16 m of wave w, lane group gl, slot m
            uint32_t *cf = &sh.coef[(p & 15) * kCoefStride + (p >> 4)]; // row r at 8 r
            uint32_t h0, h1, h2;
            split3w(scale * kp, h0, h1, h2);
            cf[0] = h0;
            cf[8] = h1;
            cf[16] = h2;
            split3w(scale * qp, h0, h1, h2);
            cf[24] = h0;
            cf[32] = h1;
            cf[40] = h2;
        }
        const float ar = L.alpha * scale;
        const float bk = L.beta * kp;
        // |b k| > 2^-64 |a r| (false when both vanish: then x = 0 * z = 0)
        const uint32_t scaled = lane_mask(fabsf(bk) > fabsf(ar) * kFormTiny);
        sh.row[p] = make_float2(self(scaled, div_refined(ar, bk), ar), __uint_as_float(sel(scaled, 0u, 4u * D)));
        const int si = p + (p >> 4);
        sh.srow[si] = self(scaled, bk, 1.0f);
        if (REFIT) sh.w2row[si] = __uint_as_float(pick(u0, u1));
        const float kq = wave_sum(kp * qp);
        if ((t & 63) == 0) sh.kq[t >> 6] = kq;
    } else {
        // (a use on this side too, so the compiler keeps the two loads ahead
        // of the code loads instead of sinking them into the branch above)
        asm volatile("" ::"v"(praw), "v"(rpv));
        const int j = tl;
        // v / c to within a hair of correct rounding (a row whose update
        // nearly cancels its decayed content amplifies any rounding of e),
        // formed here, where these waves wait for the staging of the others
        sh.vc[j] = div_refined(In<TIn>::cvt(x0), __uint_as_float(x1));
        sh.c[j] = __uint_as_float(x1);
        sh.ez[D + j] = 0.0f;
    }
    __syncthreads();
    finish_unit<N8, REFIT>(a, sh, L, w0, w1);
}

template <int N8, typename TIn, bool REFIT, bool GATED>
void launch_one(const DecodeArgs &a, unsigned units, const UnitGeom &ug, hipStream_t s) {
    hipLaunchKernelGGL((decode128_kernel<N8, TIn, REFIT, GATED>), dim3(units), dim3(256), 0, s, a, ug);
}

template <int N8, typename TIn>
void launch_in(const DecodeArgs &a, unsigned units, const UnitGeom &ug, hipStream_t s) {
    const bool refit = a.cs != nullptr;
    const bool gated = a.gate != nullptr;
    if (refit && gated) launch_one<N8, TIn, true, true>(a, units, ug, s);
    else if (refit) launch_one<N8, TIn, true, false>(a, units, ug, s);
    else if (gated) launch_one<N8, TIn, false, true>(a, units, ug, s);
    else launch_one<N8, TIn, false, false>(a, units, ug, s);
}

template <int N8>
hipError_t launch_n8(bool bf16, const DecodeArgs &a, hipStream_t s) {
    const unsigned units = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hv);
    const UnitGeom ug = unit_geom(a);
    if (bf16)
        launch_in<N8, uint16_t>(a, units, ug, s);
    else
        launch_in<N8, float>(a, units, ug, s);
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
