// Internal declarations shared by the C-ABI layer and the HIP kernels of
// libstq.so.  Not installed; the public interface is include/stq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "stq.h"

namespace stq {

// One decode launch: B sequences x Hv value heads, in place on slots[b].
struct DecodeArgs {
    const int8_t *pool8;  // [n_slots][Hv][n8][D]       read
    const uint8_t *pool4; // [n_slots][Hv][D-n8][D/2]   read
    const float *r;       // [n_slots][Hv][D]           read
    int8_t *pool8_out;    // written (equal to the read pointers when in place)
    uint8_t *pool4_out;
    float *r_out;
    const float *s32;     // [n_slots][Hv][D][D]   (FP32 format) read
    float *s32_out;       //                                      written
    const float *c;       // [Hv][D]
    const int32_t *perm;  // [Hv][D]
    const float *cs;      // [n_slots][Hv][D] per-state column factors read
    float *cs_out;        //                  and refit (REFIT format; else null)
    const float *w2;      // [Hv][D] squared row-impact weights, logical rows
    const int32_t *slots; // [B] or nullptr (identity)
    const void *q;        // [B][Hk][D]
    const void *k;        // [B][Hk][D]
    const void *v;        // [B][Hv][D]
    const float *alpha;   // [B][Hv] scalar gate (null when gate is given)
    const float *beta;    // [B][Hv]
    float *o;             // [B][Hv][D] fp32, or bf16 when o_bf16
    int32_t B, Hv, Hk, n8, n_slots;
    const float *gate;    // [B][Hv][D] per-key-row gate, logical rows, or null
    int32_t o_bf16;       // readout written as bf16 (RNE) instead of fp32
    // ragged row classes (ALLOC formats): pool8 / pool8_out are the byte
    // pools [n_slots][slot_bytes]; layout [Hv][kLayoutStride]
    const int32_t *layout;
    int64_t slot_bytes;
};

// Store readout element idx in the requested precision (wave-uniform choice).
__device__ __forceinline__ void store_o(const DecodeArgs &a, size_t idx, float v) {
    if (a.o_bf16) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        const uint32_t h = (v != v) ? 0x7FC0u : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
        reinterpret_cast<uint16_t *>(a.o)[idx] = static_cast<uint16_t>(h);
    } else {
        a.o[idx] = v;
    }
}

// Pack / dequant of B slots.
struct PackArgs {
    int8_t *pool8;
    uint8_t *pool4;
    float *r;
    const float *c;
    const int32_t *perm;
    const int32_t *slots;
    const float *S_in; // pack: [B][Hv][D][D] logical order
    float *S_out;      // dequant: [B][Hv][D][D] logical order
    float *cs;         // REFIT: [n_slots][Hv][D] per-state column factors
                       // (pack writes them, dequant reads them); else null
    const float *w2;   // REFIT: [Hv][D] squared row-impact weights
    int32_t B, Hv, n8, n_slots;
    const int32_t *layout; // ALLOC formats: [Hv][kLayoutStride]; pool8 is the byte pool
    int64_t slot_bytes;
};

// Ragged row classes (ALLOC formats).  Class k = 0..4: FP16 pivot rows and
// 8-, 6-, 4-, 2-bit rows, stored per head in that physical order.  Layout
// table per head: counts of the five classes, then the head's segment offset
// within a slot and the segment size in bytes (a multiple of 16).
constexpr int kNumClasses = 5;
constexpr int kLayoutStride = 8;
constexpr int kLayoutSegOff = 5;
constexpr int kLayoutSegBytes = 6;

// After the [Hv][kLayoutStride] table, the layout buffer holds per head the
// row-chunk load descriptors of the 128 x 128 ragged decode: for each wave w
// (rows 16 m + 4 w .. 16 m + 4 w + 3 in its slot m) and slot m, two words.
//   word 0: the slot's row base, b_k + (16 m - s_k) RB_k, for class k
//           starting at physical row s_k and segment byte b_k (row p of the
//           class at b_k + (p - s_k) RB_k, so lane group g adds g RB_k);
//   word 1: RB_k | k << 9 | shA << 16 | shB << 20 | offB << 24, where lane
//           column group c reads its two 8-byte words at
//           8 ((2c) >> shA) and offB + 8 ((2c) >> shB) past its row;
//           bit 31 set instead when the slot's four rows straddle a class
//           boundary (that slot takes the per-lane path).
// Written with the layout; zero for heads of other sizes.
constexpr int kSlotDescWords = 64;
constexpr int kLayoutWordsPerHead = kLayoutStride + kSlotDescWords;

// Row bytes of class k at head size D (FP16, 8, 6, 4, 2 bits).
__host__ __device__ inline int class_row_bytes_d(int k, int D) {
    return k == 0 ? 2 * D : (k == 1 ? D : (k == 2 ? 3 * D / 4 : (k == 3 ? D / 2 : D / 4)));
}

// The descriptors above for one head with class counts n[0..4] at D = 128.
__host__ __device__ inline void slot_descs_128(const int32_t *n, int32_t *out) {
    constexpr int D = 128;
    int s[kNumClasses], b[kNumClasses];
    s[0] = 0;
    b[0] = 0;
    for (int k = 1; k < kNumClasses; ++k) {
        s[k] = s[k - 1] + n[k - 1];
        b[k] = b[k - 1] + n[k - 1] * class_row_bytes_d(k - 1, D);
    }
    auto cls = [&](int p) { return (p >= s[1]) + (p >= s[2]) + (p >= s[3]) + (p >= s[4]); };
    // per class: shA, shB, offB (pivot: bytes 16c and 16c + 8; 8-bit: 8c;
    // 6-bit: the 8-byte words holding its nibbles and its 2-bit fields;
    // 4-bit and 2-bit: the 8-byte word holding its codes)
    constexpr int shA[kNumClasses] = {0, 1, 2, 2, 3};
    constexpr int shB[kNumClasses] = {0, 1, 3, 2, 3};
    constexpr int offB[kNumClasses] = {8, 0, D / 2, 0, 0};
    for (int w = 0; w < 4; ++w)
        for (int m = 0; m < 8; ++m) {
            const int p0 = 16 * m + 4 * w;
            const int k = cls(p0);
            int32_t *o = out + 2 * (8 * w + m);
            if (cls(p0 + 3) != k) {
                o[0] = 0;
                o[1] = static_cast<int32_t>(0x80000000u);
                continue;
            }
            const int rb = class_row_bytes_d(k, D);
            o[0] = b[k] + (16 * m - s[k]) * rb;
            o[1] = rb | (k << 9) | (shA[k] << 16) | (shB[k] << 20) | (offB[k] << 24);
        }
}

// Offline calibration of the ALLOC formats.
struct AllocCalArgs {
    const float *records; // [n_rec][Hv][D][D] fp32 states, logical rows
    int64_t n_rec;
    int32_t Hv;
    const float *c;       // [Hv][D] column factors the candidates are taken against
    double *dist;         // [Hv][D][kNumClasses] accumulated candidate distortions
    const float *alpha;   // retention: [B][Hv] scalar gate, or
    const float *gate;    //            [B][Hv][D] row gate
    int32_t B;
    double *logret;       // [Hv][D] summed log retention
    double *nret;         // [Hv] number of retention samples
};

// Row-impact calibration of the refit format.
struct ImpactArgs {
    const void *q, *k;    // [B][Hk][D]
    const float *alpha;   // [B][Hv] scalar gate (null when gate is given)
    const float *gate;    // [B][Hv][D] per-key-row gate, logical rows, or null
    const float *beta;    // [B][Hv]
    int32_t B, Hv, Hk;
    double *impact;       // [Hv][D] accumulated
    float *w2;            // [Hv][D]
};

struct CalibArgs {
    const float *records; // [n_rec][Hv][D][D]
    int64_t n_rec;
    int32_t Hv, n8;
    int32_t do_cols, do_rows;
    float *colmax;       // [Hv][D]
    double *rowscore;    // [Hv][D]
    float *colpart;      // [Hv][chunks][D]
    double *rowpart;     // [Hv][chunks][D]
    float *c;            // [Hv][D]
    int32_t *perm;       // [Hv][D], or null: finalize sets the column factors only
};

constexpr int kCalChunks = 64;

// Launchers (return hipSuccess or the launch error).  D in {16, 32, 64, 128}.
hipError_t launch_decode_mixed(int D, bool bf16, const DecodeArgs &a, hipStream_t s);
// 128 x 128 heads: a compile-time row split for n8 a multiple of 16, the
// split read at run time otherwise.
bool decode128_supported(int n8);
hipError_t launch_decode128(int n8, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_fp32(int D, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_pack(int D, const PackArgs &a, hipStream_t s);
hipError_t launch_dequant(int D, const PackArgs &a, hipStream_t s);
hipError_t launch_copy_slots_fp32(int D, const PackArgs &a, bool to_state, float *s32,
                                  hipStream_t s);
hipError_t launch_calib_accumulate(int D, const CalibArgs &a, hipStream_t s);
hipError_t launch_calib_finalize(int D, const CalibArgs &a, hipStream_t s);
hipError_t launch_impact_accumulate(int D, bool bf16, const ImpactArgs &a, hipStream_t s);
hipError_t launch_impact_finalize(int D, const ImpactArgs &a, hipStream_t s);
hipError_t launch_decode_alloc(int D, bool bf16, const DecodeArgs &a, hipStream_t s);
// 128 x 128 heads: matrix-core column sums, per-slot class branches.
hipError_t launch_decode_alloc128(bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_pack_alloc(int D, const PackArgs &a, hipStream_t s);
hipError_t launch_dequant_alloc(int D, const PackArgs &a, hipStream_t s);
hipError_t launch_alloc_distortion(int D, const AllocCalArgs &a, hipStream_t s);
hipError_t launch_alloc_retention(int D, const AllocCalArgs &a, hipStream_t s);
hipError_t launch_alloc_init_layout(int32_t *layout, int Hv, int D, int k, int seg_bytes,
                                    hipStream_t s);
hipError_t launch_fill_u32(uint32_t *dst, size_t n, uint32_t value, hipStream_t s);
hipError_t launch_fill_u64(uint64_t *dst, size_t n, uint64_t value, hipStream_t s);
hipError_t launch_iota_rows(int32_t *perm, int rows, int D, hipStream_t s);
hipError_t launch_copy_bytes(const void *src, void *dst, size_t bytes, hipStream_t s);

// Host side of the lifetime-aware assignment (alloc_host.cpp).  Inputs on the
// host: dist [Hv][D][5], logret [Hv][D], n (retention samples).  Outputs:
// counts [Hv][5] and perm [Hv][D].  Returns false for an infeasible budget or
// a nominal width outside the candidates.
bool assign_rows(int Hv, int D, const double *dist, const double *logret, double n,
                 int horizon, unsigned cand_mask, int nominal, int n_pivot, int32_t *counts,
                 int32_t *perm);

// stq_calibrate with its per-chunk partial results in colpart [Hv][kCalChunks][D]
// and rowpart [Hv][kCalChunks][D] instead of the state's own arrays (both
// device memory, 16-byte aligned).  Defined in stq_api.cpp.
stq_status calibrate_with(stq_state *st, const float *records, int64_t n_rec, uint32_t flags,
                          stq_stream_t stream, float *colpart, double *rowpart);

} // namespace stq
