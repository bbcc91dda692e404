// Ragged row classes: FP16 pivot rows and 8-, 6-, 4-, 2-bit rows per head
// (STEPQuant paper, arXiv 2609.38169: App. C.2 Table C1 for the candidate
// widths and the FP16 pivots; App. C.3 Table C2 for the step with pivots:
// reconstruct pivot rows from FP16, fit the column factors over the non-pivot
// integer rows, store pivot values in FP16).  Also the calibration statistics
// of the lifetime-aware assignment (App. A.3: mean log retention and the
// per-row candidate distortion).
//
// Storage per slot: one byte pool of slot_bytes; head h's rows occupy a
// segment at layout[h][5], in physical order pivots (2D bytes per row), 8-bit
// (D), 6-bit (3D/4: D/2 bytes of low nibbles, then D/4 bytes of 2-bit high
// parts), 4-bit (D/2), 2-bit (D/4, column j in bits 2(j%4) of byte j/4).
// Codes are two's complement; pivot rows have r = 0 and no column factor.
//
// The generic decode kernel here serves d = 16, 32, 64 (128 x 128 heads have
// their own kernel in alloc128.hip).  It uses the lane decomposition of
// decode_mixed_kernel (lane (g, c) owns columns 8c..8c+7 of rows g + (D/8) m)
// and the column-normalised arithmetic x = X / c.  A pivot row enters that arithmetic as z_ij = h_ij /
// c_j with a row factor of 1, so every row class shares the column sums, the
// update and the readout; only loads, the row factor and the stores differ
// per class.  Rows of one head are sorted by class, so a wave diverges only
// at the few row groups that straddle a class boundary.
#include <hip/hip_runtime.h>

#include "stq_internal.h"

namespace stq {
namespace {

constexpr float kRowFloor = 1.17549435082228750797e-38f; // 2^-126
constexpr float kHalfMax = 65504.0f;
constexpr float kRoundMagic = 12582912.0f; // 1.5 * 2^23

template <typename T> struct In;
template <> struct In<float> {
    static __device__ __forceinline__ float get(const void *p, size_t i) {
        return static_cast<const float *>(p)[i];
    }
};
template <> struct In<uint16_t> {
    static __device__ __forceinline__ float get(const void *p, size_t i) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
    }
};

template <int D> struct Geo {
    static constexpr int C8 = D / 8;
    static constexpr int TPU = C8 * C8;
    static constexpr int UPW = 256 / TPU;
};

template <int WIDTH> __device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WIDTH));
    return v;
}

__device__ __forceinline__ float qmax_of(int k) {
    return k == 1 ? 127.0f : (k == 2 ? 31.0f : (k == 3 ? 7.0f : 1.0f));
}

__device__ __forceinline__ float qinv_of(int k) {
    return k == 1 ? (1.0f / 127.0f) : (k == 2 ? (1.0f / 31.0f) : (k == 3 ? (1.0f / 7.0f) : 1.0f));
}

// Where physical row p of a head lives: its class and byte offset within the
// head's segment, from the five class counts.
struct RowPlace {
    int cls;
    int off;
};

template <int D>
__device__ __forceinline__ RowPlace place_row(const int32_t *lay, int p) {
    const int rb[kNumClasses] = {2 * D, D, 3 * D / 4, D / 2, D / 4};
    int start = 0, boff = 0;
    RowPlace rp{kNumClasses - 1, 0};
#pragma unroll
    for (int k = 0; k < kNumClasses; ++k) {
        const int n = lay[k];
        if (p < start + n) {
            rp.cls = k;
            rp.off = boff + (p - start) * rb[k];
            return rp;
        }
        start += n;
        boff += n * rb[k];
    }
    return rp;
}

// Class boundaries of one head, computed once per unit: first physical row
// (s1..s4) and first byte (b1..b4) of classes 1..4 (class 0 starts at 0).
struct HeadLayout {
    int s1, s2, s3, s4;
    int b1, b2, b3, b4;
};

template <int D>
__device__ __forceinline__ HeadLayout head_layout(const int32_t *lay) {
    const int n0 = lay[0], n1 = lay[1], n2 = lay[2], n3 = lay[3];
    HeadLayout L;
    L.s1 = n0;
    L.s2 = L.s1 + n1;
    L.s3 = L.s2 + n2;
    L.s4 = L.s3 + n3;
    L.b1 = n0 * (2 * D);
    L.b2 = L.b1 + n1 * D;
    L.b3 = L.b2 + n2 * (3 * D / 4);
    L.b4 = L.b3 + n3 * (D / 2);
    return L;
}

template <int D>
__device__ __forceinline__ RowPlace place_in(const HeadLayout &L, int p) {
    if (p < L.s1) return RowPlace{0, p * (2 * D)};
    if (p < L.s2) return RowPlace{1, L.b1 + (p - L.s1) * D};
    if (p < L.s3) return RowPlace{2, L.b2 + (p - L.s2) * (3 * D / 4)};
    if (p < L.s4) return RowPlace{3, L.b3 + (p - L.s3) * (D / 2)};
    return RowPlace{4, L.b4 + (p - L.s4) * (D / 4)};
}

// The 8 raw code words of this lane's chunk of one row (layout above).
struct Chunk {
    uint32_t w[4];
};

template <int D>
__device__ __forceinline__ Chunk load_chunk(const uint8_t *row, int cls, int c) {
    Chunk ch{{0u, 0u, 0u, 0u}};
    switch (cls) {
    case 0: {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + 16 * c);
        ch.w[0] = v.x; ch.w[1] = v.y; ch.w[2] = v.z; ch.w[3] = v.w;
        break;
    }
    case 1: {
        const uint2 v = *reinterpret_cast<const uint2 *>(row + 8 * c);
        ch.w[0] = v.x; ch.w[1] = v.y;
        break;
    }
    case 2:
        ch.w[0] = *reinterpret_cast<const uint32_t *>(row + 4 * c);
        ch.w[1] = *reinterpret_cast<const uint16_t *>(row + D / 2 + 2 * c);
        break;
    case 3:
        ch.w[0] = *reinterpret_cast<const uint32_t *>(row + 4 * c);
        break;
    default:
        ch.w[0] = *reinterpret_cast<const uint16_t *>(row + 2 * c);
        break;
    }
    return ch;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b & 0xFFFFu)));
}

// RNE to binary16, saturating at +-65504.
__device__ __forceinline__ uint32_t float_to_half_bits(float x) {
    x = fminf(fmaxf(x, -kHalfMax), kHalfMax);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

// Element e of an integer-class chunk as a signed integer value.
__device__ __forceinline__ float int_code(const Chunk &ch, int cls, int e) {
    switch (cls) {
    case 1: return static_cast<float>(static_cast<int8_t>(ch.w[e >> 2] >> (8 * (e & 3))));
    case 2: {
        const uint32_t u = ((ch.w[0] >> (4 * e)) & 0xFu) | (((ch.w[1] >> (2 * e)) & 0x3u) << 4);
        return static_cast<float>(static_cast<int>(u ^ 32u) - 32);
    }
    case 3: {
        const uint32_t u = (ch.w[0] >> (4 * e)) & 0xFu;
        return static_cast<float>(static_cast<int>(u ^ 8u) - 8);
    }
    default: {
        const uint32_t u = (ch.w[0] >> (2 * e)) & 0x3u;
        return static_cast<float>(static_cast<int>(u ^ 2u) - 2);
    }
    }
}

// Store the codes zq (integer classes) of this lane's chunk.
template <int D>
__device__ __forceinline__ void store_codes(uint8_t *row, int cls, int c, const int (&zq)[8]) {
    switch (cls) {
    case 1: {
        uint2 t;
        t.x = (zq[0] & 0xFF) | ((zq[1] & 0xFF) << 8) | ((zq[2] & 0xFF) << 16) | ((zq[3] & 0xFF) << 24);
        t.y = (zq[4] & 0xFF) | ((zq[5] & 0xFF) << 8) | ((zq[6] & 0xFF) << 16) | ((zq[7] & 0xFF) << 24);
        *reinterpret_cast<uint2 *>(row + 8 * c) = t;
        break;
    }
    case 2: {
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo |= static_cast<uint32_t>(zq[e] & 0xF) << (4 * e);
            hi |= static_cast<uint32_t>((zq[e] >> 4) & 0x3) << (2 * e);
        }
        *reinterpret_cast<uint32_t *>(row + 4 * c) = lo;
        *reinterpret_cast<uint16_t *>(row + D / 2 + 2 * c) = static_cast<uint16_t>(hi);
        break;
    }
    case 3: {
        uint32_t t = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) t |= static_cast<uint32_t>(zq[e] & 0xF) << (4 * e);
        *reinterpret_cast<uint32_t *>(row + 4 * c) = t;
        break;
    }
    default: {
        uint32_t t = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) t |= static_cast<uint32_t>(zq[e] & 0x3) << (2 * e);
        *reinterpret_cast<uint16_t *>(row + 2 * c) = static_cast<uint16_t>(t);
        break;
    }
    }
}

__device__ __forceinline__ void store_half_row(uint8_t *row, int c, const float (&X)[8]) {
    uint4 t;
    t.x = float_to_half_bits(X[0]) | (float_to_half_bits(X[1]) << 16);
    t.y = float_to_half_bits(X[2]) | (float_to_half_bits(X[3]) << 16);
    t.z = float_to_half_bits(X[4]) | (float_to_half_bits(X[5]) << 16);
    t.w = float_to_half_bits(X[6]) | (float_to_half_bits(X[7]) << 16);
    *reinterpret_cast<uint4 *>(row + 16 * c) = t;
}

// ------------------------------------------------------------------ decode --

template <int D, typename TIn, bool REFIT>
__global__ __launch_bounds__(256) void decode_alloc_kernel(DecodeArgs a) {
    using G = Geo<D>;
    constexpr int C8 = G::C8, TPU = G::TPU, UPW = G::UPW;
    __shared__ float s_k[UPW][D];
    __shared__ float s_q[UPW][D];
    __shared__ float s_v[UPW][D];
    __shared__ float s_c[UPW][D];
    __shared__ float s_g[UPW][D];
    __shared__ float s_e[UPW][D];
    __shared__ float s_red[UPW][2][C8][D];
    __shared__ float s_kq[UPW][C8];
    __shared__ float s_w2[REFIT ? UPW : 1][D];

    const int lt = threadIdx.x % TPU;
    const int ul = threadIdx.x / TPU;
    const int c = lt % C8;
    const int g = lt / C8;
    const long unit = static_cast<long>(blockIdx.x) * UPW + ul;
    const bool active = unit < static_cast<long>(a.B) * a.Hv;
    const int b = active ? static_cast<int>(unit / a.Hv) : 0;
    const int h = active ? static_cast<int>(unit % a.Hv) : 0;
    const int hk = h / (a.Hv / a.Hk);
    const int slot = active ? (a.slots ? a.slots[b] : b) : 0;
    const bool live = active && slot >= 0 && slot < a.n_slots;

    const int32_t *lay = a.layout + static_cast<size_t>(h) * kLayoutStride;
    const size_t seg_off = static_cast<size_t>(live ? slot : 0) * static_cast<size_t>(a.slot_bytes) +
                           static_cast<size_t>(lay[kLayoutSegOff]);
    const uint8_t *seg_in = reinterpret_cast<const uint8_t *>(a.pool8) + seg_off;
    uint8_t *seg_out = reinterpret_cast<uint8_t *>(a.pool8_out) + seg_off;
    const size_t ubase = static_cast<size_t>(live ? slot : 0) * a.Hv + h;
    const float *rr = a.r + ubase * D;
    float *rw = a.r_out + ubase * D;

    // Table C2 step 1: fetch this lane's row chunks and row factors.
    const HeadLayout hl = head_layout<D>(lay);
    Chunk ch[8];
    int cls[8];
    int roff[8];
    float rrow[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        const RowPlace pl = place_in<D>(hl, p);
        cls[m] = pl.cls;
        roff[m] = pl.off;
        rrow[m] = 0.0f;
        ch[m] = Chunk{{0u, 0u, 0u, 0u}};
        if (live) {
            rrow[m] = rr[p];
            ch[m] = load_chunk<D>(seg_in + pl.off, pl.cls, c);
        }
    }
    // Stage q, k, gate (physical row order), v and c.
    for (int idx = lt; idx < D; idx += TPU) {
        float kv = 0.0f, qv = 0.0f, vv = 0.0f, cv = 1.0f, wv = 0.0f, gv = 1.0f;
        if (live) {
            const int i = a.perm[static_cast<size_t>(h) * D + idx] & (D - 1);
            const size_t kb = (static_cast<size_t>(b) * a.Hk + hk) * D;
            kv = In<TIn>::get(a.k, kb + i);
            qv = In<TIn>::get(a.q, kb + i);
            vv = In<TIn>::get(a.v, (static_cast<size_t>(b) * a.Hv + h) * D + idx);
            cv = REFIT ? a.cs[ubase * D + idx] : a.c[static_cast<size_t>(h) * D + idx];
            if (a.gate) gv = a.gate[static_cast<size_t>(unit) * D + i];
            if (REFIT) wv = a.w2[static_cast<size_t>(h) * D + i];
        }
        s_k[ul][idx] = kv;
        s_q[ul][idx] = qv;
        s_v[ul][idx] = vv;
        s_c[ul][idx] = cv;
        s_g[ul][idx] = gv;
        if (REFIT) s_w2[ul][idx] = wv;
    }
    __syncthreads();

    float cj[8], cinv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cj[e] = s_c[ul][8 * c + e];
        cinv[e] = __builtin_amdgcn_rcpf(cj[e]);
    }

    // Decode the chunks to the column-normalised domain and accumulate this
    // lane's share of u~ = (D S / c)^T k and w~ = (D S / c)^T q.
    float z[8][8];
    float pu[8], pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pu[e] = 0.0f;
        pw[e] = 0.0f;
    }
    float kqp = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        float scale;
        if (cls[m] == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) z[m][e] = half_bits_to_float(ch[m].w[e >> 1] >> (16 * (e & 1))) * cinv[e];
            scale = 1.0f;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) z[m][e] = int_code(ch[m], cls[m], e);
            scale = rrow[m];
        }
        scale *= s_g[ul][p];
        rrow[m] = scale; // from here on: the factor applied to z
        const float kp = s_k[ul][p];
        const float qp = s_q[ul][p];
        const float rk = scale * kp;
        const float rq = scale * qp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pu[e] = __builtin_fmaf(rk, z[m][e], pu[e]);
            pw[e] = __builtin_fmaf(rq, z[m][e], pw[e]);
        }
        kqp = __builtin_fmaf(kp, qp, kqp);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s_red[ul][0][g][8 * c + e] = pu[e];
        s_red[ul][1][g][8 * c + e] = pw[e];
    }
    if (c == 0) s_kq[ul][g] = kqp;
    __syncthreads();

    // Column phase: e = v / c - a u~ and the readout (Table C2 step 3).  A row
    // gate is already inside the row factors, so the scalar gate is then 1.
    const float alpha = !active ? 0.0f : (a.gate ? 1.0f : a.alpha[unit]);
    const float beta = active ? a.beta[unit] : 0.0f;
    for (int j = lt; j < D; j += TPU) {
        float u = 0.0f, w = 0.0f, kq = 0.0f;
#pragma unroll
        for (int gg = 0; gg < C8; ++gg) {
            u += s_red[ul][0][gg][j];
            w += s_red[ul][1][gg][j];
            kq += s_kq[ul][gg];
        }
        const float cc = s_c[ul][j];
        const float e = __builtin_fmaf(-alpha, u, s_v[ul][j] / cc);
        s_e[ul][j] = e;
        const float ov = cc * __builtin_fmaf(alpha, w, (beta * kq) * e);
        if (live)
            store_o(a, static_cast<size_t>(unit) * D + j, ov);
        else if (active)
            store_o(a, static_cast<size_t>(unit) * D + j, __int_as_float(0x7fc00000));
    }
    __syncthreads();

    // Table C2 steps 2, 4-6: updated entries, row factors, codes, stores.
    float ev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ev[e] = s_e[ul][8 * c + e];
    float num[8], den[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        num[e] = 0.0f;
        den[e] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        const float ar = alpha * rrow[m];
        const float bk = beta * s_k[ul][p];
        float x[8];
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = __builtin_fmaf(ar, z[m][e], bk * ev[e]);
            mx = fmaxf(mx, fabsf(x[e]));
        }
        mx = group_max<C8>(mx); // every lane of a row shares its class
        uint8_t *row = seg_out + roff[m];
        if (cls[m] == 0) {
            float X[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) X[e] = cj[e] * x[e];
            if (live) {
                store_half_row(row, c, X);
                if (c == 0) rw[p] = 0.0f;
            }
            continue;
        }
        // row factor from the row max times fl32(1/q_b); codes by one FMA that
        // adds 1.5 * 2^23 (round half to even into the low mantissa bits)
        const int qbi = static_cast<int>(qmax_of(cls[m]));
        const float rn = fmaxf(mx * qinv_of(cls[m]), kRowFloor);
        const float mul = __builtin_amdgcn_rcpf(rn);
        int zq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int zi = __float_as_int(__builtin_fmaf(x[e], mul, kRoundMagic)) -
                           __float_as_int(kRoundMagic);
            zq[e] = min(max(zi, -qbi), qbi);
        }
        if (REFIT) {
            // sum_i w2 r' z' X = c sum_i (w2 r') z' x, sum_i w2 r'^2 z'^2
            const float wr = s_w2[ul][p] * rn;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float zf = static_cast<float>(zq[e]);
                num[e] = __builtin_fmaf(wr * zf, x[e], num[e]);
                den[e] = __builtin_fmaf((wr * rn) * zf, zf, den[e]);
            }
        }
        if (live) {
            store_codes<D>(row, cls[m], c, zq);
            if (c == 0) rw[p] = rn;
        }
    }
    if (REFIT) {
        // Table C2 step 5: column factors refit over the non-pivot integer rows.
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s_red[ul][0][g][8 * c + e] = num[e];
            s_red[ul][1][g][8 * c + e] = den[e];
        }
        __syncthreads();
        if (live) {
            for (int j = lt; j < D; j += TPU) {
                float ns = 0.0f, ds = 0.0f;
#pragma unroll
                for (int gg = 0; gg < C8; ++gg) {
                    ns += s_red[ul][0][gg][j];
                    ds += s_red[ul][1][gg][j];
                }
                const float cold = s_c[ul][j];
                a.cs_out[ubase * D + j] = ds > 0.0f ? fmaxf(cold * (ns / ds), kRowFloor) : cold;
            }
        }
    }
}

// -------------------------------------------------------- pack / dequant --

template <int D, bool REFIT>
__global__ __launch_bounds__(256) void pack_alloc_kernel(PackArgs a) {
    using G = Geo<D>;
    constexpr int C8 = G::C8, TPU = G::TPU, UPW = G::UPW;
    __shared__ float2 red[REFIT ? UPW * C8 * D : 1];
    const int lt = threadIdx.x % TPU;
    const int ul = threadIdx.x / TPU;
    const int c = lt % C8;
    const int g = lt / C8;
    const long unit = static_cast<long>(blockIdx.x) * UPW + ul;
    const bool active = unit < static_cast<long>(a.B) * a.Hv;
    const int b = active ? static_cast<int>(unit / a.Hv) : 0;
    const int h = active ? static_cast<int>(unit % a.Hv) : 0;
    const int slot = active ? (a.slots ? a.slots[b] : b) : -1;
    const bool live = slot >= 0 && slot < a.n_slots;
    const int32_t *lay = a.layout + static_cast<size_t>(h) * kLayoutStride;
    uint8_t *seg = reinterpret_cast<uint8_t *>(a.pool8) +
                   static_cast<size_t>(live ? slot : 0) * static_cast<size_t>(a.slot_bytes) +
                   static_cast<size_t>(lay[kLayoutSegOff]);
    const size_t ubase = static_cast<size_t>(live ? slot : 0) * a.Hv + h;
    float *rr = a.r + ubase * D;
    const float *S = a.S_in + static_cast<size_t>(live ? unit : 0) * D * D;
    const float *cc = a.c + static_cast<size_t>(h) * D;
    float cj[8], num[8], den[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cj[e] = cc[8 * c + e];
        num[e] = 0.0f;
        den[e] = 0.0f;
    }
#pragma unroll 1
    for (int m = 0; m < 8 && live; ++m) {
        const int p = g + C8 * m;
        const int i = a.perm[static_cast<size_t>(h) * D + p] & (D - 1);
        const RowPlace pl = place_row<D>(lay, p);
        uint8_t *row = seg + pl.off;
        const float4 s0 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c);
        const float4 s1 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c + 4);
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        if (pl.cls == 0) {
            store_half_row(row, c, sv);
            if (c == 0) rr[p] = 0.0f;
            continue;
        }
        float x[8];
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = sv[e] / cj[e];
            mx = fmaxf(mx, fabsf(x[e]));
        }
        mx = group_max<C8>(mx);
        const float qb = qmax_of(pl.cls);
        const float rn = fmaxf(mx / qb, kRowFloor);
        if (c == 0) rr[p] = rn;
        int zq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = rintf(x[e] / rn);
            y = fminf(fmaxf(y, -qb), qb);
            zq[e] = static_cast<int>(y);
        }
        if (REFIT) {
            const float wr = a.w2[static_cast<size_t>(h) * D + i] * rn;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float zf = static_cast<float>(zq[e]);
                num[e] = __builtin_fmaf(wr * zf, sv[e], num[e]);
                den[e] = __builtin_fmaf((wr * rn) * zf, zf, den[e]);
            }
        }
        store_codes<D>(row, pl.cls, c, zq);
    }
    if (REFIT) {
        float2 *ru = red + static_cast<size_t>(ul) * C8 * D;
#pragma unroll
        for (int e = 0; e < 8; ++e) ru[g * D + 8 * c + e] = make_float2(num[e], den[e]);
        __syncthreads();
        if (live) {
            for (int j = lt; j < D; j += TPU) {
                float ns = 0.0f, ds = 0.0f;
                for (int q = 0; q < C8; ++q) {
                    const float2 f = ru[q * D + j];
                    ns += f.x;
                    ds += f.y;
                }
                a.cs[ubase * D + j] = ds > 0.0f ? fmaxf(ns / ds, kRowFloor) : cc[j];
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void dequant_alloc_kernel(PackArgs a) {
    using G = Geo<D>;
    constexpr int C8 = G::C8, TPU = G::TPU, UPW = G::UPW;
    const int lt = threadIdx.x % TPU;
    const int ul = threadIdx.x / TPU;
    const int c = lt % C8;
    const int g = lt / C8;
    const long unit = static_cast<long>(blockIdx.x) * UPW + ul;
    if (unit >= static_cast<long>(a.B) * a.Hv) return; // no barrier below
    const int b = static_cast<int>(unit / a.Hv);
    const int h = static_cast<int>(unit % a.Hv);
    const int slot = a.slots ? a.slots[b] : b;
    if (slot < 0 || slot >= a.n_slots) return;
    const int32_t *lay = a.layout + static_cast<size_t>(h) * kLayoutStride;
    const uint8_t *seg = reinterpret_cast<const uint8_t *>(a.pool8) +
                         static_cast<size_t>(slot) * static_cast<size_t>(a.slot_bytes) +
                         static_cast<size_t>(lay[kLayoutSegOff]);
    const size_t ubase = static_cast<size_t>(slot) * a.Hv + h;
    const float *cc = a.cs ? a.cs + ubase * D : a.c + static_cast<size_t>(h) * D;
    float *S = a.S_out + static_cast<size_t>(unit) * D * D;
#pragma unroll 1
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        const int i = a.perm[static_cast<size_t>(h) * D + p] & (D - 1);
        const RowPlace pl = place_row<D>(lay, p);
        const Chunk ch = load_chunk<D>(seg + pl.off, pl.cls, c);
        const float r = a.r[ubase * D + p];
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (pl.cls == 0)
                y[e] = half_bits_to_float(ch.w[e >> 1] >> (16 * (e & 1)));
            else
                y[e] = (r * cc[8 * c + e]) * int_code(ch, pl.cls, e);
        }
        *reinterpret_cast<float4 *>(S + static_cast<size_t>(i) * D + 8 * c) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4 *>(S + static_cast<size_t>(i) * D + 8 * c + 4) = make_float4(y[4], y[5], y[6], y[7]);
    }
}

// ------------------------------------------------------------ calibration --

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Candidate distortions (App. A.3, KDA reconstruction distortion): one wave
// per (head, row); lanes hold columns j = lane and lane + 64.  For every
// record: the row's absmax against c gives the row factor of each integer
// width, the codes and the reconstruction, and each candidate's squared error
// is accumulated per lane; the FP16 candidate is the binary16 rounding.  The
// quotient, the max, the row factor (rounded once to fp32, as stored) and
// the codes are taken in double, so every rounding decision is the one of
// the definition.  Records are taken in order and the lane sums are reduced
// once at the end, so the result does not depend on scheduling.
template <int D>
__global__ __launch_bounds__(256) void alloc_distortion_kernel(AllocCalArgs a) {
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int row = blockIdx.x * 4 + wave; // (h, i) flattened
    if (row >= a.Hv * D) return;           // whole waves; no barrier below
    const int h = row / D;
    const int i = row % D;
    constexpr int NJ = D > 64 ? 2 : 1;
    double cv[NJ];
    bool on[NJ];
#pragma unroll
    for (int t = 0; t < NJ; ++t) {
        const int j = lane + 64 * t;
        on[t] = j < D;
        cv[t] = on[t] ? static_cast<double>(a.c[static_cast<size_t>(h) * D + j]) : 1.0;
    }
    const double floor_r = static_cast<double>(kRowFloor);
    double acc[kNumClasses] = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (long s = 0; s < a.n_rec; ++s) {
        const float *Srow = a.records + ((static_cast<size_t>(s) * a.Hv + h) * D + i) * D;
        float sv[NJ];
        double xv[NJ];
        double mx = 0.0;
#pragma unroll
        for (int t = 0; t < NJ; ++t) {
            sv[t] = on[t] ? Srow[lane + 64 * t] : 0.0f;
            xv[t] = static_cast<double>(sv[t]) / cv[t];
            mx = fmax(mx, fabs(xv[t]));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off, 64));
#pragma unroll
        for (int t = 0; t < NJ; ++t) {
            if (!on[t]) continue;
            const double S = static_cast<double>(sv[t]);
            const float hsat = fminf(fmaxf(sv[t], -kHalfMax), kHalfMax);
            const double y0 = static_cast<double>(static_cast<_Float16>(hsat));
            acc[0] += (y0 - S) * (y0 - S);
#pragma unroll
            for (int k = 1; k < kNumClasses; ++k) {
                const double qb = static_cast<double>(qmax_of(k));
                double rr = static_cast<double>(static_cast<float>(mx / qb));
                rr = fmax(rr, floor_r);
                double z = rint(xv[t] / rr);
                z = fmin(fmax(z, -qb), qb);
                const double y = (rr * cv[t]) * z;
                acc[k] += (y - S) * (y - S);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kNumClasses; ++k) acc[k] = wave_sum_d(acc[k]);
    if (lane == 0) {
        double *dst = a.dist + static_cast<size_t>(row) * kNumClasses;
#pragma unroll
        for (int k = 0; k < kNumClasses; ++k) dst[k] += acc[k];
    }
}

// Summed log retention per (head, row) (App. A.3, mean log retention): the
// scalar gate gives log(alpha) to every row of its head, the row gate
// log(d_i).  Samples are taken in order by one thread per row.
template <int D>
__global__ __launch_bounds__(128) void alloc_retention_kernel(AllocCalArgs a) {
    const int h = blockIdx.x;
    const int i = threadIdx.x;
    if (i >= D) return;
    double acc = 0.0;
    for (int b = 0; b < a.B; ++b) {
        const size_t bh = static_cast<size_t>(b) * a.Hv + h;
        const float x = a.gate ? a.gate[bh * D + i] : a.alpha[bh];
        acc += log(static_cast<double>(x));
    }
    a.logret[static_cast<size_t>(h) * D + i] += acc;
    if (i == 0) a.nret[h] += static_cast<double>(a.B);
}

// Uniform layout: every row of every head in class k, no pivots.
__global__ void alloc_init_layout_kernel(int32_t *layout, int Hv, int D, int k, int seg) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= Hv) return;
    int32_t *l = layout + static_cast<size_t>(h) * kLayoutStride;
    for (int t = 0; t < kLayoutStride; ++t) l[t] = 0;
    l[k] = D;
    l[kLayoutSegOff] = h * seg;
    l[kLayoutSegBytes] = seg;
    int32_t *desc = layout + static_cast<size_t>(Hv) * kLayoutStride + static_cast<size_t>(h) * kSlotDescWords;
    for (int t = 0; t < kSlotDescWords; ++t) desc[t] = 0;
    if (D == 128) slot_descs_128(l, desc);
}

} // namespace

hipError_t launch_alloc_init_layout(int32_t *layout, int Hv, int D, int k, int seg_bytes,
                                    hipStream_t s) {
    hipLaunchKernelGGL(alloc_init_layout_kernel, dim3((Hv + 63) / 64), dim3(64), 0, s, layout, Hv,
                       D, k, seg_bytes);
    return hipGetLastError();
}

#define STQ_ALLOC_DISPATCH(D, CALL)                         \
    switch (D) {                                            \
    case 16: { constexpr int DD = 16; CALL; } break;        \
    case 32: { constexpr int DD = 32; CALL; } break;        \
    case 64: { constexpr int DD = 64; CALL; } break;        \
    case 128: { constexpr int DD = 128; CALL; } break;      \
    default: return hipErrorInvalidValue;                   \
    }

template <int D> static unsigned alloc_unit_grid(long units) {
    return static_cast<unsigned>((units + Geo<D>::UPW - 1) / Geo<D>::UPW);
}

// The generic decode serves d = 16, 32, 64; 128 x 128 heads go to the
// matrix-core kernel of alloc128.hip.
#define STQ_ALLOC_DISPATCH_SMALL(D, CALL)                   \
    switch (D) {                                            \
    case 16: { constexpr int DD = 16; CALL; } break;        \
    case 32: { constexpr int DD = 32; CALL; } break;        \
    case 64: { constexpr int DD = 64; CALL; } break;        \
    default: return hipErrorInvalidValue;                   \
    }

hipError_t launch_decode_alloc(int D, bool bf16, const DecodeArgs &a, hipStream_t s) {
    if (D == 128) return launch_decode_alloc128(bf16, a, s);
    const long units = static_cast<long>(a.B) * a.Hv;
    const bool refit = a.cs != nullptr;
    if (bf16 && refit) {
        STQ_ALLOC_DISPATCH_SMALL(D, hipLaunchKernelGGL((decode_alloc_kernel<DD, uint16_t, true>),
                                                       dim3(alloc_unit_grid<DD>(units)), dim3(256), 0, s, a));
    } else if (bf16) {
        STQ_ALLOC_DISPATCH_SMALL(D, hipLaunchKernelGGL((decode_alloc_kernel<DD, uint16_t, false>),
                                                       dim3(alloc_unit_grid<DD>(units)), dim3(256), 0, s, a));
    } else if (refit) {
        STQ_ALLOC_DISPATCH_SMALL(D, hipLaunchKernelGGL((decode_alloc_kernel<DD, float, true>),
                                                       dim3(alloc_unit_grid<DD>(units)), dim3(256), 0, s, a));
    } else {
        STQ_ALLOC_DISPATCH_SMALL(D, hipLaunchKernelGGL((decode_alloc_kernel<DD, float, false>),
                                                       dim3(alloc_unit_grid<DD>(units)), dim3(256), 0, s, a));
    }
    return hipGetLastError();
}

hipError_t launch_pack_alloc(int D, const PackArgs &a, hipStream_t s) {
    const long units = static_cast<long>(a.B) * a.Hv;
    if (a.cs) {
        STQ_ALLOC_DISPATCH(D, hipLaunchKernelGGL((pack_alloc_kernel<DD, true>),
                                                 dim3(alloc_unit_grid<DD>(units)), dim3(256), 0, s, a));
    } else {
        STQ_ALLOC_DISPATCH(D, hipLaunchKernelGGL((pack_alloc_kernel<DD, false>),
                                                 dim3(alloc_unit_grid<DD>(units)), dim3(256), 0, s, a));
    }
    return hipGetLastError();
}

hipError_t launch_dequant_alloc(int D, const PackArgs &a, hipStream_t s) {
    const long units = static_cast<long>(a.B) * a.Hv;
    STQ_ALLOC_DISPATCH(D, hipLaunchKernelGGL((dequant_alloc_kernel<DD>),
                                             dim3(alloc_unit_grid<DD>(units)), dim3(256), 0, s, a));
    return hipGetLastError();
}

hipError_t launch_alloc_distortion(int D, const AllocCalArgs &a, hipStream_t s) {
    const unsigned rows = static_cast<unsigned>(a.Hv) * static_cast<unsigned>(D);
    STQ_ALLOC_DISPATCH(D, hipLaunchKernelGGL((alloc_distortion_kernel<DD>), dim3((rows + 3) / 4),
                                             dim3(256), 0, s, a));
    return hipGetLastError();
}

hipError_t launch_alloc_retention(int D, const AllocCalArgs &a, hipStream_t s) {
    STQ_ALLOC_DISPATCH(D, hipLaunchKernelGGL((alloc_retention_kernel<DD>), dim3(a.Hv), dim3(128), 0,
                                             s, a));
    return hipGetLastError();
}

} // namespace stq
