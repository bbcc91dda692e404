// Fused decode step over a packed 4/8-bit recurrent state (gfx950).
//
// Method: STEPQuant paper (arXiv 2609.38169), Sec. 2.1 Eq. (1) with a scalar
// gate D_t = a I, the dual-axis representation S_ij = r_i c_j z_ij of Sec. 4.3,
// the quantizer of Sec. 2.2 and the step order of App. C.3 Table C2:
// reconstruct, update, emit the readout before requantizing, derive the row
// factors, pack, write back.  One read and one write of the packed state.
//
// Work decomposition (one "unit" = one slot x value head, a D x D state):
//   - a unit is served by (D/8)^2 lanes; lane (g, c) owns the 8 columns
//     8c .. 8c+7 of the 8 physical rows p = g + (D/8) m, m = 0..7, so every
//     lane holds 64 state entries in registers for the whole step;
//   - the D/8 lanes sharing g are consecutive and hold complete rows, so the
//     per-row absmax is a reduction across D/8 adjacent lanes;
//   - an 8-bit row chunk is one 8-byte load, a 4-bit row chunk one 4-byte
//     load: both cover the same 8 columns, so the column sums of S^T k and
//     S^T q from both row widths accumulate in the same registers;
//   - column sums are finished through LDS ([g][j] partials, summed over g).
// Arithmetic is arranged in the column-normalised domain x = X / c:
//   u~_j = sum_i r_i k_i z_ij   (= u_j / c_j),   w~_j = sum_i r_i q_i z_ij
//   e_j  = v_j / c_j - a u~_j
//   x_ij = a r_i z_ij + b k_i e_j          (= X_ij / c_j)
//   o_j  = c_j (a w~_j + b (k.q) e_j)      (= sum_i X_ij q_i)
// which is Eq. (1) rearranged; it needs no per-element multiply by c.
// 4-bit codes are widened as 16 z (a sign-extended byte whose high nibble is the
// code) and the factor 1/16 is folded into the per-row multipliers.
// Quantization adds 1.5 * 2^23 inside an FMA: the sum is rounded once to an
// integer with ties to even, and the low mantissa bits are the two's-complement
// code.  The clip of Sec. 2.2 never binds here: |x| <= max|x| and
// r' = fl32(max|x| * fl32(1/q_b)) give |x / r'| <= q_b (1 + 2^-22), which
// rounds to at most q_b.
#include <hip/hip_runtime.h>

#include "stq_internal.h"

namespace stq {
namespace {

constexpr float kRoundMagic = 12582912.0f; // 1.5 * 2^23
constexpr float kRowFloor = 1.17549435082228750797e-38f; // 2^-126

template <typename T> struct In;
template <> struct In<float> {
    static __device__ __forceinline__ float get(const void *p, size_t i) {
        return static_cast<const float *>(p)[i];
    }
};
template <> struct In<uint16_t> { // bf16 bit patterns, widened exactly
    static __device__ __forceinline__ float get(const void *p, size_t i) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
    }
};

__device__ __forceinline__ float sbyte(uint32_t w, int k) {
    return static_cast<float>(static_cast<int8_t>(w >> (8 * k)));
}

// Max across the `width` consecutive lanes of a row group.
template <int WIDTH> __device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WIDTH));
    return v;
}

template <int D> struct Geo {
    static constexpr int C8 = D / 8;       // lanes per row group = column chunks
    static constexpr int TPU = C8 * C8;    // lanes per unit
    static constexpr int UPW = 256 / TPU;  // units per 256-lane workgroup
};

template <int D, typename TIn, bool REFIT>
__global__ __launch_bounds__(256) void decode_mixed_kernel(DecodeArgs a) {
    using G = Geo<D>;
    constexpr int C8 = G::C8, TPU = G::TPU, UPW = G::UPW;
    __shared__ float s_k[UPW][D];      // k in physical row order
    __shared__ float s_q[UPW][D];      // q in physical row order
    __shared__ float s_v[UPW][D];
    __shared__ float s_c[UPW][D];
    __shared__ float s_e[UPW][D];
    __shared__ float s_red[UPW][2][C8][D];
    __shared__ float s_kq[UPW][C8];
    __shared__ float s_w2[REFIT ? UPW : 1][D]; // squared row-impact weights, physical rows
    __shared__ float s_g[UPW][D];      // row gate in physical row order (1 for a scalar gate)

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
    const int n8 = a.n8;

    const size_t ubase = static_cast<size_t>(live ? slot : 0) * a.Hv + h;
    const int8_t *p8 = a.pool8 + ubase * static_cast<size_t>(n8) * D;
    const uint8_t *p4 = a.pool4 + ubase * static_cast<size_t>(D - n8) * (D / 2);
    const float *rr = a.r + ubase * D;
    int8_t *q8 = a.pool8_out + ubase * static_cast<size_t>(n8) * D;
    uint8_t *q4 = a.pool4_out + ubase * static_cast<size_t>(D - n8) * (D / 2);
    float *rw = a.r_out + ubase * D;

    // Table C2 step 1: fetch the packed rows and row factors of this lane.
    uint32_t w0[8], w1[8];
    float rrow[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        w0[m] = 0u;
        w1[m] = 0u;
        rrow[m] = 0.0f;
        if (live) {
            rrow[m] = rr[p];
            if (p < n8) {
                const uint2 t = *reinterpret_cast<const uint2 *>(p8 + static_cast<size_t>(p) * D + 8 * c);
                w0[m] = t.x;
                w1[m] = t.y;
            } else {
                w0[m] = *reinterpret_cast<const uint32_t *>(p4 + static_cast<size_t>(p - n8) * (D / 2) + 4 * c);
            }
        }
    }
    // Stage q, k (permuted to physical row order), v and c in LDS.
    for (int idx = lt; idx < D; idx += TPU) {
        float kv = 0.0f, qv = 0.0f, vv = 0.0f, cv = 1.0f, wv = 0.0f, gv = 1.0f;
        if (live) {
            const int i = a.perm[static_cast<size_t>(h) * D + idx] & (D - 1);
            const size_t kb = (static_cast<size_t>(b) * a.Hk + hk) * D;
            kv = In<TIn>::get(a.k, kb + i);
            qv = In<TIn>::get(a.q, kb + i);
            if (a.gate) gv = a.gate[static_cast<size_t>(unit) * D + i];
            vv = In<TIn>::get(a.v, (static_cast<size_t>(b) * a.Hv + h) * D + idx);
            cv = REFIT ? a.cs[ubase * D + idx] : a.c[static_cast<size_t>(h) * D + idx];
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

    // Widen the codes and accumulate this lane's share of u~ and w~.
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
        const float kp = s_k[ul][p];
        const float qp = s_q[ul][p];
        float scale;
        if (p < n8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[m][e] = sbyte(w0[m], e);
                z[m][4 + e] = sbyte(w1[m], e);
            }
            scale = rrow[m];
        } else {
            const uint32_t hi = w0[m] & 0xF0F0F0F0u;         // odd columns, x16
            const uint32_t lo = (w0[m] << 4) & 0xF0F0F0F0u;  // even columns, x16
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[m][2 * e] = sbyte(lo, e);
                z[m][2 * e + 1] = sbyte(hi, e);
            }
            scale = rrow[m] * 0.0625f;
        }
        // a row gate d_i scales the whole reconstructed row (D S has rows d_i r_i z_i)
        scale *= s_g[ul][p];
        rrow[m] = scale; // from here on: factor applied to the widened code
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

    // Column phase: finish u~, w~ and k.q; emit o (Table C2 step 3) and e.
    // With a row gate the gate is already in the row factors: scalar gate 1.
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
        const float cj = s_c[ul][j];
        const float e = __builtin_fmaf(-alpha, u, s_v[ul][j] / cj);
        s_e[ul][j] = e;
        const float ov = cj * __builtin_fmaf(alpha, w, (beta * kq) * e);
        if (live)
            store_o(a, static_cast<size_t>(unit) * D + j, ov);
        else if (active)
            store_o(a, static_cast<size_t>(unit) * D + j, __int_as_float(0x7fc00000));
    }
    __syncthreads();

    // Table C2 steps 2 and 4: x = X / c, row absmax, new row factors.
    float ev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ev[e] = s_e[ul][8 * c + e];
    float inv[8], rnv[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        const float ar = alpha * rrow[m];
        const float bk = beta * s_k[ul][p];
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = __builtin_fmaf(ar, z[m][e], bk * ev[e]);
            z[m][e] = x;
            mx = fmaxf(mx, fabsf(x));
        }
        mx = group_max<C8>(mx);
        const float qinv = (p < n8) ? (1.0f / 127.0f) : (1.0f / 7.0f);
        const float rn = fmaxf(mx * qinv, kRowFloor);
        inv[m] = __builtin_amdgcn_rcpf(rn);
        rnv[m] = rn;
        if (live && (m % C8) == (c % 8) && c < 8) rw[p] = rn;
    }
    // Table C2 step 6: codes against the stored factor, pack, write in place.
    // With REFIT, also this lane's share of the column refit sums (App. C.1):
    // sum_i w2 r' z' X = c sum_i (w2 r') z' x and sum_i w2 r'^2 z'^2.
    float num[8], den[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        num[e] = 0.0f;
        den[e] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        uint32_t bits[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            bits[e] = __float_as_uint(__builtin_fmaf(z[m][e], inv[m], kRoundMagic));
        if (REFIT) {
            const float wr = s_w2[ul][p] * rnv[m];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float zq = __uint_as_float(bits[e]) - kRoundMagic; // the code, exactly
                num[e] = __builtin_fmaf(wr * zq, z[m][e], num[e]);
                den[e] = __builtin_fmaf((wr * rnv[m]) * zq, zq, den[e]);
            }
        }
        if (!live) continue;
        if (p < n8) {
            uint2 t;
            t.x = (bits[0] & 0xFFu) | ((bits[1] & 0xFFu) << 8) | ((bits[2] & 0xFFu) << 16) | (bits[3] << 24);
            t.y = (bits[4] & 0xFFu) | ((bits[5] & 0xFFu) << 8) | ((bits[6] & 0xFFu) << 16) | (bits[7] << 24);
            *reinterpret_cast<uint2 *>(q8 + static_cast<size_t>(p) * D + 8 * c) = t;
        } else {
            uint32_t t = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) t |= (bits[e] & 0xFu) << (4 * e);
            *reinterpret_cast<uint32_t *>(q4 + static_cast<size_t>(p - n8) * (D / 2) + 4 * c) = t;
        }
    }
    if (REFIT) {
        // Table C2 step 5: refit the column factors to the new codes.
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

// Unquantized comparison path: the same step on an fp32 state (Eq. (1) with
// D_t = a I, or D_t = diag(d) over the key rows), read and written once.
template <int D, typename TIn>
__global__ __launch_bounds__(256) void decode_fp32_kernel(DecodeArgs a) {
    using G = Geo<D>;
    constexpr int C8 = G::C8, TPU = G::TPU, UPW = G::UPW;
    __shared__ float s_k[UPW][D];
    __shared__ float s_q[UPW][D];
    __shared__ float s_v[UPW][D];
    __shared__ float s_e[UPW][D];
    __shared__ float s_red[UPW][2][C8][D];
    __shared__ float s_kq[UPW][C8];
    __shared__ float s_g[UPW][D];      // row gate (1 for a scalar gate)

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
    const float *S = a.s32 + (static_cast<size_t>(live ? slot : 0) * a.Hv + h) * D * D;
    float *Sw = a.s32_out + (static_cast<size_t>(live ? slot : 0) * a.Hv + h) * D * D;

    float s[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int i = g + C8 * m;
        if (live) {
            const float4 x0 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c);
            const float4 x1 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c + 4);
            s[m][0] = x0.x; s[m][1] = x0.y; s[m][2] = x0.z; s[m][3] = x0.w;
            s[m][4] = x1.x; s[m][5] = x1.y; s[m][6] = x1.z; s[m][7] = x1.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) s[m][e] = 0.0f;
        }
    }
    for (int idx = lt; idx < D; idx += TPU) {
        float kv = 0.0f, qv = 0.0f, vv = 0.0f, gv = 1.0f;
        if (live) {
            const size_t kb = (static_cast<size_t>(b) * a.Hk + hk) * D;
            kv = In<TIn>::get(a.k, kb + idx);
            qv = In<TIn>::get(a.q, kb + idx);
            vv = In<TIn>::get(a.v, (static_cast<size_t>(b) * a.Hv + h) * D + idx);
            if (a.gate) gv = a.gate[static_cast<size_t>(unit) * D + idx];
        }
        s_k[ul][idx] = kv;
        s_q[ul][idx] = qv;
        s_v[ul][idx] = vv;
        s_g[ul][idx] = gv;
    }
    __syncthreads();

    float pu[8], pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pu[e] = 0.0f;
        pw[e] = 0.0f;
    }
    float kqp = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int i = g + C8 * m;
        const float kp = s_k[ul][i];
        const float qp = s_q[ul][i];
        const float gk = s_g[ul][i] * kp; // (D S)^T k and (D S)^T q
        const float gq = s_g[ul][i] * qp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pu[e] = __builtin_fmaf(gk, s[m][e], pu[e]);
            pw[e] = __builtin_fmaf(gq, s[m][e], pw[e]);
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
        const float e = __builtin_fmaf(-alpha, u, s_v[ul][j]);
        s_e[ul][j] = e;
        const float ov = __builtin_fmaf(alpha, w, (beta * kq) * e);
        if (live)
            store_o(a, static_cast<size_t>(unit) * D + j, ov);
        else if (active)
            store_o(a, static_cast<size_t>(unit) * D + j, __int_as_float(0x7fc00000));
    }
    __syncthreads();

    float ev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ev[e] = s_e[ul][8 * c + e];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int i = g + C8 * m;
        const float bk = beta * s_k[ul][i];
        const float ad = alpha * s_g[ul][i];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(ad, s[m][e], bk * ev[e]);
        if (live) {
            *reinterpret_cast<float4 *>(Sw + static_cast<size_t>(i) * D + 8 * c) = make_float4(x[0], x[1], x[2], x[3]);
            *reinterpret_cast<float4 *>(Sw + static_cast<size_t>(i) * D + 8 * c + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
    }
}

template <int D>
hipError_t launch_mixed_d(bool bf16, const DecodeArgs &a, hipStream_t s) {
    const long units = static_cast<long>(a.B) * a.Hv;
    const unsigned grid = static_cast<unsigned>((units + Geo<D>::UPW - 1) / Geo<D>::UPW);
    const bool refit = a.cs != nullptr;
    if (bf16 && refit)
        hipLaunchKernelGGL((decode_mixed_kernel<D, uint16_t, true>), dim3(grid), dim3(256), 0, s, a);
    else if (bf16)
        hipLaunchKernelGGL((decode_mixed_kernel<D, uint16_t, false>), dim3(grid), dim3(256), 0, s, a);
    else if (refit)
        hipLaunchKernelGGL((decode_mixed_kernel<D, float, true>), dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((decode_mixed_kernel<D, float, false>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fp32_d(bool bf16, const DecodeArgs &a, hipStream_t s) {
    const long units = static_cast<long>(a.B) * a.Hv;
    const unsigned grid = static_cast<unsigned>((units + Geo<D>::UPW - 1) / Geo<D>::UPW);
    if (bf16)
        hipLaunchKernelGGL((decode_fp32_kernel<D, uint16_t>), dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((decode_fp32_kernel<D, float>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_decode_mixed(int D, bool bf16, const DecodeArgs &a, hipStream_t s) {
    if (D == 128 && decode128_supported(a.n8)) return launch_decode128(a.n8, bf16, a, s);
    switch (D) {
    case 16: return launch_mixed_d<16>(bf16, a, s);
    case 32: return launch_mixed_d<32>(bf16, a, s);
    case 64: return launch_mixed_d<64>(bf16, a, s);
    case 128: return launch_mixed_d<128>(bf16, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_fp32(int D, bool bf16, const DecodeArgs &a, hipStream_t s) {
    switch (D) {
    case 16: return launch_fp32_d<16>(bf16, a, s);
    case 32: return launch_fp32_d<32>(bf16, a, s);
    case 64: return launch_fp32_d<64>(bf16, a, s);
    case 128: return launch_fp32_d<128>(bf16, a, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace stq
