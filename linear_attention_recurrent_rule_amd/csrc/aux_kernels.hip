// Off-the-timed-path kernels of libstq.so (gfx950): pack of a given fp32 state
// (prefill boundary), dequantized read-back, offline calibration, fills, and a
// streaming copy used as the HBM reference.
//
// Method: STEPQuant paper (arXiv 2609.38169) Sec. 2.2 (quantizer), Sec. 4.3
// (S_ij = r_i c_j z_ij), App. C.3 Table C2 (pack step), Sec. 3.2 / Sec. 4.4
// (precision map and scales calibrated offline, fixed across requests) and
// App. A.3 (each batch element of a recorded step is one calibration sample).
// Lane layout per state is the decode kernel's: lane (g, c) of a unit owns
// columns 8c..8c+7 of physical rows g + (D/8) m, m = 0..7.
#include <hip/hip_runtime.h>

#include "stq_internal.h"

namespace stq {
namespace {

constexpr float kRowFloor = 1.17549435082228750797e-38f; // 2^-126

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

template <int WIDTH> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, WIDTH);
    return v;
}

// Pack: x = S / c, r = max(fl32(max|x| / q_b), 2^-126), z = rhe(x / r)
// (Sec. 2.2 and Sec. 4.3; IEEE divisions, this path is not timed).  With
// REFIT, each state's column factors are then refit to its codes (App. C.1
// fixed-code update): c'_j = sum_i w2_i v_ij S_ij / sum_i w2_i v_ij^2 with
// v = r z, summed over the unit's rows through LDS in a fixed order.
template <int D, bool REFIT>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
    using G = Geo<D>;
    constexpr int C8 = G::C8, TPU = G::TPU, UPW = G::UPW;
    __shared__ float2 red[REFIT ? UPW * C8 * D : 1]; // [unit][row group g][column]
    const int lt = threadIdx.x % TPU;
    const int ul = threadIdx.x / TPU;
    const int c = lt % C8;
    const int g = lt / C8;
    const long unit = static_cast<long>(blockIdx.x) * UPW + ul;
    const bool active = unit < static_cast<long>(a.B) * a.Hv;
    const int b = active ? static_cast<int>(unit / a.Hv) : 0;
    const int h = active ? static_cast<int>(unit % a.Hv) : 0;
    const int slot = active ? (a.slots ? a.slots[b] : b) : -1;
    const bool live = slot >= 0 && slot < a.n_slots; // whole units, no early exit
    const int n8 = a.n8;
    const size_t ubase = static_cast<size_t>(live ? slot : 0) * a.Hv + h;
    int8_t *p8 = a.pool8 + ubase * static_cast<size_t>(n8) * D;
    uint8_t *p4 = a.pool4 + ubase * static_cast<size_t>(D - n8) * (D / 2);
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
        const float4 s0 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c);
        const float4 s1 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c + 4);
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        float x[8];
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = sv[e] / cj[e];
            mx = fmaxf(mx, fabsf(x[e]));
        }
        mx = group_max<C8>(mx);
        const bool is8 = p < n8;
        const float qb = is8 ? 127.0f : 7.0f;
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
        if (is8) {
            uint2 t;
            t.x = (zq[0] & 0xFF) | ((zq[1] & 0xFF) << 8) | ((zq[2] & 0xFF) << 16) | ((zq[3] & 0xFF) << 24);
            t.y = (zq[4] & 0xFF) | ((zq[5] & 0xFF) << 8) | ((zq[6] & 0xFF) << 16) | ((zq[7] & 0xFF) << 24);
            *reinterpret_cast<uint2 *>(p8 + static_cast<size_t>(p) * D + 8 * c) = t;
        } else {
            uint32_t t = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) t |= static_cast<uint32_t>(zq[e] & 0xF) << (4 * e);
            *reinterpret_cast<uint32_t *>(p4 + static_cast<size_t>(p - n8) * (D / 2) + 4 * c) = t;
        }
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
__global__ __launch_bounds__(256) void dequant_kernel(PackArgs a) {
    using G = Geo<D>;
    constexpr int C8 = G::C8, TPU = G::TPU, UPW = G::UPW;
    const int lt = threadIdx.x % TPU;
    const int ul = threadIdx.x / TPU;
    const int c = lt % C8;
    const int g = lt / C8;
    const long unit = static_cast<long>(blockIdx.x) * UPW + ul;
    if (unit >= static_cast<long>(a.B) * a.Hv) return;
    const int b = static_cast<int>(unit / a.Hv);
    const int h = static_cast<int>(unit % a.Hv);
    const int slot = a.slots ? a.slots[b] : b;
    float *S = a.S_out + static_cast<size_t>(unit) * D * D;
    const bool live = slot >= 0 && slot < a.n_slots;
    const int n8 = a.n8;
    const size_t ubase = static_cast<size_t>(live ? slot : 0) * a.Hv + h;
    const int8_t *p8 = a.pool8 + ubase * static_cast<size_t>(n8) * D;
    const uint8_t *p4 = a.pool4 + ubase * static_cast<size_t>(D - n8) * (D / 2);
    const float *rr = a.r + ubase * D;
    const float *cc = a.cs ? a.cs + ubase * D : a.c + static_cast<size_t>(h) * D;
#pragma unroll 1
    for (int m = 0; m < 8; ++m) {
        const int p = g + C8 * m;
        const int i = a.perm[static_cast<size_t>(h) * D + p] & (D - 1);
        float x[8];
        if (!live) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __int_as_float(0x7fc00000);
        } else {
            int zq[8];
            if (p < n8) {
                const uint2 t = *reinterpret_cast<const uint2 *>(p8 + static_cast<size_t>(p) * D + 8 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zq[e] = static_cast<int8_t>(t.x >> (8 * e));
                    zq[4 + e] = static_cast<int8_t>(t.y >> (8 * e));
                }
            } else {
                const uint32_t t = *reinterpret_cast<const uint32_t *>(p4 + static_cast<size_t>(p - n8) * (D / 2) + 4 * c);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int nib = static_cast<int>((t >> (4 * e)) & 0xFu);
                    zq[e] = nib >= 8 ? nib - 16 : nib;
                }
            }
            const float rp = rr[p];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (rp * cc[8 * c + e]) * static_cast<float>(zq[e]);
        }
        *reinterpret_cast<float4 *>(S + static_cast<size_t>(i) * D + 8 * c) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4 *>(S + static_cast<size_t>(i) * D + 8 * c + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
}

// FP32 format: move whole states between a dense [B][Hv][D][D] buffer and the
// slots of the state pool.
template <int D>
__global__ __launch_bounds__(256) void copy_slots_kernel(PackArgs a, float *s32, int to_state) {
    const long unit = blockIdx.x;
    const int b = static_cast<int>(unit / a.Hv);
    const int h = static_cast<int>(unit % a.Hv);
    const int slot = a.slots ? a.slots[b] : b;
    const bool live = slot >= 0 && slot < a.n_slots;
    float4 *pool = reinterpret_cast<float4 *>(s32 + (static_cast<size_t>(live ? slot : 0) * a.Hv + h) * D * D);
    if (to_state) {
        if (!live) return;
        const float4 *src = reinterpret_cast<const float4 *>(a.S_in + static_cast<size_t>(unit) * D * D);
        for (int t = threadIdx.x; t < D * D / 4; t += blockDim.x) pool[t] = src[t];
    } else {
        float4 *dst = reinterpret_cast<float4 *>(a.S_out + static_cast<size_t>(unit) * D * D);
        const float nan = __int_as_float(0x7fc00000);
        for (int t = threadIdx.x; t < D * D / 4; t += blockDim.x)
            dst[t] = live ? pool[t] : make_float4(nan, nan, nan, nan);
    }
}

// Calibration statistics.  Workgroup (h, chunk) folds records chunk,
// chunk + kCalChunks, ... of head h into one partial per column (max |S|) and
// per row (sum of S^2, per record in fp32, across records in fp64).  The
// partials are combined afterwards in chunk order, so results are independent
// of scheduling.
template <int D>
__global__ __launch_bounds__(256) void calib_partial_kernel(CalibArgs a) {
    constexpr int C8 = D / 8, TPU = C8 * C8;
    __shared__ float s_col[256 / C8 > 0 ? 256 / C8 : 1][D];
    const int h = blockIdx.x / kCalChunks;
    const int chunk = blockIdx.x % kCalChunks;
    const int t = threadIdx.x;
    // lanes beyond one unit's worth (D < 128) take further records in parallel
    const int sub = t / TPU;              // record sub-slot within the workgroup
    constexpr int SUBS = 256 / TPU;
    const int lt = t % TPU;
    const int c = lt % C8;
    const int g = lt / C8;
    float cmax[8];
    double racc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cmax[e] = 0.0f;
        racc[e] = 0.0;
    }
    for (int64_t rec = chunk + static_cast<int64_t>(sub) * kCalChunks; rec < a.n_rec;
         rec += static_cast<int64_t>(kCalChunks) * SUBS) {
        const float *S = a.records + (static_cast<size_t>(rec) * a.Hv + h) * D * D;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int i = g + C8 * m;
            const float4 s0 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c);
            const float4 s1 = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(i) * D + 8 * c + 4);
            const float x[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            float sq = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                cmax[e] = fmaxf(cmax[e], fabsf(x[e]));
                sq = __builtin_fmaf(x[e], x[e], sq);
            }
            sq = group_sum<C8>(sq);
            racc[m] += static_cast<double>(sq);
        }
    }
    // rows: lanes with c == 0 hold each row's total over this lane's records;
    // combine the sub-slots in order through LDS (fp64 via two passes of fp32
    // would lose bits, so sub-slots are combined sequentially in a loop).
    __shared__ double s_row[SUBS][D];
    if (c == 0) {
#pragma unroll
        for (int m = 0; m < 8; ++m) s_row[sub][g + C8 * m] = racc[m];
    }
    // columns: max over the 8 rows of this lane is in cmax; fold over g
#pragma unroll
    for (int e = 0; e < 8; ++e) s_col[t / C8][8 * c + e] = cmax[e];
    __syncthreads();
    for (int j = t; j < D; j += 256) {
        float mx = 0.0f;
        for (int r = 0; r < 256 / C8; ++r) mx = fmaxf(mx, s_col[r][j]);
        a.colpart[(static_cast<size_t>(h) * kCalChunks + chunk) * D + j] = mx;
        double acc = 0.0;
        for (int sidx = 0; sidx < SUBS; ++sidx) acc += s_row[sidx][j];
        a.rowpart[(static_cast<size_t>(h) * kCalChunks + chunk) * D + j] = acc;
    }
}

// Fold the chunk partials into the running statistics (chunk order), then, if
// asked, finalize: c = colmax (0 -> 1); row i is 8-bit when fewer than n8 rows
// beat it (higher score, or equal score and lower index); perm = 8-bit rows
// ascending, then 4-bit rows ascending.
template <int D>
__global__ __launch_bounds__(D) void calib_fold_kernel(CalibArgs a, int fold, int finalize) {
    __shared__ double s_score[D];
    __shared__ int s_sel[D];
    const int h = blockIdx.x;
    const int j = threadIdx.x;
    const size_t hj = static_cast<size_t>(h) * D + j;
    if (fold) {
        if (a.do_cols) {
            float mx = a.colmax[hj];
            for (int ch = 0; ch < kCalChunks; ++ch)
                mx = fmaxf(mx, a.colpart[(static_cast<size_t>(h) * kCalChunks + ch) * D + j]);
            a.colmax[hj] = mx;
        }
        if (a.do_rows) {
            double acc = 0.0;
            for (int ch = 0; ch < kCalChunks; ++ch)
                acc += a.rowpart[(static_cast<size_t>(h) * kCalChunks + ch) * D + j];
            a.rowscore[hj] += acc;
        }
    }
    if (!finalize) return;
    const float cm = a.colmax[hj];
    a.c[hj] = cm > 0.0f ? cm : 1.0f;
    s_score[j] = a.rowscore[hj];
    __syncthreads();
    const double mine = s_score[j];
    int beaten = 0;
    for (int i = 0; i < D; ++i) {
        const double o = s_score[i];
        beaten += (o > mine || (o == mine && i < j)) ? 1 : 0;
    }
    const int sel = beaten < a.n8 ? 1 : 0;
    s_sel[j] = sel;
    __syncthreads();
    int pos = 0;
    if (sel) {
        for (int i = 0; i < j; ++i) pos += s_sel[i];
    } else {
        int before = 0;
        for (int i = 0; i < j; ++i) before += 1 - s_sel[i];
        pos = a.n8 + before;
    }
    if (a.perm) a.perm[static_cast<size_t>(h) * D + pos] = j; // no perm: column factors only
}

__global__ void fill_u32_kernel(uint32_t *dst, size_t n, uint32_t value) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = value;
}

__global__ void fill_u64_kernel(uint64_t *dst, size_t n, uint64_t value) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = value;
}

__global__ void iota_rows_kernel(int32_t *perm, int rows, int D) {
    const size_t n = static_cast<size_t>(rows) * D;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        perm[i] = static_cast<int32_t>(i % D);
}

// Streaming copy: one 16-byte word per lane, one 4 KiB tile per workgroup
// (the fastest of the plain copy shapes measured on gfx950).
// A streaming copy with non-temporal loads and stores (the faster of the two
// on this part: about 6.4 TB/s against 6.0 TB/s for cached accesses).
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void copy_kernel(const u32x4v *__restrict__ src,
                                                   u32x4v *__restrict__ dst, size_t n) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Row impact (Sec. 4.1; App. C.1 with the scalar gate): one workgroup per
// value head walks the B samples in order; lane i accumulates
// g_i^2 = (alpha (q_i - beta k_i k.q))^2 in double, with k.q reduced in a
// fixed tree, so the sums do not depend on scheduling.
template <typename T> __device__ __forceinline__ float load_in(const void *p, size_t i);
template <> __device__ __forceinline__ float load_in<float>(const void *p, size_t i) {
    return static_cast<const float *>(p)[i];
}
template <> __device__ __forceinline__ float load_in<uint16_t>(const void *p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
}

__device__ __forceinline__ double block_sum128(double v, double *tmp) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
    __syncthreads();
    const double s = tmp[0] + tmp[1];
    __syncthreads();
    return s;
}

template <int D, typename TIn>
__global__ __launch_bounds__(128) void impact_accumulate_kernel(ImpactArgs a) {
    __shared__ double tmp[2];
    const int h = blockIdx.x;
    const int i = threadIdx.x;
    const int hk = h / (a.Hv / a.Hk);
    double acc = 0.0;
    for (int b = 0; b < a.B; ++b) {
        const size_t base = (static_cast<size_t>(b) * a.Hk + hk) * D;
        const double qi = i < D ? static_cast<double>(load_in<TIn>(a.q, base + i)) : 0.0;
        const double ki = i < D ? static_cast<double>(load_in<TIn>(a.k, base + i)) : 0.0;
        const double kq = block_sum128(ki * qi, tmp);
        // scalar gate, or the row gate d_i of the KDA form (App. C.1: g_i = d_i (q_i - b k_i k.q))
        const double al = a.gate ? (i < D ? static_cast<double>(a.gate[(static_cast<size_t>(b) * a.Hv + h) * D + i]) : 0.0)
                                 : static_cast<double>(a.alpha[static_cast<size_t>(b) * a.Hv + h]);
        const double be = a.beta[static_cast<size_t>(b) * a.Hv + h];
        const double g = al * (qi - be * ki * kq);
        acc += g * g;
    }
    if (i < D) a.impact[static_cast<size_t>(h) * D + i] += acc;
}

// w2_i = fl32((impact_i / mean impact)^(1/4)), floored at 2^-32; an all-zero
// head gets 1 (App. B.3: the row factor scales as impact^(1/8)).
template <int D>
__global__ __launch_bounds__(128) void impact_finalize_kernel(ImpactArgs a) {
    __shared__ double tmp[2];
    const int h = blockIdx.x;
    const int i = threadIdx.x;
    const double om = i < D ? a.impact[static_cast<size_t>(h) * D + i] : 0.0;
    const double mean = block_sum128(om, tmp) / D;
    if (i < D) {
        float w = 1.0f;
        if (mean > 0.0) {
            w = static_cast<float>(sqrt(sqrt(om / mean)));
            w = fmaxf(w, 2.3283064365386963e-10f); // 2^-32
        }
        a.w2[static_cast<size_t>(h) * D + i] = w;
    }
}

unsigned grid_for(size_t n, unsigned cap = 4096) {
    size_t g = (n + 255) / 256;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return static_cast<unsigned>(g);
}

template <int D> unsigned unit_grid(long units) {
    return static_cast<unsigned>((units + Geo<D>::UPW - 1) / Geo<D>::UPW);
}

} // namespace

#define STQ_DISPATCH_D(D, CALL)          \
    switch (D) {                         \
    case 16: { constexpr int DD = 16; CALL; } break;   \
    case 32: { constexpr int DD = 32; CALL; } break;   \
    case 64: { constexpr int DD = 64; CALL; } break;   \
    case 128: { constexpr int DD = 128; CALL; } break; \
    default: return hipErrorInvalidValue; \
    }

hipError_t launch_pack(int D, const PackArgs &a, hipStream_t s) {
    const long units = static_cast<long>(a.B) * a.Hv;
    if (a.cs) {
        STQ_DISPATCH_D(D, hipLaunchKernelGGL((pack_kernel<DD, true>), dim3(unit_grid<DD>(units)), dim3(256), 0, s, a));
    } else {
        STQ_DISPATCH_D(D, hipLaunchKernelGGL((pack_kernel<DD, false>), dim3(unit_grid<DD>(units)), dim3(256), 0, s, a));
    }
    return hipGetLastError();
}

hipError_t launch_impact_accumulate(int D, bool bf16, const ImpactArgs &a, hipStream_t s) {
    if (bf16) {
        STQ_DISPATCH_D(D, hipLaunchKernelGGL((impact_accumulate_kernel<DD, uint16_t>), dim3(a.Hv), dim3(128), 0, s, a));
    } else {
        STQ_DISPATCH_D(D, hipLaunchKernelGGL((impact_accumulate_kernel<DD, float>), dim3(a.Hv), dim3(128), 0, s, a));
    }
    return hipGetLastError();
}

hipError_t launch_impact_finalize(int D, const ImpactArgs &a, hipStream_t s) {
    STQ_DISPATCH_D(D, hipLaunchKernelGGL((impact_finalize_kernel<DD>), dim3(a.Hv), dim3(128), 0, s, a));
    return hipGetLastError();
}

hipError_t launch_dequant(int D, const PackArgs &a, hipStream_t s) {
    const long units = static_cast<long>(a.B) * a.Hv;
    STQ_DISPATCH_D(D, hipLaunchKernelGGL((dequant_kernel<DD>), dim3(unit_grid<DD>(units)), dim3(256), 0, s, a));
    return hipGetLastError();
}

hipError_t launch_copy_slots_fp32(int D, const PackArgs &a, bool to_state, float *s32, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(static_cast<long>(a.B) * a.Hv);
    STQ_DISPATCH_D(D, hipLaunchKernelGGL((copy_slots_kernel<DD>), dim3(grid), dim3(256), 0, s, a, s32,
                                         to_state ? 1 : 0));
    return hipGetLastError();
}

hipError_t launch_calib_accumulate(int D, const CalibArgs &a, hipStream_t s) {
    if (a.n_rec <= 0 || (!a.do_cols && !a.do_rows)) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(a.Hv * kCalChunks);
    STQ_DISPATCH_D(D, hipLaunchKernelGGL((calib_partial_kernel<DD>), dim3(grid), dim3(256), 0, s, a));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    STQ_DISPATCH_D(D, hipLaunchKernelGGL((calib_fold_kernel<DD>), dim3(a.Hv), dim3(DD), 0, s, a, 1, 0));
    return hipGetLastError();
}

hipError_t launch_calib_finalize(int D, const CalibArgs &a, hipStream_t s) {
    STQ_DISPATCH_D(D, hipLaunchKernelGGL((calib_fold_kernel<DD>), dim3(a.Hv), dim3(DD), 0, s, a, 0, 1));
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *dst, size_t n, uint32_t value, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n)), dim3(256), 0, s, dst, n, value);
    return hipGetLastError();
}

hipError_t launch_fill_u64(uint64_t *dst, size_t n, uint64_t value, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(grid_for(n)), dim3(256), 0, s, dst, n, value);
    return hipGetLastError();
}

hipError_t launch_iota_rows(int32_t *perm, int rows, int D, hipStream_t s) {
    const size_t n = static_cast<size_t>(rows) * D;
    hipLaunchKernelGGL(iota_rows_kernel, dim3(grid_for(n)), dim3(256), 0, s, perm, rows, D);
    return hipGetLastError();
}

hipError_t launch_copy_bytes(const void *src, void *dst, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const u32x4v *>(src), static_cast<u32x4v *>(dst), n);
    return hipGetLastError();
}

} // namespace stq
