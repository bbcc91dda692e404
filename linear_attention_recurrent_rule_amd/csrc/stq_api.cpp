// C ABI of libstq.so: argument validation, layout arithmetic and dispatch.
// Every check runs on the host before anything is queued; a rejected call
// leaves the stream untouched.  See include/stq.h for the contract.
#include "stq.h"

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "stq_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr uint32_t kRowFloorBits = 0x00800000u; // 2^-126
constexpr uint32_t kOneBits = 0x3f800000u;      // 1.0f

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_d(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Layout {
    size_t pool8, pool4, r, c, perm, colmax, rowscore, colpart, rowpart, s32, cs, w2, impact,
        layout, dist, logret, nret, total;
    int64_t slot_bytes;
};

bool alloc_format(int32_t fmt) { return fmt == STQ_FMT_ALLOC || fmt == STQ_FMT_ALLOC_REFIT; }
bool refit_format(int32_t fmt) { return fmt == STQ_FMT_REFIT || fmt == STQ_FMT_ALLOC_REFIT; }
bool calibrated_format(int32_t fmt) {
    return fmt == STQ_FMT_MIXED48 || fmt == STQ_FMT_REFIT || alloc_format(fmt);
}

// Row bytes of class k at head size D (FP16, 8, 6, 4, 2 bits).
int64_t class_row_bytes(int k, int64_t D) {
    switch (k) {
    case 0: return 2 * D;
    case 1: return D;
    case 2: return 3 * D / 4;
    case 3: return D / 2;
    default: return D / 4;
    }
}

int class_of_width(int bits) {
    switch (bits) {
    case 8: return 1;
    case 6: return 2;
    case 4: return 3;
    case 2: return 4;
    default: return -1;
    }
}

// Bytes of one slot of an ALLOC byte pool: room for any assignment within
// the integer budget, the pivots and the per-head padding.
int64_t alloc_slot_bytes(const stq_desc *d) {
    const int64_t H = d->n_heads_v, D = d->d_k, P = d->n_pivot, b = d->nominal_bits;
    const int64_t bytes = b * (H * D - P) * D / 8 + 2 * D * P + 16 * H;
    return (bytes + 15) / 16 * 16;
}

// Layout table rows from class counts [Hv][5], then the per-slot load
// descriptors of each head; false if a head's counts are invalid or the
// segments do not fit slot_bytes (sets *space).
bool build_layout(const stq_desc *d, int64_t slot_bytes, const int32_t *counts, int32_t *table,
                  bool *space) {
    const int H = d->n_heads_v, D = d->d_k;
    int64_t off = 0;
    *space = false;
    for (int h = 0; h < H; ++h) {
        int64_t sum = 0, seg = 0;
        for (int k = 0; k < stq::kNumClasses; ++k) {
            const int32_t n = counts[h * stq::kNumClasses + k];
            if (n < 0) return false;
            sum += n;
            seg += n * class_row_bytes(k, D);
        }
        if (sum != D) return false;
        seg = (seg + 15) / 16 * 16;
        int32_t *row = table + static_cast<size_t>(h) * stq::kLayoutStride;
        for (int t = 0; t < stq::kLayoutStride; ++t) row[t] = 0;
        for (int k = 0; k < stq::kNumClasses; ++k) row[k] = counts[h * stq::kNumClasses + k];
        row[stq::kLayoutSegOff] = static_cast<int32_t>(off);
        row[stq::kLayoutSegBytes] = static_cast<int32_t>(seg);
        int32_t *desc = table + static_cast<size_t>(H) * stq::kLayoutStride +
                        static_cast<size_t>(h) * stq::kSlotDescWords;
        for (int t = 0; t < stq::kSlotDescWords; ++t) desc[t] = 0;
        if (D == 128) stq::slot_descs_128(row, desc);
        off += seg;
    }
    if (off > slot_bytes) {
        *space = true;
        return false;
    }
    return true;
}

// Validates a descriptor; fills byte sizes of each region (0 = absent).
stq_status describe(const stq_desc *d, Layout *L) {
    if (!d) return STQ_E_ARG;
    if (d->fmt < STQ_FMT_MIXED48 || d->fmt > STQ_FMT_ALLOC_REFIT) return STQ_E_ARG;
    if (d->n_slots < 1 || d->n_heads_v < 1 || d->n_heads_k < 1) return STQ_E_SHAPE;
    if (d->n_heads_v % d->n_heads_k != 0) return STQ_E_SHAPE;
    if (d->d_k < 1 || d->d_v < 1) return STQ_E_SHAPE;
    if (d->d_k != d->d_v || !supported_d(d->d_k)) return STQ_E_UNSUPPORTED;
    if (calibrated_format(d->fmt) && (d->n8 < 0 || d->n8 > d->d_k)) return STQ_E_SHAPE;
    if (d->fmt == STQ_FMT_INT8ROW && d->n8 != d->d_k) return STQ_E_SHAPE;
    if (alloc_format(d->fmt)) {
        if (d->n8 != 0 || class_of_width(d->nominal_bits) < 0) return STQ_E_SHAPE;
        if (d->n_pivot < 0 || d->n_pivot > d->n_heads_v * d->d_k) return STQ_E_SHAPE;
    } else if (d->nominal_bits != 0 || d->n_pivot != 0) {
        return STQ_E_SHAPE;
    }
    const size_t S = static_cast<size_t>(d->n_slots), H = static_cast<size_t>(d->n_heads_v);
    const size_t D = static_cast<size_t>(d->d_k);
    std::memset(L, 0, sizeof(*L));
    if (alloc_format(d->fmt)) {
        L->slot_bytes = alloc_slot_bytes(d);
        L->pool8 = S * static_cast<size_t>(L->slot_bytes);
        L->r = S * H * D * sizeof(float);
        L->layout = H * stq::kLayoutWordsPerHead * sizeof(int32_t);
        L->dist = H * D * stq::kNumClasses * sizeof(double);
        L->logret = H * D * sizeof(double);
        L->nret = H * sizeof(double);
    } else if (d->fmt != STQ_FMT_FP32) {
        const size_t n8 = static_cast<size_t>(d->n8);
        L->pool8 = S * H * n8 * D;
        L->pool4 = S * H * (D - n8) * (D / 2);
        L->r = S * H * D * sizeof(float);
    } else {
        L->s32 = S * H * D * D * sizeof(float);
    }
    L->c = H * D * sizeof(float);
    L->perm = H * D * sizeof(int32_t);
    if (calibrated_format(d->fmt)) {
        L->colmax = H * D * sizeof(float);
        L->rowscore = H * D * sizeof(double);
        L->colpart = H * stq::kCalChunks * D * sizeof(float);
        L->rowpart = H * stq::kCalChunks * D * sizeof(double);
    }
    if (refit_format(d->fmt)) {
        L->cs = S * H * D * sizeof(float);
        L->w2 = H * D * sizeof(float);
        L->impact = H * D * sizeof(double);
    }
    L->total = round_up(L->pool8) + round_up(L->pool4) + round_up(L->r) + round_up(L->c) +
               round_up(L->perm) + round_up(L->colmax) + round_up(L->rowscore) +
               round_up(L->colpart) + round_up(L->rowpart) + round_up(L->s32) +
               round_up(L->cs) + round_up(L->w2) + round_up(L->impact) + round_up(L->layout) +
               round_up(L->dist) + round_up(L->logret) + round_up(L->nret);
    return STQ_OK;
}

// Re-validates a state handed back by the caller.
stq_status check_state(const stq_state *st) {
    if (!st) return STQ_E_ARG;
    Layout L;
    stq_status e = describe(&st->desc, &L);
    if (e != STQ_OK) return e;
    if (!st->c || !st->perm) return STQ_E_ARG;
    if (st->desc.fmt == STQ_FMT_FP32) {
        if (!st->s32 || !aligned(st->s32, 16)) return STQ_E_ARG;
    } else {
        if (!st->r || !aligned(st->pool8, 16) || !aligned(st->pool4, 16)) return STQ_E_ARG;
        if ((L.pool8 && !st->pool8) || (L.pool4 && !st->pool4)) return STQ_E_ARG;
    }
    if (calibrated_format(st->desc.fmt) &&
        (!st->colmax || !st->rowscore || !st->cal_colpart || !st->cal_rowpart))
        return STQ_E_ARG;
    if (refit_format(st->desc.fmt) && (!st->cs || !st->w2 || !st->impact ||
                                       !aligned(st->cs, 16) || !aligned(st->w2, 16)))
        return STQ_E_ARG;
    if (alloc_format(st->desc.fmt) &&
        (!st->layout || !st->dist || !st->logret || !st->nret || st->slot_bytes != L.slot_bytes))
        return STQ_E_ARG;
    return STQ_OK;
}

stq_status dev(hipError_t e) { return e == hipSuccess ? STQ_OK : STQ_E_DEVICE; }

} // namespace

extern "C" {

int32_t stq_abi_version(void) { return 7; }

const char *stq_status_str(int32_t s) {
    switch (s) {
    case STQ_OK: return "STQ_OK";
    case STQ_E_ARG: return "STQ_E_ARG: null, misaligned or invalid argument";
    case STQ_E_SHAPE: return "STQ_E_SHAPE: inconsistent dimensions";
    case STQ_E_UNSUPPORTED: return "STQ_E_UNSUPPORTED: head dimension not compiled";
    case STQ_E_SPACE: return "STQ_E_SPACE: buffer smaller than stq_state_bytes";
    case STQ_E_STATE: return "STQ_E_STATE: mixed-precision state not calibrated";
    case STQ_E_DEVICE: return "STQ_E_DEVICE: HIP launch or runtime failure";
    default: return "unknown stq_status";
    }
}

size_t stq_state_bytes(const stq_desc *desc) {
    Layout L;
    return describe(desc, &L) == STQ_OK ? L.total : 0;
}

stq_status stq_alloc_state(const stq_desc *desc, void *devp, size_t bytes, stq_stream_t stream,
                           stq_state *out) {
    if (!desc || !out || !devp) return STQ_E_ARG;
    if (!aligned(devp, kAlign)) return STQ_E_ARG;
    Layout L;
    stq_status e = describe(desc, &L);
    if (e != STQ_OK) return e;
    if (bytes < L.total) return STQ_E_SPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *p = static_cast<char *>(devp);
    stq_state st;
    std::memset(&st, 0, sizeof(st));
    st.desc = *desc;
    auto take = [&p](size_t n) -> void * {
        if (n == 0) return nullptr;
        void *q = p;
        p += round_up(n);
        return q;
    };
    st.pool8 = static_cast<int8_t *>(take(L.pool8));
    st.pool4 = static_cast<uint8_t *>(take(L.pool4));
    st.r = static_cast<float *>(take(L.r));
    st.c = static_cast<float *>(take(L.c));
    st.perm = static_cast<int32_t *>(take(L.perm));
    st.colmax = static_cast<float *>(take(L.colmax));
    st.rowscore = static_cast<double *>(take(L.rowscore));
    st.cal_colpart = static_cast<float *>(take(L.colpart));
    st.cal_rowpart = static_cast<double *>(take(L.rowpart));
    st.s32 = static_cast<float *>(take(L.s32));
    st.cs = static_cast<float *>(take(L.cs));
    st.w2 = static_cast<float *>(take(L.w2));
    st.impact = static_cast<double *>(take(L.impact));
    st.layout = static_cast<int32_t *>(take(L.layout));
    st.dist = static_cast<double *>(take(L.dist));
    st.logret = static_cast<double *>(take(L.logret));
    st.nret = static_cast<double *>(take(L.nret));
    st.slot_bytes = L.slot_bytes;
    st.calibrated = calibrated_format(desc->fmt) ? 0 : 1;

    const int D = desc->d_k;
    hipError_t he = hipSuccess;
    auto run = [&he](hipError_t x) {
        if (he == hipSuccess) he = x;
    };
    if (L.pool8) run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.pool8), L.pool8 / 4, 0u, s));
    if (L.pool4) run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.pool4), L.pool4 / 4, 0u, s));
    if (L.r) run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.r), L.r / 4, kRowFloorBits, s));
    run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.c), L.c / 4, kOneBits, s));
    run(stq::launch_iota_rows(st.perm, desc->n_heads_v, D, s));
    if (L.colmax) run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.colmax), L.colmax / 4, 0u, s));
    if (L.rowscore) run(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st.rowscore), L.rowscore / 8, 0u, s));
    if (L.s32) run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.s32), L.s32 / 4, 0u, s));
    if (L.cs) run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.cs), L.cs / 4, kOneBits, s));
    if (L.w2) run(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st.w2), L.w2 / 4, kOneBits, s));
    if (L.impact) run(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st.impact), L.impact / 8, 0u, s));
    if (L.layout) {
        // every row at the nominal width, no pivots, until a layout is chosen
        const int k = class_of_width(desc->nominal_bits);
        const int64_t seg = (D * class_row_bytes(k, D) + 15) / 16 * 16;
        run(stq::launch_alloc_init_layout(st.layout, desc->n_heads_v, D, k, static_cast<int>(seg), s));
        run(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st.dist), L.dist / 8, 0u, s));
        run(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st.logret), L.logret / 8, 0u, s));
        run(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st.nret), L.nret / 8, 0u, s));
    }
    if (he != hipSuccess) return STQ_E_DEVICE;
    *out = st;
    return STQ_OK;
}

stq_status stq_calibrate(stq_state *st, const float *records, int64_t n_rec, uint32_t flags,
                         stq_stream_t stream) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    return stq::calibrate_with(st, records, n_rec, flags, stream, st->cal_colpart,
                               st->cal_rowpart);
}

} // extern "C"

// The body of stq_calibrate with the per-chunk partial results in colpart and
// rowpart (the state's own arrays, or another buffer of the same size).
stq_status stq::calibrate_with(stq_state *st, const float *records, int64_t n_rec,
                               uint32_t flags, stq_stream_t stream, float *colpart,
                               double *rowpart) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    if (!calibrated_format(st->desc.fmt)) return STQ_E_ARG;
    const bool ragged = alloc_format(st->desc.fmt);
    const uint32_t allowed = ragged ? (STQ_CAL_RESET | STQ_CAL_COLS | STQ_CAL_FINALIZE | STQ_CAL_DIST)
                                    : (STQ_CAL_RESET | STQ_CAL_COLS | STQ_CAL_ROWS | STQ_CAL_FINALIZE);
    if (flags & ~allowed) return STQ_E_ARG;
    if (n_rec < 0) return STQ_E_SHAPE;
    const bool accumulate = (flags & (STQ_CAL_COLS | STQ_CAL_ROWS | STQ_CAL_DIST)) != 0;
    if (accumulate && n_rec > 0 && (!records || !aligned(records, 16))) return STQ_E_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = st->desc.d_k, H = st->desc.n_heads_v;
    stq::CalibArgs a;
    a.records = records;
    a.n_rec = n_rec;
    a.Hv = H;
    a.n8 = st->desc.n8;
    a.do_cols = (flags & STQ_CAL_COLS) ? 1 : 0;
    a.do_rows = (flags & STQ_CAL_ROWS) ? 1 : 0;
    a.colmax = st->colmax;
    a.rowscore = st->rowscore;
    a.colpart = colpart;
    a.rowpart = rowpart;
    a.c = st->c;
    a.perm = ragged ? nullptr : st->perm; // ragged: perm comes from stq_allocate
    if (flags & STQ_CAL_RESET) {
        if ((e = dev(stq::launch_fill_u32(reinterpret_cast<uint32_t *>(st->colmax),
                                          static_cast<size_t>(H) * D, 0u, s))) != STQ_OK)
            return e;
        if ((e = dev(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st->rowscore),
                                          static_cast<size_t>(H) * D, 0u, s))) != STQ_OK)
            return e;
        if (ragged) {
            const size_t nd = static_cast<size_t>(H) * D;
            if ((e = dev(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st->dist),
                                              nd * stq::kNumClasses, 0u, s))) != STQ_OK ||
                (e = dev(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st->logret), nd, 0u,
                                              s))) != STQ_OK ||
                (e = dev(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st->nret),
                                              static_cast<size_t>(H), 0u, s))) != STQ_OK)
                return e;
        }
    }
    if ((flags & (STQ_CAL_COLS | STQ_CAL_ROWS)) && n_rec > 0)
        if ((e = dev(stq::launch_calib_accumulate(D, a, s))) != STQ_OK) return e;
    if (flags & STQ_CAL_FINALIZE) {
        if ((e = dev(stq::launch_calib_finalize(D, a, s))) != STQ_OK) return e;
        if (!ragged) st->calibrated = 1; // ragged: stq_allocate completes it
    }
    if ((flags & STQ_CAL_DIST) && n_rec > 0) {
        stq::AllocCalArgs ca{};
        ca.records = records;
        ca.n_rec = n_rec;
        ca.Hv = H;
        ca.c = st->c;
        ca.dist = st->dist;
        if ((e = dev(stq::launch_alloc_distortion(D, ca, s))) != STQ_OK) return e;
    }
    return STQ_OK;
}

extern "C" {

stq_status stq_set_calibration(stq_state *st, const float *c, const int32_t *perm,
                               stq_stream_t stream) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    if (!calibrated_format(st->desc.fmt)) return STQ_E_ARG;
    if (!c || !perm || !aligned(c, 16) || !aligned(perm, 16)) return STQ_E_ARG;
    if (alloc_format(st->desc.fmt)) return STQ_E_ARG; // use stq_set_alloc_layout
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t n = static_cast<size_t>(st->desc.n_heads_v) * st->desc.d_k * 4;
    if ((e = dev(stq::launch_copy_bytes(c, st->c, n, s))) != STQ_OK) return e;
    if ((e = dev(stq::launch_copy_bytes(perm, st->perm, n, s))) != STQ_OK) return e;
    st->calibrated = 1;
    return STQ_OK;
}

namespace {

stq_status calibrate_impact(stq_state *st, const void *q, const void *k, int32_t dtype,
                            const float *alpha, const float *gate, const float *beta, int32_t B,
                            uint32_t flags, stq_stream_t stream) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    if (!refit_format(st->desc.fmt)) return STQ_E_ARG;
    if (flags & ~(STQ_CAL_RESET | STQ_CAL_FINALIZE)) return STQ_E_ARG;
    if (B < 0) return STQ_E_SHAPE;
    if (dtype != STQ_F32 && dtype != STQ_BF16) return STQ_E_ARG;
    const size_t el = dtype == STQ_F32 ? 4 : 2;
    const float *g_or_a = gate ? gate : alpha;
    if (B > 0 && (!q || !k || !g_or_a || !beta || !aligned(q, el) || !aligned(k, el) ||
                  !aligned(g_or_a, 4) || !aligned(beta, 4)))
        return STQ_E_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = st->desc.d_k, H = st->desc.n_heads_v;
    stq::ImpactArgs a;
    a.q = q;
    a.k = k;
    a.alpha = gate ? nullptr : alpha;
    a.gate = gate;
    a.beta = beta;
    a.B = B;
    a.Hv = H;
    a.Hk = st->desc.n_heads_k;
    a.impact = st->impact;
    a.w2 = st->w2;
    if (flags & STQ_CAL_RESET)
        if ((e = dev(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st->impact),
                                          static_cast<size_t>(H) * D, 0u, s))) != STQ_OK)
            return e;
    if (B > 0)
        if ((e = dev(stq::launch_impact_accumulate(D, dtype == STQ_BF16, a, s))) != STQ_OK) return e;
    if (flags & STQ_CAL_FINALIZE)
        if ((e = dev(stq::launch_impact_finalize(D, a, s))) != STQ_OK) return e;
    return STQ_OK;
}

} // namespace

stq_status stq_calibrate_impact(stq_state *st, const void *q, const void *k, int32_t dtype,
                                const float *alpha, const float *beta, int32_t B, uint32_t flags,
                                stq_stream_t stream) {
    return calibrate_impact(st, q, k, dtype, alpha, nullptr, beta, B, flags, stream);
}

stq_status stq_calibrate_impact_gated(stq_state *st, const void *q, const void *k, int32_t dtype,
                                      const float *gate, const float *beta, int32_t B,
                                      uint32_t flags, stq_stream_t stream) {
    if (B > 0 && !gate) return STQ_E_ARG;
    return calibrate_impact(st, q, k, dtype, nullptr, gate, beta, B, flags, stream);
}

namespace {

stq_status batch_args(const stq_state *st, const int32_t *slots, int32_t B) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    if (B < 1 || B > st->desc.n_slots) return STQ_E_SHAPE;
    if (slots && !aligned(slots, 4)) return STQ_E_ARG;
    return STQ_OK;
}

// Debug check of the slot precondition, enabled by setting STQ_CHECK_SLOTS in
// the environment: the slot list is copied to the host (which synchronises
// the stream) and a slot in range that appears twice is rejected.
stq_status check_slots_distinct(const int32_t *slots, int32_t B, int32_t n_slots,
                                hipStream_t stream) {
    if (!slots || std::getenv("STQ_CHECK_SLOTS") == nullptr) return STQ_OK;
    std::vector<int32_t> h(static_cast<size_t>(B));
    if (hipMemcpyAsync(h.data(), slots, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                       stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return STQ_E_DEVICE;
    std::vector<char> seen(static_cast<size_t>(n_slots), 0);
    for (int32_t s : h) {
        if (s < 0 || s >= n_slots) continue; // skipped by the kernels
        if (seen[static_cast<size_t>(s)]) return STQ_E_ARG;
        seen[static_cast<size_t>(s)] = 1;
    }
    return STQ_OK;
}

stq::PackArgs pack_args(const stq_state *st, const int32_t *slots, int32_t B) {
    stq::PackArgs a{};
    a.pool8 = st->pool8;
    a.pool4 = st->pool4;
    a.r = st->r;
    a.c = st->c;
    a.perm = st->perm;
    a.slots = slots;
    a.S_in = nullptr;
    a.S_out = nullptr;
    a.cs = refit_format(st->desc.fmt) ? st->cs : nullptr;
    a.w2 = refit_format(st->desc.fmt) ? st->w2 : nullptr;
    a.B = B;
    a.Hv = st->desc.n_heads_v;
    a.n8 = st->desc.n8;
    a.n_slots = st->desc.n_slots;
    a.layout = alloc_format(st->desc.fmt) ? st->layout : nullptr;
    a.slot_bytes = st->slot_bytes;
    return a;
}

} // namespace

stq_status stq_pack_state(const stq_state *st, const float *S, const int32_t *slots, int32_t B,
                          stq_stream_t stream) {
    stq_status e = batch_args(st, slots, B);
    if (e != STQ_OK) return e;
    if (!S || !aligned(S, 16)) return STQ_E_ARG;
    if (calibrated_format(st->desc.fmt) && !st->calibrated) return STQ_E_STATE;
    if ((e = check_slots_distinct(slots, B, st->desc.n_slots, static_cast<hipStream_t>(stream))) != STQ_OK)
        return e;
    stq::PackArgs a = pack_args(st, slots, B);
    a.S_in = S;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (st->desc.fmt == STQ_FMT_FP32) return dev(stq::launch_copy_slots_fp32(st->desc.d_k, a, true, st->s32, s));
    if (alloc_format(st->desc.fmt)) return dev(stq::launch_pack_alloc(st->desc.d_k, a, s));
    return dev(stq::launch_pack(st->desc.d_k, a, s));
}

stq_status stq_dequant_state(const stq_state *st, const int32_t *slots, int32_t B, float *S_out,
                             stq_stream_t stream) {
    stq_status e = batch_args(st, slots, B);
    if (e != STQ_OK) return e;
    if (!S_out || !aligned(S_out, 16)) return STQ_E_ARG;
    stq::PackArgs a = pack_args(st, slots, B);
    a.S_out = S_out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (st->desc.fmt == STQ_FMT_FP32) return dev(stq::launch_copy_slots_fp32(st->desc.d_k, a, false, st->s32, s));
    if (alloc_format(st->desc.fmt)) return dev(stq::launch_dequant_alloc(st->desc.d_k, a, s));
    return dev(stq::launch_dequant(st->desc.d_k, a, s));
}

namespace {

bool same_desc(const stq_desc &x, const stq_desc &y) {
    return x.n_slots == y.n_slots && x.n_heads_v == y.n_heads_v && x.n_heads_k == y.n_heads_k &&
           x.d_k == y.d_k && x.d_v == y.d_v && x.n8 == y.n8 && x.fmt == y.fmt &&
           x.nominal_bits == y.nominal_bits && x.n_pivot == y.n_pivot;
}

// [p, p + n) and [q, q + n) overlap without being the same range
bool partial_overlap(const void *p, const void *q, size_t n) {
    if (!p || !q || n == 0 || p == q) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + n && b < a + n;
}

// Exactly one of alpha (scalar gate, [B][Hv]) and gate (row gate, [B][Hv][d_k])
// is non-null.
stq_status decode(const stq_state *src, const stq_state *dst, const int32_t *slots, int32_t B,
                  const void *q, const void *k, const void *v, int32_t dtype, const float *alpha,
                  const float *gate, const float *beta, void *o, stq_stream_t stream) {
    stq_status e = batch_args(src, slots, B);
    if (e != STQ_OK) return e;
    if ((e = check_state(dst)) != STQ_OK) return e;
    if (!same_desc(src->desc, dst->desc)) return STQ_E_SHAPE;
    const bool o_bf16 = (dtype & STQ_OUT_BF16) != 0;
    dtype &= ~STQ_OUT_BF16;
    if (dtype != STQ_F32 && dtype != STQ_BF16) return STQ_E_ARG;
    const size_t el = dtype == STQ_F32 ? 4 : 2;
    const float *g_or_a = gate ? gate : alpha;
    if (!q || !k || !v || !g_or_a || !beta || !o) return STQ_E_ARG;
    if (!aligned(q, el) || !aligned(k, el) || !aligned(v, el) || !aligned(g_or_a, 4) ||
        !aligned(beta, 4) || !aligned(o, o_bf16 ? 2 : 4))
        return STQ_E_ARG;
    if (calibrated_format(src->desc.fmt) && !src->calibrated) return STQ_E_STATE;
    if ((e = check_slots_distinct(slots, B, src->desc.n_slots, static_cast<hipStream_t>(stream))) !=
        STQ_OK)
        return e;
    const bool refit = refit_format(src->desc.fmt);
    Layout L;
    describe(&src->desc, &L);
    if (partial_overlap(src->pool8, dst->pool8, L.pool8) || partial_overlap(src->pool4, dst->pool4, L.pool4) ||
        partial_overlap(src->r, dst->r, L.r) || partial_overlap(src->s32, dst->s32, L.s32) ||
        partial_overlap(src->cs, dst->cs, L.cs))
        return STQ_E_ARG;
    stq::DecodeArgs a{};
    a.pool8 = src->pool8;
    a.pool4 = src->pool4;
    a.r = src->r;
    a.pool8_out = dst->pool8;
    a.pool4_out = dst->pool4;
    a.r_out = dst->r;
    a.s32 = src->s32;
    a.s32_out = dst->s32;
    a.c = src->c;
    a.perm = src->perm;
    a.cs = refit ? src->cs : nullptr;
    a.cs_out = refit ? dst->cs : nullptr;
    a.w2 = refit ? src->w2 : nullptr;
    a.slots = slots;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = gate ? nullptr : alpha;
    a.gate = gate;
    a.beta = beta;
    a.o = static_cast<float *>(o);
    a.o_bf16 = o_bf16 ? 1 : 0;
    a.B = B;
    a.Hv = src->desc.n_heads_v;
    a.Hk = src->desc.n_heads_k;
    a.n8 = src->desc.n8;
    a.n_slots = src->desc.n_slots;
    a.layout = alloc_format(src->desc.fmt) ? src->layout : nullptr;
    a.slot_bytes = src->slot_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == STQ_BF16;
    if (src->desc.fmt == STQ_FMT_FP32) return dev(stq::launch_decode_fp32(src->desc.d_k, bf16, a, s));
    if (alloc_format(src->desc.fmt)) return dev(stq::launch_decode_alloc(src->desc.d_k, bf16, a, s));
    return dev(stq::launch_decode_mixed(src->desc.d_k, bf16, a, s));
}

} // namespace

stq_status stq_decode_step(const stq_state *st, const int32_t *slots, int32_t B, const void *q,
                           const void *k, const void *v, int32_t dtype, const float *alpha,
                           const float *beta, void *o, stq_stream_t stream) {
    if (!alpha) return STQ_E_ARG;
    return decode(st, st, slots, B, q, k, v, dtype, alpha, nullptr, beta, o, stream);
}

stq_status stq_decode_step_into(const stq_state *src, const stq_state *dst, const int32_t *slots,
                                int32_t B, const void *q, const void *k, const void *v,
                                int32_t dtype, const float *alpha, const float *beta, void *o,
                                stq_stream_t stream) {
    if (!src || !dst || !alpha) return STQ_E_ARG;
    return decode(src, dst, slots, B, q, k, v, dtype, alpha, nullptr, beta, o, stream);
}

stq_status stq_decode_step_gated(const stq_state *src, const stq_state *dst, const int32_t *slots,
                                 int32_t B, const void *q, const void *k, const void *v,
                                 int32_t dtype, const float *gate, const float *beta, void *o,
                                 stq_stream_t stream) {
    if (!src || !dst || !gate) return STQ_E_ARG;
    return decode(src, dst, slots, B, q, k, v, dtype, nullptr, gate, beta, o, stream);
}

stq_status stq_calibrate_retention(stq_state *st, const float *alpha, const float *gate,
                                   int32_t B, uint32_t flags, stq_stream_t stream) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    if (!alloc_format(st->desc.fmt)) return STQ_E_ARG;
    if (flags & ~STQ_CAL_RESET) return STQ_E_ARG;
    if (B < 0) return STQ_E_SHAPE;
    if (B > 0) {
        if ((alpha == nullptr) == (gate == nullptr)) return STQ_E_ARG;
        if (!aligned(alpha ? alpha : gate, 4)) return STQ_E_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = st->desc.d_k, H = st->desc.n_heads_v;
    if (flags & STQ_CAL_RESET) {
        if ((e = dev(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st->logret),
                                          static_cast<size_t>(H) * D, 0u, s))) != STQ_OK ||
            (e = dev(stq::launch_fill_u64(reinterpret_cast<uint64_t *>(st->nret),
                                          static_cast<size_t>(H), 0u, s))) != STQ_OK)
            return e;
    }
    if (B == 0) return STQ_OK;
    stq::AllocCalArgs a{};
    a.Hv = H;
    a.alpha = alpha;
    a.gate = gate;
    a.B = B;
    a.logret = st->logret;
    a.nret = st->nret;
    return dev(stq::launch_alloc_retention(D, a, s));
}

// The candidate set of an assignment: 0 picks Table C1's set for the nominal
// width; otherwise only integer classes, and the nominal width among them.
static bool candidate_mask(int nominal, uint32_t candidates, uint32_t *mask) {
    uint32_t m = candidates;
    if (m == 0) m = nominal <= 4 ? 0x1Eu : 0x0Eu; // {8,6,4,2} or {8,6,4}
    const int k = class_of_width(nominal);
    if ((m & ~0x1Eu) || k < 0 || !(m & (1u << k))) return false;
    *mask = m;
    return true;
}

stq_status stq_assign_rows(int32_t n_heads_v, int32_t d_k, const double *dist,
                           const double *logret, double nret, int32_t horizon,
                           uint32_t candidates, int32_t nominal_bits, int32_t n_pivot,
                           int32_t *counts, int32_t *perm) {
    if (n_heads_v < 1 || d_k < 1 || !dist || !logret || !counts || !perm) return STQ_E_ARG;
    if (static_cast<int64_t>(n_heads_v) * d_k > (int64_t{1} << 24)) return STQ_E_SHAPE;
    uint32_t mask = 0;
    if (horizon < 1 || !(nret > 0.0) || !candidate_mask(nominal_bits, candidates, &mask))
        return STQ_E_ARG;
    if (n_pivot < 0 || n_pivot > n_heads_v * d_k) return STQ_E_ARG;
    return stq::assign_rows(n_heads_v, d_k, dist, logret, nret, horizon, mask, nominal_bits,
                            n_pivot, counts, perm)
               ? STQ_OK
               : STQ_E_ARG;
}

stq_status stq_allocate(stq_state *st, int32_t horizon, uint32_t candidates,
                        stq_stream_t stream) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    if (!alloc_format(st->desc.fmt) || horizon < 1) return STQ_E_ARG;
    const int nominal = st->desc.nominal_bits;
    uint32_t mask = 0;
    if (!candidate_mask(nominal, candidates, &mask)) return STQ_E_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = st->desc.d_k, H = st->desc.n_heads_v;
    const size_t nd = static_cast<size_t>(H) * D;
    std::vector<double> dist(nd * stq::kNumClasses), logret(nd), nret(H);
    if (hipMemcpyAsync(dist.data(), st->dist, dist.size() * sizeof(double), hipMemcpyDeviceToHost,
                       s) != hipSuccess ||
        hipMemcpyAsync(logret.data(), st->logret, nd * sizeof(double), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipMemcpyAsync(nret.data(), st->nret, H * sizeof(double), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return STQ_E_DEVICE;
    if (!(nret[0] > 0.0)) return STQ_E_STATE;
    std::vector<int32_t> counts(static_cast<size_t>(H) * stq::kNumClasses), perm(nd);
    if ((e = stq_assign_rows(H, D, dist.data(), logret.data(), nret[0], horizon, mask, nominal,
                             st->desc.n_pivot, counts.data(), perm.data())) != STQ_OK)
        return e;
    std::vector<int32_t> table(static_cast<size_t>(H) * stq::kLayoutWordsPerHead);
    bool space = false;
    if (!build_layout(&st->desc, st->slot_bytes, counts.data(), table.data(), &space))
        return space ? STQ_E_SPACE : STQ_E_ARG;
    if (hipMemcpyAsync(st->layout, table.data(), table.size() * sizeof(int32_t),
                       hipMemcpyHostToDevice, s) != hipSuccess ||
        hipMemcpyAsync(st->perm, perm.data(), perm.size() * sizeof(int32_t), hipMemcpyHostToDevice,
                       s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return STQ_E_DEVICE;
    st->calibrated = 1;
    return STQ_OK;
}

stq_status stq_set_alloc_layout(stq_state *st, const int32_t *counts, const float *c,
                                const int32_t *perm, stq_stream_t stream) {
    stq_status e = check_state(st);
    if (e != STQ_OK) return e;
    if (!alloc_format(st->desc.fmt)) return STQ_E_ARG;
    if (!counts || !c || !perm || !aligned(c, 16) || !aligned(perm, 16)) return STQ_E_ARG;
    const int D = st->desc.d_k, H = st->desc.n_heads_v;
    std::vector<int32_t> table(static_cast<size_t>(H) * stq::kLayoutWordsPerHead);
    bool space = false;
    if (!build_layout(&st->desc, st->slot_bytes, counts, table.data(), &space))
        return space ? STQ_E_SPACE : STQ_E_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t n = static_cast<size_t>(H) * D * 4;
    if ((e = dev(stq::launch_copy_bytes(c, st->c, n, s))) != STQ_OK) return e;
    if ((e = dev(stq::launch_copy_bytes(perm, st->perm, n, s))) != STQ_OK) return e;
    if (hipMemcpyAsync(st->layout, table.data(), table.size() * sizeof(int32_t),
                       hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return STQ_E_DEVICE;
    st->calibrated = 1;
    return STQ_OK;
}

stq_status stq_stream_copy(const void *src, void *dst, size_t bytes, stq_stream_t stream) {
    if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16) || bytes % 16 != 0) return STQ_E_ARG;
    return dev(stq::launch_copy_bytes(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

} // extern "C"
