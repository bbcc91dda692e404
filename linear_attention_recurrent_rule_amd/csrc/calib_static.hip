// stq_calibrate_static: stq_calibrate for callers that cannot allocate device
// memory, with its per-chunk partial results in a fixed array of the library
// instead of the state's own partial arrays.
//
// The array lives in device memory for as long as the library is loaded (one
// copy per GPU).  Host code never passes the array's name to a kernel: its
// device address is looked up once per device, with that device current, and
// kept; every later use goes through that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "stq.h"
#include "stq_internal.h"

namespace {

// Partials of one call: [Hv][kCalChunks][D] fp32 column maxima, then (at the
// next 256-byte boundary) [Hv][kCalChunks][D] fp64 row sums: 768 bytes per
// (head, key row), so 8192 head rows (Hv * d_k, e.g. 64 heads of 128) take
// 6 MiB.
constexpr size_t kMaxHeadRows = 8192;
constexpr size_t kPartBytesPerRow = static_cast<size_t>(stq::kCalChunks) * (4 + 8);
constexpr size_t kScratchBytes = kMaxHeadRows * kPartBytesPerRow;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// The device address of this device's copy of the array (looked up on the
// first call on that device, which is current here).
void *scratch_address(int device) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[device] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return nullptr;
        g_ptr[device] = p;
    }
    return g_ptr[device];
}

} // namespace

extern "C" stq_status stq_calibrate_static(stq_state *st, const float *records, int64_t n_rec,
                                           uint32_t flags, stq_stream_t stream) {
    if (!st) return STQ_E_ARG;
    if (st->desc.n_heads_v < 1 || st->desc.d_k < 1) return STQ_E_SHAPE;
    const size_t rows = static_cast<size_t>(st->desc.n_heads_v) * static_cast<size_t>(st->desc.d_k);
    const size_t col_bytes = round256(rows * stq::kCalChunks * sizeof(float));
    if (col_bytes + rows * stq::kCalChunks * sizeof(double) > kScratchBytes) return STQ_E_SPACE;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices)
        return STQ_E_DEVICE;
    unsigned char *base = static_cast<unsigned char *>(scratch_address(device));
    if (base == nullptr) return STQ_E_DEVICE;
    // every partial that the fold reads is written earlier in the same call,
    // so nothing left by a previous call needs clearing
    return stq::calibrate_with(st, records, n_rec, flags, stream,
                               reinterpret_cast<float *>(base),
                               reinterpret_cast<double *>(base + col_bytes));
}
