// kron_quantize_noalloc: kron_quantize with its scratch space in a fixed device
// array of the library instead of a caller workspace, for callers that cannot
// allocate (code under stream capture, tight serving loops).
//
// The array `scratch` below is a file-scope device variable: every GPU the
// library runs on holds one copy of KQ_NOALLOC_SCRATCH_BYTES until the process
// ends.  In host code its name is only a host-side stand-in, never a device
// address: the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and kept in `g_scratch`.  Every call on a
// device shares that device's array, so calls that overlap on one GPU (two
// streams, two threads) race on it; the array keeps the last call's contents.
// Nothing in it has to start at zero: the solver writes every scratch value it
// reads (the factors, the running values and the scales are initialised by the
// solver's first kernels, errors are written before they are read, and stale
// band operands are masked by selects).
#include <mutex>

#include "kq_common.hpp"

namespace kq {

kq_status quantize_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const void*, int64_t, const void*,
                            int64_t, const kq_quantizer*, int8_t*, int64_t, void*, int64_t, double*, void*,
                            hipStream_t, bool);
size_t quantize_workspace_bytes(kq_dtype dtype, int64_t m, int64_t n);
kq_status quantize_checked_args(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* U_A,
                                int64_t lda, const void* U_B, int64_t ldb, const kq_quantizer* q, int8_t* codes,
                                int64_t ldc, void* V, int64_t ldv, double* loss_dev, const char* who);

static __device__ __align__(256) char scratch[KQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch[MAX_DEVICES];  // device address of `scratch`, per device

// The device address of the current device's scratch array (set up on the
// device's first call).
static kq_status scratch_for_current_device(void** out) {
    int dev = -1;
    KQ_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) {
        set_error("kron_quantize_noalloc: device index out of range");
        return KQ_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        KQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) {
            set_error("kron_quantize_noalloc: hipGetSymbolAddress returned no address");
            return KQ_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KQ_OK;
}

}  // namespace kq

using namespace kq;

extern "C" kq_status kron_quantize_noalloc(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                                           const void* U_A, int64_t lda, const void* U_B, int64_t ldb,
                                           const kq_quantizer* q, int8_t* codes, int64_t ldc, void* V, int64_t ldv,
                                           double* loss_dev, void* stream) {
    set_error("");
    kq_status s = quantize_checked_args(dtype, m, n, W, ldw, U_A, lda, U_B, ldb, q, codes, ldc, V, ldv, loss_dev,
                                        "kron_quantize_noalloc");
    if (s != KQ_OK || m == 0 || n == 0) return s;
    const size_t need = quantize_workspace_bytes(dtype, m, n);
    if (need > size_t(KQ_NOALLOC_SCRATCH_BYTES)) {
        set_error("kron_quantize_noalloc: an m x n problem of this dtype needs " + std::to_string(need) +
                  " bytes of scratch; the fixed array holds " + std::to_string(size_t(KQ_NOALLOC_SCRATCH_BYTES)) +
                  " (use kron_quantize with a workspace)");
        return KQ_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    s = scratch_for_current_device(&ws);
    if (s != KQ_OK) return s;
    return quantize_dispatch(dtype, m, n, W, ldw, U_A, lda, U_B, ldb, q, codes, ldc, V, ldv, loss_dev, ws,
                             static_cast<hipStream_t>(stream), true);
}
