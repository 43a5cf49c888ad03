// C ABI of the kronq library: argument validation and dispatch.  Every check that
// can be made on the host happens here, before anything is enqueued.
#include <cmath>
#include <string>

#include "kq_common.hpp"

namespace kq {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

kq_status hip_fail(hipError_t e, const char* what) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return KQ_ERR_HIP;
}

size_t quantize_workspace_bytes(kq_dtype dtype, int64_t m, int64_t n);
size_t prepare_workspace_bytes(int64_t d);
size_t loss_workspace_bytes(int64_t m, int64_t n);
kq_status quantize_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const void*, int64_t, const void*,
                            int64_t, const kq_quantizer*, int8_t*, int64_t, void*, int64_t, double*, void*,
                            hipStream_t, bool);
kq_status prepare_dispatch(kq_dtype, int64_t, const void*, int64_t, double, void*, int64_t, double*, double*,
                           int32_t*, void*, hipStream_t);
kq_status factor_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, void*, int64_t, double, double,
                          hipStream_t);
kq_status loss_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const void*, int64_t, const void*, int64_t,
                        const void*, int64_t, double, double*, void*, hipStream_t);
kq_status scales_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, int, int, void*, hipStream_t);
size_t kronecker_workspace_bytes(kq_dtype, int64_t, int64_t, int64_t);
size_t biip_workspace_bytes(kq_dtype, int64_t, int64_t);
kq_status biip_forward_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const void*, int64_t, const void*,
                                int64_t, const int8_t*, const int8_t*, void*, int64_t, void*, int64_t, void*, int64_t,
                                void*, void*, void*, hipStream_t);
kq_status biip_inverse_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const int8_t*, const int8_t*,
                                const void*, const void*, void*, int64_t, void*, hipStream_t);
kq_status kronecker_dispatch(kq_dtype, int, int64_t, int64_t, int64_t, const void*, int64_t, const void*, int64_t, int,
                             double, void*, int64_t, void*, int64_t, int32_t*, void*, hipStream_t);
kq_status waterkron_scales_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const void*, int64_t, double,
                                    void*, void*, hipStream_t);
kq_status waterkron_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const void*, int64_t, const void*,
                             int64_t, const void*, const void*, int32_t*, int64_t, void*, int64_t, double*, void*,
                             hipStream_t);

// Largest supported matrix edge: keeps every tile index and padded extent in int.
constexpr int64_t MAX_DIM = 1 << 16;

static kq_status invalid(const std::string& msg) {
    set_error(msg);
    return KQ_ERR_INVALID_ARG;
}

static bool dtype_ok(kq_dtype d) { return d == KQ_F32 || d == KQ_F64; }

static kq_status check_ws(void* ws, size_t have, size_t need, const char* op) {
    if (need == 0) return KQ_OK;
    if (!ws || have < need) {
        set_error(std::string(op) + ": workspace of " + std::to_string(need) + " bytes required, got " +
                  std::to_string(ws ? have : 0));
        return KQ_ERR_WORKSPACE;
    }
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) {
        set_error(std::string(op) + ": workspace must be 256-byte aligned");
        return KQ_ERR_WORKSPACE;
    }
    return KQ_OK;
}

// The host-checkable arguments of the quantize entry points (everything but the
// scratch space).  KQ_OK with m == 0 or n == 0 means: nothing to do.
kq_status quantize_checked_args(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* U_A,
                                int64_t lda, const void* U_B, int64_t ldb, const kq_quantizer* q, int8_t* codes,
                                int64_t ldc, void* V, int64_t ldv, double* loss_dev, const char* who) {
    const std::string f(who);
    if (!dtype_ok(dtype)) return invalid(f + ": dtype must be KQ_F32 or KQ_F64");
    if (m < 0 || n < 0 || m > MAX_DIM || n > MAX_DIM) return invalid(f + ": m, n must be in [0, 65536]");
    if (!q) return invalid(f + ": null quantizer");
    if (q->bits < 2 || q->bits > 8) return invalid(f + ": bits must be in [2, 8]");
    if (q->per_row != 0 && q->per_row != 1) return invalid(f + ": per_row must be 0 or 1");
    if (m == 0 || n == 0) {
        if (loss_dev) return invalid(f + ": no loss for an empty matrix");
        return KQ_OK;
    }
    if (!W || !U_A || !codes || !V || !q->scales) return invalid(f + ": null pointer");
    if (ldw < n || lda < n || ldc < n || ldv < n || (U_B && ldb < m)) return invalid(f + ": leading dimension too small");
    return KQ_OK;
}

}  // namespace kq

using namespace kq;

extern "C" {

int32_t kron_abi_version(void) { return 4; }

const char* kron_status_string(kq_status s) {
    switch (s) {
        case KQ_OK: return "ok";
        case KQ_ERR_INVALID_ARG: return "invalid argument";
        case KQ_ERR_NOT_PD: return "factor not positive definite";
        case KQ_ERR_WORKSPACE: return "workspace too small";
        case KQ_ERR_HIP: return "HIP runtime error";
        case KQ_ERR_UNSUPPORTED: return "unsupported";
    }
    return "unknown status";
}

const char* kron_last_error(void) { return g_last_error.c_str(); }

size_t kron_workspace_bytes(int op, kq_dtype dtype, int64_t m, int64_t n) {
    if (!dtype_ok(dtype) || m < 0 || n < 0 || m > MAX_DIM || n > MAX_DIM) return 0;
    switch (op) {
        case KQ_OP_FACTOR: return 0;
        case KQ_OP_PREPARE: return m > 0 ? prepare_workspace_bytes(m) : 0;
        case KQ_OP_QUANTIZE: return (m > 0 && n > 0) ? quantize_workspace_bytes(dtype, m, n) : 0;
        case KQ_OP_LOSS: return (m > 0 && n > 0) ? loss_workspace_bytes(m, n) : 0;
    }
    return 0;
}

kq_status kron_factor_accumulate(kq_dtype dtype, int64_t rows, int64_t dim, const void* X, int64_t ldx, void* S,
                                 int64_t lds, double alpha, double beta, void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_factor_accumulate: dtype must be KQ_F32 or KQ_F64");
    if (rows < 0 || dim < 0 || dim > MAX_DIM || rows > (int64_t(1) << 30))
        return invalid("kron_factor_accumulate: rows must be in [0, 2^30] and dim in [0, 65536]");
    if (dim == 0) return KQ_OK;
    if (!S || (rows > 0 && !X)) return invalid("kron_factor_accumulate: null pointer");
    if (ldx < dim || lds < dim) return invalid("kron_factor_accumulate: leading dimension smaller than dim");
    if (!std::isfinite(alpha) || !std::isfinite(beta)) return invalid("kron_factor_accumulate: non-finite alpha/beta");
    return factor_dispatch(dtype, rows, dim, X, ldx, S, lds, alpha, beta, static_cast<hipStream_t>(stream));
}

kq_status kron_prepare(kq_dtype dtype, int64_t dim, const void* A, int64_t lda, double damp_rel, void* U, int64_t ldu,
                       double* trace_out, double* lambda_out, int32_t* info_dev, void* ws, size_t ws_bytes,
                       void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_prepare: dtype must be KQ_F32 or KQ_F64");
    if (dim < 1 || dim > MAX_DIM) return invalid("kron_prepare: dim must be in [1, 65536]");
    if (!A || !U) return invalid("kron_prepare: null pointer");
    if (lda < dim || ldu < dim) return invalid("kron_prepare: leading dimension smaller than dim");
    if (!(damp_rel >= 0.0) || !std::isfinite(damp_rel)) return invalid("kron_prepare: damp_rel must be finite and >= 0");
    kq_status s = check_ws(ws, ws_bytes, prepare_workspace_bytes(dim), "kron_prepare");
    if (s != KQ_OK) return s;
    return prepare_dispatch(dtype, dim, A, lda, damp_rel, U, ldu, trace_out, lambda_out, info_dev, ws,
                            static_cast<hipStream_t>(stream));
}

kq_status kron_row_scales(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, int32_t bits,
                          int32_t per_row, void* scales, void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_row_scales: dtype must be KQ_F32 or KQ_F64");
    if (m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM) return invalid("kron_row_scales: m, n must be in [1, 65536]");
    if (!W || !scales) return invalid("kron_row_scales: null pointer");
    if (ldw < n) return invalid("kron_row_scales: ldw < n");
    if (bits < 2 || bits > 8) return invalid("kron_row_scales: bits must be in [2, 8]");
    if (per_row != 0 && per_row != 1) return invalid("kron_row_scales: per_row must be 0 or 1");
    return scales_dispatch(dtype, m, n, W, ldw, bits, per_row, scales, static_cast<hipStream_t>(stream));
}

kq_status kron_quantize(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* U_A, int64_t lda,
                        const void* U_B, int64_t ldb, const kq_quantizer* q, int8_t* codes, int64_t ldc, void* V,
                        int64_t ldv, double* loss_dev, void* ws, size_t ws_bytes, void* stream) {
    set_error("");
    kq_status s = quantize_checked_args(dtype, m, n, W, ldw, U_A, lda, U_B, ldb, q, codes, ldc, V, ldv, loss_dev,
                                        "kron_quantize");
    if (s != KQ_OK || m == 0 || n == 0) return s;
    s = check_ws(ws, ws_bytes, quantize_workspace_bytes(dtype, m, n), "kron_quantize");
    if (s != KQ_OK) return s;
    return quantize_dispatch(dtype, m, n, W, ldw, U_A, lda, U_B, ldb, q, codes, ldc, V, ldv, loss_dev, ws,
                             static_cast<hipStream_t>(stream), true);
}

kq_status kron_quantize_per_diagonal(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                                     const void* U_A, int64_t lda, const void* U_B, int64_t ldb,
                                     const kq_quantizer* q, int8_t* codes, int64_t ldc, void* V, int64_t ldv,
                                     double* loss_dev, void* ws, size_t ws_bytes, void* stream) {
    set_error("");
    kq_status s = quantize_checked_args(dtype, m, n, W, ldw, U_A, lda, U_B, ldb, q, codes, ldc, V, ldv, loss_dev,
                                        "kron_quantize_per_diagonal");
    if (s != KQ_OK || m == 0 || n == 0) return s;
    s = check_ws(ws, ws_bytes, quantize_workspace_bytes(dtype, m, n), "kron_quantize_per_diagonal");
    if (s != KQ_OK) return s;
    return quantize_dispatch(dtype, m, n, W, ldw, U_A, lda, U_B, ldb, q, codes, ldc, V, ldv, loss_dev, ws,
                             static_cast<hipStream_t>(stream), false);
}

size_t kron_kronecker_workspace_bytes(kq_dtype dtype, int64_t samples, int64_t n, int64_t m) {
    if (!dtype_ok(dtype) || samples < 1 || samples > (int64_t(1) << 30) || n < 1 || m < 1 || n > MAX_DIM ||
        m > MAX_DIM)
        return 0;
    return kronecker_workspace_bytes(dtype, samples, n, m);
}

kq_status kron_factor_kronecker(kq_dtype dtype, int32_t method, int64_t samples, int64_t n, int64_t m, const void* Xa,
                                int64_t ldxa, const void* Xb, int64_t ldxb, int32_t iters, double damp_rel, void* A,
                                int64_t lda, void* B, int64_t ldb, int32_t* info_dev, void* ws, size_t ws_bytes,
                                void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_factor_kronecker: dtype must be KQ_F32 or KQ_F64");
    if (method != KQ_KRON_FROBENIUS && method != KQ_KRON_FLIPFLOP)
        return invalid("kron_factor_kronecker: method must be KQ_KRON_FROBENIUS or KQ_KRON_FLIPFLOP");
    if (samples < 1 || samples > (int64_t(1) << 30) || n < 1 || m < 1 || n > MAX_DIM || m > MAX_DIM)
        return invalid("kron_factor_kronecker: samples must be in [1, 2^30] and n, m in [1, 65536]");
    if (iters < 1 || iters > 64) return invalid("kron_factor_kronecker: iters must be in [1, 64]");
    if (!Xa || !Xb || !A || !B) return invalid("kron_factor_kronecker: null pointer");
    if (ldxa < n || ldxb < m || lda < n || ldb < m) return invalid("kron_factor_kronecker: leading dimension too small");
    if (!(damp_rel >= 0.0) || !std::isfinite(damp_rel))
        return invalid("kron_factor_kronecker: damp_rel must be finite and >= 0");
    kq_status s = check_ws(ws, ws_bytes, kronecker_workspace_bytes(dtype, samples, n, m), "kron_factor_kronecker");
    if (s != KQ_OK) return s;
    return kronecker_dispatch(dtype, method, samples, n, m, Xa, ldxa, Xb, ldxb, iters, damp_rel, A, lda, B, ldb,
                              info_dev, ws, static_cast<hipStream_t>(stream));
}

size_t kron_biip_workspace_bytes(kq_dtype dtype, int64_t m, int64_t n) {
    if (!dtype_ok(dtype) || m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM) return 0;
    return biip_workspace_bytes(dtype, m, n);
}

kq_status kron_biip_forward(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* A,
                            int64_t lda, const void* B, int64_t ldb, const int8_t* signs_n, const int8_t* signs_m,
                            void* W_out, int64_t ldwo, void* A_out, int64_t ldao, void* B_out, int64_t ldbo,
                            void* scale_a, void* scale_b, void* ws, size_t ws_bytes, void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_biip_forward: dtype must be KQ_F32 or KQ_F64");
    if (m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM) return invalid("kron_biip_forward: m, n must be in [1, 65536]");
    if (!W || !A || !B || !signs_n || !signs_m || !W_out || !A_out || !B_out || !scale_a || !scale_b)
        return invalid("kron_biip_forward: null pointer");
    if (ldw < n || lda < n || ldb < m || ldwo < n || ldao < n || ldbo < m)
        return invalid("kron_biip_forward: leading dimension too small");
    kq_status s = check_ws(ws, ws_bytes, biip_workspace_bytes(dtype, m, n), "kron_biip_forward");
    if (s != KQ_OK) return s;
    return biip_forward_dispatch(dtype, m, n, W, ldw, A, lda, B, ldb, signs_n, signs_m, W_out, ldwo, A_out, ldao, B_out,
                                 ldbo, scale_a, scale_b, ws, static_cast<hipStream_t>(stream));
}

kq_status kron_biip_inverse(kq_dtype dtype, int64_t m, int64_t n, const void* V2, int64_t ldv2, const int8_t* signs_n,
                            const int8_t* signs_m, const void* scale_a, const void* scale_b, void* V, int64_t ldv,
                            void* ws, size_t ws_bytes, void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_biip_inverse: dtype must be KQ_F32 or KQ_F64");
    if (m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM) return invalid("kron_biip_inverse: m, n must be in [1, 65536]");
    if (!V2 || !signs_n || !signs_m || !scale_a || !scale_b || !V) return invalid("kron_biip_inverse: null pointer");
    if (ldv2 < n || ldv < n) return invalid("kron_biip_inverse: leading dimension too small");
    kq_status s = check_ws(ws, ws_bytes, biip_workspace_bytes(dtype, m, n), "kron_biip_inverse");
    if (s != KQ_OK) return s;
    return biip_inverse_dispatch(dtype, m, n, V2, ldv2, signs_n, signs_m, scale_a, scale_b, V, ldv, ws,
                                 static_cast<hipStream_t>(stream));
}

kq_status kron_waterkron_scales(kq_dtype dtype, int64_t m, int64_t n, const void* U_A, int64_t lda, const void* U_B,
                                int64_t ldb, double step, void* alpha, void* beta, void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_waterkron_scales: dtype must be KQ_F32 or KQ_F64");
    if (m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM) return invalid("kron_waterkron_scales: m, n must be in [1, 65536]");
    if (!U_A || !alpha || !beta) return invalid("kron_waterkron_scales: null pointer");
    if (lda < n || (U_B && ldb < m)) return invalid("kron_waterkron_scales: leading dimension too small");
    if (!(step > 0.0) || !std::isfinite(step)) return invalid("kron_waterkron_scales: step must be finite and > 0");
    return waterkron_scales_dispatch(dtype, m, n, U_A, lda, U_B, ldb, step, alpha, beta,
                                     static_cast<hipStream_t>(stream));
}

kq_status kron_quantize_waterkron(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* U_A,
                                  int64_t lda, const void* U_B, int64_t ldb, const void* alpha, const void* beta,
                                  int32_t* codes, int64_t ldc, void* V, int64_t ldv, double* loss_dev, void* ws,
                                  size_t ws_bytes, void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_quantize_waterkron: dtype must be KQ_F32 or KQ_F64");
    if (m < 0 || n < 0 || m > MAX_DIM || n > MAX_DIM) return invalid("kron_quantize_waterkron: m, n must be in [0, 65536]");
    if (m == 0 || n == 0) {
        if (loss_dev) return invalid("kron_quantize_waterkron: no loss for an empty matrix");
        return KQ_OK;
    }
    if (!W || !U_A || !alpha || !beta || !codes || !V) return invalid("kron_quantize_waterkron: null pointer");
    if (ldw < n || lda < n || ldc < n || ldv < n || (U_B && ldb < m))
        return invalid("kron_quantize_waterkron: leading dimension too small");
    kq_status s = check_ws(ws, ws_bytes, quantize_workspace_bytes(dtype, m, n), "kron_quantize_waterkron");
    if (s != KQ_OK) return s;
    return waterkron_dispatch(dtype, m, n, W, ldw, U_A, lda, U_B, ldb, alpha, beta, codes, ldc, V, ldv, loss_dev, ws,
                              static_cast<hipStream_t>(stream));
}

kq_status kron_loss(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* V, int64_t ldv,
                    const void* A, int64_t lda, const void* B, int64_t ldb, double damp_rel, double* loss_dev, void* ws,
                    size_t ws_bytes, void* stream) {
    set_error("");
    if (!dtype_ok(dtype)) return invalid("kron_loss: dtype must be KQ_F32 or KQ_F64");
    if (m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM) return invalid("kron_loss: m, n must be in [1, 65536]");
    if (!W || !V || !A || !loss_dev) return invalid("kron_loss: null pointer");
    if (ldw < n || ldv < n || lda < n || (B && ldb < m)) return invalid("kron_loss: leading dimension too small");
    if (!(damp_rel >= 0.0) || !std::isfinite(damp_rel)) return invalid("kron_loss: damp_rel must be finite and >= 0");
    kq_status s = check_ws(ws, ws_bytes, loss_workspace_bytes(m, n), "kron_loss");
    if (s != KQ_OK) return s;
    return loss_dispatch(dtype, m, n, W, ldw, V, ldv, A, lda, B, ldb, damp_rel, loss_dev, ws,
                         static_cast<hipStream_t>(stream));
}

}  // extern "C"
