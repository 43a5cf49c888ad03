/*
 * kronq.h -- C ABI of the MI355X (gfx950) library for two-sided GPTQ:
 * GPTQ adaptive rounding of an m x n weight matrix W under a Kronecker-factored
 * Hessian A (x) B (A: n x n input curvature, B: m x m output curvature).
 *
 * Sources: "FastKron: Efficient Quantization with Kronecker-Factored Hessians"
 * (section 2: the solver; section 2.6: the side costs; section 3.2: Kronecker
 * factors), "WaterKron and FlipFlop Hessian" (section 2 notation; section 2.4:
 * scales are handed to the algorithm), the BaKron and GPTQ-2D abstracts, the
 * pith.science review of BaKron, and the KronQ page (sensitivity score).
 *
 * Conventions shared by every entry point
 *  - Matrices are row-major with an explicit leading dimension (elements, >= the
 *    number of columns).  W, V are m x n; A, U_A are n x n; B, U_B are m x m.
 *  - Every data pointer is DEVICE memory owned by the caller.  The library never
 *    allocates or frees device memory; scratch space comes from the caller's
 *    workspace (size from kron_workspace_bytes, alignment 256 bytes).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *    work is enqueued asynchronously on it; the only host synchronisation is
 *    kron_prepare with info_dev == NULL.
 *  - Host-checkable errors (null pointers, sizes, leading dimensions, bits,
 *    workspace size) are reported before anything is enqueued.  A failed HIP call
 *    returns KQ_ERR_HIP; kron_last_error() then holds the HIP message.
 *  - Floating-point type of every real array is `dtype` (fp32 or fp64).  The
 *    factor preparation always computes in fp64.
 *  - Calls are re-entrant; the only library state is a thread-local error string.
 */
#ifndef KRONQ_H
#define KRONQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KQ_F32 = 0, KQ_F64 = 1 } kq_dtype;

typedef enum {
    KQ_OK = 0,
    KQ_ERR_INVALID_ARG = 1, /* bad pointer, size, leading dimension or option   */
    KQ_ERR_NOT_PD = 2,      /* kron_prepare: damped factor not positive definite */
    KQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required        */
    KQ_ERR_HIP = 4,         /* a HIP runtime call failed                         */
    KQ_ERR_UNSUPPORTED = 5  /* valid request the library does not implement      */
} kq_status;

/* Operation codes for kron_workspace_bytes. */
enum { KQ_OP_FACTOR = 0, KQ_OP_PREPARE = 1, KQ_OP_QUANTIZE = 2, KQ_OP_LOSS = 3 };

/*
 * Base quantizer: a symmetric uniform grid with codes in [-2^(bits-1),
 * 2^(bits-1)-1] and value s * code (WaterKron page section 2.4: scales are chosen
 * up front and handed to the algorithm; FastKron page section 2.1: 'round' is
 * replaced by the map to the closest alphabet element, here round half to even
 * of x / s, then clamp).
 *   bits     2..8
 *   per_row  1: scales has m entries (one per output row); 0: one entry
 *   scales   device array of dtype, each >= 0; a zero scale gives code 0, V = 0
 */
typedef struct {
    int32_t bits;
    int32_t per_row;
    const void* scales;
} kq_quantizer;

/*
 * Workspace bytes needed by an operation (0 if none):
 *   KQ_OP_FACTOR   (m = rows, n = dim)   -> 0
 *   KQ_OP_PREPARE  (m = dim, n ignored)
 *   KQ_OP_QUANTIZE (m, n)                -> covers both the two-sided and B = I modes
 *   KQ_OP_LOSS     (m, n)
 * Returns 0 for invalid arguments as well.
 */
size_t kron_workspace_bytes(int op, kq_dtype dtype, int64_t m, int64_t n);

/*
 * K-FAC factor accumulation: S <- beta * S + alpha * X^T X.
 * FastKron page section 3.2 ('Marginal', an independence assumption) and section
 * 2.6 (accumulating the Hessian from the calibration set): with the N samples of
 * the module input as rows of X and alpha = 1/N, S becomes A = E[a a^T]; with
 * output-gradient rows it becomes B = E[b b^T].
 *   X   rows x dim, leading dimension ldx >= dim
 *   S   dim x dim, lds >= dim; the full symmetric matrix is written.  When beta
 *       is 0, S is not read (it may hold anything).
 * Runs on fp32 / fp64 matrix cores.  No workspace.
 */
kq_status kron_factor_accumulate(kq_dtype dtype, int64_t rows, int64_t dim, const void* X,
                                 int64_t ldx, void* S, int64_t lds, double alpha, double beta,
                                 void* stream);

/*
 * Damped factor: A_d = A + damp_rel * (tr(A) / dim) * I (the small damping that
 * makes PSD factors invertible, WaterKron page section 2 "Notation"), then the
 * upper-triangular U with positive diagonal and U^T U = A_d^{-1}; U^T is the lower
 * Cholesky factor of A_d^{-1} used by the solver (BaKron review, key machinery).
 * Computed in fp64 as U = RevCholesky(A_d)^{-T}: a blocked Cholesky of the
 * index-reversed A_d followed by a blocked triangular inverse.
 *   A          dim x dim symmetric (only read), lda >= dim
 *   U          dim x dim output, ldu >= dim; the strictly lower part is set to 0
 *   trace_out  optional device double: tr(A) before damping
 *   lambda_out optional device double: the added diagonal damp_rel * tr(A) / dim
 *   info_dev   optional device int32.  Non-NULL: the call is asynchronous and
 *              *info_dev becomes 0, or k > 0 when the factorisation (which runs
 *              from the last index of A_d towards the first) met a non-positive
 *              pivot at its k-th step; U is then undefined.  NULL: the call waits
 *              for the stream and returns KQ_ERR_NOT_PD in that case.
 *   ws         workspace of kron_workspace_bytes(KQ_OP_PREPARE, dtype, dim, 0)
 * The KronQ sensitivity score of a sublayer is trace_out(A) * trace_out(B).
 */
kq_status kron_prepare(kq_dtype dtype, int64_t dim, const void* A, int64_t lda, double damp_rel,
                       void* U, int64_t ldu, double* trace_out, double* lambda_out,
                       int32_t* info_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * Scales for the base quantizer from W: s_i = max_j |W_ij| / (2^(bits-1) - 1)
 * per row (per_row = 1, m outputs) or the same over the whole tensor (one
 * output).  A helper for callers; kron_quantize takes any non-negative scales.
 */
kq_status kron_row_scales(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                          int32_t bits, int32_t per_row, void* scales, void* stream);

/*
 * Two-sided GPTQ (FastKron / BaKron): the codes that GPTQ on vecop(W) with Hessian
 * A_d (x) B_d produces (FastKron page section 2.2), computed anti-diagonal by
 * anti-diagonal (section 2.3) with the error feedback batched by a recursion over
 * anti-diagonal ranges (sections 2.4-2.5).  In exact arithmetic every valid
 * processing order gives the same output (section 2.5); in floating point the
 * order of the feedback sums can move values that sit within rounding of a grid
 * midpoint.
 *   W      m x n input weights (not modified), ldw >= n
 *   U_A    n x n upper factor from kron_prepare (U_A^T U_A = A_d^{-1}), lda >= n
 *   U_B    m x m upper factor of B_d, ldb >= m; NULL means B = I, which is
 *          standard one-sided GPTQ with input curvature A
 *   q      base quantizer (see kq_quantizer)
 *   codes  m x n int8 output, ldc >= n
 *   V      m x n output, V_ij = s_i * codes_ij, ldv >= n
 *   loss_dev  optional device double (NULL: not computed): the proxy loss of the
 *          result, tr(B_d (V - W) A_d (V - W)^T) with the damped factors U_A, U_B
 *          stand for, taken from the solver's rounding errors Delta: the error
 *          feedback makes V - W = L~_B Delta L~_A^T (FastKron page section 2.2), so the loss is
 *          sum_ij (Delta_ij / ((U_B)_ii (U_A)_jj))^2, summed in fp64 in a fixed
 *          order.  It equals kron_loss on the same factors up to the rounding of
 *          the feedback sums (about 1e-6 relative in fp32, 1e-12 in fp64);
 *          kron_loss recomputes it from W and V alone.  Must be NULL if m or n is 0.
 *   ws     workspace of kron_workspace_bytes(KQ_OP_QUANTIZE, dtype, m, n)
 * Non-finite W or scales give unspecified codes.
 */
kq_status kron_quantize(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                        const void* U_A, int64_t lda, const void* U_B, int64_t ldb,
                        const kq_quantizer* q, int8_t* codes, int64_t ldc, void* V, int64_t ldv,
                        double* loss_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * Proxy loss D_{A,B} = tr(B_d (V - W) A_d (V - W)^T) (WaterKron page section 1,
 * item 1; FastKron page section 2.2) with E = V - W, A_d = A + damp_rel tr(A)/n I,
 * B_d likewise; damp_rel = 0 gives the undamped loss.  Computed in fp64 as
 * sum_ij (B_d)_ij (E A_d E^T)_ij when n <= m, else sum_ij (A_d)_ij (E^T B_d E)_ij
 * (the same value for symmetric factors, at 3/4 of the flops of forming both
 * B_d E and E A_d when m = n); B = I gives sum_ij E_ij (E A_d)_ij.
 *   A  n x n, B  m x m, both symmetric (each is read as its own transpose);
 *      B = NULL means B = I
 *   loss_dev  device double output
 *   ws  workspace of kron_workspace_bytes(KQ_OP_LOSS, dtype, m, n)
 */
kq_status kron_loss(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                    const void* V, int64_t ldv, const void* A, int64_t lda, const void* B,
                    int64_t ldb, double damp_rel, double* loss_dev, void* ws, size_t ws_bytes,
                    void* stream);

/* Short static description of a status code. */
const char* kron_status_string(kq_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char* kron_last_error(void);

/* ABI version of this header: 2 (kron_quantize gained loss_dev). */
int32_t kron_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KRONQ_H */
