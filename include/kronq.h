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
 *    workspace (size from kron_workspace_bytes, alignment 256 bytes), except for
 *    kron_quantize_noalloc, whose scratch is a fixed array in the library.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *    work is enqueued asynchronously on it; the only host synchronisation is
 *    kron_prepare with info_dev == NULL.
 *  - Host-checkable errors (null pointers, sizes, leading dimensions, bits,
 *    workspace size) are reported before anything is enqueued.  A failed HIP call
 *    returns KQ_ERR_HIP; kron_last_error() then holds the HIP message.
 *  - Floating-point type of every real array is `dtype` (fp32 or fp64).  The
 *    factor preparation always computes in fp64.
 *  - Calls are re-entrant; the only library state is a thread-local error string
 *    (and the per-GPU scratch array of kron_quantize_noalloc).
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
 * anti-diagonal ranges (sections 2.4-2.5).  The matrix is cut into 32 x 32
 * tiles; the recursion's leaves, chunks of 16 tile-diagonals, each run as one
 * persistent launch in which a tile starts as soon as the outputs it reads of
 * the tiles before it in its row and column have arrived (it polls them).
 * Every wait inside that launch is bounded, by 2^18 polls or by the decimal
 * value of the environment variable KQ_CHUNK_SPIN_LIMIT read at the call: a
 * wait that reaches the bound (which the task order rules out for the default)
 * ends the launch early, with NaN in V for the tiles that gave up.  In exact arithmetic every valid
 * processing order gives the same output (section 2.5); in floating point the
 * order of the feedback sums can move values that sit within rounding of a grid
 * midpoint.
 *   W      m x n input weights (not modified), ldw >= n
 *   U_A    n x n upper factor from kron_prepare (U_A^T U_A = A_d^{-1}), lda >= n
 *   U_B    m x m upper factor of B_d, ldb >= m; NULL means B = I, which is
 *          standard one-sided GPTQ with input curvature A: every row is then its
 *          own problem, and the library runs the recursive lazily batched GPTQ
 *          of FastKron page section 2.4 (column ranges halved down to 64-column
 *          leaves, the feedback between them as dense products), at one-sided cost
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
 * kron_quantize with the two-sided leaves launched one kernel per tile-diagonal
 * instead of on the persistent wavefront solver.  The codes, V and loss are
 * bitwise those of kron_quantize (the same operations in the same order); only
 * the schedule differs.  kron_quantize runs each chunk of 16 tile-diagonals of
 * 32 x 32 tiles in one persistent launch whose workgroups hold a compute unit
 * while they wait for the tiles before them (FastKron page, section 2.3: the
 * tiles of a tile-diagonal are independent; BaKron review, key_machinery: a
 * wavefront over anti-diagonals); this call never waits inside a kernel, so it
 * is the one for callers that share the GPU with other long-running work.  At
 * 4096 x 4096 fp32 on MI355X it takes about 4.7 ms against 4.3 ms.  Arguments,
 * workspace (the same size), errors and U_B = NULL (the one-sided path,
 * unchanged) are as for kron_quantize.
 */
kq_status kron_quantize_per_diagonal(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                                     const void* U_A, int64_t lda, const void* U_B, int64_t ldb,
                                     const kq_quantizer* q, int8_t* codes, int64_t ldc, void* V,
                                     int64_t ldv, double* loss_dev, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * WaterKron two-sided rate allocation (WaterKron page, section 3; section 2.4
 * for WaterSIC, its B = I case): the column scales alpha_j proportional to
 * 1 / L^(A)_jj and row scales beta_i proportional to 1 / L^(B)_ii, L the reverse
 * Cholesky factor of the damped factor.  With U from kron_prepare,
 * U = RevCholesky(A_d)^{-T}, so 1 / L_jj = U_jj:
 *   alpha_j = step * U_A[j][j]   (the product formed in fp64, rounded once)
 *   beta_i  = U_B[i][i]          (1 when U_B is NULL, B = I)
 * `step` (> 0) is the free proportionality constant: the grid step in the
 * geometry where every entry's rounding error weighs the same in the loss.
 *   alpha  device array of n entries of dtype (output)
 *   beta   device array of m entries of dtype (output)
 */
kq_status kron_waterkron_scales(kq_dtype dtype, int64_t m, int64_t n, const void* U_A, int64_t lda,
                                const void* U_B, int64_t ldb, double step, void* alpha, void* beta,
                                void* stream);

/*
 * Two-sided GPTQ with the WaterKron alphabet (WaterKron page, section 2.1):
 * entry (i, j) of V is beta_i alpha_j Z_ij with Z an unbounded integer matrix
 * (meant for entropy coding).  The solver is kron_quantize's, with the grid
 * step of entry (i, j) s_ij = beta_i * alpha_j (one rounding in dtype) and
 * z_ij = rne(x_ij / s_ij) without clipping (codes are held as int32 and clamped
 * only at +-2^30).  U_B = NULL is WaterSIC (one-sided, column scales only when
 * beta = 1).
 *   alpha  n column scales (> 0), beta  m row scales (> 0), device, dtype
 *   codes  m x n int32 output, ldc >= n
 *   V      m x n output, V_ij = (beta_i alpha_j) codes_ij
 *   loss_dev, ws  as for kron_quantize (same workspace size)
 */
kq_status kron_quantize_waterkron(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                                  const void* U_A, int64_t lda, const void* U_B, int64_t ldb,
                                  const void* alpha, const void* beta, int32_t* codes, int64_t ldc,
                                  void* V, int64_t ldv, double* loss_dev, void* ws, size_t ws_bytes,
                                  void* stream);

/* Kronecker approximation methods for kron_factor_kronecker. */
typedef enum { KQ_KRON_FROBENIUS = 0, KQ_KRON_FLIPFLOP = 1 } kq_kron_method;

/* Workspace bytes of kron_factor_kronecker for N samples, n inputs, m outputs
 * (0 for invalid arguments). */
size_t kron_kronecker_workspace_bytes(kq_dtype dtype, int64_t samples, int64_t n, int64_t m);

/*
 * Kronecker approximation A (x) B of H = E[a a^T (x) b b^T] from paired samples
 * (WaterKron page, section 5 and Table 1; FastKron page section 3.2): the
 * alternating fixed-point iteration started from B_0 = I, `iters` full updates
 * (A, then B):
 *   KQ_KRON_FLIPFLOP   A <- (1/(N m)) sum_s (b_s^T B_d^{-1} b_s) a_s a_s^T,
 *                      B <- (1/(N n)) sum_s (a_s^T A_d^{-1} a_s) b_s b_s^T
 *                      (the flip-flop matrix-normal maximum-likelihood iteration
 *                      the WaterKron page cites; M_d = M + damp_rel tr(M)/d I)
 *   KQ_KRON_FROBENIUS  A <- sum_s (b_s^T B b_s) a_s a_s^T / (N ||B||_F^2),
 *                      B <- sum_s (a_s^T A a_s) b_s b_s^T / (N ||A||_F^2)
 *                      (alternating least squares for ||H - A (x) B||_F; damp_rel
 *                      unused)
 * iters = 1 with FlipFlop and damp_rel = 0 gives A = E[|b|^2 a a^T] / m.
 *   Xa  N x n activation rows (ldxa >= n), Xb  N x m gradient rows (ldxb >= m),
 *       row s of both is one sample
 *   A   n x n output (lda >= n), B  m x m output (ldb >= m), full symmetric
 *   iters     1..64
 *   info_dev  FlipFlop only, as for kron_prepare: non-NULL receives 0 or the
 *             failing pivot step of the first damped factor that was not
 *             positive definite (asynchronous); NULL makes the call wait and
 *             return KQ_ERR_NOT_PD in that case
 *   ws  workspace of kron_kronecker_workspace_bytes(dtype, N, n, m)
 */
kq_status kron_factor_kronecker(kq_dtype dtype, int32_t method, int64_t samples, int64_t n, int64_t m,
                                const void* Xa, int64_t ldxa, const void* Xb, int64_t ldxb, int32_t iters,
                                double damp_rel, void* A, int64_t lda, void* B, int64_t ldb,
                                int32_t* info_dev, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of kron_biip_forward / kron_biip_inverse (0 if invalid). */
size_t kron_biip_workspace_bytes(kq_dtype dtype, int64_t m, int64_t n);

/*
 * KronQ bidirectional incoherence processing (KronQ page, section
 * "Kronecker-Factored Quantization": BiIP and Theorem 1).  With
 * s_A = diag(A)^{-1/4}, s_B = diag(B)^{-1/4} (1 where a diagonal entry is not
 * positive) and the randomised Walsh-Hadamard rotations Q = (I (x) H_h/sqrt(h))
 * diag(signs) (Sylvester H_h on blocks of h = the largest power of two dividing
 * the dimension, at most 4096; signs are +-1 drawn by the caller):
 *   W_out = Q_B S_B W S_A Q_A^T              (m x n)
 *   A_out = Q_A S_A^{-1} A S_A^{-1} Q_A^T     (n x n)
 *   B_out = Q_B S_B^{-1} B S_B^{-1} Q_B^T     (m x m)
 * so tr(B E A E^T) is unchanged when E is mapped back by kron_biip_inverse.
 * Quantize W_out with factors from A_out, B_out, then map V back.
 *   signs_n, signs_m  device int8 arrays of n and m entries (negative: -1)
 *   scale_a, scale_b  device outputs s_A (n), s_B (m), dtype; kron_biip_inverse
 *                     takes them back
 *   ws  workspace of kron_biip_workspace_bytes(dtype, m, n)
 * Every pass reads and writes its matrix once (HBM-bound).
 */
kq_status kron_biip_forward(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* A,
                            int64_t lda, const void* B, int64_t ldb, const int8_t* signs_n,
                            const int8_t* signs_m, void* W_out, int64_t ldwo, void* A_out, int64_t ldao,
                            void* B_out, int64_t ldbo, void* scale_a, void* scale_b, void* ws,
                            size_t ws_bytes, void* stream);

/* V = S_B^{-1} Q_B^T V2 Q_A S_A^{-1}: a result of the processed problem (m x n)
 * back in the original coordinates, with the signs and scales of the forward
 * call.  Same workspace. */
kq_status kron_biip_inverse(kq_dtype dtype, int64_t m, int64_t n, const void* V2, int64_t ldv2,
                            const int8_t* signs_n, const int8_t* signs_m, const void* scale_a,
                            const void* scale_b, void* V, int64_t ldv, void* ws, size_t ws_bytes,
                            void* stream);

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

/*
 * For callers that cannot allocate device memory (code under HIP stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): kron_quantize
 * with the same arguments and results but no workspace argument.  Its scratch
 * space is a fixed array of KQ_NOALLOC_SCRATCH_BYTES in the library's device
 * memory, one per GPU, held from the library's first use on that GPU until the
 * process ends; the call itself allocates nothing.  The array is found on the
 * device that is current at the call, which must be the device of `stream`.
 *   - Sizes whose scratch need (kron_workspace_bytes(KQ_OP_QUANTIZE, dtype, m,
 *     n)) exceeds KQ_NOALLOC_SCRATCH_BYTES return KQ_ERR_WORKSPACE before
 *     anything is enqueued: e.g. fp32 up to 1600 x 1600 two-sided fits.
 *   - Every call on one GPU uses that GPU's single array: calls that overlap on
 *     one GPU (other streams, other threads) race and give undefined results.
 *     Calls ordered on one stream are safe.
 */
#define KQ_NOALLOC_SCRATCH_BYTES (64u << 20)
kq_status kron_quantize_noalloc(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                                const void* U_A, int64_t lda, const void* U_B, int64_t ldb,
                                const kq_quantizer* q, int8_t* codes, int64_t ldc, void* V, int64_t ldv,
                                double* loss_dev, void* stream);

/* Short static description of a status code. */
const char* kron_status_string(kq_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char* kron_last_error(void);

/* ABI version of this header: 4 (2: kron_quantize gained loss_dev; 3: the WaterKron
 * entry points, kron_factor_kronecker, the BiIP transforms and kron_quantize_noalloc;
 * 4: kron_quantize on the persistent wavefront solver, kron_quantize_per_diagonal). */
int32_t kron_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KRONQ_H */
