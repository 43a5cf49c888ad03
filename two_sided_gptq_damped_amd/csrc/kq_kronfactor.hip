// Kronecker approximations H ~ A (x) B of H = E[a a^T (x) b b^T] from paired
// samples (rows a_s of Xa, N x n, and b_s of Xb, N x m), for gfx950.
//
// What is computed (WaterKron page, section 5 and Table 1: alternating
// fixed-point iterations started from the identity; FastKron page section 3.2):
//   FlipFlop   A_{k+1} = (1/(N m)) sum_s (b_s^T B_k,d^{-1} b_s) a_s a_s^T
//              B_{k+1} = (1/(N n)) sum_s (a_s^T A_{k+1},d^{-1} a_s) b_s b_s^T
//              (the flip-flop matrix-normal maximum-likelihood iteration the
//              page cites, with the damped inverses M_d = M + delta tr(M)/d I)
//   Frobenius  A_{k+1} = sum_s (b_s^T B_k b_s) a_s a_s^T / (N ||B_k||_F^2)
//              B_{k+1} = sum_s (a_s^T A_{k+1} a_s) b_s b_s^T / (N ||A_{k+1}||_F^2)
//              (the same iteration with A_{k+1}, B_k in place of their
//              inverses: alternating least squares for ||H - A (x) B||_F)
// B_0 = I.  Each half-step is
//   1. the per-sample weights q_s = x_s^T M x_s: for FlipFlop M = M_d^{-1} =
//      U^T U with U from the library's damped factor preparation, so
//      q_s = ||U x_s||^2; for Frobenius M is the factor itself.  Both are one
//      product X Op(M) on the matrix cores whose 64 x 64 tiles reduce their
//      rows on the way out (squares, or products with X), partial sums per
//      (sample, column tile) in fp64, then a fixed-order row sum;
//   2. Y = diag(q_s c) X with c = 1/m (1/n) or 1/||M||_F^2;
//   3. the new factor (1/N) X^T Y with the library's SYRK tiles.
#include <algorithm>

#include "kq_common.hpp"

namespace kq {

kq_status syrk_dispatch(kq_dtype, int64_t, int64_t, const void*, int64_t, const void*, int64_t, void*, int64_t, double,
                        double, hipStream_t);
size_t prepare_workspace_bytes(int64_t d);
kq_status prepare_dispatch(kq_dtype, int64_t, const void*, int64_t, double, void*, int64_t, double*, double*,
                           int32_t*, void*, hipStream_t);

// Partial sums of q_s over column tile Q: rows 64 P .. 64 P + 63 of X (N x d)
// times Op(M)'s columns 64 Q ..  TRI: Op(M)(k, c) = U[c][k] (U upper, so only
// k >= 64 Q contributes) and the partial is sum_c (X U^T)[s][c]^2.  Otherwise
// Op(M) = M (symmetric) and the partial is sum_c (X M)[s][c] X[s][c].
template <typename T, bool TRI>
__global__ __launch_bounds__(GEMM_THREADS) void quadform_partial_kernel(const T* __restrict__ X, int64_t ldx,
                                                                        const T* __restrict__ M, int64_t ldm, int N,
                                                                        int d, int tiles, double* __restrict__ part) {
    __shared__ GemmSmem<T> sm;
    __shared__ double red[TILE][TILE + 1];
    const int Q = blockIdx.x, P = blockIdx.y;
    const int k0 = TRI ? Q * TILE : 0;
    WaveAcc<T> acc;
    acc.zero();
    const T* A = X + int64_t(P) * TILE * ldx + k0;
    if (TRI)  // B(k, c) = U[64 Q + c][k0 + k]
        tile_gemm<T, T, false, true, true>(A, ldx, M + int64_t(Q) * TILE * ldm + k0, ldm, N - P * TILE, d - Q * TILE,
                                           d - k0, sm, acc);
    else  // B(k, c) = M[k][64 Q + c]
        tile_gemm<T, T, false, false, true>(A, ldx, M + Q * TILE, ldm, N - P * TILE, d - Q * TILE, d, sm, acc);
    for_each_acc(acc, [&](int r, int c, T v) {
        double e = 0.0;
        const int s = P * TILE + r, j = Q * TILE + c;
        if (s < N && j < d) e = TRI ? double(v) * double(v) : double(v) * double(X[int64_t(s) * ldx + j]);
        red[r][c] = e;
    });
    __syncthreads();
    if (threadIdx.x < TILE) {
        const int s = P * TILE + threadIdx.x;
        double t = 0.0;
        for (int c = 0; c < TILE; ++c) t += red[threadIdx.x][c];
        if (s < N) part[int64_t(s) * tiles + Q] = t;
    }
}

// Y[s][:] = (q_s * coef) X[s][:] with q_s = sum of the row's partials (fixed
// order) and coef = scale, divided by *norm when norm is given.
template <typename T>
__global__ void scale_rows_kernel(const T* __restrict__ X, int64_t ldx, int N, int d, const double* __restrict__ part,
                                  int tiles, double scale, const double* __restrict__ norm, T* __restrict__ Y,
                                  int64_t ldy) {
    const int s = blockIdx.x;
    if (s >= N) return;
    double q = 0.0;
    for (int t = 0; t < tiles; ++t) q += part[int64_t(s) * tiles + t];
    const double c = norm ? scale / *norm : scale;
    const T f = T(q * c);
    for (int j = threadIdx.x; j < d; j += blockDim.x) Y[int64_t(s) * ldy + j] = f * X[int64_t(s) * ldx + j];
}

// ||M||_F^2 of a d x d matrix in fp64, fixed order: FROB_PARTS workgroups take
// rows round-robin, then one workgroup adds their sums.
constexpr int FROB_PARTS = 512;

template <typename T>
__global__ __launch_bounds__(256) void frob2_partial_kernel(const T* __restrict__ M, int64_t ldm, int d,
                                                            double* __restrict__ part) {
    __shared__ double red[256];
    double t = 0.0;
    for (int i = blockIdx.x; i < d; i += gridDim.x)
        for (int j = threadIdx.x; j < d; j += 256) {
            const double v = double(M[int64_t(i) * ldm + j]);
            t = __builtin_fma(v, v, t);
        }
    const double tot = block_sum_256(t, red);
    if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void frob2_final_kernel(const double* __restrict__ part, double* __restrict__ out) {
    __shared__ double red[256];
    double t = 0.0;
    for (int i = threadIdx.x; i < FROB_PARTS; i += 256) t += part[i];
    const double tot = block_sum_256(t, red);
    if (threadIdx.x == 0) *out = tot;
}

template <typename T>
__global__ void identity_kernel(T* __restrict__ M, int64_t ldm, int d) {
    const int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (e >= int64_t(d) * d) return;
    const int i = int(e / d), j = int(e % d);
    M[int64_t(i) * ldm + j] = i == j ? T(1) : T(0);
}

// out = the first nonzero of info[0 .. count) (0 if none).
__global__ void first_nonzero_kernel(const int32_t* __restrict__ info, int count, int32_t* __restrict__ out) {
    if (threadIdx.x != 0) return;
    int32_t v = 0;
    for (int i = 0; i < count && v == 0; ++i) v = info[i];
    *out = v;
}

__global__ void zero_ints_kernel(int32_t* __restrict__ p, int count) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

constexpr int KRON_MAX_ITERS = 64;

struct KronLayout {
    size_t off_U, off_pws, off_Y, off_part, off_scal, off_info, bytes;
};

static KronLayout kron_layout(kq_dtype dtype, int64_t N, int64_t n, int64_t m) {
    const size_t es = dtype == KQ_F64 ? 8 : 4;
    const int64_t d = std::max(n, m);
    const int64_t ldy = round_up(d, 4);
    KronLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    L.off_U = take(size_t(d) * size_t(d) * es);
    L.off_pws = take(prepare_workspace_bytes(d));
    L.off_Y = take(size_t(N) * size_t(ldy) * es);
    L.off_part = take(size_t(N) * size_t((d + TILE - 1) / TILE) * sizeof(double));
    L.off_scal = take((FROB_PARTS + 1) * sizeof(double));
    L.off_info = take(2 * KRON_MAX_ITERS * sizeof(int32_t));
    L.bytes = off;
    return L;
}

size_t kronecker_workspace_bytes(kq_dtype dtype, int64_t N, int64_t n, int64_t m) {
    return kron_layout(dtype, N, n, m).bytes;
}

template <typename T>
static kq_status kronecker_typed(int method, int64_t N, int64_t n, int64_t m, const T* Xa, int64_t ldxa, const T* Xb,
                                 int64_t ldxb, int iters, double damp_rel, T* A, int64_t lda, T* B, int64_t ldb,
                                 int32_t* info_dev, void* ws, hipStream_t st) {
    const kq_dtype dtype = sizeof(T) == 8 ? KQ_F64 : KQ_F32;
    const KronLayout L = kron_layout(dtype, N, n, m);
    char* base = static_cast<char*>(ws);
    T* U = reinterpret_cast<T*>(base + L.off_U);
    void* pws = base + L.off_pws;
    T* Y = reinterpret_cast<T*>(base + L.off_Y);
    double* part = reinterpret_cast<double*>(base + L.off_part);
    double* norm = reinterpret_cast<double*>(base + L.off_scal);
    int32_t* info = reinterpret_cast<int32_t*>(base + L.off_info);
    const bool flipflop = method == KQ_KRON_FLIPFLOP;

    hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(2 * KRON_MAX_ITERS), 0, st, info, 2 * KRON_MAX_ITERS);
    KQ_LAUNCHED("zero_ints_kernel");
    hipLaunchKernelGGL(identity_kernel<T>, dim3(unsigned((m * m + 255) / 256)), dim3(256), 0, st, B, ldb, int(m));
    KQ_LAUNCHED("identity_kernel");

    // One half-step: the factor F (d_out x d_out) from samples Xo weighted by the
    // quadratic forms of the other factor G (d_in x d_in) on its samples Xi.
    auto half = [&](const T* G, int64_t ldg, int64_t d_in, const T* Xi, int64_t ldxi, const T* Xo, int64_t ldxo,
                    int64_t d_out, T* F, int64_t ldf, int32_t* inf) -> kq_status {
        const int tiles = int((d_in + TILE - 1) / TILE);
        const dim3 grid(unsigned(tiles), unsigned((N + TILE - 1) / TILE));
        if (flipflop) {
            kq_status s = prepare_dispatch(dtype, d_in, G, ldg, damp_rel, U, d_in, nullptr, nullptr, inf, pws, st);
            if (s != KQ_OK) return s;
            hipLaunchKernelGGL((quadform_partial_kernel<T, true>), grid, dim3(GEMM_THREADS), 0, st, Xi, ldxi, U, d_in,
                               int(N), int(d_in), tiles, part);
        } else {
            hipLaunchKernelGGL(frob2_partial_kernel<T>, dim3(FROB_PARTS), dim3(256), 0, st, G, ldg, int(d_in),
                               norm + 1);
            KQ_LAUNCHED("frob2_partial_kernel");
            hipLaunchKernelGGL(frob2_final_kernel, dim3(1), dim3(256), 0, st, norm + 1, norm);
            KQ_LAUNCHED("frob2_final_kernel");
            hipLaunchKernelGGL((quadform_partial_kernel<T, false>), grid, dim3(GEMM_THREADS), 0, st, Xi, ldxi, G, ldg,
                               int(N), int(d_in), tiles, part);
        }
        KQ_LAUNCHED("quadform_partial_kernel");
        const int64_t ldy = round_up(d_out, 4);
        hipLaunchKernelGGL(scale_rows_kernel<T>, dim3(unsigned(N)), dim3(256), 0, st, Xo, ldxo, int(N), int(d_out),
                           part, tiles, flipflop ? 1.0 / double(d_in) : 1.0, flipflop ? nullptr : norm, Y, ldy);
        KQ_LAUNCHED("scale_rows_kernel");
        return syrk_dispatch(dtype, N, d_out, Xo, ldxo, Y, ldy, F, ldf, 1.0 / double(N), 0.0, st);
    };
    for (int k = 0; k < iters; ++k) {
        kq_status s = half(B, ldb, m, Xb, ldxb, Xa, ldxa, n, A, lda, info + 2 * k);
        if (s != KQ_OK) return s;
        s = half(A, lda, n, Xa, ldxa, Xb, ldxb, m, B, ldb, info + 2 * k + 1);
        if (s != KQ_OK) return s;
    }
    if (info_dev) {
        hipLaunchKernelGGL(first_nonzero_kernel, dim3(1), dim3(64), 0, st, info, 2 * iters, info_dev);
        KQ_LAUNCHED("first_nonzero_kernel");
    } else if (flipflop) {
        int32_t h[2 * KRON_MAX_ITERS];
        KQ_HIP(hipMemcpyAsync(h, info, sizeof(int32_t) * 2 * iters, hipMemcpyDeviceToHost, st));
        KQ_HIP(hipStreamSynchronize(st));
        for (int i = 0; i < 2 * iters; ++i)
            if (h[i] != 0) {
                set_error("kron_factor_kronecker: a damped factor of iteration " + std::to_string(i / 2 + 1) +
                          " is not positive definite (pivot step " + std::to_string(h[i]) + ")");
                return KQ_ERR_NOT_PD;
            }
    }
    return KQ_OK;
}

kq_status kronecker_dispatch(kq_dtype dtype, int method, int64_t N, int64_t n, int64_t m, const void* Xa,
                             int64_t ldxa, const void* Xb, int64_t ldxb, int iters, double damp_rel, void* A,
                             int64_t lda, void* B, int64_t ldb, int32_t* info_dev, void* ws, hipStream_t st) {
    if (dtype == KQ_F64)
        return kronecker_typed<double>(method, N, n, m, static_cast<const double*>(Xa), ldxa,
                                       static_cast<const double*>(Xb), ldxb, iters, damp_rel, static_cast<double*>(A),
                                       lda, static_cast<double*>(B), ldb, info_dev, ws, st);
    return kronecker_typed<float>(method, N, n, m, static_cast<const float*>(Xa), ldxa, static_cast<const float*>(Xb),
                                  ldxb, iters, damp_rel, static_cast<float*>(A), lda, static_cast<float*>(B), ldb,
                                  info_dev, ws, st);
}

}  // namespace kq
