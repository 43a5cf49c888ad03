// Factor preparation for two-sided GPTQ, computed in fp64 on gfx950.
//
// A_d = A + damp_rel * (tr A / d) I (WaterKron page, section 2 "Notation": a
// small damping makes the PSD factors invertible), then the upper-triangular U
// with U^T U = A_d^{-1} (its transpose is the lower Cholesky factor of the
// inverse used by the solver; pith.science review of BaKron, key machinery).
//
// Route: U = RevCholesky(A_d)^{-T} with RevCholesky(M) the lower L, L^T L = M
// (WaterKron page notation).  With J the index reversal and C = J A_d J:
// C = L_c L_c^T (ordinary Cholesky), RevCholesky(A_d) = J L_c^T J and therefore
// U = J L_c^{-1} J.  Steps, all on 64 x 64 fp64 blocks of a padded dp x dp copy:
//   1. trace and damping; C = J A_d J (identity in the padding)
//   2. right-looking blocked Cholesky: diagonal-block factor + its inverse,
//      panel (C_ik <- C_ik L_kk^{-T}) and trailing update (C_ij -= C_ik C_jk^T),
//      the last two on fp64 matrix cores
//   3. blocked lower-triangular inverse, one block row at a time:
//      Li_ik = -L_ii^{-1} sum_{k<=j<i} L_ij Li_jk
//   4. U[r][c] = Li[d-1-r][d-1-c] for c >= r, 0 below the diagonal.
#include "kq_common.hpp"

namespace kq {

template <typename TIn>
__global__ void trace_kernel(const TIn* __restrict__ A, int64_t lda, int d, double* __restrict__ out) {
    __shared__ double red[1024];
    double s = 0.0;
    for (int i = threadIdx.x; i < d; i += blockDim.x) s += double(A[int64_t(i) * lda + i]);
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (int(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = red[0];
}

__global__ void set_int_kernel(int32_t* p, int32_t v) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

template <typename TIn>
__global__ void build_reversed_kernel(const TIn* __restrict__ A, int64_t lda, int d, int dp,
                                      const double* __restrict__ trace, double damp_rel,
                                      double* __restrict__ C, double* trace_out, double* lambda_out) {
    const double lam = damp_rel * (*trace) / double(d);
    const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (idx == 0) {
        if (trace_out) *trace_out = *trace;
        if (lambda_out) *lambda_out = lam;
    }
    if (idx >= int64_t(dp) * dp) return;
    const int i = int(idx / dp), j = int(idx % dp);
    double v;
    if (i < d && j < d)
        v = double(A[int64_t(d - 1 - i) * lda + (d - 1 - j)]) + (i == j ? lam : 0.0);
    else
        v = (i == j) ? 1.0 : 0.0;
    C[idx] = v;
}

// Cholesky of the diagonal block C[k][k] in LDS (unblocked, right-looking), and
// the inverse of the factor by forward substitution.  Writes L (zero above the
// diagonal) back into C and L^{-1} into Dinv[k].  A pivot that is not > 0
// records its 1-based position in *info (first failure only) and continues
// with a unit pivot so the remaining kernels stay finite.
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ C, int dp, int k,
                                                         double* __restrict__ Dinv, int32_t* __restrict__ info) {
    constexpr int P = TILE + 1;
    __shared__ double L[TILE * P];
    __shared__ double X[TILE * P];
    __shared__ int failed;
    const int t = threadIdx.x;
    double* blk = C + int64_t(k) * TILE * dp + int64_t(k) * TILE;
    for (int e = t; e < TILE * TILE; e += 256) L[(e >> 6) * P + (e & 63)] = blk[int64_t(e >> 6) * dp + (e & 63)];
    if (t == 0) failed = 0;
    __syncthreads();
    for (int j = 0; j < TILE; ++j) {
        if (t == 0) {
            double p = L[j * P + j];
            if (!(p > 0.0)) {
                if (!failed && *info == 0) *info = k * TILE + j + 1;
                failed = 1;
                p = 1.0;
            }
            L[j * P + j] = sqrt(p);
        }
        __syncthreads();
        const double piv = L[j * P + j];
        for (int i = j + 1 + t; i < TILE; i += 256) L[i * P + j] /= piv;
        __syncthreads();
        // trailing lower triangle: rows i > j, columns c in (j, i]
        const int rem = TILE - 1 - j;
        for (int e = t; e < rem * rem; e += 256) {
            const int i = j + 1 + e / rem, c = j + 1 + e % rem;
            if (c <= i) L[i * P + c] -= L[i * P + j] * L[c * P + j];
        }
        __syncthreads();
    }
    // inverse of the lower factor, one column per thread
    if (t < TILE) {
        const int c = t;
        for (int i = 0; i < TILE; ++i) {
            double x;
            if (i < c) {
                x = 0.0;
            } else {
                double s = (i == c) ? 1.0 : 0.0;
                for (int j = c; j < i; ++j) s -= L[i * P + j] * X[j * P + c];
                x = s / L[i * P + i];
            }
            X[i * P + c] = x;
        }
    }
    __syncthreads();
    double* dinv = Dinv + int64_t(k) * TILE * TILE;
    for (int e = t; e < TILE * TILE; e += 256) {
        const int r = e >> 6, c = e & 63;
        blk[int64_t(r) * dp + c] = c <= r ? L[r * P + c] : 0.0;
        dinv[e] = X[r * P + c];
    }
}

// C[i][k] <- C[i][k] * Dinv[k]^T for the block rows i > k.
__global__ __launch_bounds__(GEMM_THREADS) void potrf_panel_kernel(double* __restrict__ C, int dp, int k,
                                                                   const double* __restrict__ Dinv) {
    __shared__ GemmSmem<double> sm;
    const int i = k + 1 + blockIdx.x;
    double* blk = C + int64_t(i) * TILE * dp + int64_t(k) * TILE;
    WaveAcc<double> acc;
    acc.zero();
    // B(kk, c) = Dinv[k][c][kk]
    tile_gemm<double, double, false, true, false>(blk, dp, Dinv + int64_t(k) * TILE * TILE, TILE, TILE, TILE, TILE, sm,
                                                  acc);
    __syncthreads();
    for_each_acc(acc, [&](int r, int c, double v) { blk[int64_t(r) * dp + c] = v; });
}

// C[i][j] -= C[i][k] C[j][k]^T for k < j <= i.
__global__ __launch_bounds__(GEMM_THREADS) void potrf_trailing_kernel(double* __restrict__ C, int dp, int k) {
    const int i = k + 1 + blockIdx.y, j = k + 1 + blockIdx.x;
    if (j > i) return;
    __shared__ GemmSmem<double> sm;
    WaveAcc<double> acc;
    acc.zero();
    const double* A = C + int64_t(i) * TILE * dp + int64_t(k) * TILE;
    const double* B = C + int64_t(j) * TILE * dp + int64_t(k) * TILE;  // B(kk, c) = C[j*64+c][k*64+kk]
    tile_gemm<double, double, false, true, false>(A, dp, B, dp, TILE, TILE, TILE, sm, acc);
    double* out = C + int64_t(i) * TILE * dp + int64_t(j) * TILE;
    for_each_acc(acc, [&](int r, int c, double v) { out[int64_t(r) * dp + c] -= v; });
}

// Block row i of the inverse, first part: Li[i][k] = sum_{k<=j<i} L[i][j] Li[j][k]
// for k < i (grid.x = i), plus Li[i][i] = Dinv[i] (block grid.x == i).
__global__ __launch_bounds__(GEMM_THREADS) void trtri_row_kernel(const double* __restrict__ C, double* __restrict__ Li,
                                                                 int dp, int i, const double* __restrict__ Dinv) {
    const int k = blockIdx.x;
    double* out = Li + int64_t(i) * TILE * dp + int64_t(k) * TILE;
    if (k == i) {
        const double* src = Dinv + int64_t(i) * TILE * TILE;
        for (int e = threadIdx.x; e < TILE * TILE; e += GEMM_THREADS) out[int64_t(e >> 6) * dp + (e & 63)] = src[e];
        return;
    }
    __shared__ GemmSmem<double> sm;
    WaveAcc<double> acc;
    acc.zero();
    const double* A = C + int64_t(i) * TILE * dp + int64_t(k) * TILE;   // L[i][k..i-1]
    const double* B = Li + int64_t(k) * TILE * dp + int64_t(k) * TILE;  // Li[k..i-1][k]
    tile_gemm<double, double, false, false, false>(A, dp, B, dp, TILE, TILE, (i - k) * TILE, sm, acc);
    for_each_acc(acc, [&](int r, int c, double v) { out[int64_t(r) * dp + c] = v; });
}

// Second part: Li[i][k] <- -Dinv[i] Li[i][k] for k < i.
__global__ __launch_bounds__(GEMM_THREADS) void trtri_scale_kernel(double* __restrict__ Li, int dp, int i,
                                                                   const double* __restrict__ Dinv) {
    const int k = blockIdx.x;
    double* blk = Li + int64_t(i) * TILE * dp + int64_t(k) * TILE;
    __shared__ GemmSmem<double> sm;
    WaveAcc<double> acc;
    acc.zero();
    tile_gemm<double, double, false, false, false>(Dinv + int64_t(i) * TILE * TILE, TILE, blk, dp, TILE, TILE, TILE,
                                                   sm, acc);
    __syncthreads();
    for_each_acc(acc, [&](int r, int c, double v) { blk[int64_t(r) * dp + c] = -v; });
}

template <typename TOut>
__global__ void flip_kernel(const double* __restrict__ Li, int dp, int d, TOut* __restrict__ U, int64_t ldu) {
    const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (idx >= int64_t(d) * d) return;
    const int r = int(idx / d), c = int(idx % d);
    U[int64_t(r) * ldu + c] = c >= r ? TOut(Li[int64_t(d - 1 - r) * dp + (d - 1 - c)]) : TOut(0);
}

// ------------------------------------------------------------------- host side

struct PrepareLayout {
    int64_t dp, nt;
    size_t off_C, off_Li, off_Dinv, off_scal, bytes;
};

PrepareLayout prepare_layout(int64_t d) {
    PrepareLayout L;
    L.dp = round_up(d, TILE);
    L.nt = L.dp / TILE;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    L.off_C = take(size_t(L.dp) * L.dp * 8);
    L.off_Li = take(size_t(L.dp) * L.dp * 8);
    L.off_Dinv = take(size_t(L.nt) * TILE * TILE * 8);
    L.off_scal = take(64);
    L.bytes = off;
    return L;
}

size_t prepare_workspace_bytes(int64_t d) { return prepare_layout(d).bytes; }

template <typename T>
kq_status prepare_typed(int64_t d, const T* A, int64_t lda, double damp_rel, T* U, int64_t ldu, double* trace_out,
                        double* lambda_out, int32_t* info_dev, void* ws, hipStream_t st) {
    const PrepareLayout L = prepare_layout(d);
    char* base = static_cast<char*>(ws);
    double* C = reinterpret_cast<double*>(base + L.off_C);
    double* Li = reinterpret_cast<double*>(base + L.off_Li);
    double* Dinv = reinterpret_cast<double*>(base + L.off_Dinv);
    double* trace = reinterpret_cast<double*>(base + L.off_scal);
    int32_t* info_ws = reinterpret_cast<int32_t*>(base + L.off_scal + 16);
    int32_t* info = info_dev ? info_dev : info_ws;
    const int dp = int(L.dp), nt = int(L.nt);

    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(64), 0, st, info, 0);
    KQ_LAUNCHED("set_int_kernel");
    hipLaunchKernelGGL(trace_kernel<T>, dim3(1), dim3(1024), 0, st, A, lda, int(d), trace);
    KQ_LAUNCHED("trace_kernel");
    const int64_t cnt = int64_t(dp) * dp;
    hipLaunchKernelGGL(build_reversed_kernel<T>, dim3(unsigned((cnt + 255) / 256)), dim3(256), 0, st, A, lda, int(d),
                       dp, trace, damp_rel, C, trace_out, lambda_out);
    KQ_LAUNCHED("build_reversed_kernel");
    for (int k = 0; k < nt; ++k) {
        hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, st, C, dp, k, Dinv, info);
        KQ_LAUNCHED("potrf_diag_kernel");
        const int rest = nt - k - 1;
        if (rest > 0) {
            hipLaunchKernelGGL(potrf_panel_kernel, dim3(rest), dim3(GEMM_THREADS), 0, st, C, dp, k, Dinv);
            KQ_LAUNCHED("potrf_panel_kernel");
            hipLaunchKernelGGL(potrf_trailing_kernel, dim3(rest, rest), dim3(GEMM_THREADS), 0, st, C, dp, k);
            KQ_LAUNCHED("potrf_trailing_kernel");
        }
    }
    for (int i = 0; i < nt; ++i) {
        hipLaunchKernelGGL(trtri_row_kernel, dim3(i + 1), dim3(GEMM_THREADS), 0, st, C, Li, dp, i, Dinv);
        KQ_LAUNCHED("trtri_row_kernel");
        if (i > 0) {
            hipLaunchKernelGGL(trtri_scale_kernel, dim3(i), dim3(GEMM_THREADS), 0, st, Li, dp, i, Dinv);
            KQ_LAUNCHED("trtri_scale_kernel");
        }
    }
    const int64_t ucnt = d * d;
    hipLaunchKernelGGL(flip_kernel<T>, dim3(unsigned((ucnt + 255) / 256)), dim3(256), 0, st, Li, dp, int(d), U, ldu);
    KQ_LAUNCHED("flip_kernel");
    if (!info_dev) {
        int32_t h = 0;
        KQ_HIP(hipMemcpyAsync(&h, info_ws, sizeof(int32_t), hipMemcpyDeviceToHost, st));
        KQ_HIP(hipStreamSynchronize(st));
        if (h != 0) {
            set_error("kron_prepare: damped factor is not positive definite (pivot step " + std::to_string(h) + ")");
            return KQ_ERR_NOT_PD;
        }
    }
    return KQ_OK;
}

kq_status prepare_dispatch(kq_dtype dtype, int64_t d, const void* A, int64_t lda, double damp_rel, void* U,
                           int64_t ldu, double* trace_out, double* lambda_out, int32_t* info_dev, void* ws,
                           hipStream_t st) {
    if (dtype == KQ_F64)
        return prepare_typed<double>(d, static_cast<const double*>(A), lda, damp_rel, static_cast<double*>(U), ldu,
                                     trace_out, lambda_out, info_dev, ws, st);
    return prepare_typed<float>(d, static_cast<const float*>(A), lda, damp_rel, static_cast<float*>(U), ldu, trace_out,
                                lambda_out, info_dev, ws, st);
}

}  // namespace kq
