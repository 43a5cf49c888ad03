// K-FAC factor accumulation, proxy loss and scale helper for gfx950.
#include <algorithm>

#include "kq_common.hpp"

namespace kq {

// ------------------------------------------------------- factor accumulation
// S <- beta S + alpha X^T X (FastKron page, section 3.2 'Marginal' factors and
// section 2.6's accumulation over the calibration set), on the 64 x 64 tiles of
// the lower triangle (I >= J); each tile and its mirror are written, so the full
// symmetric matrix is produced, and a diagonal tile writes each element once.
// Work items: the T (T - 1) / 2 tiles below the diagonal, one workgroup each,
// and the T diagonal tiles in pairs.  At T = 64 that is 2048 workgroups, a
// whole number of the 8-per-CU rounds, where one workgroup per tile would leave
// 32 tiles to a second round; the 32 pair items come first so that they start
// in the first wave of dispatches.
// EXACT: dim is a multiple of 64, rows of 16 and ldx of 4, so every operand load
// is in range and vector aligned and the bounds checks are dropped.
// The weighted form S <- beta S + alpha X^T Y with Y = diag(w) X (the FlipFlop /
// Frobenius factor updates) runs the same tiles with Y as the right operand:
// X^T diag(w) X is symmetric, so the lower tiles and their mirrors give it all.
template <typename T, bool EXACT>
__device__ __forceinline__ void syrk_tile(const T* __restrict__ X, int64_t ldx, const T* __restrict__ Y, int64_t ldy,
                                          int rows, int dim, T* __restrict__ S, int64_t lds, T alpha, T beta, int I,
                                          int J, GemmSmem<T>& sm) {
    WaveAcc<T> acc;
    acc.zero();
    const int mv = dim - I * TILE, nv = dim - J * TILE;
    // A(r, k) = X[k][I*64 + r]; B(k, c) = Y[k][J*64 + c]
    tile_gemm<T, T, true, false, !EXACT>(X + I * TILE, ldx, Y + J * TILE, ldy, mv, nv, rows, sm, acc);
    // A diagonal tile keeps its lower triangle and mirrors it, so S is exactly
    // symmetric also when Y differs from X (X^T diag(w) X computed as x_r (w x_c)
    // and x_c (w x_r) would round differently).
    for_each_acc(acc, [&](int r, int c, T v) {
        if (r >= mv || c >= nv || (I == J && c > r)) return;
        const int64_t gi = int64_t(I) * TILE + r, gj = int64_t(J) * TILE + c;
        T* p = S + gi * lds + gj;
        *p = beta == T(0) ? alpha * v : beta * *p + alpha * v;
        if (gi != gj) {
            T* q = S + gj * lds + gi;
            *q = beta == T(0) ? alpha * v : beta * *q + alpha * v;
        }
    });
}

template <typename T, bool EXACT>
__global__ __launch_bounds__(GEMM_THREADS) void syrk_kernel(const T* __restrict__ X, int64_t ldx,
                                                            const T* __restrict__ Y, int64_t ldy, int rows, int dim,
                                                            T* __restrict__ S, int64_t lds, T alpha, T beta,
                                                            int tiles) {
    __shared__ GemmSmem<T> sm;
    const int npairs = (tiles + 1) / 2;
    const int item = blockIdx.x;
    if (item < npairs) {  // diagonal tiles 2 item and 2 item + 1
        syrk_tile<T, EXACT>(X, ldx, Y, ldy, rows, dim, S, lds, alpha, beta, 2 * item, 2 * item, sm);
        if (2 * item + 1 < tiles)
            syrk_tile<T, EXACT>(X, ldx, Y, ldy, rows, dim, S, lds, alpha, beta, 2 * item + 1, 2 * item + 1, sm);
        return;
    }
    // below the diagonal: o = I (I - 1) / 2 + J with J < I
    const int o = item - npairs;
    int I = int((1.0 + sqrt(1.0 + 8.0 * o)) * 0.5);
    while (I * (I - 1) / 2 > o) --I;
    while ((I + 1) * I / 2 <= o) ++I;
    syrk_tile<T, EXACT>(X, ldx, Y, ldy, rows, dim, S, lds, alpha, beta, I, o - I * (I - 1) / 2, sm);
}

// S <- beta S + alpha X^T Y, Y = X or diag(w) X (same leading-dimension rules).
kq_status syrk_dispatch(kq_dtype dtype, int64_t rows, int64_t dim, const void* X, int64_t ldx, const void* Y,
                        int64_t ldy, void* S, int64_t lds, double alpha, double beta, hipStream_t st) {
    const int tiles = int((dim + TILE - 1) / TILE);
    const size_t es = dtype == KQ_F64 ? 8 : 4;
    const bool exact = dim % TILE == 0 && rows % KSTEP == 0 && ldx % 4 == 0 && ldy % 4 == 0 &&
                       reinterpret_cast<uintptr_t>(X) % (4 * es) == 0 && reinterpret_cast<uintptr_t>(Y) % (4 * es) == 0;
    const dim3 grid(unsigned((tiles + 1) / 2 + tiles * (tiles - 1) / 2)), block(GEMM_THREADS);
    if (dtype == KQ_F64) {
        auto k = exact ? syrk_kernel<double, true> : syrk_kernel<double, false>;
        hipLaunchKernelGGL(k, grid, block, 0, st, static_cast<const double*>(X), ldx, static_cast<const double*>(Y),
                           ldy, int(rows), int(dim), static_cast<double*>(S), lds, alpha, beta, tiles);
    } else {
        auto k = exact ? syrk_kernel<float, true> : syrk_kernel<float, false>;
        hipLaunchKernelGGL(k, grid, block, 0, st, static_cast<const float*>(X), ldx, static_cast<const float*>(Y), ldy,
                           int(rows), int(dim), static_cast<float*>(S), lds, float(alpha), float(beta), tiles);
    }
    KQ_LAUNCHED("syrk_kernel");
    return KQ_OK;
}

kq_status factor_dispatch(kq_dtype dtype, int64_t rows, int64_t dim, const void* X, int64_t ldx, void* S, int64_t lds,
                          double alpha, double beta, hipStream_t st) {
    return syrk_dispatch(dtype, rows, dim, X, ldx, X, ldx, S, lds, alpha, beta, st);
}

// ------------------------------------------------------------------ the loss
// tr(B_d E A_d E^T) with E = V - W, A_d = A + lam_A I, B_d = B + lam_B I, in fp64
// on matrix cores over zero-padded fp64 copies (the damping folded into the
// copies' diagonals).  A_d and B_d are symmetric, so with G = E A_d E^T (m x m)
// and H = E^T B_d E (n x n), both symmetric,
//   tr(B_d E A_d E^T) = sum_ij (B_d)_ij G_ij = sum_ij (A_d)_ij H_ij.
// The cheaper form is taken: one full product (E A_d, or B_d E) and the upper
// triangle of tiles of the symmetric one, each tile's weighted sum formed as it
// leaves the matrix cores (off-diagonal tiles count twice).  Flops
// m n (2 n + m) for G when n <= m, m n (2 m + n) for H otherwise, against
// 2 m n (m + n) for the two full products B_d E and E A_d.  B = I needs only
// sum_ij E_ij (E A_d)_ij.  Partial sums per tile, then one fixed-order pass.
//
// Every product reads its left operand k-major (E through its transpose E^T,
// B_d as itself, being symmetric) and its right operand row-major, so both
// tiles arrive in LDS in the order the matrix cores read them.  The full
// product uses 128 x 128 output blocks: half the operand traffic per flop of a
// 64 x 64 block, which is what an fp64 product of this size is short of.  (The
// symmetric product keeps 64 x 64 tiles: its triangle of 128 x 128 tiles is too
// few to spread evenly over the CUs, and splitting their K ranges to even it out
// scatters the blocks over the operands and loses the shared cache lines.)

template <typename TIn>
__global__ void diag_trace_kernel(const TIn* __restrict__ A, int64_t lda, int d, double* __restrict__ out) {
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

// dst (rp x cp, fp64) = src (rows x cols) zero-padded; with sub != nullptr,
// dst = src - sub; with trace != nullptr, damp_rel * trace / rows is added on the
// diagonal of the square src.
template <typename TIn>
__global__ void pad_copy_kernel(const TIn* __restrict__ src, int64_t lds, const TIn* __restrict__ sub, int64_t ldsub,
                                int rows, int cols, int rp, int cp, const double* __restrict__ trace, double damp_rel,
                                double* __restrict__ dst) {
    const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (idx >= int64_t(rp) * cp) return;
    const int r = int(idx / cp), c = int(idx % cp);
    double v = 0.0;
    if (r < rows && c < cols) {
        v = double(src[int64_t(r) * lds + c]);
        if (sub) v -= double(sub[int64_t(r) * ldsub + c]);
        if (trace && r == c) v += damp_rel * (*trace) / rows;
    }
    dst[idx] = v;
}

// dstT (cp x rp, fp64) = (src - sub)^T zero-padded, through a 32 x 32 LDS tile
// so that reads and writes are both row-contiguous.  Block (32, 8), grid
// (cp / 32, rp / 32).
template <typename TIn>
__global__ void pad_diff_transpose_kernel(const TIn* __restrict__ src, int64_t lds, const TIn* __restrict__ sub,
                                          int64_t ldsub, int rows, int cols, int rp, double* __restrict__ dstT) {
    __shared__ double tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32, tx = threadIdx.x, ty = threadIdx.y;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = r0 + ty + 8 * q, c = c0 + tx;
        double v = 0.0;
        if (r < rows && c < cols) v = double(src[int64_t(r) * lds + c]) - double(sub[int64_t(r) * ldsub + c]);
        tile[ty + 8 * q][tx] = v;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = c0 + ty + 8 * q;
        dstT[int64_t(c) * rp + r0 + tx] = tile[tx][ty + 8 * q];
    }
}

// C (M x N) = At^T B with At K x M and B K x N row-major fp64, M, N multiples of
// 128 and K of 16.  One 256-thread workgroup per 128 x 128 block, each wave a
// 64 x 64 quarter (4 x 4 v_mfma_f64_16x16x4 blocks), K in 16-deep slices through
// double-buffered LDS, both operands stored k-major.
constexpr int BIG = 128;
constexpr int BIG_S = BIG + 16;  // LDS row stride: rows k and k + 1 start 32 banks apart

struct __attribute__((aligned(16))) BigSmem {
    double a[2][KSTEP * BIG_S];
    double b[2][KSTEP * BIG_S];
};

// acc += At[k0:k1, a-cols]^T B[k0:k1, b-cols] for one 128 x 128 block; At and B
// point at the block's first column, rows k are ld apart.  All 256 threads call
// it (it contains barriers); k1 - k0 is a multiple of 16.
__device__ __forceinline__ void big_mma(const double* __restrict__ a0, int lda, const double* __restrict__ b0,
                                        int ldb, int k0, int k1, BigSmem& sm, f64x4 (&acc)[4][4]) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wy = w >> 1, wx = w & 1;
    const int lk = t >> 4, lq = (t & 15) * 8;  // loader: slice row lk, 8 consecutive columns from lq
    f64x2 ra[4], rb[4];
    auto fetch = [&](int k) {
        const f64x2* pa = reinterpret_cast<const f64x2*>(a0 + int64_t(k + lk) * lda + lq);
        const f64x2* pb = reinterpret_cast<const f64x2*>(b0 + int64_t(k + lk) * ldb + lq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ra[e] = pa[e];
            rb[e] = pb[e];
        }
    };
    auto stash = [&](int buf) {
        f64x2* sa = reinterpret_cast<f64x2*>(sm.a[buf] + lk * BIG_S + lq);
        f64x2* sb = reinterpret_cast<f64x2*>(sm.b[buf] + lk * BIG_S + lq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sa[e] = ra[e];
            sb[e] = rb[e];
        }
    };
    const int nk = (k1 - k0) / KSTEP;
    fetch(k0);
    __syncthreads();  // earlier readers of sm are done
    stash(0);
    __syncthreads();
    const int kr = lane >> 4, ix = lane & 15;
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        if (s + 1 < nk) fetch(k0 + (s + 1) * KSTEP);
        const double* As = sm.a[cur];
        const double* Bs = sm.b[cur];
#pragma unroll
        for (int kk = 0; kk < KSTEP; kk += 4) {
            double av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = As[(kk + kr) * BIG_S + wy * 64 + 16 * i + ix];
                bv[i] = Bs[(kk + kr) * BIG_S + wx * 64 + 16 * i + ix];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < nk) {
            stash(cur ^ 1);
            __syncthreads();
        }
    }
}

__device__ __forceinline__ void big_zero(f64x4 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0;
}

// Visit the accumulators with their block coordinates: D register r of a 16 x 16
// block sits at row lane / 16 + 4 r, column lane % 16.
template <typename Fn>
__device__ __forceinline__ void big_for_each(const f64x4 (&acc)[4][4], Fn&& fn) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wy = w >> 1, wx = w & 1, kr = lane >> 4, ix = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) fn(wy * 64 + 16 * i + kr + 4 * r, wx * 64 + 16 * j + ix, acc[i][j][r]);
}

__global__ __launch_bounds__(GEMM_THREADS) void gemm_tn_f64_big_kernel(const double* __restrict__ At, int lda,
                                                                       const double* __restrict__ B, int ldb,
                                                                       double* __restrict__ C, int ldc, int K) {
    __shared__ BigSmem sm;
    const int I = blockIdx.y, J = blockIdx.x;
    f64x4 acc[4][4];
    big_zero(acc);
    big_mma(At + int64_t(I) * BIG, lda, B + int64_t(J) * BIG, ldb, 0, K, sm, acc);
    double* out = C + int64_t(I) * BIG * ldc + int64_t(J) * BIG;
    big_for_each(acc, [&](int r, int c, double v) { out[int64_t(r) * ldc + c] = v; });
}

// One 64 x 64 tile (I <= J) of a symmetric product S = X^T Y (X, Y: K x W
// row-major), weighted by the damped factor F:
//   partial[tile] = w sum_rc F[I r][J c] S_IJ[r][c],  w = 1 on the diagonal, 2 above.
// Tiles are numbered J (J + 1) / 2 + I over the upper triangle.  64 x 64 tiles
// rather than 128 x 128: the triangle then has enough tiles to spread evenly
// over the CUs.  The K range of each tile is cut into SYM_KSPLIT parts, one
// workgroup each (part-major, so workgroups running together read the same rows
// of X and Y): the triangle's tile count is rarely a multiple of the resident
// workgroups, and quarter-size pieces shrink the last, partly filled round.
constexpr int SYM_KSPLIT = 4;

__global__ __launch_bounds__(GEMM_THREADS) void loss_sym_kernel(const double* __restrict__ X,
                                                                const double* __restrict__ Y, int ld, int K,
                                                                const double* __restrict__ F, int ldf, int ntiles,
                                                                double* __restrict__ partial) {
    __shared__ GemmSmem<double> sm;
    __shared__ double red[GEMM_THREADS];
    const int kpart = blockIdx.x / ntiles, b = blockIdx.x - kpart * ntiles;
    const int kl = K / SYM_KSPLIT;
    int J = int((sqrt(8.0 * b + 1.0) - 1.0) * 0.5);
    while (J * (J + 1) / 2 > b) --J;
    while ((J + 1) * (J + 2) / 2 <= b) ++J;
    const int I = b - J * (J + 1) / 2;
    WaveAcc<double> acc;
    acc.zero();
    // A(r, k) = X[k][I*64 + r], B(k, c) = Y[k][J*64 + c] over this part's rows k
    const int64_t k0 = int64_t(kpart) * kl * ld;
    tile_gemm<double, double, true, false, false>(X + k0 + int64_t(I) * TILE, ld, Y + k0 + int64_t(J) * TILE, ld, TILE,
                                                  TILE, kl, sm, acc);
    const double* f = F + int64_t(I) * TILE * ldf + int64_t(J) * TILE;
    double s = 0.0;
    for_each_acc(acc, [&](int r, int c, double v) { s = __builtin_fma(f[int64_t(r) * ldf + c], v, s); });
    const double tot = block_sum_256(s, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = I == J ? tot : 2.0 * tot;
}

// B = I: partial sums of E * Q (Q = E A_d), one per block, in a fixed order.
__global__ void loss_partial_kernel(const double* __restrict__ Q, const double* __restrict__ E, int64_t count,
                                    double* __restrict__ partial) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x)
        s = __builtin_fma(E[i], Q[i], s);
    const double tot = block_sum_256(s, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = tot;
}

__global__ void loss_final_kernel(const double* __restrict__ partial, int count, double* __restrict__ out) {
    __shared__ double red[256];
    double s = 0.0;
    for (int i = threadIdx.x; i < count; i += blockDim.x) s += partial[i];
    const double tot = block_sum_256(s, red);
    if (threadIdx.x == 0) *out = tot;
}

constexpr int LOSS_BLOCKS = 1024;
struct LossLayout {
    int64_t mp, np;  // padded to 128
    int npart;       // partial sums
    bool rows;       // G = E A_d E^T (m x m) rather than H = E^T B_d E (n x n)
    size_t off_E, off_Et, off_Q, off_A, off_B, off_scal, bytes;
};

LossLayout loss_layout(int64_t m, int64_t n) {
    LossLayout L;
    L.mp = round_up(m, BIG);
    L.np = round_up(n, BIG);
    L.rows = n <= m;
    const int64_t t = (L.rows ? L.mp : L.np) / TILE;
    L.npart = int(std::max<int64_t>(LOSS_BLOCKS, t * (t + 1) / 2 * SYM_KSPLIT));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    L.off_E = take(size_t(L.mp) * L.np * 8);
    L.off_Et = L.off_E;  // a path reads E or E^T, never both
    L.off_Q = take(size_t(L.mp) * L.np * 8);
    L.off_A = take(size_t(L.np) * L.np * 8);
    L.off_B = take(size_t(L.mp) * L.mp * 8);
    L.off_scal = take((size_t(L.npart) + 8) * 8);
    L.bytes = off;
    return L;
}

size_t loss_workspace_bytes(int64_t m, int64_t n) { return loss_layout(m, n).bytes; }

template <typename T>
kq_status loss_typed(int64_t m, int64_t n, const T* W, int64_t ldw, const T* V, int64_t ldv, const T* A, int64_t lda,
                     const T* B, int64_t ldb, double damp_rel, double* loss_dev, void* ws, hipStream_t st) {
    const LossLayout L = loss_layout(m, n);
    char* base = static_cast<char*>(ws);
    double* E = reinterpret_cast<double*>(base + L.off_E);
    double* Et = reinterpret_cast<double*>(base + L.off_Et);
    double* Q = reinterpret_cast<double*>(base + L.off_Q);
    double* Ap = reinterpret_cast<double*>(base + L.off_A);
    double* Bp = reinterpret_cast<double*>(base + L.off_B);
    double* scal = reinterpret_cast<double*>(base + L.off_scal);
    double *trA = scal, *trB = scal + 1, *partial = scal + 8;
    const int mp = int(L.mp), np = int(L.np);
    auto blocks = [](int64_t count) { return dim3(unsigned((count + 255) / 256)); };

    if (!B || L.rows) {  // the products read E only through E^T
        hipLaunchKernelGGL(pad_diff_transpose_kernel<T>, dim3(np / 32, mp / 32), dim3(32, 8), 0, st, V, ldv, W, ldw,
                           int(m), int(n), mp, Et);
        KQ_LAUNCHED("pad_diff_transpose_kernel");
    } else {
        hipLaunchKernelGGL(pad_copy_kernel<T>, blocks(int64_t(mp) * np), dim3(256), 0, st, V, ldv, W, ldw, int(m),
                           int(n), mp, np, (const double*)nullptr, 0.0, E);
        KQ_LAUNCHED("pad_copy_kernel");
    }
    hipLaunchKernelGGL(diag_trace_kernel<T>, dim3(1), dim3(1024), 0, st, A, lda, int(n), trA);
    KQ_LAUNCHED("diag_trace_kernel");
    hipLaunchKernelGGL(pad_copy_kernel<T>, blocks(int64_t(np) * np), dim3(256), 0, st, A, lda, (const T*)nullptr,
                       int64_t(0), int(n), int(n), np, np, trA, damp_rel, Ap);
    KQ_LAUNCHED("pad_copy_kernel");
    int nparts = LOSS_BLOCKS;
    if (!B) {  // Q^T = A_d E^T (A_d symmetric: its own transpose), then sum E^T * Q^T
        hipLaunchKernelGGL(gemm_tn_f64_big_kernel, dim3(mp / BIG, np / BIG), dim3(GEMM_THREADS), 0, st, Ap, np, Et,
                           mp, Q, mp, np);
        KQ_LAUNCHED("gemm_tn_f64_big_kernel");
        hipLaunchKernelGGL(loss_partial_kernel, dim3(LOSS_BLOCKS), dim3(256), 0, st, Q, Et, int64_t(mp) * np, partial);
        KQ_LAUNCHED("loss_partial_kernel");
    } else {
        hipLaunchKernelGGL(diag_trace_kernel<T>, dim3(1), dim3(1024), 0, st, B, ldb, int(m), trB);
        KQ_LAUNCHED("diag_trace_kernel");
        hipLaunchKernelGGL(pad_copy_kernel<T>, blocks(int64_t(mp) * mp), dim3(256), 0, st, B, ldb, (const T*)nullptr,
                           int64_t(0), int(m), int(m), mp, mp, trB, damp_rel, Bp);
        KQ_LAUNCHED("pad_copy_kernel");
        if (L.rows) {  // Q^T = A_d E^T; G = Q E^T = (Q^T)^T E^T weighted by B_d
            hipLaunchKernelGGL(gemm_tn_f64_big_kernel, dim3(mp / BIG, np / BIG), dim3(GEMM_THREADS), 0, st, Ap, np,
                               Et, mp, Q, mp, np);
            KQ_LAUNCHED("gemm_tn_f64_big_kernel");
            const int t = mp / TILE;
            nparts = t * (t + 1) / 2 * SYM_KSPLIT;
            hipLaunchKernelGGL(loss_sym_kernel, dim3(nparts), dim3(GEMM_THREADS), 0, st, Q, Et, mp, np, Bp, mp,
                               t * (t + 1) / 2, partial);
        } else {  // P = B_d E (B_d its own transpose); H = P^T E weighted by A_d
            hipLaunchKernelGGL(gemm_tn_f64_big_kernel, dim3(np / BIG, mp / BIG), dim3(GEMM_THREADS), 0, st, Bp, mp, E,
                               np, Q, np, mp);
            KQ_LAUNCHED("gemm_tn_f64_big_kernel");
            const int t = np / TILE;
            nparts = t * (t + 1) / 2 * SYM_KSPLIT;
            hipLaunchKernelGGL(loss_sym_kernel, dim3(nparts), dim3(GEMM_THREADS), 0, st, Q, E, np, mp, Ap, np,
                               t * (t + 1) / 2, partial);
        }
        KQ_LAUNCHED("loss_sym_kernel");
    }
    hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, st, partial, nparts, loss_dev);
    KQ_LAUNCHED("loss_final_kernel");
    return KQ_OK;
}

kq_status loss_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* V, int64_t ldv,
                        const void* A, int64_t lda, const void* B, int64_t ldb, double damp_rel, double* loss_dev,
                        void* ws, hipStream_t st) {
    if (dtype == KQ_F64)
        return loss_typed<double>(m, n, static_cast<const double*>(W), ldw, static_cast<const double*>(V), ldv,
                                  static_cast<const double*>(A), lda, static_cast<const double*>(B), ldb, damp_rel,
                                  loss_dev, ws, st);
    return loss_typed<float>(m, n, static_cast<const float*>(W), ldw, static_cast<const float*>(V), ldv,
                             static_cast<const float*>(A), lda, static_cast<const float*>(B), ldb, damp_rel, loss_dev,
                             ws, st);
}

// ------------------------------------------------------------------- scales
// s_i = max_j |W_ij| / (2^(bits-1) - 1) per row, or over the whole tensor.

template <typename T>
struct Bits;
template <>
struct Bits<float> {
    typedef unsigned int U;
    static __device__ U to(float x) { return __float_as_uint(x); }
    static __device__ float from(U u) { return __uint_as_float(u); }
};
template <>
struct Bits<double> {
    typedef unsigned long long U;
    static __device__ U to(double x) { return (U)__double_as_longlong(x); }
    static __device__ double from(U u) { return __longlong_as_double((long long)u); }
};

template <typename T>
__global__ void clear_scalar_kernel(T* p) {
    if (threadIdx.x == 0) *p = T(0);
}

// One block per row.  Non-negative floats order like their bit patterns, so the
// tensor-wide maximum is an integer atomic max on the bits.
template <typename T>
__global__ void row_absmax_kernel(const T* __restrict__ W, int64_t ldw, int n, int per_row, T qmax,
                                  T* __restrict__ scales) {
    __shared__ T red[256];
    const int r = blockIdx.x;
    T mx = T(0);
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
        const T a = fabs(W[int64_t(r) * ldw + c]);
        mx = a > mx ? a : mx;
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (int(threadIdx.x) < w) red[threadIdx.x] = red[threadIdx.x] > red[threadIdx.x + w] ? red[threadIdx.x] : red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (per_row)
            scales[r] = red[0] / qmax;
        else
            atomicMax(reinterpret_cast<typename Bits<T>::U*>(scales), Bits<T>::to(red[0]));
    }
}

template <typename T>
__global__ void divide_scalar_kernel(T* p, T q) {
    if (threadIdx.x == 0) *p = *p / q;
}

template <typename T>
kq_status scales_typed(int64_t m, int64_t n, const T* W, int64_t ldw, int bits, int per_row, T* scales, hipStream_t st) {
    const T qmax = T((1 << (bits - 1)) - 1);
    if (!per_row) {
        hipLaunchKernelGGL(clear_scalar_kernel<T>, dim3(1), dim3(64), 0, st, scales);
        KQ_LAUNCHED("clear_scalar_kernel");
    }
    hipLaunchKernelGGL(row_absmax_kernel<T>, dim3(unsigned(m)), dim3(256), 0, st, W, ldw, int(n), per_row, qmax, scales);
    KQ_LAUNCHED("row_absmax_kernel");
    if (!per_row) {
        hipLaunchKernelGGL(divide_scalar_kernel<T>, dim3(1), dim3(64), 0, st, scales, qmax);
        KQ_LAUNCHED("divide_scalar_kernel");
    }
    return KQ_OK;
}

// WaterKron steps (WaterKron page, section 3): alpha_j = step * U_A[j, j] and
// beta_i = U_B[i, i] (1 when B = I), the reciprocals of the reverse Cholesky
// diagonals up to the free factor step.  The product is formed in fp64 and
// rounded once to T.
template <typename T>
__global__ void waterkron_scales_kernel(const T* __restrict__ UA, int64_t lda, const T* __restrict__ UB, int64_t ldb,
                                        int m, int n, double step, T* __restrict__ alpha, T* __restrict__ beta) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) alpha[i] = T(step * double(UA[int64_t(i) * lda + i]));
    if (i < m) beta[i] = UB ? UB[int64_t(i) * ldb + i] : T(1);
}

kq_status waterkron_scales_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* UA, int64_t lda, const void* UB,
                                    int64_t ldb, double step, void* alpha, void* beta, hipStream_t st) {
    const int64_t d = m > n ? m : n;
    const dim3 grid(unsigned((d + 255) / 256)), block(256);
    if (dtype == KQ_F64)
        hipLaunchKernelGGL(waterkron_scales_kernel<double>, grid, block, 0, st, static_cast<const double*>(UA), lda,
                           static_cast<const double*>(UB), ldb, int(m), int(n), step, static_cast<double*>(alpha),
                           static_cast<double*>(beta));
    else
        hipLaunchKernelGGL(waterkron_scales_kernel<float>, grid, block, 0, st, static_cast<const float*>(UA), lda,
                           static_cast<const float*>(UB), ldb, int(m), int(n), step, static_cast<float*>(alpha),
                           static_cast<float*>(beta));
    KQ_LAUNCHED("waterkron_scales_kernel");
    return KQ_OK;
}

kq_status scales_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, int bits, int per_row,
                          void* scales, hipStream_t st) {
    if (dtype == KQ_F64)
        return scales_typed<double>(m, n, static_cast<const double*>(W), ldw, bits, per_row, static_cast<double*>(scales),
                                    st);
    return scales_typed<float>(m, n, static_cast<const float*>(W), ldw, bits, per_row, static_cast<float*>(scales), st);
}

}  // namespace kq
