// Two-sided GPTQ solver (FastKron / BaKron) for gfx950.
//
// What is computed (FastKron page, sections 2.2-2.5): with the normalised
// factors L~_A = N_A^T, L~_B = N_B^T (N = diag(U)^{-1} U, unit upper triangular),
// the codes Z and errors Delta such that for every entry (i, j)
//   x_ij = W_ij + (L~_B Delta L~_A^T)_ij - Delta_ij   (feedback of entries <= (i, j))
//   z_ij = clamp(rne(x_ij / s_i)),  v_ij = s_i z_ij,  Delta_ij = v_ij - x_ij.
// Updates flow only to the bottom-right (section 2.3), so entries on one
// anti-diagonal i + j = k are independent.
//
// Schedule.  The matrix is cut into 64 x 64 tiles; tiles with I + J = K form
// tile-diagonal K, and tiles of one tile-diagonal are independent for the same
// reason.  solve(K0, K1) over tile-diagonal ranges follows section 2.5's
// recursion: solve(K0, mid), add the errors of the first half to the second half
// with two batched products (stage 1: T1 = Delta_band N_A restricted to the tiles
// it can reach; stage 2: X += N_B^T T1 on the tiles of diagonals [mid, K1)), then
// solve(mid, K1).  A leaf is one tile-diagonal: every tile on it runs the
// element-level anti-diagonal sweep of its 64 x 64 entries (127 steps) with the
// in-tile feedback, one workgroup per tile.
//
// Workspace layout (row-major, padded to multiples of 64 with zero weights,
// unit scales and identity factors, so padding never reaches a real entry):
//   NA  np x np   normalised input factor
//   NB  mp x mp   normalised output factor (absent when B = I)
//   X   mp x np   running pre-rounding values (starts as W)
//   D   mp x np   errors Delta
//   T1  mp x np   stage-1 products
//   S   mp        per-row scales
#include "kq_common.hpp"

namespace kq {

// N[r][c] = U[r][c] / U[r][r] for c >= r inside d x d; identity in the padding.
template <typename T>
__global__ void normalize_factor_kernel(const T* __restrict__ U, int64_t ldu, int d, int dp,
                                        T* __restrict__ N) {
    const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (idx >= int64_t(dp) * dp) return;
    const int r = int(idx / dp), c = int(idx % dp);
    T v;
    if (r < d && c < d)
        v = (c >= r) ? U[int64_t(r) * ldu + c] / U[int64_t(r) * ldu + r] : T(0);
    else
        v = (r == c) ? T(1) : T(0);
    N[idx] = v;
}

template <typename T>
__global__ void init_solver_kernel(const T* __restrict__ W, int64_t ldw, int m, int n, int mp, int np,
                                   const T* __restrict__ scales, int per_row, T* __restrict__ X,
                                   T* __restrict__ S) {
    const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (idx < int64_t(mp) * np) {
        const int r = int(idx / np), c = int(idx % np);
        X[idx] = (r < m && c < n) ? W[int64_t(r) * ldw + c] : T(0);
    }
    if (idx < mp) {
        const int r = int(idx);
        S[r] = r < m ? scales[per_row ? r : 0] : T(1);
    }
}

// Leaf: one tile-diagonal K.  Workgroup = one 64 x 64 tile, 1024 threads; thread
// (w, l) owns column l and rows w, w+16, w+32, w+48.  Right-looking in-tile
// feedback: after the entries of element anti-diagonal d are rounded, every
// later entry of the tile adds the contribution of the entry to its left in the
// same row (Delta * L~_A) and of the entry above it in the same column
// (L~_B * R, R = row-accumulated error); only the tile's own diagonal blocks of
// the factors are needed, everything from earlier tiles is already in X.
template <typename T>
__global__ __launch_bounds__(1024) void leaf_kernel(const T* __restrict__ X, T* __restrict__ D,
                                                    const T* __restrict__ NA, const T* __restrict__ NB,
                                                    const T* __restrict__ S, int np, int mp, int Mt,
                                                    int Nt, int K, int m, int n, int qmin, int qmax,
                                                    int8_t* __restrict__ Z, int64_t ldz,
                                                    T* __restrict__ V, int64_t ldv) {
    constexpr int P = TILE + 1;
    __shared__ T sNA[TILE * P];  // sNA[b'][b] = N_A[J*64+b'][J*64+b]
    __shared__ T sNB[TILE * P];  // sNB[a'][a] = N_B[I*64+a'][I*64+a]
    __shared__ T dD[2][TILE];    // errors of the current element diagonal, by row
    __shared__ T dR[2][TILE];    // row-accumulated errors of the diagonal, by column
    __shared__ T sS[TILE];

    const int ilo = K - Nt + 1 > 0 ? K - Nt + 1 : 0;
    const int I = ilo + blockIdx.x;
    const int ihi = K < Mt - 1 ? K : Mt - 1;
    if (I > ihi) return;
    const int J = K - I;
    const int t = threadIdx.x, w = t >> 6, l = t & 63;

    for (int e = t; e < TILE * TILE; e += 1024) {
        const int r = e >> 6, c = e & 63;
        sNA[r * P + c] = NA[int64_t(J * TILE + r) * np + J * TILE + c];
        sNB[r * P + c] = NB ? NB[int64_t(I * TILE + r) * mp + I * TILE + c] : T(r == c);
    }
    if (t < TILE) sS[t] = S[I * TILE + t];

    T acc[4], rp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i] = X[int64_t(I * TILE + w + 16 * i) * np + J * TILE + l];
        rp[i] = T(0);
    }
    __syncthreads();

    const T tqmin = T(qmin), tqmax = T(qmax);
    for (int d = 0; d < 2 * TILE - 1; ++d) {
        const int buf = d & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int a = w + 16 * i;
            if (a + l == d) {
                T z, v;
                quantize(acc[i], sS[a], tqmin, tqmax, z, v);
                const T delta = v - acc[i];
                dD[buf][a] = delta;
                dR[buf][l] = rp[i] + delta;
                const int64_t gi = int64_t(I) * TILE + a, gj = int64_t(J) * TILE + l;
                D[gi * np + gj] = delta;
                if (gi < m && gj < n) {
                    Z[gi * ldz + gj] = int8_t(z);
                    V[gi * ldv + gj] = v;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int a = w + 16 * i;
            if (a + l > d) {
                const int bs = d - a;  // row source (a, bs) on diagonal d
                if (bs >= 0 && bs < l) {
                    const T c = dD[buf][a] * sNA[bs * P + l];
                    acc[i] += c;
                    rp[i] += c;
                }
                const int as = d - l;  // column source (as, l) on diagonal d
                if (as >= 0 && as < a) acc[i] += sNB[as * P + a] * dR[buf][l];
            }
        }
    }
}

// Stage 1 of the band propagation at node [K0, K1) with split mid:
// T1[I', J] = sum_{J' in source band, J' <= J} Delta[I', J'] N_A[J', J]
// for every tile (I', J) that a target tile (I >= I', J) of diagonals [mid, K1)
// reads.  Grid: x = column offset within the row's window, y = source row.
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS) void band_stage1_kernel(const T* __restrict__ D,
                                                                   const T* __restrict__ NA,
                                                                   T* __restrict__ T1, int np, int Nt,
                                                                   int K0, int mid, int K1, int row0) {
    __shared__ GemmSmem<T> sm;
    const int Ip = row0 + blockIdx.y;
    const int jlo = K0 - Ip > 0 ? K0 - Ip : 0;
    const int J = jlo + blockIdx.x;
    const int jend = K1 - Ip < Nt ? K1 - Ip : Nt;
    if (J >= jend) return;
    const int khi = J < mid - 1 - Ip ? J : mid - 1 - Ip;  // inclusive
    WaveAcc<T> acc;
    acc.zero();
    if (khi >= jlo) {
        const T* A = D + int64_t(Ip) * TILE * np + int64_t(jlo) * TILE;
        const T* B = NA + int64_t(jlo) * TILE * np + int64_t(J) * TILE;
        tile_gemm<T, T, false, false, false>(A, np, B, np, TILE, TILE, (khi - jlo + 1) * TILE, sm, acc);
    }
    T* out = T1 + int64_t(Ip) * TILE * np + int64_t(J) * TILE;
    for_each_acc(acc, [&](int r, int c, T v) { out[int64_t(r) * np + c] = v; });
}

// Stage 2: X[I, J] += sum_{I'} N_B[I', I]^T T1[I', J] for the tiles of
// diagonals [mid, K1).  With B = I only the I' = I term exists (N_B = identity).
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS) void band_stage2_kernel(const T* __restrict__ T1,
                                                                   const T* __restrict__ NB,
                                                                   T* __restrict__ X, int np, int mp,
                                                                   int Mt, int Nt, int K0, int mid) {
    __shared__ GemmSmem<T> sm;
    const int K = mid + blockIdx.y;
    const int ilo = K - Nt + 1 > 0 ? K - Nt + 1 : 0;
    const int I = ilo + blockIdx.x;
    const int ihi = K < Mt - 1 ? K : Mt - 1;
    if (I > ihi) return;
    const int J = K - I;
    const int klo = K0 - J > 0 ? K0 - J : 0;
    const int khi = I < mid - 1 ? I : mid - 1;
    if (klo > khi) return;
    T* out = X + int64_t(I) * TILE * np + int64_t(J) * TILE;
    if (!NB) {
        if (I < klo || I > khi) return;
        const T* src = T1 + int64_t(I) * TILE * np + int64_t(J) * TILE;
        for (int e = threadIdx.x; e < TILE * TILE; e += GEMM_THREADS) {
            const int r = e >> 6, c = e & 63;
            out[int64_t(r) * np + c] += src[int64_t(r) * np + c];
        }
        return;
    }
    WaveAcc<T> acc;
    acc.zero();
    const T* A = NB + int64_t(klo) * TILE * mp + int64_t(I) * TILE;  // A(r, k) = NB[k][r]
    const T* B = T1 + int64_t(klo) * TILE * np + int64_t(J) * TILE;
    tile_gemm<T, T, true, false, false>(A, mp, B, np, TILE, TILE, (khi - klo + 1) * TILE, sm, acc);
    for_each_acc(acc, [&](int r, int c, T v) { out[int64_t(r) * np + c] += v; });
}

// ------------------------------------------------------------------- host side

struct SolverLayout {
    int64_t mp, np, Mt, Nt;
    size_t bytes;
    size_t off_NA, off_NB, off_X, off_D, off_T1, off_S;
};

SolverLayout solver_layout(kq_dtype dtype, int64_t m, int64_t n) {
    SolverLayout L;
    const size_t es = dtype == KQ_F64 ? 8 : 4;
    L.mp = round_up(m, TILE);
    L.np = round_up(n, TILE);
    L.Mt = L.mp / TILE;
    L.Nt = L.np / TILE;
    size_t off = 0;
    auto take = [&](size_t count) {
        size_t o = off;
        off += align256(count * es);
        return o;
    };
    L.off_NA = take(size_t(L.np) * L.np);
    L.off_NB = take(size_t(L.mp) * L.mp);
    L.off_X = take(size_t(L.mp) * L.np);
    L.off_D = take(size_t(L.mp) * L.np);
    L.off_T1 = take(size_t(L.mp) * L.np);
    L.off_S = take(size_t(L.mp));
    L.bytes = off;
    return L;
}

template <typename T>
struct SolverRun {
    const SolverLayout& L;
    int m, n, qmin, qmax;
    T *NA, *NB, *X, *D, *T1, *S;
    int8_t* Z;
    int64_t ldz;
    T* V;
    int64_t ldv;
    hipStream_t st;

    kq_status leaf(int K) {
        const int ilo = K - int(L.Nt) + 1 > 0 ? K - int(L.Nt) + 1 : 0;
        const int ihi = K < int(L.Mt) - 1 ? K : int(L.Mt) - 1;
        hipLaunchKernelGGL(leaf_kernel<T>, dim3(ihi - ilo + 1), dim3(1024), 0, st, X, D, NA, NB, S,
                           int(L.np), int(L.mp), int(L.Mt), int(L.Nt), K, m, n, qmin, qmax, Z, ldz, V, ldv);
        KQ_LAUNCHED("leaf_kernel");
        return KQ_OK;
    }

    kq_status propagate(int K0, int mid, int K1) {
        const int Mt = int(L.Mt), Nt = int(L.Nt);
        // stage 1 rows: I' with a source tile in [K0, mid): K0 - Nt < I' < mid
        const int row0 = K0 - Nt + 1 > 0 ? K0 - Nt + 1 : 0;
        const int row1 = mid < Mt ? mid : Mt;  // exclusive
        if (row1 > row0) {
            hipLaunchKernelGGL(band_stage1_kernel<T>, dim3(K1 - K0, row1 - row0), dim3(GEMM_THREADS), 0, st,
                               D, NA, T1, int(L.np), Nt, K0, mid, K1, row0);
            KQ_LAUNCHED("band_stage1_kernel");
        }
        const int width = Mt < Nt ? Mt : Nt;
        hipLaunchKernelGGL(band_stage2_kernel<T>, dim3(width, K1 - mid), dim3(GEMM_THREADS), 0, st, T1, NB, X,
                           int(L.np), int(L.mp), Mt, Nt, K0, mid);
        KQ_LAUNCHED("band_stage2_kernel");
        return KQ_OK;
    }

    kq_status solve(int K0, int K1) {
        if (K1 - K0 == 1) return leaf(K0);
        const int mid = (K0 + K1) / 2;
        kq_status s = solve(K0, mid);
        if (s != KQ_OK) return s;
        s = propagate(K0, mid, K1);
        if (s != KQ_OK) return s;
        return solve(mid, K1);
    }
};

template <typename T>
kq_status quantize_typed(int64_t m, int64_t n, const T* W, int64_t ldw, const T* UA, int64_t lda, const T* UB,
                         int64_t ldb, const kq_quantizer* q, int8_t* codes, int64_t ldc, T* V, int64_t ldv,
                         void* ws, hipStream_t st) {
    const SolverLayout L = solver_layout(sizeof(T) == 8 ? KQ_F64 : KQ_F32, m, n);
    char* base = static_cast<char*>(ws);
    SolverRun<T> run{L, int(m), int(n), -(1 << (q->bits - 1)), (1 << (q->bits - 1)) - 1,
                     reinterpret_cast<T*>(base + L.off_NA), UB ? reinterpret_cast<T*>(base + L.off_NB) : nullptr,
                     reinterpret_cast<T*>(base + L.off_X), reinterpret_cast<T*>(base + L.off_D),
                     reinterpret_cast<T*>(base + L.off_T1), reinterpret_cast<T*>(base + L.off_S),
                     codes, ldc, V, ldv, st};
    const int threads = 256;
    auto blocks = [&](int64_t count) { return dim3(unsigned((count + threads - 1) / threads)); };
    hipLaunchKernelGGL(normalize_factor_kernel<T>, blocks(L.np * L.np), dim3(threads), 0, st, UA, lda, int(n),
                       int(L.np), run.NA);
    KQ_LAUNCHED("normalize_factor_kernel");
    if (UB) {
        hipLaunchKernelGGL(normalize_factor_kernel<T>, blocks(L.mp * L.mp), dim3(threads), 0, st, UB, ldb, int(m),
                           int(L.mp), run.NB);
        KQ_LAUNCHED("normalize_factor_kernel");
    }
    hipLaunchKernelGGL(init_solver_kernel<T>, blocks(L.mp * L.np), dim3(threads), 0, st, W, ldw, int(m), int(n),
                       int(L.mp), int(L.np), static_cast<const T*>(q->scales), q->per_row, run.X, run.S);
    KQ_LAUNCHED("init_solver_kernel");
    return run.solve(0, int(L.Mt + L.Nt - 1));
}

size_t quantize_workspace_bytes(kq_dtype dtype, int64_t m, int64_t n) { return solver_layout(dtype, m, n).bytes; }

kq_status quantize_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* UA,
                            int64_t lda, const void* UB, int64_t ldb, const kq_quantizer* q, int8_t* codes,
                            int64_t ldc, void* V, int64_t ldv, void* ws, hipStream_t st) {
    if (dtype == KQ_F64)
        return quantize_typed<double>(m, n, static_cast<const double*>(W), ldw, static_cast<const double*>(UA), lda,
                                      static_cast<const double*>(UB), ldb, q, codes, ldc, static_cast<double*>(V),
                                      ldv, ws, st);
    return quantize_typed<float>(m, n, static_cast<const float*>(W), ldw, static_cast<const float*>(UA), lda,
                                 static_cast<const float*>(UB), ldb, q, codes, ldc, static_cast<float*>(V), ldv, ws,
                                 st);
}

}  // namespace kq
