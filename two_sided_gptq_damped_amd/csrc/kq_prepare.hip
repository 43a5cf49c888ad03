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
//      panel (C_ik <- C_ik L_kk^{-T}) and updates (C_ij -= C_ik C_jk^T) in two
//      levels (inside a panel of PANEL block columns, then the whole trailing
//      matrix once per panel), the last two on fp64 matrix cores
//   3. lower-triangular inverse by recursive halving of the block range,
//      one pair of matrix-core launches per recursion level
//   4. U[r][c] = Li[d-1-r][d-1-c] for c >= r, 0 below the diagonal.
#include <algorithm>

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

// Lane l's copy of another lane's double (the lane index must be uniform).
__device__ __forceinline__ double readlane_f64(double v, int l) {
    const long long b = __double_as_longlong(v);
    const unsigned lo = unsigned(__builtin_amdgcn_readlane(int(b & 0xffffffffll), l));
    const unsigned hi = unsigned(__builtin_amdgcn_readlane(int(b >> 32), l));
    return __longlong_as_double((long long)((unsigned long long)hi << 32 | lo));
}

// Cholesky of the diagonal block C[k][k] and the inverse of its factor.
//
// Factor: left-looking over four 16-column panels.  For panel p (columns c0..c0+15)
// the waves first subtract the contribution of the finished columns
// (L[r][c] -= sum_{q < c0} L[r][q] L[c][q], one 16-row block per wave on the
// matrix cores); then one wave factors the panel in
// registers, lane i holding row c0 + i: per column, the pivot and the column
// entries of the other panel rows are broadcast with readlane, so a column costs
// no LDS round trip and no workgroup barrier.
// Inverse: the four 16 x 16 diagonal blocks are inverted by forward substitution,
// one wave each (lane = column); then the blocks below the diagonal follow by
// distance d = 1..3 on the matrix cores: T = sum_{q=j}^{i-1} L_iq X_qj,
// X_ij = -X_ii T.
// Writes L^{-1} into Dinv[k] (the block of L itself is used only through it).  A pivot
// that is not > 0 records its 1-based position in *info (first failure only) and
// continues with a unit pivot so the remaining kernels stay finite.
// One v_mfma_f64_16x16x4 step: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; register r of the result holds row l / 16 + 4 r, column l % 16.
__device__ __forceinline__ f64x4 mma16(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

constexpr int DP = TILE + 1;  // row stride of the diagonal-block arrays
struct DiagSmem {
    double L[TILE * DP];
    double X[TILE * DP];
    double rdiag[TILE];  // 1 / L[j][j]
    double colj[64];     // the panel column being eliminated, one entry per lane
};

// Factor the diagonal block k held in sm.L (full 64 x 64, lower part used) by
// the 256 threads of the workgroup; writes L into C and L^{-1} into Dinv[k].
__device__ __forceinline__ void diag_factor(double* __restrict__ C, int dp, int k, double* __restrict__ Dinv,
                            int32_t* __restrict__ info, DiagSmem& sm) {
    constexpr int P = DP;
    constexpr int PW = 16;  // panel width
    double* const L = sm.L;
    double* const X = sm.X;
    double* const rdiag = sm.rdiag;
    double* const colj = sm.colj;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int ix = lane & 15, kr = lane >> 4;  // 16 x 16 x 4 operand position: row / column ix, k kr
    __syncthreads();  // the block the caller's threads wrote into L is complete
    bool failed = false;  // uniform in wave 0, the only writer of *info
    for (int p = 0; p < TILE / PW; ++p) {
        const int c0 = PW * p;
        if (p > 0) {
            // row block rb = p + w of the panel: L[rb][p] -= L[rb][0:p] L[p][0:p]^T
            // (whole 16 x 16 blocks; the upper triangle of the diagonal block is
            // never read)
            if (w < TILE / PW - p) {
                const int rb = p + w;
                f64x4 acc = {0.0, 0.0, 0.0, 0.0};
                for (int q = 0; q < c0; q += 4)
                    acc = mma16(L[(PW * rb + ix) * P + q + kr], L[(c0 + ix) * P + q + kr], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) L[(PW * rb + kr + 4 * r) * P + c0 + ix] -= acc[r];
            }
            __syncthreads();
        }
        if (w == 0) {
            const int r = c0 + lane;
            const bool live = r < TILE;
            double a[PW];
#pragma unroll
            for (int j = 0; j < PW; ++j) a[j] = (live && c0 + j <= r) ? L[r * P + c0 + j] : 0.0;
            int fail_col = -1;  // first non-positive pivot of this panel (uniform)
            double dnext = readlane_f64(a[0], 0);
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                double d = dnext;
                if (!(d > 0.0)) {
                    fail_col = fail_col < 0 ? j : fail_col;
                    d = 1.0;
                }
                // 1/sqrt(d) from the hardware estimate and one Newton step (it
                // squares the estimate's relative error)
                double inv = __builtin_amdgcn_rsq(d);
                inv = inv * __builtin_fma(-0.5 * d * inv, inv, 1.5);
                const double piv = d * inv;
                if (lane == 0) rdiag[c0 + j] = inv;
                a[j] = lane > j ? a[j] * inv : (lane == j ? piv : a[j]);
                // Column j + 1, which the next pivot needs, is updated with a
                // register broadcast (lane j + 1's a[j]); the later columns get their
                // multipliers through LDS (one wave: its LDS accesses complete in
                // order, no barrier needed), off the chain of pivots.
                if (j + 1 < PW) {
                    a[j + 1] = __builtin_fma(-a[j], readlane_f64(a[j], j + 1), a[j + 1]);
                    dnext = readlane_f64(a[j + 1], j + 1);
                }
                if (j + 2 < PW) {
                    colj[lane] = a[j];
#pragma unroll
                    for (int c = j + 2; c < PW; ++c) a[c] = __builtin_fma(-a[j], colj[c], a[c]);
                }
            }
            if (fail_col >= 0 && lane == 0 && !failed && *info == 0) *info = k * TILE + c0 + fail_col + 1;
            failed = failed || fail_col >= 0;
            if (live) {
#pragma unroll
                for (int j = 0; j < PW; ++j)
                    if (c0 + j <= r) L[r * P + c0 + j] = a[j];
            }
        }
        __syncthreads();
    }
    // diagonal 16 x 16 blocks of the inverse: wave w, block w, lane = column.
    // Forward substitution, column-oriented: once x[q] is known it is taken out
    // of every later row, so the dependent chain is 16 steps long; each row
    // still receives its terms in order q = 0, 1, ...
    if (lane < PW) {
        const int i0 = PW * w, c = lane;
        double x[PW];
#pragma unroll
        for (int r = 0; r < PW; ++r) x[r] = r == c ? 1.0 : 0.0;
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            x[q] *= rdiag[i0 + q];
#pragma unroll
            for (int r = q + 1; r < PW; ++r) x[r] = __builtin_fma(-L[(i0 + r) * P + i0 + q], x[q], x[r]);
        }
#pragma unroll
        for (int r = 0; r < PW; ++r) X[(i0 + r) * P + i0 + c] = x[r];
    }
    __syncthreads();
    // blocks below the diagonal, by distance d = ib - jb, one wave per block:
    // T = sum_{q=jb}^{ib-1} L[ib][q] X[q][jb], then X[ib][jb] = -X[ib][ib] T.  The
    // 16 x 16 x 4 product leaves rows kr + 4 r of T in register r, which is how
    // the k-group r of the second product's right operand is laid out, so T
    // never leaves the registers.
#pragma unroll
    for (int d = 1; d < TILE / PW; ++d) {
        if (w < TILE / PW - d) {
            const int jb = w, ib = w + d;
            f64x4 tacc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int q = PW * jb; q < PW * ib; q += 4)
                tacc = mma16(L[(PW * ib + ix) * P + q + kr], X[(q + kr) * P + PW * jb + ix], tacc);
            f64x4 xacc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int g = 0; g < 4; ++g) xacc = mma16(X[(PW * ib + ix) * P + PW * ib + 4 * g + kr], tacc[g], xacc);
#pragma unroll
            for (int r = 0; r < 4; ++r) X[(PW * ib + kr + 4 * r) * P + PW * jb + ix] = -xacc[r];
        }
        __syncthreads();
    }
    // L^{-1} to Dinv (blocks above the 16 x 16 block diagonal were never written:
    // zeros).  L[k][k] itself is not stored: every later step reads the diagonal
    // block only through its inverse.
    double* dinv = Dinv + int64_t(k) * TILE * TILE;
    for (int e = t; e < TILE * TILE; e += 256) {
        const int r = e >> 6, c = e & 63;
        dinv[e] = (c >> 4) > (r >> 4) ? 0.0 : X[r * P + c];
    }
}

// The first diagonal block (the others are factored inside the trailing update
// of the step before, see potrf_update_kernel).
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ C, int dp, int k,
                                                         double* __restrict__ Dinv, int32_t* __restrict__ info) {
    __shared__ DiagSmem sm;
    const double* blk = C + int64_t(k) * TILE * dp + int64_t(k) * TILE;
    double v[TILE * TILE / 256];  // all loads in flight before the LDS stores wait on them
#pragma unroll
    for (int q = 0; q < TILE * TILE / 256; ++q) {
        const int e = threadIdx.x + 256 * q;
        v[q] = blk[int64_t(e >> 6) * dp + (e & 63)];
    }
#pragma unroll
    for (int q = 0; q < TILE * TILE / 256; ++q) {
        const int e = threadIdx.x + 256 * q;
        sm.L[(e >> 6) * DP + (e & 63)] = v[q];
    }
    diag_factor(C, dp, k, Dinv, info, sm);
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

// Two-level blocking: the factorisation takes panels of PANEL block columns.
// Inside a panel, step k updates only the panel's later columns (k < j < panel
// end) with block column k; after the panel's last step one update with the
// panel's PANEL columns at once (K = PANEL * 64 = 512) brings the whole trailing
// matrix up to date.  The trailing matrix is then read and written once per
// panel rather than once per block column: at d = 14336 about 31 GB streamed
// instead of about 245 GB.  The updates keep two 32-deep K slices in flight.
constexpr int PANEL = 8;

// C[i][j] -= sum_{k0 <= k < k0 + kw} C[i][k] C[j][k]^T for the blocks t0 <= j <= i,
// j < jend, with t0 = k0 + kw.  Workgroup 0 takes block (t0, t0): it updates it
// into LDS and goes on to factor it (diag_factor), so the next diagonal
// factorisation runs while the other blocks are updated.  The other blocks are
// numbered row by row over the trapezoid (r = i - t0, c = j - t0, c <= r, c < w with
// w = jend - t0): q = r (r + 1) / 2 + c for r < w, then w (w + 1) / 2 + (r - w) w + c;
// workgroup q (q >= 1) takes block q.
__device__ __forceinline__ void trapezoid_index(int q, int w, int& r, int& c) {
    const int tri = w * (w + 1) / 2;
    if (q < tri) {
        r = int((sqrt(8.0 * q + 1.0) - 1.0) * 0.5);
        while (r * (r + 1) / 2 > q) --r;
        while ((r + 1) * (r + 2) / 2 <= q) ++r;
        c = q - r * (r + 1) / 2;
    } else {
        r = w + (q - tri) / w;
        c = (q - tri) % w;
    }
}

__global__ __launch_bounds__(GEMM_THREADS) void potrf_update_kernel(double* __restrict__ C, int dp, int k0, int kw,
                                                                    int jend, double* __restrict__ Dinv,
                                                                    int32_t* __restrict__ info) {
    __shared__ union {
        GemmSmemK<double, 2 * KSTEP> g;
        DiagSmem d;
    } sm;
    const int t0 = k0 + kw;
    int i, j;
    if (blockIdx.x == 0) {
        i = j = t0;
    } else {
        int r, c;
        trapezoid_index(int(blockIdx.x), jend - t0, r, c);
        i = t0 + r;
        j = t0 + c;
    }
    WaveAcc<double> acc;
    acc.zero();
    const double* A = C + int64_t(i) * TILE * dp + int64_t(k0) * TILE;
    const double* B = C + int64_t(j) * TILE * dp + int64_t(k0) * TILE;  // B(kk, c) = C[j*64+c][k0*64+kk]
    double* out = C + int64_t(i) * TILE * dp + int64_t(j) * TILE;
    const bool diag = blockIdx.x == 0;
    double pre[WaveAcc<double>::NREG];  // the diagonal block, loaded while the product runs
    if (diag) {
        const int t = threadIdx.x & 255, lane = t & 63, w = t >> 6;
#pragma unroll
        for (int r = 0; r < WaveAcc<double>::NREG; ++r)
            pre[r] = out[int64_t((w >> 1) * 32 + WaveAcc<double>::row(r, lane)) * dp + (w & 1) * 32 +
                         WaveAcc<double>::col(r, lane)];
    }
    tile_gemm_masked_k2<double, 2 * KSTEP, false, true>(A, dp, B, dp, kw * TILE, sm.g, acc, NoMask(), NoMask());
    if (diag) {
        __syncthreads();  // the product's LDS reads are done before L overwrites them
        const int t = threadIdx.x & 255, lane = t & 63, w = t >> 6;
#pragma unroll
        for (int r = 0; r < WaveAcc<double>::NREG; ++r)
            sm.d.L[((w >> 1) * 32 + WaveAcc<double>::row(r, lane)) * DP + (w & 1) * 32 + WaveAcc<double>::col(r, lane)] =
                pre[r] - acc.get(r);
        diag_factor(C, dp, t0, Dinv, info, sm.d);
        return;
    }
    for_each_acc(acc, [&](int r, int c, double v) { out[int64_t(r) * dp + c] -= v; });
}

// Lower-triangular inverse by recursive halving over block ranges:
// inv([[L11, 0], [L21, L22]]) = [[X11, 0], [-X22 L21 X11, X22]].  Diagonal blocks
// come from the factorisation (Dinv); each recursion level is two launches
// covering all nodes of the level (nodes of one level are disjoint):
//   stage a: Tm[i][j] = sum_{j <= k < mid} L[i][k] Li[k][j]        (L21 X11)
//   stage b: Li[i][j] = -sum_{mid <= k <= i} Li[i][k] Tm[k][j]     (-X22 (L21 X11))
// for i in [mid, hi), j in [lo, mid) with lo = node * 2h, mid = lo + h.
__global__ void trtri_diag_kernel(double* __restrict__ Li, int dp, const double* __restrict__ Dinv) {
    const int k = blockIdx.x;
    double* out = Li + int64_t(k) * TILE * dp + int64_t(k) * TILE;
    const double* src = Dinv + int64_t(k) * TILE * TILE;
    for (int e = threadIdx.x; e < TILE * TILE; e += blockDim.x) out[int64_t(e >> 6) * dp + (e & 63)] = src[e];
}

// The K range of output tile (i, j) is triangular in j (stage a: mid - j tiles)
// or in i (stage b: i - mid + 1 tiles), so one workgroup takes a pair of tiles
// whose ranges add up to the same length: j and lo + h - 1 - (j - lo) in stage a,
// i and hi - 1 - (i - mid) in stage b.  Every workgroup of a level then does the
// same work.
__global__ __launch_bounds__(GEMM_THREADS) void trtri_level_a_kernel(const double* __restrict__ C,
                                                                     const double* __restrict__ Li,
                                                                     double* __restrict__ Tm, int dp, int nt, int h) {
    const int lo = blockIdx.z * 2 * h, mid = lo + h;
    const int hi = lo + 2 * h < nt ? lo + 2 * h : nt;
    const int i = mid + blockIdx.y;
    if (i >= hi) return;
    __shared__ GemmSmem<double> sm;
    const int jpair[2] = {lo + int(blockIdx.x), lo + h - 1 - int(blockIdx.x)};
    for (int q = 0; q < (jpair[0] == jpair[1] ? 1 : 2); ++q) {
        const int j = jpair[q];
        WaveAcc<double> acc;
        acc.zero();
        const double* A = C + int64_t(i) * TILE * dp + int64_t(j) * TILE;
        const double* B = Li + int64_t(j) * TILE * dp + int64_t(j) * TILE;
        tile_gemm<double, double, false, false, false>(A, dp, B, dp, TILE, TILE, (mid - j) * TILE, sm, acc);
        double* out = Tm + int64_t(i) * TILE * dp + int64_t(j) * TILE;
        for_each_acc(acc, [&](int r, int c, double v) { out[int64_t(r) * dp + c] = v; });
    }
}

__global__ __launch_bounds__(GEMM_THREADS) void trtri_level_b_kernel(double* __restrict__ Li,
                                                                     const double* __restrict__ Tm, int dp, int nt,
                                                                     int h) {
    const int lo = blockIdx.z * 2 * h, mid = lo + h;
    const int hi = lo + 2 * h < nt ? lo + 2 * h : nt;
    const int ipair[2] = {mid + int(blockIdx.y), hi - 1 - int(blockIdx.y)};
    if (ipair[0] > ipair[1]) return;
    const int j = lo + blockIdx.x;
    __shared__ GemmSmem<double> sm;
    for (int q = 0; q < (ipair[0] == ipair[1] ? 1 : 2); ++q) {
        const int i = ipair[q];
        WaveAcc<double> acc;
        acc.zero();
        const double* A = Li + int64_t(i) * TILE * dp + int64_t(mid) * TILE;
        const double* B = Tm + int64_t(mid) * TILE * dp + int64_t(j) * TILE;
        tile_gemm<double, double, false, false, false>(A, dp, B, dp, TILE, TILE, (i - mid + 1) * TILE, sm, acc);
        double* out = Li + int64_t(i) * TILE * dp + int64_t(j) * TILE;
        for_each_acc(acc, [&](int r, int c, double v) { out[int64_t(r) * dp + c] = -v; });
    }
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
    size_t off_C, off_Li, off_Tm, off_Dinv, off_scal, bytes;
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
    L.off_Tm = take(size_t(L.dp) * L.dp * 8);
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
    double* Tm = reinterpret_cast<double*>(base + L.off_Tm);
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
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, st, C, dp, 0, Dinv, info);
    KQ_LAUNCHED("potrf_diag_kernel");
    // blocks of the update of [t0, nt) x [t0, jend): the trapezoid below the diagonal
    auto update = [&](int k0, int kw, int jend) {
        const int t0 = k0 + kw, rows = nt - t0, w = jend - t0;
        const int blocks = w * (w + 1) / 2 + (rows - w) * w;
        hipLaunchKernelGGL(potrf_update_kernel, dim3(blocks), dim3(GEMM_THREADS), 0, st, C, dp, k0, kw, jend, Dinv,
                           info);
    };
    for (int p0 = 0; p0 < nt; p0 += PANEL) {
        const int p1 = std::min(p0 + PANEL, nt);
        for (int k = p0; k < p1 && k + 1 < nt; ++k) {
            hipLaunchKernelGGL(potrf_panel_kernel, dim3(nt - k - 1), dim3(GEMM_THREADS), 0, st, C, dp, k, Dinv);
            KQ_LAUNCHED("potrf_panel_kernel");
            if (k + 1 < p1) {  // the panel's later columns, and the next diagonal block
                update(k, 1, p1);
                KQ_LAUNCHED("potrf_update_kernel");
            }
        }
        if (p1 < nt) {  // the whole trailing matrix with the panel's columns, and block p1
            update(p0, p1 - p0, nt);
            KQ_LAUNCHED("potrf_update_kernel");
        }
    }
    hipLaunchKernelGGL(trtri_diag_kernel, dim3(nt), dim3(256), 0, st, Li, dp, Dinv);
    KQ_LAUNCHED("trtri_diag_kernel");
    for (int h = 1; h < nt; h *= 2) {
        const int nodes = (nt + 2 * h - 1) / (2 * h);
        const int half = (h + 1) / 2;  // tile pairs per row (stage a) or column (stage b)
        hipLaunchKernelGGL(trtri_level_a_kernel, dim3(half, h, nodes), dim3(GEMM_THREADS), 0, st, C, Li, Tm, dp, nt,
                           h);
        KQ_LAUNCHED("trtri_level_a_kernel");
        hipLaunchKernelGGL(trtri_level_b_kernel, dim3(h, half, nodes), dim3(GEMM_THREADS), 0, st, Li, Tm, dp, nt, h);
        KQ_LAUNCHED("trtri_level_b_kernel");
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
