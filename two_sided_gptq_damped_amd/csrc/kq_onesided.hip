// One-sided GPTQ (B = I) for gfx950: the recursive, lazily batched form.
//
// What is computed (FastKron page, section 2.1 and section 2.4's GPTQ-recursive
// with lazy batch updates; one-sided GPTQ is the two-sided solver with B = I,
// section 2.2): every row of W is its own problem.  With N = diag(U_A)^{-1} U_A
// (unit upper triangular, N[j', j] = U_A[j', j] / U_A[j', j']) and the row's
// scale s,
//   x_j = W_j + sum_{j' < j} Delta_j' N[j', j],
//   z_j = clamp(rne(x_j / s)),  v_j = s z_j,  Delta_j = v_j - x_j,
// columns in order.  The feedback is batched over column ranges:
//   solve(j0, j1) = solve(j0, mid); X[:, mid:j1] += Delta[:, j0:mid] N[j0:mid, mid:j1];
//                   solve(mid, j1)
// down to 64-column leaves.  All of the method's work, m n (n - 1) flops, is in
// those dense rectangular products (matrix cores) except the leaves' in-block
// triangles (m n 63 flops), and the sequential depth is n / 64 leaves.
//
// Leaf: one lane per row, the block's 64 pre-rounding values in registers and
// the 64 x 64 diagonal block of N in LDS (read as wave-wide broadcasts).  The
// sweep over the block's columns is right-looking: once column j is rounded its
// error is added to the row's later columns, so each column's chain is its own
// rounding plus one fused multiply-add.  Rows do not interact; the only
// barriers guard the LDS staging of the row block.  The quotient x / s is
// formed as x * (1/s), as in the two-sided leaf.
//
// Workspace (the two-sided solver's layout; the output-factor and stage buffers
// are not touched): NA np x np, X mp x np (starts as W), D mp x np (errors),
// S mp.  Padding as there: zero weights, unit scales, identity factor.
#include <type_traits>

#include "kq_common.hpp"

namespace kq {

constexpr int OS_BLK = 64;   // columns per leaf
constexpr int OS_ROWS = 64;  // rows per leaf workgroup: one wave, one row per lane

__device__ __forceinline__ float os_clamp(float x, float lo, float hi) { return __builtin_amdgcn_fmed3f(x, lo, hi); }
__device__ __forceinline__ double os_clamp(double x, double lo, double hi) { return kclamp(x, lo, hi); }

// The value v of lane l (wave-uniform l).
__device__ __forceinline__ float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ double lane_value(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(u)), l);
    const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(u >> 32)), l);
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

// Leaf over columns [j0, j0 + 64) for rows r0 = 64 blockIdx.x .. r0 + 63.
// Global memory is read and written row by row (16-byte accesses, coalesced),
// through the LDS tile xs that holds one row per lane (pitch 68: 16-byte
// aligned rows, and a wave's 16-byte accesses cover all banks evenly).  The
// 64 columns are taken in four sub-blocks of 16: a sub-block's pre-rounding
// values sit in registers for its sweep (right-looking: once column j is
// rounded its error goes into the sub-block's later columns), then its 16
// errors are applied to the row's later sub-blocks in LDS, four columns at a
// time.  The sub-block loop is not unrolled, so the code a lone wave runs is a
// few kilobytes that stay in the instruction cache.
// ENTRY (the WaterKron alphabet): entry (i, j) has the step S[i] * C[j] and the
// codes are int32.
template <typename T, bool ENTRY>
__global__ __launch_bounds__(OS_ROWS) void onesided_leaf_kernel(const T* __restrict__ X, T* __restrict__ D,
                                                                const T* __restrict__ NA, const T* __restrict__ S,
                                                                const T* __restrict__ C, int np, int j0, int m, int n,
                                                                int qmin, int qmax,
                                                                std::conditional_t<ENTRY, int32_t, int8_t>* __restrict__ Z,
                                                                int64_t ldz, T* __restrict__ V, int64_t ldv) {
    constexpr int SB = 16;                       // sub-block width
    constexpr int VN = 16 / sizeof(T);           // entries per 16-byte access
    constexpr int SP = OS_BLK + 16 / sizeof(T);  // xs row pitch: 68 fp32 / 66 fp64
    typedef T VT __attribute__((ext_vector_type(VN)));
    // cf[j][jj] = N[j0 + j][j0 + jj] strictly above the diagonal, 0 elsewhere
    __shared__ __attribute__((aligned(16))) T cf[OS_BLK][OS_BLK];
    __shared__ __attribute__((aligned(16))) T xs[OS_ROWS * SP];
    // codes: int8 packed four per word, or int32 (ENTRY); rows padded by one word
    __shared__ uint32_t zs[ENTRY ? OS_BLK : OS_BLK / 4][OS_ROWS + 1];
    const int lane = threadIdx.x, r0 = blockIdx.x * OS_ROWS;
    // 16-byte loads: LPR lanes cover one 64-entry row, RPI rows per instruction,
    // so the whole row block and the coefficient block are in flight at once
    constexpr int LPR = OS_BLK / VN, RPI = 64 / LPR, NI = OS_ROWS / RPI;
    const int lr = lane / LPR, lc = (lane % LPR) * VN;
    {
        VT xa[NI], ca[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
            xa[i] = *reinterpret_cast<const VT*>(X + int64_t(r0 + RPI * i + lr) * np + j0 + lc);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            ca[i] = *reinterpret_cast<const VT*>(NA + int64_t(j0 + RPI * i + lr) * np + j0 + lc);
#pragma unroll
        for (int i = 0; i < NI; ++i) *reinterpret_cast<VT*>(&xs[(RPI * i + lr) * SP + lc]) = xa[i];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            VT c = ca[i];
#pragma unroll
            for (int e = 0; e < VN; ++e)
                if (lc + e <= RPI * i + lr) c[e] = T(0);
            *reinterpret_cast<VT*>(&cf[RPI * i + lr][lc]) = c;
        }
    }
    const T s = S[r0 + lane];
    const T rs = s == T(0) ? T(0) : T(1) / s;
    const T tqmin = T(qmin), tqmax = T(qmax);
    T* const xr = xs + lane * SP;
    __syncthreads();
#pragma unroll 1
    for (int c0 = 0; c0 < OS_BLK; c0 += SB) {
        T x[SB];
#pragma unroll
        for (int q = 0; q < SB / VN; ++q) {
            const VT v = *reinterpret_cast<const VT*>(xr + c0 + VN * q);
#pragma unroll
            for (int e = 0; e < VN; ++e) x[VN * q + e] = v[e];
        }
        uint32_t zp[SB / 4] = {};
        T se[ENTRY ? SB : 1], rse[ENTRY ? SB : 1];  // per-entry steps and their reciprocals
        if (ENTRY) {
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                se[j] = s * C[j0 + c0 + j];
                rse[j] = se[j] == T(0) ? T(0) : T(1) / se[j];
            }
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const T sj = ENTRY ? se[j] : s, rj = ENTRY ? rse[j] : rs;
            const T z = os_clamp(krint(x[j] * rj), tqmin, tqmax);
            const T d = sj * z - x[j];
            x[j] = d;  // from here on x[j] holds the error
            if (ENTRY)
                zs[c0 + j][lane] = uint32_t(int(z));
            else
                zp[j >> 2] |= (uint32_t(int(z)) & 0xffu) << (8 * (j & 3));
#pragma unroll
            for (int q = (j + 1) / VN; q < SB / VN; ++q) {
                const VT c = *reinterpret_cast<const VT*>(&cf[c0 + j][c0 + VN * q]);
#pragma unroll
                for (int e = 0; e < VN; ++e)
                    if (VN * q + e > j) x[VN * q + e] = kfma(d, c[e], x[VN * q + e]);
            }
        }
#pragma unroll
        for (int q = 0; q < SB / VN; ++q) {
            VT v;
#pragma unroll
            for (int e = 0; e < VN; ++e) v[e] = x[VN * q + e];
            *reinterpret_cast<VT*>(xr + c0 + VN * q) = v;
        }
        if (!ENTRY) {
#pragma unroll
            for (int q = 0; q < SB / 4; ++q) zs[c0 / 4 + q][lane] = zp[q];
        }
        // the sub-block's errors into the row's later columns, VN at a time
#pragma unroll 2
        for (int g = c0 + SB; g < OS_BLK; g += VN) {
            VT acc = *reinterpret_cast<const VT*>(xr + g);
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const VT c = *reinterpret_cast<const VT*>(&cf[c0 + j][g]);
#pragma unroll
                for (int e = 0; e < VN; ++e) acc[e] = kfma(x[j], c[e], acc[e]);
            }
            *reinterpret_cast<VT*>(xr + g) = acc;
        }
    }
    __syncthreads();  // every lane's row of errors and codes is complete
#pragma unroll
    for (int i = 0; i < NI; ++i)
        *reinterpret_cast<VT*>(D + int64_t(r0 + RPI * i + lr) * np + j0 + lc) =
            *reinterpret_cast<const VT*>(&xs[(RPI * i + lr) * SP + lc]);
    // Z and V = s z row by row; row rr's scale is lane rr's s, read across the wave
    const bool col_ok = j0 + lane < n;
    const T cl = ENTRY ? C[j0 + lane] : T(1);  // this lane's column scale
    for (int rr = 0; rr < OS_ROWS && r0 + rr < m; ++rr) {
        const int z = ENTRY ? int(zs[lane][rr]) : int(int8_t(uint8_t(zs[lane >> 2][rr] >> (8 * (lane & 3)))));
        const T sr = ENTRY ? lane_value(s, rr) * cl : lane_value(s, rr);
        if (col_ok) {
            Z[int64_t(r0 + rr) * ldz + j0 + lane] = std::remove_reference_t<decltype(Z[0])>(z);
            V[int64_t(r0 + rr) * ldv + j0 + lane] = sr * T(z);
        }
    }
}

// X[:, mid:j1] += D[:, j0:mid] N[j0:mid, mid:j1] on 64 x 64 output blocks: block
// (Q, P) covers columns mid + 64 Q and rows 64 P.  Q runs fastest, so blocks that
// share the row panel of D are dispatched together.
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS) void onesided_update_kernel(const T* __restrict__ D,
                                                                       const T* __restrict__ NA, T* __restrict__ X,
                                                                       int np, int j0, int mid) {
    __shared__ GemmSmem<T> sm;
    const int Q = blockIdx.x, P = blockIdx.y;
    WaveAcc<T> acc;
    acc.zero();
    const T* A = D + int64_t(P) * TILE * np + j0;
    const T* B = NA + int64_t(j0) * np + mid + Q * TILE;
    tile_gemm<T, T, false, false, false>(A, np, B, np, TILE, TILE, mid - j0, sm, acc);
    T* out = X + int64_t(P) * TILE * np + mid + Q * TILE;
    for_each_acc(acc, [&](int rr, int cc, T v) { out[int64_t(rr) * np + cc] += v; });
}

template <typename T>
struct OneSidedRun {
    int m, n, mp, np, qmin, qmax;
    const T* NA;
    T *X, *D;
    const T *S, *C;  // C: column scales (WaterKron mode) or nullptr
    void* Z;         // int8 codes, int32 in the WaterKron mode
    int64_t ldz;
    T* V;
    int64_t ldv;
    hipStream_t st;

    kq_status leaf(int j0) {
        if (C)
            hipLaunchKernelGGL((onesided_leaf_kernel<T, true>), dim3(unsigned(mp / OS_ROWS)), dim3(OS_ROWS), 0, st, X, D,
                               NA, S, C, np, j0, m, n, qmin, qmax, static_cast<int32_t*>(Z), ldz, V, ldv);
        else
            hipLaunchKernelGGL((onesided_leaf_kernel<T, false>), dim3(unsigned(mp / OS_ROWS)), dim3(OS_ROWS), 0, st, X,
                               D, NA, S, C, np, j0, m, n, qmin, qmax, static_cast<int8_t*>(Z), ldz, V, ldv);
        KQ_LAUNCHED("onesided_leaf_kernel");
        return KQ_OK;
    }
    kq_status update(int j0, int mid, int j1) {
        hipLaunchKernelGGL(onesided_update_kernel<T>, dim3(unsigned((j1 - mid) / TILE), unsigned(mp / TILE)),
                           dim3(GEMM_THREADS), 0, st, D, NA, X, np, j0, mid);
        KQ_LAUNCHED("onesided_update_kernel");
        return KQ_OK;
    }
    kq_status solve(int j0, int j1) {
        if (j1 - j0 <= OS_BLK) return leaf(j0);
        const int blocks = (j1 - j0) / OS_BLK;
        const int mid = j0 + OS_BLK * (blocks / 2);
        kq_status s = solve(j0, mid);
        if (s != KQ_OK) return s;
        s = update(j0, mid, j1);
        if (s != KQ_OK) return s;
        return solve(mid, j1);
    }
};

// mp, np: multiples of 64 (the padded extents of the workspace buffers).
template <typename T>
kq_status onesided_solve(int m, int n, int mp, int np, int qmin, int qmax, const T* NA, T* X, T* D, const T* S,
                         const T* C, void* Z, int64_t ldz, T* V, int64_t ldv, hipStream_t st) {
    OneSidedRun<T> run{m, n, mp, np, qmin, qmax, NA, X, D, S, C, Z, ldz, V, ldv, st};
    return run.solve(0, np);
}

template kq_status onesided_solve<float>(int, int, int, int, int, int, const float*, float*, float*, const float*,
                                         const float*, void*, int64_t, float*, int64_t, hipStream_t);
template kq_status onesided_solve<double>(int, int, int, int, int, int, const double*, double*, double*,
                                          const double*, const double*, void*, int64_t, double*, int64_t,
                                          hipStream_t);

}  // namespace kq
