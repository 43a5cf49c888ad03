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
// down to chunks of four 64-column leaves; inside a chunk each leaf first pulls
// the products of the chunk's earlier leaves, X[:, leaf] += Delta[:, chunk start
// : leaf] N[.., leaf], then sweeps.  All of the method's work, m n (n - 1) flops,
// is in those dense rectangular products (matrix cores) except the leaves'
// in-block triangles (m n 63 flops), and the sequential depth is n / 64 leaves.
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
constexpr int OS_ROWS = 64;  // rows per leaf workgroup
constexpr int OS_CHUNK = 4;  // leaves per chunk: the recursion's lowest unit

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

// Leaf over columns [j0, j0 + 64) for rows r0 = 64 blockIdx.x .. r0 + 63, four
// waves of 16 rows.  Each row is spread over the four lanes of a quad: lane q of
// the quad owns the columns c = 4 i + q (i < 16), so every lane holds a quarter
// of the row's later columns at every step.  The sweep is right-looking and
// fully unrolled over the 64 columns: the owner of column j (lane j mod 4) rounds
// it, a DPP quad broadcast hands its error to the row's other three lanes, and
// each lane adds error * N[j][c] to its columns c > j (the ones with i >= j / 4,
// known at compile time; the few with c <= j get an exact zero coefficient).  The
// coefficients sit in LDS per lane class, cq[q][j][i] = N[j0 + j][j0 + 4 i + q]
// strictly above the diagonal and 0 elsewhere, so a lane reads its four
// consecutive i with one 16-byte access, and the lanes of a class share the
// address (an LDS broadcast).  Global memory is read and written row by row
// (16-byte accesses, coalesced) through the LDS tile xs (pitch 68 fp32 / 66 fp64).
// ENTRY (the WaterKron alphabet): entry (i, j) has the step S[i] * C[j] and the
// codes are int32.
constexpr int OS_THREADS = 256;  // four waves
constexpr int OS_WROWS = 16;     // rows per wave: four lanes per row

// v of lane q of this lane's quad (q a constant: a DPP quad_perm broadcast).
template <int Q>
__device__ __forceinline__ float quad_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), Q * 0x55, 0xf, 0xf, false));
}
template <int Q>
__device__ __forceinline__ double quad_bcast(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_mov_dpp(int(uint32_t(u)), Q * 0x55, 0xf, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_mov_dpp(int(uint32_t(u >> 32)), Q * 0x55, 0xf, 0xf, false);
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

template <typename T, bool ENTRY, int J>
struct OsSweep {
    // column J: rounding by its owner, then its error into the later columns
    static __device__ __forceinline__ void step(T (&x)[16], const T* __restrict__ cqr, int q, T s, T rs,
                                                const T* __restrict__ C, int j0, T tqmin, T tqmax,
                                                std::conditional_t<ENTRY, int32_t, int8_t>* __restrict__ zcol) {
        constexpr int I = J >> 2, QJ = J & 3;
        T sj = s, rj = rs;
        if (ENTRY) {
            sj = s * C[j0 + J];
            rj = sj == T(0) ? T(0) : T(1) / sj;
        }
        const T z = os_clamp(krint(x[I] * rj), tqmin, tqmax);
        const T d = sj * z - x[I];
        const bool own = q == QJ;
        if (own) {
            x[I] = d;  // from here on the owner's x[I] holds the error
            zcol[J * (OS_ROWS + 1)] = std::conditional_t<ENTRY, int32_t, int8_t>(int(z));
        }
        const T db = quad_bcast<QJ>(d);
        // columns 4 i + q > J for i >= I (the owner's own column J, and the
        // columns 4 I + q <= J of the lanes before it, have zero coefficients)
        const T* cj = cqr + J * 16;
#pragma unroll
        for (int g = I >> 2; g < 4; ++g) {
            typedef T V4 __attribute__((ext_vector_type(4)));
            V4 c;
            if (sizeof(T) == 4) {
                c = *reinterpret_cast<const V4*>(cj + 4 * g);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) c[e] = cj[4 * g + e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * g + e >= I) x[4 * g + e] = kfma(db, c[e], x[4 * g + e]);
        }
        OsSweep<T, ENTRY, J + 1>::step(x, cqr, q, s, rs, C, j0, tqmin, tqmax, zcol);
    }
};
template <typename T, bool ENTRY>
struct OsSweep<T, ENTRY, OS_BLK> {
    static __device__ __forceinline__ void step(T (&)[16], const T*, int, T, T, const T*, int, T, T,
                                                std::conditional_t<ENTRY, int32_t, int8_t>*) {}
};

template <typename T, bool ENTRY>
__global__ __launch_bounds__(OS_THREADS) void onesided_leaf_kernel(const T* __restrict__ X, T* __restrict__ D,
                                                                   const T* __restrict__ NA, const T* __restrict__ S,
                                                                   const T* __restrict__ C, int np, int c0, int j0,
                                                                   int m, int n, int qmin, int qmax,
                                                                   std::conditional_t<ENTRY, int32_t, int8_t>* __restrict__ Z,
                                                                   int64_t ldz, T* __restrict__ V, int64_t ldv) {
    using CodeT = std::conditional_t<ENTRY, int32_t, int8_t>;
    constexpr int VN = 16 / sizeof(T);           // entries per 16-byte access
    constexpr int SP = OS_BLK + 16 / sizeof(T);  // xs row pitch: 68 fp32 / 66 fp64
    typedef T VT __attribute__((ext_vector_type(VN)));
    __shared__ __attribute__((aligned(16))) T cq[4][OS_BLK][16];
    __shared__ __attribute__((aligned(16))) T xs[OS_ROWS * SP];
    __shared__ CodeT zs[OS_BLK][OS_ROWS + 1];  // zs[column][row]
    __shared__ GemmSmem<T> sg;                  // the chunk product's staging
    const int t = threadIdx.x, r0 = blockIdx.x * OS_ROWS;
    // 16-byte loads: LPR threads cover one 64-entry row, RPI rows per pass
    constexpr int LPR = OS_BLK / VN, RPI = OS_THREADS / LPR, NI = OS_ROWS / RPI;
    const int lr = t / LPR, lc = (t % LPR) * VN;
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
            const int j = RPI * i + lr;
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                const int c = lc + e;
                cq[c & 3][j][c >> 2] = c > j ? ca[i][e] : T(0);
            }
        }
    }
    // the chunk's earlier leaves: X[rows, j0:j0+64] += D[rows, c0:j0] N[c0:j0, j0:j0+64]
    if (j0 > c0) {
        WaveAcc<T> acc;
        acc.zero();
        tile_gemm<T, T, false, false, false>(D + int64_t(r0) * np + c0, np, NA + int64_t(c0) * np + j0, np, TILE,
                                             TILE, j0 - c0, sg, acc);
        for_each_acc(acc, [&](int r, int c, T v) { xs[r * SP + c] += v; });
    }
    const int w = t >> 6, lane = t & 63, q = lane & 3;
    const int row = OS_WROWS * w + (lane >> 2);  // this lane's row in the block
    const T s = S[r0 + row];
    const T rs = s == T(0) ? T(0) : T(1) / s;
    __syncthreads();
    T x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = xs[row * SP + 4 * i + q];
    OsSweep<T, ENTRY, 0>::step(x, &cq[q][0][0], q, s, rs, C, j0, T(qmin), T(qmax), &zs[0][row]);
#pragma unroll
    for (int i = 0; i < 16; ++i) xs[row * SP + 4 * i + q] = x[i];
    __syncthreads();  // every row's errors and codes are complete
#pragma unroll
    for (int i = 0; i < NI; ++i)
        *reinterpret_cast<VT*>(D + int64_t(r0 + RPI * i + lr) * np + j0 + lc) =
            *reinterpret_cast<const VT*>(&xs[(RPI * i + lr) * SP + lc]);
    // Z and V = step * z: column t % 64, rows t / 64 + 4 k
    const int col = t & 63;
    const bool col_ok = j0 + col < n;
    const T cl = ENTRY ? C[j0 + col] : T(1);
#pragma unroll 4
    for (int rr = t >> 6; rr < OS_ROWS; rr += OS_THREADS / 64) {
        if (r0 + rr >= m || !col_ok) continue;
        const int z = int(zs[col][rr]);
        Z[int64_t(r0 + rr) * ldz + j0 + col] = CodeT(z);
        V[int64_t(r0 + rr) * ldv + j0 + col] = S[r0 + rr] * cl * T(z);
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

    kq_status leaf(int c0, int j0) {
        if (C)
            hipLaunchKernelGGL((onesided_leaf_kernel<T, true>), dim3(unsigned(mp / OS_ROWS)), dim3(OS_THREADS), 0, st, X,
                               D, NA, S, C, np, c0, j0, m, n, qmin, qmax, static_cast<int32_t*>(Z), ldz, V, ldv);
        else
            hipLaunchKernelGGL((onesided_leaf_kernel<T, false>), dim3(unsigned(mp / OS_ROWS)), dim3(OS_THREADS), 0, st, X,
                               D, NA, S, C, np, c0, j0, m, n, qmin, qmax, static_cast<int8_t*>(Z), ldz, V, ldv);
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
        const int blocks = (j1 - j0) / OS_BLK;
        if (blocks <= OS_CHUNK) {  // a chunk: each leaf pulls its earlier leaves' products
            for (int l = 0; l < blocks; ++l) {
                const kq_status s = leaf(j0, j0 + OS_BLK * l);
                if (s != KQ_OK) return s;
            }
            return KQ_OK;
        }
        const int chunks = (blocks + OS_CHUNK - 1) / OS_CHUNK;
        const int mid = j0 + OS_BLK * OS_CHUNK * (chunks / 2);
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
