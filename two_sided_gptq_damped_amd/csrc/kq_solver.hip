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
// Schedule.  The matrix is cut into 32 x 32 scheduling tiles; tiles with
// I + J = K form tile-diagonal K and are independent for the same reason.
// solve(K0, K1) over tile-diagonal ranges follows section 2.5's recursion:
// solve(K0, mid); add the errors of the first half to the second half with two
// batched products; solve(mid, K1):
//   stage 1  T1[I', J] = sum_{J' : K0 <= I'+J' < mid} Delta[I', J'] N_A[J', J]
//            for the tiles (I', J) a target can read (K0 <= I'+J < K1, I' < mid)
//   stage 2  X[I, J] += sum_{I'} N_B[I', I]^T T1[I', J] for mid <= I+J < K1.
// Both stages run on 64 x 64 matrix-core output blocks (2 x 2 scheduling tiles)
// and mask at 32-tile granularity: source tiles outside the band and T1 tiles not
// written by this node read as zero, targets outside the band are not written.
// A leaf is one tile-diagonal: each 32 x 32 tile runs the element-level
// anti-diagonal sweep (63 steps) with the in-tile feedback, one workgroup per tile.
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

constexpr int ST = 32;    // scheduling tile edge
constexpr int CHUNK = 8;  // tile-diagonals per recursion leaf (chunk)

// N[r][c] = U[r][c] / U[r][r] for c >= r inside d x d; identity in the padding.
// Rows blockIdx.y, + gridDim.y, ...; each thread four consecutive columns (dp is
// a multiple of 64, so they are in range and the store is 16-byte aligned).
template <typename T>
__global__ void normalize_factor_kernel(const T* __restrict__ U, int64_t ldu, int d, int dp,
                                        T* __restrict__ N);

template <typename T>
__global__ void init_solver_kernel(const T* __restrict__ W, int64_t ldw, int m, int n, int mp, int np,
                                   const T* __restrict__ scales, int per_row, T* __restrict__ X,
                                   T* __restrict__ S);

// Four consecutive elements (16-byte aligned), from global memory or LDS.
template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
    f32x4 v;
    __device__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
    __device__ void store(float* p) const { *reinterpret_cast<f32x4*>(p) = v; }
    __device__ float operator[](int j) const { return v[j]; }
    __device__ void set(int j, float x) { v[j] = x; }
};
template <>
struct Vec4<double> {
    f64x2 lo, hi;
    __device__ void load(const double* p) {
        lo = reinterpret_cast<const f64x2*>(p)[0];
        hi = reinterpret_cast<const f64x2*>(p)[1];
    }
    __device__ void store(double* p) const {
        reinterpret_cast<f64x2*>(p)[0] = lo;
        reinterpret_cast<f64x2*>(p)[1] = hi;
    }
    __device__ double operator[](int j) const { return j < 2 ? lo[j] : hi[j - 2]; }
    __device__ void set(int j, double x) {
        if (j < 2)
            lo[j] = x;
        else
            hi[j - 2] = x;
    }
};

// Leaf: the tiles of one tile-diagonal K, one 512-thread workgroup per 32 x 32
// tile.  In the sweep thread t owns two entries of column b = t % 32, rows
// (2g - b + i) mod 32 with g = t / 32 (see the layouts below).  Right-looking
// in-tile feedback: after the entries of
// element anti-diagonal d are rounded, each later entry adds the contribution of
// the rounded entry in its row (Delta * L~_A) and of the one in its column
// (L~_B * R, R the row-accumulated error).  One wave rounds four consecutive
// diagonals per round and one barrier separates the rounds (the exchange
// arrays hold every round's values, so nothing is overwritten while read);
// finished errors and codes go to LDS for the epilogue.
//
// The tile's diagonal factor blocks sit in LDS with their unit diagonal
// replaced by 0 and an extra all-zero row / column; a source that does not exist
// (off the tile) is mapped to that zero line.  Because N is upper triangular,
// every update whose source is not strictly to the left / above its target then
// multiplies by an exact zero, so the updates need no predicates (finished
// entries only ever receive +0).  The exchange arrays start at zero so the
// multiplied values are always finite.
//
// Chunks.  The recursion stops at chunks of consecutive tile-diagonals
// [c0, c1); inside a chunk the feedback between tiles is pulled by each leaf
// (left-looking, the per-entry form of section 2.4 at tile granularity).  For
// tile (I, J) on diagonal K of the chunk, with the chunk-local row-propagated
// errors
//   T1c[I', J] = sum_{J' <= J, I' + J' >= c0} Delta[I', J'] N_A[J', J]
// (written by tile (I', J)'s own leaf), the chunk's contribution is
//   rowpart = sum_{c0 - I <= J' < J} Delta[I, J'] N_A[J', J]
//   X[I, J] += N_B[I, I]^T rowpart + sum_{c0 - J <= I' < I} N_B[I', I]^T T1c[I', J]
// and after the sweep the leaf writes T1c[I, J] = rowpart + Delta[I, J] N_A[J, J]
// for the later diagonals of its chunk.  With B = I only rowpart is added.  The
// 32 x 32 x 32 products run on the matrix cores: their operands are staged
// k-major in LDS and each wave owns one 16 x 16 quadrant of one of the two sums,
// over all of its slices, so the sums need no reduction across waves.
//
// The quotient x / s is formed as x * (1/s) (1/s rounded once per row): within
// two ulps of the IEEE quotient, so it can change a rounding decision only for
// values that sit within ~1e-15 (fp64) or ~1e-7 (fp32) grid units of a
// midpoint.  A zero scale has 1/s = 0, so q = 0 and the code is 0 with no test
// (for finite x).
__device__ __forceinline__ float clamp_fast(float x, float lo, float hi) { return __builtin_amdgcn_fmed3f(x, lo, hi); }
__device__ __forceinline__ double clamp_fast(double x, double lo, double hi) { return kclamp(x, lo, hi); }
template <typename T>
__device__ __forceinline__ void quantize_fast(T x, T s, T rs, T qmin, T qmax, T& z, T& v) {
    z = clamp_fast(krint(x * rs), qmin, qmax);  // one median-of-three for fp32 (finite x)
    v = s * z;
}

// The value of v in the next lower lane of the wave (lane 0 gets 0): a DPP
// shift of the whole wave by one lane.  With bound_ctrl the lane without a
// source reads 0, so the shift can ride on the FMA that consumes it.
__device__ __forceinline__ float lane_below(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ double lane_below(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(u)), 0x138, 0xf, 0xf, true);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(u >> 32)), 0x138, 0xf, 0xf, true);
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

// N consecutive LDS entries as one vector access.
// v of lane l - 32 in the upper half of the wave (lanes 32..63); the lower half
// keeps its own v (permlane32_swap of v with itself).
__device__ __forceinline__ float lanes_up32(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_permlane32_swap(u, u, false, false)[0]);
}
__device__ __forceinline__ double lanes_up32(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const unsigned lo = unsigned(u), hi = unsigned(u >> 32);
    const unsigned slo = __builtin_amdgcn_permlane32_swap(lo, lo, false, false)[0];
    const unsigned shi = __builtin_amdgcn_permlane32_swap(hi, hi, false, false)[0];
    return __builtin_bit_cast(double, (uint64_t(shi) << 32) | slo);
}

template <typename T>
__global__ void normalize_factor_kernel(const T* __restrict__ U, int64_t ldu, int d, int dp,
                                        T* __restrict__ N) {
    const int c0 = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (c0 >= dp) return;
    for (int r = blockIdx.y; r < dp; r += gridDim.y) {
        const T* row = U + int64_t(r) * ldu;
        const T diag = r < d ? row[r] : T(1);
        Vec4<T> v;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + u;
            T x;
            if (r < d && c < d)
                x = (c >= r) ? row[c] / diag : T(0);
            else
                x = (r == c) ? T(1) : T(0);
            v.set(u, x);
        }
        v.store(N + int64_t(r) * dp + c0);
    }
}

// X = W zero-padded to mp x np; S = the scales, unit in the padding.  Rows as in
// normalize_factor_kernel, four consecutive columns per thread.
template <typename T>
__global__ void init_solver_kernel(const T* __restrict__ W, int64_t ldw, int m, int n, int mp, int np,
                                   const T* __restrict__ scales, int per_row, T* __restrict__ X,
                                   T* __restrict__ S) {
    const int c0 = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    for (int r = blockIdx.y; r < mp; r += gridDim.y) {
        if (blockIdx.x == 0 && threadIdx.x == 0) S[r] = r < m ? scales[per_row ? r : 0] : T(1);
        if (c0 >= np) continue;
        Vec4<T> v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v.set(u, (r < m && c0 + u < n) ? W[int64_t(r) * ldw + c0 + u] : T(0));
        v.store(X + int64_t(r) * np + c0);
    }
}

template <typename T, int N>
struct VecN {
    typedef T V __attribute__((ext_vector_type(N)));
    V v;
    __device__ void load(const T* p) { v = *reinterpret_cast<const V*>(p); }
    __device__ void store(T* p) const { *reinterpret_cast<V*>(p) = v; }
    __device__ T operator[](int j) const { return v[j]; }
    __device__ void set(int j, T x) { v[j] = x; }
};

// One wave's 16 x 16 block on the matrix cores: acc += A (16 x KD) B (KD x 16)
// with A(r, k) = As[k * SA + r] and B(k, c) = Bs[k * SB + c].  Operand lanes
// A[r = l % 16][k = l / 16], B[k = l / 16][c = l % 16]; result register r of lane
// l sits at row 4 (l / 16) + r (fp32) or l / 16 + 4 r (fp64), column l % 16
// (measured on gfx950).
template <typename T>
struct Q16;
template <>
struct Q16<float> {
    f32x4 c;
    __device__ void zero() { c = f32x4{0.f, 0.f, 0.f, 0.f}; }
    template <int SA, int SB, int KD>
    __device__ void mma(const float* As, const float* Bs, int lane) {
        const int kr = lane >> 4, ix = lane & 15;
#pragma unroll
        for (int kk = 0; kk < KD; kk += 4)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(As[(kk + kr) * SA + ix], Bs[(kk + kr) * SB + ix], c, 0, 0, 0);
    }
    __device__ float get(int r) const { return c[r]; }
    static __device__ __forceinline__ int row(int r, int lane) { return 4 * (lane >> 4) + r; }
    static __device__ __forceinline__ int col(int, int lane) { return lane & 15; }
};
template <>
struct Q16<double> {
    f64x4 c;
    __device__ void zero() { c = f64x4{0.0, 0.0, 0.0, 0.0}; }
    template <int SA, int SB, int KD>
    __device__ void mma(const double* As, const double* Bs, int lane) {
        const int kr = lane >> 4, ix = lane & 15;
#pragma unroll
        for (int kk = 0; kk < KD; kk += 4)
            c = __builtin_amdgcn_mfma_f64_16x16x4f64(As[(kk + kr) * SA + ix], Bs[(kk + kr) * SB + ix], c, 0, 0, 0);
    }
    __device__ double get(int r) const { return c[r]; }
    static __device__ __forceinline__ int row(int r, int lane) { return (lane >> 4) + 4 * r; }
    static __device__ __forceinline__ int col(int, int lane) { return lane & 15; }
};

constexpr int LEAF_THREADS = 512;   // the chunk products and the table set-up
constexpr int SWEEP_THREADS = 512;  // the sweep: two entries per thread
constexpr int LEAF_E = ST * ST / SWEEP_THREADS;

template <typename T>
__global__ __launch_bounds__(LEAF_THREADS) void leaf_kernel(const T* __restrict__ X, T* __restrict__ D,
                                                   const T* __restrict__ NA, const T* __restrict__ NB,
                                                   const T* __restrict__ S, T* __restrict__ T1c, int np, int mp,
                                                   int Mt, int Nt, int K, int c0, int c1, int m, int n, int qmin,
                                                   int qmax, int8_t* __restrict__ Z, int64_t ldz,
                                                   T* __restrict__ V, int64_t ldv) {
    constexpr int PB = ST + 4;  // 16-byte aligned rows for the vector reads
    constexpr int PA = ST + 1;  // column ST is the zero sentinel
    constexpr int PK = ST + 4;  // k-major staging rows, 16-byte aligned
    __shared__ __attribute__((aligned(16))) T sNB[(ST + 1) * PB];  // sNB[as][a] = N_B[..as][..a], row ST = 0
    __shared__ T sNAt[ST * PA];                                    // sNAt[b][bs] = N_A[..bs][..b], col ST = 0
    constexpr int RD = 2 * LEAF_E;                      // diagonals per sweep round (one wave's two groups)
    constexpr int NROUND = (2 * ST - 1 + RD - 1) / RD;  // sweep rounds
    // chunk operands of up to BATCH slices: A(r, k) at [k][r], B(k, c) at [k][c]
    constexpr int MAXS = 2 * (CHUNK - 1);                  // most slices a leaf needs
    constexpr int BATCH = sizeof(T) == 4 ? MAXS : MAXS / 2;  // staged together (LDS budget)
    __shared__ __attribute__((aligned(16))) T stg[BATCH][2][ST * PK];
    T* const bufA = stg[0][0];
    T* const bufB = stg[0][1];

    const int ilo = K - Nt + 1 > 0 ? K - Nt + 1 : 0;
    const int I = ilo + blockIdx.x;
    const int ihi = K < Mt - 1 ? K : Mt - 1;
    if (I > ihi) return;
    const int J = K - I;
    // threads t < 256 also work in the block layout (four rows each); all
    // LEAF_THREADS threads take part in the sweep
    const int t = threadIdx.x, tb = t & 255, w = tb >> 6, l = tb & 63;
    const bool blk = t < 256;
    const int b = l & 31, r0 = 8 * w + 4 * (l >> 5);
    const int fgrp = t >> 8;                    // staging loads: slices rotate over the 256-thread groups
    const int wv = t >> 6, lane = t & 63;  // chunk products: wave, lane
    const int q8 = tb >> 3, c4 = 4 * (tb & 7);  // this thread's share of a 32 x 32 staging load

    // chunk sources: row tiles J' in [jl, J), column tiles I' in [il, I)
    const int jl = c0 - I > 0 ? c0 - I : 0;
    const int il = c0 - J > 0 ? c0 - J : 0;
    const int n1 = J - jl;
    const int n2 = NB ? I - il : 0;
    const int ns = n1 + n2;
    constexpr int NFG = LEAF_THREADS / 256;
    constexpr int SLOTS = (BATCH + NFG - 1) / NFG;  // slices of a batch held by one thread
    Vec4<T> pa[SLOTS], pb[SLOTS];
    auto fetch = [&](int sl, Vec4<T>& va, Vec4<T>& vb) {
        if (sl < n1) {
            const int jp = jl + sl;
            va.load(D + int64_t(I * ST + q8) * np + jp * ST + c4);   // A(r = q8, k = c4 + j)
            vb.load(NA + int64_t(jp * ST + q8) * np + J * ST + c4);  // B(k = q8, c = c4 + j)
        } else {
            const int ip = il + sl - n1;
            va.load(NB + int64_t(ip * ST + q8) * mp + I * ST + c4);  // A(r = c4 + j, k = q8)
            vb.load(T1c + int64_t(ip * ST + q8) * np + J * ST + c4); // B(k = q8, c = c4 + j)
        }
    };
    // every load of the first batch is in flight before anything waits on one
#pragma unroll
    for (int v = 0; v < SLOTS; ++v) {
        const int u = NFG * v + fgrp;
        if (u < BATCH && u < ns) fetch(u, pa[v], pb[v]);
    }

    constexpr int FE = ST * ST / LEAF_THREADS;  // factor-block entries per thread
    T fnb[FE], fna[FE];                         // kept for the sweep's tables
#pragma unroll
    for (int u = 0; u < FE; ++u) {
        const int e = t + u * LEAF_THREADS, r = e >> 5, c = e & 31;
        const T nb = NB ? NB[int64_t(I * ST + r) * mp + I * ST + c] : T(0);
        fnb[u] = r == c ? T(0) : nb;
        sNB[r * PB + c] = fnb[u];
        const T na = NA[int64_t(J * ST + r) * np + J * ST + c];
        fna[u] = r == c ? T(0) : na;
        sNAt[c * PA + r] = fna[u];
    }
    if (t < ST) {
        sNB[ST * PB + t] = T(0);
        sNAt[t * PA + ST] = T(0);
    }

    // Two layouts of the tile over the threads, both with column b = t % 32:
    //   block layout  threads t < 256, rows r0 + i (four each): vector LDS reads,
    //                 coalesced global access, the chunk products;
    //   sweep layout  threads t < SWEEP_THREADS, rows ar[i] = (E g - b + i) mod 32
    //                 with g = t / 32 and E = LEAF_E entries each: entry i of every
    //                 thread lies on an element diagonal congruent to i mod E, and
    //                 all entries of diagonal d sit in slot d % E of group
    //                 (d mod 32) / E.
    constexpr int E = LEAF_E;
    const int g = t >> 5;  // sweep layout: column b, rows (E g - b + i) mod 32
    int ar[E], dg[E];
    T x[E], rp[E], sc[E], rs[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        ar[i] = (E * g - b + i) & (ST - 1);
        dg[i] = b + ar[i];
        sc[i] = S[I * ST + ar[i]];
        rs[i] = sc[i] == T(0) ? T(0) : T(1) / sc[i];
        rp[i] = T(0);
    }
    T acc[4], crow[4], ccol[4], sblk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i] = blk ? X[int64_t(I * ST + r0 + i) * np + J * ST + b] : T(0);
        sblk[i] = blk ? S[I * ST + r0 + i] : T(0);
        crow[i] = T(0);
        ccol[i] = T(0);
    }
    __syncthreads();

    // ---- chunk prologue: rowpart (crow) and the column feedback (ccol), block layout
    if (ns > 0) {
        // Wave wv owns the 16 x 16 quadrant qd = wv % 4 of one part: the row part
        // (rowpart) for wv < 4 and the column part for wv >= 4, accumulated over all
        // of that part's slices, so no partial sums cross waves.  With B = I there
        // is no column part: the two halves take the row slices of even and odd
        // index and their quadrants are added once at the end.
        const int part = wv >> 2, qd = wv & 3, qr = 16 * (qd >> 1), qc = 16 * (qd & 1);
        const bool split = NB == nullptr;
        Q16<T> pq;
        pq.zero();
        for (int sb = 0; sb < ns; sb += BATCH) {
            if (sb > 0) {
                __syncthreads();  // the previous batch is consumed
#pragma unroll
                for (int v = 0; v < SLOTS; ++v) {
                    const int u = NFG * v + fgrp;
                    if (u < BATCH && sb + u < ns) fetch(sb + u, pa[v], pb[v]);
                }
            }
#pragma unroll
            for (int v = 0; v < SLOTS; ++v) {
                const int u = NFG * v + fgrp;
                if (u < BATCH && sb + u < ns) {
                    if (sb + u < n1) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) stg[u][0][(c4 + j) * PK + q8] = pa[v][j];
                    } else {
                        pa[v].store(stg[u][0] + q8 * PK + c4);
                    }
                    pb[v].store(stg[u][1] + q8 * PK + c4);
                }
            }
            __syncthreads();
            // this wave's slices of the batch: its part's, or every other one
            const int nbat = ns - sb < BATCH ? ns - sb : BATCH;
            int u0, u1, du;
            if (split) {
                u0 = (sb + part) & 1 ? 1 : 0;
                u1 = nbat;
                du = 2;
            } else if (part == 0) {
                u0 = 0;
                u1 = n1 - sb < nbat ? (n1 - sb > 0 ? n1 - sb : 0) : nbat;
                du = 1;
            } else {
                u0 = n1 - sb > 0 ? n1 - sb : 0;
                u1 = nbat;
                du = 1;
            }
            for (int u = u0; u < u1; u += du)
                pq.template mma<PK, PK, ST>(stg[u][0] + qr, stg[u][1] + qc, lane);
        }
        // the quadrants reach the block layout through the staging area:
        // park[0] = rowpart (also the right operand of the in-tile column
        // feedback), park[1] = the column part
        const bool nbs = NB && n1 > 0;  // the in-tile column feedback strict(N_B[I, I])^T rowpart
        T* park = reinterpret_cast<T*>(stg);
        static_assert(sizeof(stg) >= 2 * ST * ST * sizeof(T), "staging area too small");
        auto park_quadrant = [&]() {
            T* q = park + part * ST * ST + qr * ST + qc;
#pragma unroll
            for (int r = 0; r < 4; ++r) q[Q16<T>::row(r, lane) * ST + Q16<T>::col(r, lane)] = pq.get(r);
        };
        __syncthreads();  // staged operands consumed
        if (part == 0 || !nbs) park_quadrant();
        if (nbs) {
            __syncthreads();  // rowpart complete
            if (part == 1) {
                // strict(N_B[I, I])^T (r, k) = N_B[k][r], k-major in sNB already
                pq.template mma<PB, ST, ST>(sNB + qr, park + qc, lane);
                park_quadrant();
            }
        }
        __syncthreads();
        if (blk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const T p0 = park[(r0 + i) * ST + b], p1 = park[ST * ST + (r0 + i) * ST + b];
                crow[i] = split ? p0 + p1 : p0;
                ccol[i] = split ? T(0) : p1;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += crow[i] + ccol[i];
    }

    // ---- to the sweep layout through LDS, and the sweep's factor tables
    // The staging area is free from here on.  Beside bufA / bufB it holds the
    // factor coefficients in the form the sweep reads them: the coefficient of
    // diagonal d's source for the entry (a, b) sits at a fixed offset from a
    // per-entry base,
    //   cB[(d - b + ST) PB + a] = N_B[d - b][a]   (column source (d - b, b))
    //   cA[b PT + d - a + ST]   = N_A[d - a][b]   (row source (a, d - a)),
    // zero wherever the source lies off the tile (and, as in sNB / sNAt, on and
    // below the diagonal), so the unrolled sweep spends no arithmetic on addresses.
    constexpr int NRB = 3 * ST + 4;  // rows of cB; d - b + ST stays in [1, NRB) for d <= 2 ST + 3
    constexpr int PT = 3 * ST + 4;   // row pitch of cA (even: lanes step PT + 1 apart)
    T* const cB = stg[0][0] + 2 * ST * PK;
    T* const cA = cB + NRB * PB;
    // the sweep's exchange, one slice per round: errors by row, row-accumulated
    // errors by column
    T* const xD = cA + ST * PT;            // [round][row][diagonal of the round]
    T* const xR = xD + NROUND * ST * RD;  // [round][column][diagonal of the round]
    static_assert(2 * ST * PK + NRB * PB + ST * PT + 2 * NROUND * ST * RD <= sizeof(stg) / sizeof(T),
                  "staging area too small");
    static_assert((2 * ST * PK + NRB * PB + ST * PT) % 8 == 0, "32-byte aligned exchange slices");
    __syncthreads();  // the prologue's reads of the staging area are done
    if (blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) bufA[(r0 + i) * PK + b] = acc[i];
    }
    {
        // zero lines, four entries per store: cB rows [0, ST) and [2 ST, NRB), cA
        // columns [0, ST) and [2 ST, PT) of every row; then the factor entries
        constexpr int ZB0 = ST * PB / 4, ZB1 = (NRB - 2 * ST) * PB / 4;
        constexpr int ZAR = ST / 4 + (PT - 2 * ST) / 4;  // per cA row
        static_assert(PB % 4 == 0 && PT % 4 == 0 && (2 * ST * PK) % 4 == 0, "16-byte table lines");
        Vec4<T> z4;
#pragma unroll
        for (int j = 0; j < 4; ++j) z4.set(j, T(0));
        for (int u = t; u < ZB0 + ZB1 + ST * ZAR; u += LEAF_THREADS) {
            T* q;
            if (u < ZB0) {
                q = cB + 4 * u;
            } else if (u < ZB0 + ZB1) {
                q = cB + 2 * ST * PB + 4 * (u - ZB0);
            } else {
                const int v = u - ZB0 - ZB1, r = v / ZAR, k = v - r * ZAR;
                q = cA + r * PT + (k < ST / 4 ? 4 * k : 2 * ST + 4 * (k - ST / 4));
            }
            z4.store(q);
        }
#pragma unroll
        for (int u = 0; u < FE; ++u) {
            const int e = t + u * LEAF_THREADS, r = e >> 5, c = e & 31;
            cB[(r + ST) * PB + c] = fnb[u];  // N_B[r][c]
            cA[c * PT + ST + r] = fna[u];    // N_A[r][c]
        }
    }
    __syncthreads();
    if (t >= SWEEP_THREADS) return;  // the later barriers wait for the sweep's waves only
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = bufA[ar[i] * PK + b];

    // ---- the sweep: 2 ST - 1 element anti-diagonals, four per round.
    // Slot i of group g holds diagonal 2 g + i (and 2 g + i + 32, entries past the
    // tile's main anti-diagonal), so the four diagonals d0 .. d0 + 3 of round
    // d0 / 4 sit in the two groups of one wave, the round's producer: its lower
    // half-wave (group 2 w) holds d0 in slot 0 and d0 + 1 in slot 1, its upper half
    // (group 2 w + 1) d0 + 2 and d0 + 3.  For the entry (a, b) on diagonal D and an
    // earlier diagonal d of the round, the column source (d - b, b) is slot d mod 2
    // of lane b of the group holding d, and the row source (a, d - a) is the same
    // slot of lane b - (D - d).  So the producer rounds d0, gives d0's feedback to
    // its d0 + 1 entries (a lane shift brings the row source) and rounds d0 + 1;
    // permlane32_swap then hands the lower half's errors to the upper half at the
    // same lane, lane shifts line up the row sources, and the upper half takes the
    // feedback of d0 and d0 + 1, rounds d0 + 2, passes its feedback on within the
    // half and rounds d0 + 3.  One barrier publishes the round; every wave then adds
    // the feedback of d0, d0 + 1, d0 + 2, d0 + 3 to its entries in turn: the same
    // operations in the same order as one diagonal at a time.  The next round's
    // producer does so right before its own chain, in one stretch of code.
    // Sources that do not exist have zero coefficients and every value exchanged
    // is finite, so a group writes all of its slots, and diagonal 2 ST - 1 (the
    // last round's fourth, outside the tile) contributes nothing.  A rounded
    // entry's error and code go straight to bufB (k-major, for the epilogue) and
    // bufA; each entry of bufA is read (as x) and later written by the same thread.
    static_assert(E == 2 && RD == 4, "the sweep holds two entries per thread, four diagonals per round");
    using VR = VecN<T, RD>;
    const T tqmin = T(qmin), tqmax = T(qmax);
    const T* pB[E];  // + d PB: N_B coefficient of diagonal d for slot k
    const T* pA[E];  // + d: N_A coefficient of diagonal d for slot k
#pragma unroll
    for (int k = 0; k < E; ++k) {
        pB[k] = cB + (ST - b) * PB + ar[k];
        pA[k] = cA + b * PT + ST - ar[k];
    }
    const bool upper = (g & 1) != 0;  // the half-wave holding the round's last two diagonals
    // coefficients of the round's diagonals d0 + m for slot k
    auto coef = [&](int d0, T (&nb)[RD][E], T (&na)[RD][E]) {
#pragma unroll
        for (int m = 0; m < RD; ++m)
#pragma unroll
            for (int k = 0; k < E; ++k) {
                nb[m][k] = pB[k][(d0 + m) * PB];
                na[m][k] = pA[k][d0 + m];
            }
    };
    // the producer's chain for round r (diagonals d0 = 4 r ..), then its publication
    auto chain = [&](int r, const T (&nb)[RD][E], const T (&na)[RD][E]) {
        const int d0 = RD * r;
        // lower half: d0 in slot 0, d0 + 1 in slot 1 (the upper half computes the
        // same operations on its own entries; nothing of that is kept)
        T z0, z1, v;
        quantize_fast(x[0], sc[0], rs[0], tqmin, tqmax, z0, v);
        const T e0 = v - x[0];
        const T q0 = rp[0] + e0;
        const T el = lane_below(e0);  // row source of slot 1 on d0
        const T x1 = kfma(el, na[0][1], kfma(nb[0][1], q0, x[1]));
        quantize_fast(x1, sc[1], rs[1], tqmin, tqmax, z1, v);
        const T e1 = v - x1;
        const T q1 = kfma(el, na[0][1], rp[1]) + e1;
        // the lower half's errors at the same lane of the upper half
        const T se0 = lanes_up32(e0), se1 = lanes_up32(e1), sq0 = lanes_up32(q0), sq1 = lanes_up32(q1);
        const T e0s1 = lane_below(se0), e0s2 = lane_below(e0s1), e0s3 = lane_below(e0s2);
        const T e1s1 = lane_below(se1), e1s2 = lane_below(e1s1);
        // upper half: d0 + 2 in slot 0, after the feedback of d0 and d0 + 1
        T z2, z3;
        T x2 = kfma(e0s2, na[0][0], kfma(nb[0][0], sq0, x[0]));
        x2 = kfma(e1s1, na[1][0], kfma(nb[1][0], sq1, x2));
        T r2 = kfma(e0s2, na[0][0], rp[0]);
        r2 = kfma(e1s1, na[1][0], r2);
        quantize_fast(x2, sc[0], rs[0], tqmin, tqmax, z2, v);
        const T e2 = v - x2;
        const T q2 = r2 + e2;
        // d0 + 3 in slot 1, after the feedback of d0, d0 + 1 and d0 + 2
        T x3 = kfma(e0s3, na[0][1], kfma(nb[0][1], sq0, x[1]));
        x3 = kfma(e1s2, na[1][1], kfma(nb[1][1], sq1, x3));
        T r3 = kfma(e0s3, na[0][1], rp[1]);
        r3 = kfma(e1s2, na[1][1], r3);
        const T e2l = lane_below(e2);  // row source of slot 1 on d0 + 2
        x3 = kfma(e2l, na[2][1], kfma(nb[2][1], q2, x3));
        r3 = kfma(e2l, na[2][1], r3);
        quantize_fast(x3, sc[1], rs[1], tqmin, tqmax, z3, v);
        const T e3 = v - x3;
        const T q3 = r3 + e3;
        if (g == ((d0 & (ST - 1)) >> 1) || g == ((d0 & (ST - 1)) >> 1) + 1) {
            // each half publishes its two diagonals: errors by row, row-accumulated errors by column
            const int m0 = upper ? 2 : 0;
            const T ea = upper ? e2 : e0, eb = upper ? e3 : e1;
            xD[(r * ST + ar[0]) * RD + m0] = ea;
            xD[(r * ST + ar[1]) * RD + m0 + 1] = eb;
            xR[(r * ST + b) * RD + m0] = upper ? q2 : q0;
            xR[(r * ST + b) * RD + m0 + 1] = upper ? q3 : q1;
            if (dg[0] == d0 + m0) {
                bufB[b * PK + ar[0]] = ea;
                bufA[ar[0] * PK + b] = upper ? z2 : z0;
            }
            if (dg[1] == d0 + m0 + 1) {
                bufB[b * PK + ar[1]] = eb;
                bufA[ar[1] * PK + b] = upper ? z3 : z1;
            }
        }
    };
    // every entry takes round r's feedback
    auto feedback = [&](const VR& rv, const VR (&dd)[E], const T (&nb)[RD][E], const T (&na)[RD][E]) {
#pragma unroll
        for (int j = 0; j < E; ++j)
#pragma unroll
            for (int m = 0; m < RD; ++m) {
                x[j] = kfma(dd[j][m], na[m][j], kfma(nb[m][j], rv[m], x[j]));
                rp[j] = kfma(dd[j][m], na[m][j], rp[j]);
            }
    };
    auto producer = [&](int r) { return (RD * r & (ST - 1)) / RD; };  // wave of groups 2 w, 2 w + 1
    // coefficients of round r (cnb / cna, its feedback) and of round r + 1 (read
    // after round r's barrier, for the next producer's chain)
    const int wvu = __builtin_amdgcn_readfirstlane(wv);  // wave-uniform: scalar branches on the producer
    T cnb[RD][E], cna[RD][E];
    coef(0, cnb, cna);
    if (wvu == producer(0)) chain(0, cnb, cna);
#pragma unroll
    for (int r = 0; r < NROUND; ++r) {
        __syncthreads();  // round r's errors are published
        if (r + 1 == NROUND) break;  // every entry is rounded
        VR rv, dd[E];
        rv.load(xR + (r * ST + b) * RD);
#pragma unroll
        for (int j = 0; j < E; ++j) dd[j].load(xD + (r * ST + ar[j]) * RD);
        T nnb[RD][E], nna[RD][E];
        coef(RD * (r + 1), nnb, nna);
        if (wvu == producer(r + 1)) {
            feedback(rv, dd, cnb, cna);
            chain(r + 1, nnb, nna);
        } else {
            feedback(rv, dd, cnb, cna);
        }
#pragma unroll
        for (int m = 0; m < RD; ++m)
#pragma unroll
            for (int k = 0; k < E; ++k) {
                cnb[m][k] = nnb[m][k];
                cna[m][k] = nna[m][k];
            }
    }
    // the last round's barrier made the errors and codes in bufB / bufA complete
    if (!blk) return;  // no barriers follow
    T dblk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t gi = int64_t(I) * ST + r0 + i, gj = int64_t(J) * ST + b;
        dblk[i] = bufB[b * PK + r0 + i];
        const T z = bufA[(r0 + i) * PK + b];
        D[gi * np + gj] = dblk[i];
        if (gi < m && gj < n) {
            Z[gi * ldz + gj] = int8_t(z);
            V[gi * ldv + gj] = sblk[i] * z;
        }
    }
    // ---- chunk epilogue: T1c[I, J] = rowpart + Delta + Delta strict(N_A[J, J])
    if (NB && K + 1 < c1) {
        T o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = crow[i] + dblk[i];
#pragma unroll 8
        for (int k = 0; k < ST; ++k) {
            Vec4<T> d4;
            d4.load(bufB + k * PK + r0);
            const T nak = sNAt[b * PA + k];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = kfma(d4[i], nak, o[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) T1c[int64_t(I * ST + r0 + i) * np + J * ST + b] = o[i];
    }
}

// Stage 1 at node [K0, K1) with split mid, on 64-row block P and 64-column block Q.
// Band GEMMs run split-K inside the workgroup: their launches have few blocks
// with long K ranges in the lower recursion levels, so each block gets G = 2
// groups of four waves (deterministic reduction, see tile_gemm_masked_splitk).
// Four groups shorten a lone solve's small launches a little, but two leave
// more of the device to the other work in flight beside them.
template <typename T>
struct Band {
    static constexpr int G = 2;  // stage 1: groups per block
    static constexpr int THREADS = 256 * G;
    // Stage 2 has half the blocks of stage 1 at the top node with twice the K
    // each; there four-wave blocks at full occupancy balance better than split K.
    static constexpr int THREADS2 = GEMM_THREADS;
};

template <typename T>
__global__ __launch_bounds__(Band<T>::THREADS) void band_stage1_kernel(const T* __restrict__ D,
                                                                       const T* __restrict__ NA,
                                                                       T* __restrict__ T1, int np, int Nt, int K0,
                                                                       int mid, int K1, int P0) {
    __shared__ SplitSmem<T, Band<T>::G> sm;
    const int P = P0 + blockIdx.y;
    const int I0 = 2 * P;  // first 32-row tile of the block
    const int jlo = K0 - I0 - 1 > 0 ? K0 - I0 - 1 : 0;
    const int jend = K1 - I0 < Nt ? K1 - I0 : Nt;  // exclusive, over both rows
    // the row's last block first: its K range is the longest at the top node
    const int Q = ((jend - 1) >> 1) - int(blockIdx.x);
    if (jend <= 0 || Q < (jlo >> 1)) return;
    const int kl = jlo;
    int kh = 2 * Q + 1;
    if (mid - 1 - I0 < kh) kh = mid - 1 - I0;
    if (Nt - 1 < kh) kh = Nt - 1;
    WaveAcc<T> acc;
    acc.zero();
    if (kh >= kl) {
        const T* A = D + int64_t(I0) * ST * np + int64_t(kl) * ST;
        const T* B = NA + int64_t(kl) * ST * np + int64_t(Q) * TILE;
        auto ma = [=](int r, int k) {
            const int s = I0 + (r >> 5) + kl + (k >> 5);  // tile-diagonal of the source tile
            return s >= K0 && s < mid;
        };
        tile_gemm_masked_splitk<T, Band<T>::G, false, false>(A, np, B, np, (kh - kl + 1) * ST, sm, acc, ma,
                                                             NoMask());
    }
    if (threadIdx.x >= 256) return;  // group 0 holds the product
    T* out = T1 + int64_t(I0) * ST * np + int64_t(Q) * TILE;
    for_each_acc(acc, [&](int r, int c, T v) { out[int64_t(r) * np + c] = v; });
}

// Stage 2: X[I, J] += sum_{I'} N_B[I', I]^T T1[I', J] for the tiles of diagonals
// [mid, K1), on 64 x 64 target block (P, Q) of block-diagonal sig = P + Q.
// KS: K-slice depth of the product (16 at the top node, where many blocks share
// each CU; 32 below, where a block's loads are its only latency hiding).
// Block order: a 1-D grid walks the target blocks by block row P from the last
// to the first (sig ascending within a row).  The K range of block (P, Q) grows
// with P (at the top node it is 2 P + 2 tiles), so the long blocks are
// dispatched first and the short ones fill in behind them, and no workgroup is
// spent on an empty position.
template <typename T, int KS>
__global__ __launch_bounds__(Band<T>::THREADS2) void band_stage2_kernel(const T* __restrict__ T1,
                                                                        const T* __restrict__ NB,
                                                                        T* __restrict__ X, int np, int mp, int Mt,
                                                                        int Nt, int K0, int mid, int K1, int sig0,
                                                                        int sig1) {
    __shared__ GemmSmemK<T, KS> sm;
    const int Mb = Mt >> 1, Nb = Nt >> 1;
    int sig = 0, P = -1;
    for (int b = blockIdx.x, p = Mb - 1; p >= 0; --p) {
        const int lo = sig0 > p ? sig0 : p, hi = sig1 < p + Nb - 1 ? sig1 : p + Nb - 1;
        const int cnt = hi >= lo ? hi - lo + 1 : 0;
        if (b < cnt) {
            P = p;
            sig = lo + b;
            break;
        }
        b -= cnt;
    }
    if (P < 0) return;
    const int Q = sig - P;
    const int I0 = 2 * P, J0 = 2 * Q;
    auto in_band = [=](int r, int c) {
        const int k = I0 + (r >> 5) + J0 + (c >> 5);
        return k >= mid && k < K1;
    };
    auto t1_valid = [=](int ip, int j) {  // T1 tile written by this node's stage 1
        const int k = ip + j;
        return ip < mid && k >= K0 && k < K1;
    };
    T* out = X + int64_t(I0) * ST * np + int64_t(J0) * ST;
    if (!NB) {
        const T* src = T1 + int64_t(I0) * ST * np + int64_t(J0) * ST;
        for (int e = threadIdx.x; e < TILE * TILE; e += Band<T>::THREADS2) {
            const int r = e >> 6, c = e & 63;
            if (in_band(r, c) && t1_valid(I0 + (r >> 5), J0 + (c >> 5)))
                out[int64_t(r) * np + c] += src[int64_t(r) * np + c];
        }
        return;
    }
    const int kl = K0 - J0 - 1 > 0 ? K0 - J0 - 1 : 0;
    const int kh = I0 + 1 < mid - 1 ? I0 + 1 : mid - 1;
    if (kl > kh) return;
    WaveAcc<T> acc;
    acc.zero();
    const T* A = NB + int64_t(kl) * ST * mp + int64_t(I0) * ST;  // A(r, k) = NB[k][r]
    const T* B = T1 + int64_t(kl) * ST * np + int64_t(J0) * ST;
    auto mb = [=](int k, int c) { return t1_valid(kl + (k >> 5), J0 + (c >> 5)); };
    if (KS == KSTEP)  // the top node: many blocks per CU hide the loads
        tile_gemm_masked_k<T, KS, true, false>(A, mp, B, np, (kh - kl + 1) * ST, sm, acc, NoMask(), mb);
    else
        tile_gemm_masked_k2<T, KS, true, false>(A, mp, B, np, (kh - kl + 1) * ST, sm, acc, NoMask(), mb);
    for_each_acc(acc, [&](int r, int c, T v) {
        if (in_band(r, c)) out[int64_t(r) * np + c] += v;
    });
}

// Proxy loss of the result from the solver's errors.  The feedback gives
// V - W = L~_B Delta L~_A^T exactly in exact arithmetic (FastKron page, section
// 2.2), and A_d^{-1} = U_A^T U_A with U_A = diag(U_A) N_A makes
// A_d = L~_A^{-T} diag(U_A)^{-2} L~_A^{-1} (likewise B_d), so
//   tr(B_d (V - W) A_d (V - W)^T) = sum_ij (Delta_ij / (U_B,ii U_A,jj))^2.
// Rows go round-robin over ELOSS_PARTS workgroups; every sum runs in a fixed
// order, so the result is deterministic.
constexpr int ELOSS_PARTS = 2048;

template <typename T>
__global__ void diag_recip_kernel(const T* __restrict__ U, int64_t ldu, int d, double* __restrict__ out) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < d) out[j] = 1.0 / double(U[int64_t(j) * ldu + j]);
}

template <typename T>
__global__ __launch_bounds__(256) void error_loss_partial_kernel(const T* __restrict__ D, int64_t np, int m, int n,
                                                                 const double* __restrict__ ra,
                                                                 const double* __restrict__ rb,
                                                                 double* __restrict__ partial) {
    __shared__ double red[256];
    // four independent sums, so four loads per thread are in flight at once
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    for (int i = blockIdx.x; i < m; i += gridDim.x) {
        const double ri = rb ? rb[i] : 1.0;
        const T* row = D + int64_t(i) * np;
        for (int j0 = threadIdx.x; j0 < n; j0 += 4 * 256) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + 256 * u;
                if (j < n) {
                    const double q = double(row[j]) * ra[j] * ri;
                    s[u] = __builtin_fma(q, q, s[u]);
                }
            }
        }
    }
    const double tot = block_sum_256((s[0] + s[1]) + (s[2] + s[3]), red);
    if (threadIdx.x == 0) partial[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void error_loss_final_kernel(const double* __restrict__ partial, int count,
                                                               double* __restrict__ out) {
    __shared__ double red[256];
    double s = 0.0;
    for (int i = threadIdx.x; i < count; i += blockDim.x) s += partial[i];
    const double tot = block_sum_256(s, red);
    if (threadIdx.x == 0) *out = tot;
}

// ------------------------------------------------------------------- host side

struct SolverLayout {
    int64_t mp, np, Mt, Nt;  // padded extents; tile counts in 32-tiles
    size_t bytes;
    size_t off_NA, off_NB, off_X, off_D, off_T1, off_S, off_L;
};

SolverLayout solver_layout(kq_dtype dtype, int64_t m, int64_t n) {
    SolverLayout L;
    const size_t es = dtype == KQ_F64 ? 8 : 4;
    L.mp = round_up(m, TILE);
    L.np = round_up(n, TILE);
    L.Mt = L.mp / ST;
    L.Nt = L.np / ST;
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
    L.off_L = off;  // loss scratch (fp64): 1 / U_A,jj, 1 / U_B,ii, partial sums
    off += align256((size_t(L.np) + size_t(L.mp) + ELOSS_PARTS) * sizeof(double));
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

    kq_status leaf(int K, int c0, int c1) {
        const int Mt = int(L.Mt), Nt = int(L.Nt);
        const int ilo = K - Nt + 1 > 0 ? K - Nt + 1 : 0;
        const int ihi = K < Mt - 1 ? K : Mt - 1;
        hipLaunchKernelGGL(leaf_kernel<T>, dim3(ihi - ilo + 1), dim3(LEAF_THREADS), 0, st, X, D, NA, NB, S, T1, int(L.np),
                           int(L.mp), Mt, Nt, K, c0, c1, m, n, qmin, qmax, Z, ldz, V, ldv);
        KQ_LAUNCHED("leaf_kernel");
        return KQ_OK;
    }

    kq_status propagate(int K0, int mid, int K1) {
        const int Mt = int(L.Mt), Nt = int(L.Nt);
        // stage 1 rows I' with a source tile in [K0, mid): K0 - Nt < I' < mid
        const int row0 = K0 - Nt + 1 > 0 ? K0 - Nt + 1 : 0;
        const int row1 = mid < Mt ? mid : Mt;  // exclusive
        if (row1 > row0) {
            const int P0 = row0 >> 1, P1 = (row1 - 1) >> 1;
            hipLaunchKernelGGL(band_stage1_kernel<T>, dim3((K1 - K0) / 2 + 2, P1 - P0 + 1), dim3(Band<T>::THREADS), 0,
                               st, D, NA, T1, int(L.np), Nt, K0, mid, K1, P0);
            KQ_LAUNCHED("band_stage1_kernel");
        }
        // stage 2 target block-diagonals sig with [2 sig, 2 sig + 2] meeting [mid, K1)
        const int sig0 = (mid - 1) >> 1 > 0 ? (mid - 1) >> 1 : 0;
        int sig1 = (K1 - 1) >> 1;
        const int sigmax = int(L.Mt / 2 + L.Nt / 2 - 2);
        if (sig1 > sigmax) sig1 = sigmax;
        if (sig1 >= sig0) {
            const bool top = K0 == 0 && K1 == int(L.Mt + L.Nt - 1);
            auto kern = top ? band_stage2_kernel<T, KSTEP> : band_stage2_kernel<T, 2 * KSTEP>;
            int total = 0;  // target blocks
            for (int p = 0; p < Mt / 2; ++p) {
                const int lo = sig0 > p ? sig0 : p, hi = sig1 < p + Nt / 2 - 1 ? sig1 : p + Nt / 2 - 1;
                total += hi >= lo ? hi - lo + 1 : 0;
            }
            hipLaunchKernelGGL(kern, dim3(total), dim3(Band<T>::THREADS2), 0, st, T1, NB, X, int(L.np), int(L.mp),
                               Mt, Nt, K0, mid, K1, sig0, sig1);
            KQ_LAUNCHED("band_stage2_kernel");
        }
        return KQ_OK;
    }

    kq_status solve(int K0, int K1) {
        if (K1 - K0 <= CHUNK) {
            for (int K = K0; K < K1; ++K) {
                const kq_status s = leaf(K, K0, K1);
                if (s != KQ_OK) return s;
            }
            return KQ_OK;
        }
        const int chunks = (K1 - K0 + CHUNK - 1) / CHUNK;
        const int mid = K0 + CHUNK * (chunks / 2);
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
                         double* loss_dev, void* ws, hipStream_t st) {
    const SolverLayout L = solver_layout(sizeof(T) == 8 ? KQ_F64 : KQ_F32, m, n);
    char* base = static_cast<char*>(ws);
    SolverRun<T> run{L, int(m), int(n), -(1 << (q->bits - 1)), (1 << (q->bits - 1)) - 1,
                     reinterpret_cast<T*>(base + L.off_NA), UB ? reinterpret_cast<T*>(base + L.off_NB) : nullptr,
                     reinterpret_cast<T*>(base + L.off_X), reinterpret_cast<T*>(base + L.off_D),
                     reinterpret_cast<T*>(base + L.off_T1), reinterpret_cast<T*>(base + L.off_S),
                     codes, ldc, V, ldv, st};
    const int threads = 256;
    auto blocks = [&](int64_t count) { return dim3(unsigned((count + threads - 1) / threads)); };
    auto rows = [&](int64_t cols, int64_t nrows) {  // the kernels loop over rows beyond the grid's y extent
        return dim3(unsigned((cols / 4 + threads - 1) / threads), unsigned(nrows < 65535 ? nrows : 65535));
    };
    hipLaunchKernelGGL(normalize_factor_kernel<T>, rows(L.np, L.np), dim3(threads), 0, st, UA, lda, int(n),
                       int(L.np), run.NA);
    KQ_LAUNCHED("normalize_factor_kernel");
    if (UB) {
        hipLaunchKernelGGL(normalize_factor_kernel<T>, rows(L.mp, L.mp), dim3(threads), 0, st, UB, ldb, int(m),
                           int(L.mp), run.NB);
        KQ_LAUNCHED("normalize_factor_kernel");
    }
    hipLaunchKernelGGL(init_solver_kernel<T>, rows(L.np, L.mp), dim3(threads), 0, st, W, ldw, int(m), int(n),
                       int(L.mp), int(L.np), static_cast<const T*>(q->scales), q->per_row, run.X, run.S);
    KQ_LAUNCHED("init_solver_kernel");
    const kq_status s = run.solve(0, int(L.Mt + L.Nt - 1));
    if (s != KQ_OK || !loss_dev) return s;
    double* ra = reinterpret_cast<double*>(base + L.off_L);
    double* rb = ra + L.np;
    double* part = rb + L.mp;
    hipLaunchKernelGGL(diag_recip_kernel<T>, blocks(n), dim3(threads), 0, st, UA, lda, int(n), ra);
    KQ_LAUNCHED("diag_recip_kernel");
    if (UB) {
        hipLaunchKernelGGL(diag_recip_kernel<T>, blocks(m), dim3(threads), 0, st, UB, ldb, int(m), rb);
        KQ_LAUNCHED("diag_recip_kernel");
    }
    hipLaunchKernelGGL(error_loss_partial_kernel<T>, dim3(ELOSS_PARTS), dim3(256), 0, st, run.D, L.np, int(m),
                       int(n), ra, UB ? rb : nullptr, part);
    KQ_LAUNCHED("error_loss_partial_kernel");
    hipLaunchKernelGGL(error_loss_final_kernel, dim3(1), dim3(256), 0, st, part, ELOSS_PARTS, loss_dev);
    KQ_LAUNCHED("error_loss_final_kernel");
    return KQ_OK;
}

size_t quantize_workspace_bytes(kq_dtype dtype, int64_t m, int64_t n) { return solver_layout(dtype, m, n).bytes; }

kq_status quantize_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* UA,
                            int64_t lda, const void* UB, int64_t ldb, const kq_quantizer* q, int8_t* codes,
                            int64_t ldc, void* V, int64_t ldv, double* loss_dev, void* ws, hipStream_t st) {
    if (dtype == KQ_F64)
        return quantize_typed<double>(m, n, static_cast<const double*>(W), ldw, static_cast<const double*>(UA), lda,
                                      static_cast<const double*>(UB), ldb, q, codes, ldc, static_cast<double*>(V),
                                      ldv, loss_dev, ws, st);
    return quantize_typed<float>(m, n, static_cast<const float*>(W), ldw, static_cast<const float*>(UA), lda,
                                 static_cast<const float*>(UB), ldb, q, codes, ldc, static_cast<float*>(V), ldv,
                                 loss_dev, ws, st);
}

}  // namespace kq
