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
// batched products; solve(mid, K1).  The feedback is separable: the error
// Delta[I', J'] reaches X[I, J] as N_B[I', I]^T Delta[I', J'] N_A[J', J].  The
// row-propagated errors sum_{J' <= J} Delta[I', J'] N_A[J', J] of tile (I', J) are
// accumulated in R by the nodes before the tile's chunk; the tile's leaf
// completes them and writes the complete tile to RF.  At node [K0, K1) with split
// mid, for the targets of diagonals [mid, K1):
//   stage 1  R[I', J] += sum_{J' : K0 <= I'+J' < mid} Delta[I', J'] N_A[J', J]
//   stage 2  X[I, J] += sum_{I' : K0 <= I'+J < mid} N_B[I', I]^T RF[I', J]
// (stage 2 reads only left-half tiles, whose RF is complete).  Each (source,
// target) pair passes through one stage-1 or leaf row product and one stage-2
// or leaf column product, so the band work is the method's own m n (m + n) up to
// tile granularity.  Both stages run on 64 x 64 matrix-core output blocks
// (2 x 2 scheduling tiles) and mask at 32-tile granularity: source tiles outside
// the band read as zero, targets outside the band are not written.
// The recursion stops at chunks of CHUNK tile-diagonals.  Each 32 x 32 tile of a
// chunk runs the element-level anti-diagonal sweep (63 steps) with the in-tile
// feedback, one workgroup per tile, after pulling the feedback of the chunk's
// earlier tiles.  One persistent launch runs a whole chunk (chunk_kernel): its
// workgroups draw tile tasks in tile-diagonal order and a tile starts as soon as
// the outputs it reads of the tiles before it in its row and column have
// arrived: it polls them (see kq_chunk_sched.hpp).
//
// Workspace layout (row-major, padded to multiples of 64 with zero weights,
// unit scales and identity factors, so padding never reaches a real entry):
//   NA  np x np   normalised input factor
//   NB  mp x mp   normalised output factor
// (B = I does not come here: kron_quantize runs the one-sided path for it.)
//   X   mp x np   running pre-rounding values (starts as W)
//   D   mp x np   errors Delta
//   R   mp x np   row-propagated errors accumulated for the tiles not yet swept (zero at the start)
//   RF  mp x np   each swept tile's complete row-propagated errors (its leaf writes them)
//   P   2 x min(Mt, Nt) x 2 x 32 x 32   the leaves' pre-accumulated chunk products
//   S   mp        per-row scales
//   C   np        per-column scales (the WaterKron mode only; unit in the padding)
//   F   int32 words of the persistent chunk solver (a ticket counter per chunk,
//       an abort word), zeroed per call; in that solver D and RF start as an
//       unreachable bit pattern (a signalling NaN) that marks a value as not yet
//       written
// In the WaterKron mode (kron_quantize_waterkron) entry (i, j) has the grid step
// S[i] * C[j] (one rounding) and int32 codes clamped only at +-2^30.
#include <cstdlib>
#include <type_traits>

#include "kq_common.hpp"
#include "kq_chunk_sched.hpp"

namespace kq {

constexpr int ST = 32;  // scheduling tile edge (CHUNK, the tile-diagonals of a chunk, is in kq_chunk_sched.hpp)

// Byte offsets of the solver's arrays in its workspace (see the layout above),
// from the 32-tile counts and the element size alone, so that a kernel finds
// every array from the workspace base (its launch then carries one pointer).
// The padded extents are multiples of 64, so every array size is a multiple of
// 256 bytes and the arrays are 256-byte aligned.
struct WsOffsets {
    int64_t NA, NB, X, D, R, RF, P, S, C, F, end;
};
// The bit pattern that marks a handed-over value (D, RF) as not yet written in
// the persistent solver: a signalling NaN, which no arithmetic result is (IEEE
// operations quiet a signalling NaN), so every value a leaf stores differs from it.
template <typename T>
__host__ __device__ constexpr auto unwritten_bits() {
    if constexpr (sizeof(T) == 4)
        return uint32_t(0xFFA5A5A5u);
    else
        return uint64_t(0xFFF4A5A5A5A5A5A5ull);
}

// the chunk solver's words: one ticket counter per chunk, one abort word (int32)
__host__ __device__ inline int64_t flag_words(int64_t Mt, int64_t Nt) {
    return (Mt + Nt - 1 + CHUNK - 1) / CHUNK + 1;
}
__host__ __device__ inline WsOffsets ws_offsets(int64_t Mt, int64_t Nt, int64_t es) {
    const int64_t mp = Mt * ST, np = Nt * ST;
    WsOffsets o;
    o.NA = 0;
    o.NB = o.NA + np * np * es;
    o.X = o.NB + mp * mp * es;
    o.D = o.X + mp * np * es;
    o.R = o.D + mp * np * es;
    o.RF = o.R + mp * np * es;
    o.P = o.RF + mp * np * es;  // two tile-diagonals of two 32 x 32 parts per tile
    o.S = o.P + 2 * 2 * ST * ST * (Mt < Nt ? Mt : Nt) * es;
    o.C = o.S + mp * es;
    o.F = o.C + np * es;
    o.end = o.F + (flag_words(Mt, Nt) * 4 + 255) / 256 * 256;
    return o;
}

// N[r][c] = U[r][c] / U[r][r] for c >= r inside d x d; identity in the padding.
// Rows blockIdx.y, + gridDim.y, ...; each thread four consecutive columns (dp is
// a multiple of 64, so they are in range and the store is 16-byte aligned).
template <typename T>
__global__ void normalize_factor_kernel(const T* __restrict__ U, int64_t ldu, int d, int dp,
                                        T* __restrict__ N);

template <typename T>
__global__ void init_solver_kernel(const T* __restrict__ W, int64_t ldw, int m, int n, int mp, int np,
                                   const T* __restrict__ scales, int per_row, const T* __restrict__ col_scales,
                                   T* __restrict__ X, T* __restrict__ S, T* __restrict__ C, T* __restrict__ R,
                                   T* __restrict__ D, T* __restrict__ RF);

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
// entries only ever receive +0).  Every exchange slot a round reads is written
// by that round's producer before the round's barrier, so nothing left in that
// LDS by the prologue reaches a product, and every multiplied value is finite.
//
// Chunks.  The recursion stops at chunks of consecutive tile-diagonals
// [c0, c1); inside a chunk the feedback between tiles is pulled by each leaf
// (left-looking, the per-entry form of section 2.4 at tile granularity).  For
// tile (I, J) on diagonal K of the chunk:
//   rowpart = R[I, J] + sum_{c0 - I <= J' < J} Delta[I, J'] N_A[J', J]
//   X[I, J] += N_B[I, I]^T rowpart + sum_{c0 - J <= I' < I} N_B[I', I]^T RF[I', J]
// (RF[I', J] of the chunk's earlier tiles is complete), and after the sweep the
// leaf writes RF[I, J] = rowpart + Delta[I, J] N_A[J, J].  Both come out of the
// sweep: N_B[I, I]^T rowpart is rowpart plus the in-tile column feedback of
// rowpart, and the sweep's row-accumulated errors start at rowpart, so its column
// feedback carries that part and every entry's final row-accumulated value is
// its entry of RF[I, J].  The sums over the
// slices before diagonal K - 1 are pre-accumulated by launch K - 1 (see the
// kernel), or in the persistent solver by the tile's own task while the
// freshest slices are still being swept, so the leaf itself multiplies only the
// two freshest slices after they arrive.  The
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

// X = W zero-padded to mp x np; S = the scales, unit in the padding; with column
// scales, C = them, unit in the padding; R (when given) = 0; D and RF (when
// given) = the unwritten pattern.  Rows as in normalize_factor_kernel,
// four consecutive columns per thread.
template <typename T>
__global__ void init_solver_kernel(const T* __restrict__ W, int64_t ldw, int m, int n, int mp, int np,
                                   const T* __restrict__ scales, int per_row, const T* __restrict__ col_scales,
                                   T* __restrict__ X, T* __restrict__ S, T* __restrict__ C, T* __restrict__ R,
                                   T* __restrict__ D, T* __restrict__ RF) {
    const int c0 = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (col_scales && blockIdx.y == 0 && c0 < np) {
#pragma unroll
        for (int u = 0; u < 4; ++u) C[c0 + u] = c0 + u < n ? col_scales[c0 + u] : T(1);
    }
    for (int r = blockIdx.y; r < mp; r += gridDim.y) {
        if (blockIdx.x == 0 && threadIdx.x == 0) S[r] = r < m ? scales[per_row ? r : 0] : T(1);
        if (c0 >= np) continue;
        Vec4<T> v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v.set(u, (r < m && c0 + u < n) ? W[int64_t(r) * ldw + c0 + u] : T(0));
        v.store(X + int64_t(r) * np + c0);
        if (R) {
#pragma unroll
            for (int u = 0; u < 4; ++u) v.set(u, T(0));
            v.store(R + int64_t(r) * np + c0);
        }
        if (D) {  // D and RF: not yet written (the persistent solver polls for them)
#pragma unroll
            for (int u = 0; u < 4; ++u) v.set(u, __builtin_bit_cast(T, unwritten_bits<T>()));
            v.store(D + int64_t(r) * np + c0);
            v.store(RF + int64_t(r) * np + c0);
        }
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
    __device__ void set(int r, float v) { c[r] = v; }
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
    __device__ void set(int r, double v) { c[r] = v; }
    static __device__ __forceinline__ int row(int r, int lane) { return (lane >> 4) + 4 * r; }
    static __device__ __forceinline__ int col(int, int lane) { return lane & 15; }
};

constexpr int LEAF_THREADS = 512;   // the chunk products and the table set-up
constexpr int SWEEP_THREADS = 512;  // the sweep: two entries per thread
constexpr int LEAF_E = ST * ST / SWEEP_THREADS;
static_assert(SWEEP_THREADS == LEAF_THREADS, "every thread of the leaf takes part in the sweep");

template <bool ENTRY>
using CodeT = std::conditional_t<ENTRY, int32_t, int8_t>;

// Device-coherent stores (agent-scope relaxed atomics) of the data that chunk
// tasks hand to one another: it goes through the device's coherence point, so
// no cache needs a write-back or an invalidation at a hand-over.
template <bool CO, typename T>
__device__ __forceinline__ void co_st(T* p, T v) {
    if constexpr (CO)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}
// Four consecutive elements at element offset off (this lane's) from a base
// that is the same for the whole wave: with CO one 16-byte (fp32) or two
// (fp64) device-coherent buffer loads (cache policy sc1), the form of an
// agent-scope atomic load, four elements wide.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int CPOL_SC1 = 16;  // buffer-load cache policy: device scope
template <bool CO, typename T>
__device__ __forceinline__ void co_ld4(Vec4<T>& v, const T* base, int off) {
    if constexpr (CO) {
        // raw buffer over the wave's base (0x20000: 32-bit data format, no
        // swizzle); offsets stay far below the 2 GiB record count
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, 0x7fffffff, 0x00020000);
        if constexpr (sizeof(T) == 4) {
            v.v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off * 4, 0, CPOL_SC1));
        } else {
            v.lo = __builtin_bit_cast(f64x2, __builtin_amdgcn_raw_buffer_load_b128(r, off * 8, 0, CPOL_SC1));
            v.hi = __builtin_bit_cast(f64x2, __builtin_amdgcn_raw_buffer_load_b128(r, off * 8 + 16, 0, CPOL_SC1));
        }
    } else {
        v.load(base + off);
    }
}

template <typename T>
__device__ __forceinline__ bool unwritten(const Vec4<T>& v) {
    using U = decltype(unwritten_bits<T>());
    bool any = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) any |= __builtin_bit_cast(U, v[j]) == unwritten_bits<T>();
    return any;
}

// Bound on a chunk task's wait for one value, in polls (each a device-coherent
// load and a short sleep, about a microsecond): far beyond any wait of a
// running chunk (a whole chunk takes a few hundred microseconds), so it only
// ends a wait that could never be satisfied; the task then raises the abort
// word, every later wait returns at once and the swept tiles store NaN in V.
constexpr uint32_t CHUNK_SPIN_LIMIT = 1u << 18;  // the default; the environment variable
                                                 // KQ_CHUNK_SPIN_LIMIT overrides it per call

// One leaf task on tile idx of tile-diagonal Kt of chunk [c0, c1): the sweep of
// the tile, or (pre) the pre-accumulation of its chunk products over every
// slice but its two freshest.  CHAINED: the task runs inside the persistent
// chunk solver, sums the older slices' products itself (no pre tasks there) and
// polls every handed-over value it reads until it is written (see
// kq_chunk_sched.hpp); otherwise the launch order provides the dependencies (a
// launch per tile-diagonal, the pre role on its own workgroups).
template <typename T, bool ENTRY, bool CHAINED>
__device__ __forceinline__ void leaf_task(bool pre, int Kt, int idx, int c0, int c1, int Mt, int Nt, int qmin,
                                          int qmax, char* __restrict__ ws, int m, int n,
                                          CodeT<ENTRY>* __restrict__ Z, int64_t ldz, T* __restrict__ V,
                                          int64_t ldv, uint32_t spin_limit = CHUNK_SPIN_LIMIT) {
    const WsOffsets wo = ws_offsets(Mt, Nt, sizeof(T));
    const int np = Nt * ST, mp = Mt * ST, pt = Mt < Nt ? Mt : Nt;
    T* const D = reinterpret_cast<T*>(ws + wo.D);
    T* const R = reinterpret_cast<T*>(ws + wo.R);
    T* const RF = reinterpret_cast<T*>(ws + wo.RF);
    T* const P = reinterpret_cast<T*>(ws + wo.P);
    const T* const NA = reinterpret_cast<const T*>(ws + wo.NA);
    const T* const NB = reinterpret_cast<const T*>(ws + wo.NB);
    const T* const X = reinterpret_cast<const T*>(ws + wo.X);
    const T* const S = reinterpret_cast<const T*>(ws + wo.S);
    const T* const CS = reinterpret_cast<const T*>(ws + wo.C);
    constexpr int PB = ST + 4;  // 16-byte aligned rows for the vector reads
    constexpr int PK = ST + 4;  // k-major staging rows, 16-byte aligned
    constexpr int RD = 2 * LEAF_E;                      // diagonals per sweep round (one wave's two groups)
    constexpr int NROUND = (2 * ST - 1 + RD - 1) / RD;  // sweep rounds
    // Chunk operands of up to BATCH slices: A(r, k) at [k][r], B(k, c) at [k][c]
    // (the precompute workgroups), or the leaf's layout below.
    constexpr int BATCH = 7;  // staged together (LDS budget)
    __shared__ __attribute__((aligned(16))) T stg[BATCH][2][ST * PK];
    // The leaf's LDS: the sweep's factor tables cB and cA (in the form the sweep
    // reads them, see below), the tile in the two layouts' exchange bufA / bufB,
    // and the sweep's exchange xD / xR (one slice per round: errors by row,
    // row-accumulated errors by column).  bufA .. xR are free until the sweep, so
    // the prologue stages its two slices there (slice 0 in bufA / bufB, slice 1
    // at xD); it parks its products at pk, past the sweep's arrays, so the
    // sweep can start as soon as they are read.
    constexpr int NRB = 3 * ST + 4;  // rows of cB; d - b + ST stays in [1, NRB) for d <= 2 ST + 3
    constexpr int PT = 3 * ST + 4;   // row pitch of cA (even: lanes step PT + 1 apart)
    T* const cB = &stg[0][0][0];
    T* const cA = cB + NRB * PB;
    T* const bufA = cA + ST * PT;
    T* const bufB = bufA + ST * PK;
    T* const xD = bufB + ST * PK;          // [round][row][diagonal of the round]
    T* const xR = xD + NROUND * ST * RD;  // [round][column][diagonal of the round]
    T* const pk = xR + NROUND * ST * RD;  // the prologue's products: rowpart, then the column part
    T* const junk = pk + 2 * ST * ST;     // one slot per lane for the sweep's discarded stores
    static_assert(NRB * PB + ST * PT + 2 * ST * PK + 2 * NROUND * ST * RD + 2 * ST * ST + 64 <=
                      sizeof(stg) / sizeof(T),
                  "staging area too small");
    static_assert((NRB * PB + ST * PT) % 4 == 0 && (NRB * PB + ST * PT + 2 * ST * PK) % 8 == 0,
                  "16-byte aligned bufA / bufB, 32-byte aligned exchange slices");
    static_assert(2 * ST * PK + 2 * ST * ST <= 2 * ST * PK + 2 * NROUND * ST * RD, "prologue staging fits");

    // P holds the pre-accumulated products of two tile-diagonals (slot
    // (Kt & 1) pt + idx); the chunk solver keeps them in registers instead.
    const int I = (Kt - Nt + 1 > 0 ? Kt - Nt + 1 : 0) + idx;
    if (I > (Kt < Mt - 1 ? Kt : Mt - 1)) return;
    const int J = Kt - I;
    // threads t < 256 also work in the block layout (four rows each); all
    // LEAF_THREADS threads take part in the sweep
    int t = threadIdx.x;
    // Opaque to the optimiser in the chunk solver's task loop: the thread's
    // addresses are then recomputed per task rather than kept live across it.
    if constexpr (CHAINED) asm volatile("" : "+v"(t));
    const int tb = t & 255, w = tb >> 6, l = tb & 63;
    const bool blk = t < 256;
    const int b = l & 31, r0 = 8 * w + 4 * (l >> 5);
    const int fgrp = t >> 8;                    // staging loads: slices rotate over the 256-thread groups
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;  // wave (uniform: scalar branches), lane
    const int q8 = tb >> 3, c4 = 4 * (tb & 7);  // this thread's share of a 32 x 32 staging load
    // chunk products: wave wv owns the 16 x 16 quadrant qd = wv % 4 of one part, the
    // row part (rowpart) for wv < 4 and the column part for wv >= 4, accumulated
    // over all of that part's slices, so no partial sums cross waves
    const int part = wv >> 2, qd = wv & 3, qr = 16 * (qd >> 1), qc = 16 * (qd & 1);
    T* const Pt = P + (int64_t((Kt & 1) * pt + idx) * 2 + part) * ST * ST + qr * ST + qc;
    // the chunk solver's abort word (CHAINED); s_aborted: a wait of this task gave up
    int* const abort_word = reinterpret_cast<int*>(ws + wo.F) + (Mt + Nt - 1 + CHUNK - 1) / CHUNK;
    __shared__ int s_aborted;
    if constexpr (CHAINED) {
        if (t == 0) s_aborted = 0;
        __syncthreads();
    }

    // chunk sources of the tile: row tiles J' in [jl, J), column tiles I' in [il, I);
    // the freshest of each (J - 1, I - 1) lies on diagonal Kt - 1
    const int jl = c0 - I > 0 ? c0 - I : 0;
    const int il = c0 - J > 0 ? c0 - J : 0;
    const int n1all = J - jl;
    const int n2all = I - il;
    // the slices multiplied next: row slices [jb, jb + n1), column slices
    // [ib, ib + n2): the older ones (pre, and first in the chunk solver), then
    // the freshest (the leaf), staged in stg (older) or the leaf's buffers
    bool older = pre || CHAINED;
    int jb, ib, n1, n2, ns;
    auto select_slices = [&]() {
        jb = older ? jl : J - 1;
        ib = older ? il : I - 1;
        n1 = older ? (n1all > 1 ? n1all - 1 : 0) : (n1all > 0 ? 1 : 0);
        n2 = older ? (n2all > 1 ? n2all - 1 : 0) : (n2all > 0 ? 1 : 0);
        ns = n1 + n2;
    };
    select_slices();
    constexpr int NFG = LEAF_THREADS / 256;
    constexpr int SLOTS = (BATCH + NFG - 1) / NFG;  // slices of a batch held by one thread
    Vec4<T> pa[SLOTS], pb[SLOTS];
    auto fetch = [&](int sl, Vec4<T>& va, Vec4<T>& vb) {
        if (sl < n1) {
            const int jp = jb + sl;
            co_ld4<CHAINED>(va, D + int64_t(I * ST) * np + jp * ST, q8 * np + c4);  // A(r = q8, k = c4 + j)
            vb.load(NA + int64_t(jp * ST + q8) * np + J * ST + c4);  // B(k = q8, c = c4 + j)
        } else {
            const int ip = ib + sl - n1;
            va.load(NB + int64_t(ip * ST + q8) * mp + I * ST + c4);  // A(r = c4 + j, k = q8)
            co_ld4<CHAINED>(vb, RF + int64_t(ip * ST) * np + J * ST, q8 * np + c4);  // B(k = q8, c = c4 + j)
        }
    };
    // chained: the handed-over operand of slice sl (the errors D of a row slice,
    // RF of a column slice) is polled until every value is written (device-
    // coherent loads; the writer stores each value once per call)
    auto settle = [&](int sl, Vec4<T>& va, Vec4<T>& vb) {
        if constexpr (CHAINED) {
            const bool row = sl < n1;
            Vec4<T>& v = row ? va : vb;
            const T* const bp = row ? D + int64_t(I * ST) * np + (jb + sl) * ST
                                    : RF + int64_t((ib + sl - n1) * ST) * np + J * ST;
            for (uint32_t it = 0; unwritten(v); ++it) {
                if (it >= spin_limit) {
                    __hip_atomic_store(abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    atomicOr(&s_aborted, 1);
                    break;
                }
                if ((it & 63) == 63 && __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                    atomicOr(&s_aborted, 1);
                    break;
                }
                __builtin_amdgcn_s_sleep(4);  // about 0.1 us between polls: less load traffic, same hand-over time
                co_ld4<CHAINED>(v, bp, q8 * np + c4);
            }
        }
    };
    // every load of the first batch is in flight before anything waits on one
    // (chained: once the slices are final, after the tile's own loads)
    auto first_batch = [&]() {
#pragma unroll
        for (int v = 0; v < SLOTS; ++v) {
            const int u = NFG * v + fgrp;
            if (u < BATCH && u < ns) fetch(u, pa[v], pb[v]);
        }
    };
    first_batch();
    // operand op (0: A, 1: B) of staged slice u
    auto slot = [&](int u, int op) -> T* {
        return older ? stg[u][op] : (u == 0 ? bufA : xD) + op * ST * PK;
    };
    // pq += this wave's part over the workgroup's slices, staged in batches
    auto products = [&](Q16<T>& pq) {
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
                    settle(sb + u, pa[v], pb[v]);
                    if (sb + u < n1) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) slot(u, 0)[(c4 + j) * PK + q8] = pa[v][j];
                    } else {
                        pa[v].store(slot(u, 0) + q8 * PK + c4);
                    }
                    pb[v].store(slot(u, 1) + q8 * PK + c4);
                }
            }
            __syncthreads();
            // this wave's slices of the batch: those of its part
            const int nbat = ns - sb < BATCH ? ns - sb : BATCH;
            int u0, u1;
            if (part == 0) {
                u0 = 0;
                u1 = n1 - sb < nbat ? (n1 - sb > 0 ? n1 - sb : 0) : nbat;
            } else {
                u0 = n1 - sb > 0 ? n1 - sb : 0;
                u1 = nbat;
            }
            for (int u = u0; u < u1; ++u)
                pq.template mma<PK, PK, ST>(slot(u, 0) + qr, slot(u, 1) + qc, lane);
        }
    };
    // the row part starts from R[I, J]: the row-propagated errors of every source
    // before the chunk, accumulated by the band products of the recursion
    T* const Rt = R + int64_t(I * ST + qr) * np + J * ST + qc;
    if (pre) {
        Q16<T> pq;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            pq.set(r, part == 0 ? Rt[int64_t(Q16<T>::row(r, lane)) * np + Q16<T>::col(r, lane)] : T(0));
        products(pq);
#pragma unroll
        for (int r = 0; r < 4; ++r) Pt[Q16<T>::row(r, lane) * ST + Q16<T>::col(r, lane)] = pq.get(r);
        return;
    }
    // the leaf: this wave's quadrant of the pre-accumulated products, or at the
    // chunk's first diagonal (no chunk sources) R[I, J] alone
    // (one wave-uniform source and stride, so the loads need no select)
    const T* const psrc = Kt > c0 ? Pt : Rt;
    const int pld = Kt > c0 ? ST : np;
    const bool pzero = Kt == c0 && part == 1;
    T pin[4];
    if constexpr (CHAINED) {
        // the older slices' products, from R[I, J] (zero for the column part)
        Q16<T> pq;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            pq.set(r, part == 0 ? Rt[int64_t(Q16<T>::row(r, lane)) * np + Q16<T>::col(r, lane)] : T(0));
        products(pq);
#pragma unroll
        for (int r = 0; r < 4; ++r) pin[r] = pq.get(r);
        __syncthreads();  // the staging area is free for the leaf's tables
        older = false;
        select_slices();  // the freshest slices, multiplied after the wait below
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            pin[r] = pzero ? T(0) : psrc[Q16<T>::row(r, lane) * pld + Q16<T>::col(r, lane)];
    }

    constexpr int FE = ST * ST / LEAF_THREADS;  // factor-block entries per thread
    T fnb[FE], fna[FE];
#pragma unroll
    for (int u = 0; u < FE; ++u) {
        const int e = t + u * LEAF_THREADS, r = e >> 5, c = e & 31;
        fnb[u] = NB[int64_t(I * ST + r) * mp + I * ST + c];
        fna[u] = NA[int64_t(J * ST + r) * np + J * ST + c];
    }
    // The sweep's factor tables: the coefficient of diagonal d's source for the
    // entry (a, b) sits at a fixed offset from a per-entry base,
    //   cB[(d - b + ST) PB + a] = N_B[d - b][a]   (column source (d - b, b))
    //   cA[b PT + d - a + ST]   = N_A[d - a][b]   (row source (a, d - a)),
    // zero wherever the source lies off the tile (and on and below the
    // diagonal: the unit diagonal is replaced by 0), so the unrolled sweep spends no arithmetic on
    // addresses.  First the zero lines, four entries per store (cB rows [0, ST)
    // and [2 ST, NRB), cA columns [0, ST) and [2 ST, PT) of every row), while the
    // loads are in flight; the factor entries follow once the prologue's products
    // are issued (the tables are read only by the sweep).
    {
        constexpr int ZB0 = ST * PB / 4, ZB1 = (NRB - 2 * ST) * PB / 4;
        constexpr int ZAR = ST / 4 + (PT - 2 * ST) / 4;  // per cA row
        static_assert(PB % 4 == 0 && PT % 4 == 0, "16-byte table lines");
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
    const T csb = ENTRY ? CS[J * ST + b] : T(1);  // this thread's column scale
#pragma unroll
    for (int i = 0; i < E; ++i) {
        ar[i] = (E * g - b + i) & (ST - 1);
        dg[i] = b + ar[i];
        x[i] = X[int64_t(I * ST + ar[i]) * np + J * ST + b];
        sc[i] = ENTRY ? S[I * ST + ar[i]] * csb : S[I * ST + ar[i]];
        rs[i] = sc[i] == T(0) ? T(0) : T(1) / sc[i];
    }
    T sblk[4];  // the block layout's row scales (V in the epilogue)
#pragma unroll
    for (int i = 0; i < 4; ++i) sblk[i] = ENTRY ? S[I * ST + r0 + i] * csb : S[I * ST + r0 + i];
    // chained: the tile's own data is on its way; now wait for the freshest
    // slices and the pre-accumulated products
    if constexpr (CHAINED) first_batch();

    // ---- prologue: rowpart (crow) and the chunk's column part (ccol), block layout.
    // X gets rowpart + the column part here; the in-tile column feedback of
    // rowpart, strict(N_B[I, I])^T rowpart, comes from the sweep: its
    // row-accumulated values start at rowpart (rp below), so every entry's
    // column sources pass their rowpart on with their errors, and each entry's
    // final row-accumulated value is R[I, J] = rowpart + Delta N_A[J, J].
    {
        Q16<T> pq;
#pragma unroll
        for (int r = 0; r < 4; ++r) pq.set(r, pin[r]);
        products(pq);  // the freshest slices
        // the tables' factor entries, while the products run
#pragma unroll
        for (int u = 0; u < FE; ++u) {
            const int e = t + u * LEAF_THREADS, r = e >> 5, c = e & 31;
            if (r == c) {
                fnb[u] = T(0);
                fna[u] = T(0);
            }
            cB[(r + ST) * PB + c] = fnb[u];  // N_B[r][c]
            cA[c * PT + ST + r] = fna[u];    // N_A[r][c]
        }
        // the quadrants reach the sweep layout through pk (row-major):
        // pk[0] = rowpart, pk[1] = the column part
        {
            T* q = pk + part * ST * ST + qr * ST + qc;
#pragma unroll
            for (int r = 0; r < 4; ++r) q[Q16<T>::row(r, lane) * ST + Q16<T>::col(r, lane)] = pq.get(r);
        }
        __syncthreads();  // the products and the tables are complete
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const T rowpart = pk[ar[i] * ST + b];
            x[i] += rowpart + pk[ST * ST + ar[i] * ST + b];
            rp[i] = rowpart;
        }
    }

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
        // The producer wave holds exactly the groups of d0 .. d0 + 3, so every lane
        // publishes its half's two diagonals: errors by row, row-accumulated
        // errors by column.
        const int m0 = upper ? 2 : 0;
        const T ea = upper ? e2 : e0, eb = upper ? e3 : e1;
        xD[(r * ST + ar[0]) * RD + m0] = ea;
        xD[(r * ST + ar[1]) * RD + m0 + 1] = eb;
        xR[(r * ST + b) * RD + m0] = upper ? q2 : q0;
        xR[(r * ST + b) * RD + m0 + 1] = upper ? q3 : q1;
        // A rounded entry's error and code also go to bufB / bufA.  A slot whose
        // entry lies on the diagonal 32 later (rounds before the middle) writes its
        // stand-in values there too: the entry's own round overwrites them.  After
        // the middle such entries are done, and those lanes write to junk instead.
        const bool late = RD * r >= ST;
        const bool keep0 = !late || dg[0] == d0 + m0, keep1 = !late || dg[1] == d0 + m0 + 1;
        *(keep0 ? bufB + b * PK + ar[0] : junk + lane) = ea;
        *(keep0 ? bufA + ar[0] * PK + b : junk + lane) = upper ? z2 : z0;
        *(keep1 ? bufB + b * PK + ar[1] : junk + lane) = eb;
        *(keep1 ? bufA + ar[1] * PK + b : junk + lane) = upper ? z3 : z1;
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
    T cnb[RD][E], cna[RD][E];
    coef(0, cnb, cna);
    if (wv == producer(0)) chain(0, cnb, cna);
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
        if (wv == producer(r + 1)) {
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
    // The last round's barrier made the errors and codes in bufB / bufA and every
    // entry's final row-accumulated value in xR complete.  Epilogue: waves 0..3
    // write RF[I, J] = rowpart + Delta N_A[J, J] (read by the later leaves of the
    // chunk and by the band products of the later nodes), gathered from the
    // rounds that published it; waves 4..7 store Delta, the codes and V.
    // (the errors and RF first: the tiles waiting on them poll for them)
    T zv[4];
    if (blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = r0 + i + b;  // the entry's element diagonal
            co_st<CHAINED>(RF + int64_t(I * ST + r0 + i) * np + J * ST + b, xR[((d / RD) * ST + b) * RD + d % RD]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t gi = int64_t(I) * ST + r0 + i, gj = int64_t(J) * ST + b;
            zv[i] = bufA[(r0 + i) * PK + b];
            co_st<CHAINED>(D + gi * np + gj, bufB[b * PK + r0 + i]);
        }
    }
    if (!blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t gi = int64_t(I) * ST + r0 + i, gj = int64_t(J) * ST + b;
            if (gi < m && gj < n) {
                Z[gi * ldz + gj] = CodeT<ENTRY>(zv[i]);
                V[gi * ldv + gj] = CHAINED && s_aborted ? T(__builtin_nan("")) : sblk[i] * zv[i];
            }
        }
    }
}

// Launch K: workgroups [0, nk) sweep the tiles of diagonal K.  When diagonal
// K + 1 lies in the same chunk, workgroups [nk + xpad, nk + xpad + nk1)
// pre-accumulate its tiles' chunk products over every slice that is final
// before this launch (all but the two on diagonal K) into P, so that leaf
// K + 1 adds only the freshest two slices.  Workgroup b runs on XCD b mod 8
// (each XCD has its own L2); the xpad idle workgroups put the workgroup that
// writes a tile's P on the XCD where the next launch sweeps that tile (index
// idx in both), so the leaf reads P from its own L2.  The arguments the kernel
// starts with come first (the launch preloads them into scalar registers); the
// arrays are found from the workspace base.
template <typename T, bool ENTRY>
__global__ __launch_bounds__(LEAF_THREADS) void leaf_kernel(int K, int c0, int c1, int Mt, int Nt, int qmin, int qmax,
                                                   char* __restrict__ ws, int m, int n,
                                                   CodeT<ENTRY>* __restrict__ Z, int64_t ldz, T* __restrict__ V,
                                                   int64_t ldv) {
    const int nk = diag_tiles(K, Mt, Nt);
    const bool pre = int(blockIdx.x) >= nk;
    const int xpad = (8 - nk % 8) % 8;
    const int idx = pre ? int(blockIdx.x) - nk - xpad : int(blockIdx.x);
    if (idx < 0) return;
    leaf_task<T, ENTRY, false>(pre, pre ? K + 1 : K, idx, c0, c1, Mt, Nt, qmin, qmax, ws, m, n, Z, ldz, V, ldv);
}

// The persistent chunk solver: one launch runs every leaf task of the chunk
// [c0, c1) (the sweeps of its tile-diagonals and the pre-accumulation of their
// chunk products), each workgroup drawing tickets until the chunk is done.  A
// tile's sweep starts as soon as its two neighbours before it are swept and its
// products are pre-accumulated, without waiting for the rest of the previous
// tile-diagonal or for a launch; the task order is in kq_chunk_sched.hpp.
template <typename T, bool ENTRY>
__global__ __launch_bounds__(LEAF_THREADS) void chunk_kernel(int c0, int c1, int Mt, int Nt, int qmin, int qmax,
                                                    char* __restrict__ ws, int m, int n,
                                                    CodeT<ENTRY>* __restrict__ Z, int64_t ldz, T* __restrict__ V,
                                                    int64_t ldv, uint32_t spin_limit) {
    const WsOffsets wo = ws_offsets(Mt, Nt, sizeof(T));
    int* const counter = reinterpret_cast<int*>(ws + wo.F) + c0 / CHUNK;
    __shared__ int s_ticket;
    for (;;) {
        __syncthreads();  // the previous task is done with the LDS and s_ticket
        if (threadIdx.x == 0)
            s_ticket = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const ChunkTask tk = chunk_task(__builtin_amdgcn_readfirstlane(s_ticket), c0, c1, Mt, Nt);
        if (tk.Kt < 0) return;
        leaf_task<T, ENTRY, true>(false, tk.Kt, tk.idx, c0, c1, Mt, Nt, qmin, qmax, ws, m, n, Z, ldz, V, ldv,
                                  spin_limit);
    }
}

// Stage 1 at node [K0, K1) with split mid: for the target tiles (I', J) of
// diagonals [mid, K1),
//   R[I', J] += sum_{J' : K0 <= I' + J' < mid} Delta[I', J'] N_A[J', J],
// on 64-row block P and 64-column block Q.  R starts at zero; it gathers each
// tile's row-propagated errors over the nodes whose left half holds a source of
// the tile's row, and the tile's leaf completes it.
//
// Stage 2 at the same node: for the target tiles (I, J) of diagonals [mid, K1),
//   X[I, J] += sum_{I' : K0 <= I' + J < mid} N_B[I', I]^T R[I', J],
// the column feedback of the left half's complete row-propagated tiles (every
// source of R[I', J] lies on a diagonal before mid, so each of them was swept
// already and R[I', J] is final).  Right-half sources reach X at the lower nodes
// and in the leaves, so each (source, target) pair is applied once.
//
// The two stages touch disjoint data (stage 1 writes R of right-half tiles,
// stage 2 reads R of left-half tiles and writes X), so one launch per node runs
// both: blocks [0, n1) are stage 1's, the rest stage 2's.  Each block is a 64 x 64
// output computed split-K by G = 2 groups of four waves (deterministic
// reduction, see tile_gemm_masked_splitk): the small launches of the lower
// recursion levels have few blocks with long K ranges.  Masks work at 32-tile
// granularity; a masked operand element is replaced by zero with a select, so
// the stale contents of tiles outside the band never reach a sum.
template <typename T>
struct Band {
    static constexpr int G = 2;  // groups per block
    static constexpr int THREADS = 256 * G;
};

// Stage 1 block: row block P, the qi-th column block counted from the row's last
// (the last has the longest K range at the top node).
template <typename T, bool SPLIT, typename Smem>
__device__ void band_stage1(const T* __restrict__ D, const T* __restrict__ NA, T* __restrict__ R, int np,
                            int Nt, int K0, int mid, int K1, int P, int qi, Smem& sm) {
    const int I0 = 2 * P;  // first 32-row tile of the block
    const int jlo = K0 - I0 - 1 > 0 ? K0 - I0 - 1 : 0;
    const int jend = K1 - I0 < Nt ? K1 - I0 : Nt;  // exclusive, over both rows
    const int qlo = (mid - I0 - 1 > 0 ? mid - I0 - 1 : 0) >> 1;  // first block with a target in [mid, K1)
    const int Q = ((jend - 1) >> 1) - qi;
    if (jend <= 0 || Q < qlo) return;
    const int kl = jlo;
    int kh = 2 * Q + 1;
    if (mid - 1 - I0 < kh) kh = mid - 1 - I0;
    if (Nt - 1 < kh) kh = Nt - 1;
    if (kh < kl) return;  // no source: nothing to add
    WaveAcc<T> acc;
    acc.zero();
    const T* A = D + int64_t(I0) * ST * np + int64_t(kl) * ST;
    const T* B = NA + int64_t(kl) * ST * np + int64_t(Q) * TILE;
    auto ma = [=](int r, int k) {
        const int s = I0 + (r >> 5) + kl + (k >> 5);  // tile-diagonal of the source tile
        return s >= K0 && s < mid;
    };
    // wave (wy, wx): sources (I0 + wy, kl + kt), target tile (I0 + wy, 2 Q + wx)
    auto lv = [=](int wy, int wx, int kt) {
        const int s = I0 + wy + kl + kt, k = I0 + wy + 2 * Q + wx;
        return s >= K0 && s < mid && k >= mid && k < K1;
    };
    if constexpr (SPLIT) {
        tile_gemm_masked_splitk<T, Band<T>::G, false, false>(A, np, B, np, (kh - kl + 1) * ST, sm, acc, ma, NoMask(),
                                                             lv);
        if (threadIdx.x >= 256) return;  // group 0 holds the product
    } else {
        tile_gemm_masked_k2<T, 2 * KSTEP, false, false>(A, np, B, np, (kh - kl + 1) * ST, sm, acc, ma, NoMask(), lv);
    }
    T* out = R + int64_t(I0) * ST * np + int64_t(Q) * TILE;
    for_each_acc(acc, [&](int r, int c, T v) {
        const int k = I0 + (r >> 5) + 2 * Q + (c >> 5);  // the target tile's diagonal
        if (k >= mid && k < K1) out[int64_t(r) * np + c] += v;
    });
}

// Stage 2 block bi: target blocks (P, Q) of block-diagonal sig = P + Q in
// [sig0, sig1], walked by block row P from the last to the first (sig ascending
// within a row), so the blocks with long K ranges are dispatched first and no
// workgroup is spent on an empty position.
// The product runs split-K over the workgroup's two groups (SPLIT, in the
// 512-thread launch shared with stage 1) or on one 256-thread group with two
// 32-deep slices in flight (a launch of its own).
template <typename T, bool SPLIT, typename Smem>
__device__ void band_stage2(const T* __restrict__ R, const T* __restrict__ NB, T* __restrict__ X, int np, int mp,
                            int Mt, int Nt, int K0, int mid, int K1, int sig0, int sig1, int bi, Smem& sm) {
    const int Mb = Mt >> 1, Nb = Nt >> 1;
    int sig = 0, P = -1;
    for (int b = bi, p = Mb - 1; p >= 0; --p) {
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
    const int kl = K0 - J0 - 1 > 0 ? K0 - J0 - 1 : 0;
    const int kh = I0 + 1 < mid - 1 - J0 ? I0 + 1 : mid - 1 - J0;
    if (kl > kh) return;
    auto src_valid = [=](int ip, int j) {  // a complete tile R[I', J] of the left half
        const int k = ip + j;
        return k >= K0 && k < mid;
    };
    WaveAcc<T> acc;
    acc.zero();
    const T* A = NB + int64_t(kl) * ST * mp + int64_t(I0) * ST;  // A(r, k) = NB[k][r]
    const T* B = R + int64_t(kl) * ST * np + int64_t(J0) * ST;
    auto mb = [=](int k, int c) { return src_valid(kl + (k >> 5), J0 + (c >> 5)); };
    // wave (wy, wx): sources R[kl + kt, J0 + wx], target tile (I0 + wy, J0 + wx)
    auto lv = [=](int wy, int wx, int kt) {
        const int k = I0 + wy + J0 + wx;
        return src_valid(kl + kt, J0 + wx) && k >= mid && k < K1;
    };
    if constexpr (SPLIT) {
        tile_gemm_masked_splitk<T, Band<T>::G, true, false>(A, mp, B, np, (kh - kl + 1) * ST, sm, acc, NoMask(), mb,
                                                            lv);
        if (threadIdx.x >= 256) return;  // group 0 holds the product
    } else {
        tile_gemm_masked_k2<T, 2 * KSTEP, true, false>(A, mp, B, np, (kh - kl + 1) * ST, sm, acc, NoMask(), mb, lv);
    }
    T* out = X + int64_t(I0) * ST * np + int64_t(J0) * ST;
    for_each_acc(acc, [&](int r, int c, T v) {
        const int k = I0 + (r >> 5) + J0 + (c >> 5);
        if (k >= mid && k < K1) out[int64_t(r) * np + c] += v;
    });
}

// Both stages of node [K0, K1): blocks [0, n1) are stage 1's (row blocks P0 ..,
// nq column blocks each), the rest stage 2's (none when stage 2 has its own launch).
template <typename T>
__global__ __launch_bounds__(Band<T>::THREADS) void band_kernel(const T* __restrict__ D, const T* __restrict__ NA,
                                                                const T* __restrict__ NB, T* __restrict__ R,
                                                                const T* __restrict__ RF,
                                                                T* __restrict__ X, int np, int mp, int Mt, int Nt,
                                                                int K0, int mid, int K1, int P0, int nq, int n1,
                                                                int sig0, int sig1) {
    __shared__ SplitSmem<T, Band<T>::G> sm;
    const int b = blockIdx.x;
    if (b < n1)
        band_stage1<T, true>(D, NA, R, np, Nt, K0, mid, K1, P0 + b / nq, b % nq, sm);
    else
        band_stage2<T, true>(RF, NB, X, np, mp, Mt, Nt, K0, mid, K1, sig0, sig1, b - n1, sm);
}

// Stage 1 alone, one 256-thread workgroup per target block (the large nodes).
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS) void band_stage1_kernel(const T* __restrict__ D, const T* __restrict__ NA,
                                                                   T* __restrict__ R, int np, int Nt, int K0, int mid,
                                                                   int K1, int P0, int nq) {
    __shared__ GemmSmemK<T, 2 * KSTEP> sm;
    const int b = blockIdx.x;
    band_stage1<T, false>(D, NA, R, np, Nt, K0, mid, K1, P0 + b / nq, b % nq, sm);
}

// Stage 2 alone, one 256-thread workgroup per target block.
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS) void band_stage2_kernel(const T* __restrict__ R, const T* __restrict__ NB,
                                                                   T* __restrict__ X, int np, int mp, int Mt, int Nt,
                                                                   int K0, int mid, int K1, int sig0, int sig1) {
    __shared__ GemmSmemK<T, 2 * KSTEP> sm;
    band_stage2<T, false>(R, NB, X, np, mp, Mt, Nt, K0, mid, K1, sig0, sig1, int(blockIdx.x), sm);
}

// Nodes of up to BAND_FUSE_MAX blocks run both stages in one launch: there the
// launches are short and latency-bound, and the two stages overlap.  Larger
// nodes run each stage on 256-thread workgroups (more of them per CU, two slices
// in flight), which do better once the launch fills the device.
constexpr int BAND_FUSE_MAX = 1200;

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

// The bound on one wait of the persistent chunk solver: CHUNK_SPIN_LIMIT, or
// the value of the environment variable KQ_CHUNK_SPIN_LIMIT (a decimal count of
// polls), read per call.  A small value makes waits end early on purpose: the
// launch then still drains, with NaN in V (how the bound's exit path is tested).
static uint32_t chunk_spin_limit() {
    const char* e = std::getenv("KQ_CHUNK_SPIN_LIMIT");
    if (!e || !*e) return CHUNK_SPIN_LIMIT;
    char* end = nullptr;
    const unsigned long v = std::strtoul(e, &end, 10);
    return (end && *end == '\0' && v <= 0xffffffffu) ? uint32_t(v) : CHUNK_SPIN_LIMIT;
}

__global__ void zero_words_kernel(int* __restrict__ p, int64_t count) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

// ------------------------------------------------------------------- host side

constexpr int CHUNK_GRID = 256;  // workgroups of a persistent chunk launch: one per compute unit

struct SolverLayout {
    int64_t mp, np, Mt, Nt;  // padded extents; tile counts in 32-tiles
    size_t bytes;
    size_t off_NA, off_NB, off_X, off_D, off_R, off_RF, off_P, off_S, off_C, off_F, off_L;
};

SolverLayout solver_layout(kq_dtype dtype, int64_t m, int64_t n) {
    SolverLayout L;
    const size_t es = dtype == KQ_F64 ? 8 : 4;
    L.mp = round_up(m, TILE);
    L.np = round_up(n, TILE);
    L.Mt = L.mp / ST;
    L.Nt = L.np / ST;
    static_assert(TILE % 64 == 0, "array sizes stay multiples of 256 bytes");
    const WsOffsets o = ws_offsets(L.Mt, L.Nt, int64_t(es));
    L.off_NA = size_t(o.NA);
    L.off_NB = size_t(o.NB);
    L.off_X = size_t(o.X);
    L.off_D = size_t(o.D);
    L.off_R = size_t(o.R);
    L.off_RF = size_t(o.RF);
    L.off_P = size_t(o.P);
    L.off_S = size_t(o.S);
    L.off_C = size_t(o.C);
    L.off_F = size_t(o.F);
    L.off_L = align256(size_t(o.end));  // loss scratch (fp64): 1 / U_A,jj, 1 / U_B,ii, partial sums
    L.bytes = L.off_L + align256((size_t(L.np) + size_t(L.mp) + ELOSS_PARTS) * sizeof(double));
    return L;
}

template <typename T>
struct SolverRun {
    const SolverLayout& L;
    int m, n, qmin, qmax;
    T *NA, *NB, *X, *D, *R, *RF, *P, *S;
    T* C;     // column scales (WaterKron mode) or nullptr
    void* Z;  // int8 codes, or int32 in the WaterKron mode
    int64_t ldz;
    T* V;
    int64_t ldv;
    hipStream_t st;
    char* ws;  // the workspace base (the leaves find their arrays from it)
    bool chained;  // chunks on the persistent chunk solver, else a launch per tile-diagonal and role
    uint32_t spin_limit;  // the chunk solver's bound on one wait, in polls

    kq_status leaf(int K, int c0, int c1) {
        const int Mt = int(L.Mt), Nt = int(L.Nt);
        auto tiles = [&](int k) {  // tiles on tile-diagonal k
            return (k < Mt - 1 ? k : Mt - 1) - (k - Nt + 1 > 0 ? k - Nt + 1 : 0) + 1;
        };
        // the sweep of diagonal K, and the chunk products of K + 1 when it is in
        // the chunk (behind up to 7 idle workgroups that align them with the XCDs)
        const dim3 grid(tiles(K) + (K + 1 < c1 ? (8 - tiles(K) % 8) % 8 + tiles(K + 1) : 0));
        if (C)
            hipLaunchKernelGGL((leaf_kernel<T, true>), grid, dim3(LEAF_THREADS), 0, st, K, c0, c1, Mt, Nt, qmin,
                               qmax, ws, m, n, static_cast<int32_t*>(Z), ldz, V, ldv);
        else
            hipLaunchKernelGGL((leaf_kernel<T, false>), grid, dim3(LEAF_THREADS), 0, st, K, c0, c1, Mt, Nt, qmin,
                               qmax, ws, m, n, static_cast<int8_t*>(Z), ldz, V, ldv);
        KQ_LAUNCHED("leaf_kernel");
        return KQ_OK;
    }

    kq_status propagate(int K0, int mid, int K1) {
        const int Mt = int(L.Mt), Nt = int(L.Nt);
        // stage 1 rows I' with a source tile in [K0, mid): K0 - Nt < I' < mid
        const int row0 = K0 - Nt + 1 > 0 ? K0 - Nt + 1 : 0;
        const int row1 = mid < Mt ? mid : Mt;  // exclusive
        const int P0 = row0 >> 1;
        const int nq = (K1 - mid) / 2 + 2;  // column blocks per row block: targets in [mid, K1)
        const int n1 = row1 > row0 ? nq * (((row1 - 1) >> 1) - P0 + 1) : 0;
        // stage 2 target block-diagonals sig with [2 sig, 2 sig + 2] meeting [mid, K1)
        const int sig0 = (mid - 1) >> 1 > 0 ? (mid - 1) >> 1 : 0;
        int sig1 = (K1 - 1) >> 1;
        const int sigmax = int(L.Mt / 2 + L.Nt / 2 - 2);
        if (sig1 > sigmax) sig1 = sigmax;
        int n2 = 0;  // target blocks
        for (int p = 0; p < Mt / 2 && sig1 >= sig0; ++p) {
            const int lo = sig0 > p ? sig0 : p, hi = sig1 < p + Nt / 2 - 1 ? sig1 : p + Nt / 2 - 1;
            n2 += hi >= lo ? hi - lo + 1 : 0;
        }
        const bool fuse = n1 + n2 <= BAND_FUSE_MAX;
        if (fuse && n1 + n2 > 0) {
            hipLaunchKernelGGL(band_kernel<T>, dim3(n1 + n2), dim3(Band<T>::THREADS), 0, st, D, NA, NB, R, RF, X,
                               int(L.np), int(L.mp), Mt, Nt, K0, mid, K1, P0, nq, n1, sig0, sig1);
            KQ_LAUNCHED("band_kernel");
        }
        if (!fuse && n1 > 0) {
            hipLaunchKernelGGL(band_stage1_kernel<T>, dim3(n1), dim3(GEMM_THREADS), 0, st, D, NA, R, int(L.np), Nt, K0,
                               mid, K1, P0, nq);
            KQ_LAUNCHED("band_stage1_kernel");
        }
        if (!fuse && n2 > 0) {
            hipLaunchKernelGGL(band_stage2_kernel<T>, dim3(n2), dim3(GEMM_THREADS), 0, st, RF, NB, X, int(L.np),
                               int(L.mp), Mt, Nt, K0, mid, K1, sig0, sig1);
            KQ_LAUNCHED("band_stage2_kernel");
        }
        return KQ_OK;
    }

    // the leaf tasks of chunk [c0, c1) in one persistent launch
    kq_status chunk(int c0, int c1) {
        const int Mt = int(L.Mt), Nt = int(L.Nt);
        const int tasks = chunk_tasks(c0, c1, Mt, Nt);
        const dim3 grid(tasks < CHUNK_GRID ? tasks : CHUNK_GRID);
        if (C)
            hipLaunchKernelGGL((chunk_kernel<T, true>), grid, dim3(LEAF_THREADS), 0, st, c0, c1, Mt, Nt, qmin, qmax,
                               ws, m, n, static_cast<int32_t*>(Z), ldz, V, ldv, spin_limit);
        else
            hipLaunchKernelGGL((chunk_kernel<T, false>), grid, dim3(LEAF_THREADS), 0, st, c0, c1, Mt, Nt, qmin,
                               qmax, ws, m, n, static_cast<int8_t*>(Z), ldz, V, ldv, spin_limit);
        KQ_LAUNCHED("chunk_kernel");
        return KQ_OK;
    }

    kq_status solve(int K0, int K1) {
        if (K1 - K0 <= CHUNK) {
            if (chained) return chunk(K0, K1);
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
kq_status onesided_solve(int m, int n, int mp, int np, int qmin, int qmax, const T* NA, T* X, T* D, const T* S,
                         const T* C, void* Z, int64_t ldz, T* V, int64_t ldv, hipStream_t st);

// The base quantizer as the solver sees it: the step of entry (i, j) is
// row_scales[per_row ? i : 0], times col_scales[j] when given; codes clamped to
// [qmin, qmax] and stored as int8, or as int32 when col_scales is given (the
// WaterKron alphabet).
template <typename T>
struct QuantSpec {
    const T* row_scales;
    int per_row;
    const T* col_scales;
    int qmin, qmax;
    void* codes;
    int64_t ldc;
    bool chained;  // two-sided leaves on the persistent chunk solver
};

template <typename T>
kq_status quantize_typed(int64_t m, int64_t n, const T* W, int64_t ldw, const T* UA, int64_t lda, const T* UB,
                         int64_t ldb, const QuantSpec<T>& q, T* V, int64_t ldv, double* loss_dev, void* ws,
                         hipStream_t st) {
    const SolverLayout L = solver_layout(sizeof(T) == 8 ? KQ_F64 : KQ_F32, m, n);
    char* base = static_cast<char*>(ws);
    SolverRun<T> run{L, int(m), int(n), q.qmin, q.qmax,
                     reinterpret_cast<T*>(base + L.off_NA), reinterpret_cast<T*>(base + L.off_NB),
                     reinterpret_cast<T*>(base + L.off_X), reinterpret_cast<T*>(base + L.off_D),
                     reinterpret_cast<T*>(base + L.off_R), reinterpret_cast<T*>(base + L.off_RF),
                     reinterpret_cast<T*>(base + L.off_P),
                     reinterpret_cast<T*>(base + L.off_S),
                     q.col_scales ? reinterpret_cast<T*>(base + L.off_C) : nullptr, q.codes, q.ldc, V, ldv, st, base,
                     q.chained, chunk_spin_limit()};
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
                       int(L.mp), int(L.np), q.row_scales, q.per_row, q.col_scales, run.X, run.S, run.C,
                       UB ? run.R : nullptr, UB && run.chained ? run.D : nullptr, run.RF);
    KQ_LAUNCHED("init_solver_kernel");
    if (UB && run.chained) {  // the chunk solver's ticket counters and abort word start at zero
        const int64_t nw = flag_words(L.Mt, L.Nt);
        hipLaunchKernelGGL(zero_words_kernel, blocks(nw), dim3(threads), 0, st,
                           reinterpret_cast<int*>(base + L.off_F), nw);
        KQ_LAUNCHED("zero_words_kernel");
    }
    // B = I: one-sided GPTQ, rows independent, recursive over column ranges
    const kq_status s = UB ? run.solve(0, int(L.Mt + L.Nt - 1))
                           : onesided_solve<T>(int(m), int(n), int(L.mp), int(L.np), run.qmin, run.qmax, run.NA,
                                               run.X, run.D, run.S, run.C, q.codes, q.ldc, V, ldv, st);
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

template <typename T>
kq_status quantize_as(int64_t m, int64_t n, const void* W, int64_t ldw, const void* UA, int64_t lda, const void* UB,
                      int64_t ldb, const QuantSpec<T>& q, void* V, int64_t ldv, double* loss_dev, void* ws,
                      hipStream_t st) {
    return quantize_typed<T>(m, n, static_cast<const T*>(W), ldw, static_cast<const T*>(UA), lda,
                             static_cast<const T*>(UB), ldb, q, static_cast<T*>(V), ldv, loss_dev, ws, st);
}

kq_status quantize_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* UA,
                            int64_t lda, const void* UB, int64_t ldb, const kq_quantizer* q, int8_t* codes,
                            int64_t ldc, void* V, int64_t ldv, double* loss_dev, void* ws, hipStream_t st,
                            bool chained) {
    const int qmin = -(1 << (q->bits - 1)), qmax = (1 << (q->bits - 1)) - 1;
    if (dtype == KQ_F64)
        return quantize_as<double>(m, n, W, ldw, UA, lda, UB, ldb,
                                   {static_cast<const double*>(q->scales), q->per_row, nullptr, qmin, qmax, codes, ldc,
                                    chained},
                                   V, ldv, loss_dev, ws, st);
    return quantize_as<float>(m, n, W, ldw, UA, lda, UB, ldb,
                              {static_cast<const float*>(q->scales), q->per_row, nullptr, qmin, qmax, codes, ldc,
                               chained},
                              V,
                              ldv, loss_dev, ws, st);
}

// WaterKron: steps beta_i alpha_j, int32 codes clamped only at +-2^30 (exact in
// fp32 and fp64; far beyond any code a finite step gives for finite weights).
constexpr int WK_CODE_BOUND = 1 << 30;

kq_status waterkron_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* UA,
                             int64_t lda, const void* UB, int64_t ldb, const void* alpha, const void* beta,
                             int32_t* codes, int64_t ldc, void* V, int64_t ldv, double* loss_dev, void* ws,
                             hipStream_t st) {
    if (dtype == KQ_F64)
        return quantize_as<double>(m, n, W, ldw, UA, lda, UB, ldb,
                                   {static_cast<const double*>(beta), 1, static_cast<const double*>(alpha),
                                    -WK_CODE_BOUND, WK_CODE_BOUND, codes, ldc, true},
                                   V, ldv, loss_dev, ws, st);
    return quantize_as<float>(m, n, W, ldw, UA, lda, UB, ldb,
                              {static_cast<const float*>(beta), 1, static_cast<const float*>(alpha), -WK_CODE_BOUND,
                               WK_CODE_BOUND, codes, ldc, true},
                              V, ldv, loss_dev, ws, st);
}

}  // namespace kq
