// Shared device and host helpers of the kronq HIP library (gfx950 only).
//
// The matrix-core tile used by every dense contraction in the library is a
// 64 x 64 output block computed by one 256-thread workgroup (four wave64s in a
// 2 x 2 arrangement, 32 x 32 outputs per wave), K consumed 16 at a time through
// double-buffered LDS.  fp32 uses v_mfma_f32_32x32x2f32, fp64 uses
// v_mfma_f64_16x16x4f64 (four 16 x 16 blocks per wave).  Operand lane layouts
// (measured on gfx950):
//   f32 32x32x2 : A[i=l%32][k=l/32], B[k=l/32][j=l%32],
//                 D reg r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32
//   f64 16x16x4 : A[i=l%16][k=l/16], B[k=l/16][j=l%16],
//                 D reg r -> row l/16 + 4*r, col l%16
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/kronq.h"

namespace kq {

constexpr int TILE = 64;     // solver / GEMM tile edge
constexpr int KSTEP = 16;    // K slice staged in LDS per iteration
constexpr int GEMM_THREADS = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ host side

void set_error(const std::string& msg);
kq_status hip_fail(hipError_t e, const char* what);

#define KQ_HIP(expr)                                                   \
    do {                                                               \
        hipError_t kq_e_ = (expr);                                     \
        if (kq_e_ != hipSuccess) return ::kq::hip_fail(kq_e_, #expr);  \
    } while (0)

#define KQ_LAUNCHED(name)                                              \
    do {                                                               \
        hipError_t kq_e_ = hipGetLastError();                          \
        if (kq_e_ != hipSuccess) return ::kq::hip_fail(kq_e_, name);   \
    } while (0)

inline int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Simple bump allocator over the caller's workspace.
struct Carve {
    char* base;
    size_t used = 0;
    explicit Carve(void* p) : base(static_cast<char*>(p)) {}
    template <typename T>
    T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
        used += align256(count * sizeof(T));
        return p;
    }
};

// ---------------------------------------------------------------- device side

// Precision-preserving scalar helpers (the plain __builtin_fma / rint / fmin
// are the double-precision builtins and would promote float arguments).
__device__ __forceinline__ float kfma(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double kfma(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ __forceinline__ float krint(float x) { return __builtin_rintf(x); }
__device__ __forceinline__ double krint(double x) { return __builtin_rint(x); }
__device__ __forceinline__ float kclamp(float x, float lo, float hi) { return __builtin_fminf(__builtin_fmaxf(x, lo), hi); }
__device__ __forceinline__ double kclamp(double x, double lo, double hi) { return __builtin_fmin(__builtin_fmax(x, lo), hi); }

// Base quantizer: z = clamp(rne(x / s)), v = s * z.  IEEE division (HIP's default
// correctly rounded divide), rint = round half to even.  s == 0 gives z = v = 0.
template <typename T>
__device__ __forceinline__ void quantize(T x, T s, T qmin, T qmax, T& z, T& v) {
    if (s == T(0)) {
        z = T(0);
        v = T(0);
        return;
    }
    const T r = kclamp(krint(x / s), qmin, qmax);
    z = r;
    v = s * r;
}

template <typename T>
struct LdsStride;
template <>
struct LdsStride<float> {
    static constexpr int value = 68;  // 16-byte aligned rows, spreads banks
};
template <>
struct LdsStride<double> {
    static constexpr int value = 66;
};

// Per-wave accumulator of a 32 x 32 block of the 64 x 64 tile.
template <typename T>
struct WaveAcc;

template <>
struct WaveAcc<float> {
    f32x16 c;
    __device__ void zero() {
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = 0.f;
    }
    // As/Bs: one 16-deep K slice, element (k, idx) at [k * S + idx].
    __device__ void mma(const float* As, const float* Bs, int wy, int wx, int lane) {
        constexpr int S = LdsStride<float>::value;
        const int kr = lane >> 5, ix = lane & 31;
#pragma unroll
        for (int kk = 0; kk < KSTEP; kk += 2) {
            float a = As[(kk + kr) * S + wy * 32 + ix];
            float b = Bs[(kk + kr) * S + wx * 32 + ix];
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
        }
    }
    static constexpr int NREG = 16;
    __device__ float get(int r) const { return c[r]; }
    __device__ void add(int r, float v) { c[r] += v; }
    // Position of register r inside the wave's 32 x 32 block.
    static __device__ __forceinline__ int row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
    static __device__ __forceinline__ int col(int r, int lane) { return lane & 31; }
};

template <>
struct WaveAcc<double> {
    f64x4 c[2][2];
    __device__ void zero() {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) c[i][j][r] = 0.0;
    }
    __device__ void mma(const double* As, const double* Bs, int wy, int wx, int lane) {
        constexpr int S = LdsStride<double>::value;
        const int kr = lane >> 4, ix = lane & 15;
#pragma unroll
        for (int kk = 0; kk < KSTEP; kk += 4) {
            double a0 = As[(kk + kr) * S + wy * 32 + ix];
            double a1 = As[(kk + kr) * S + wy * 32 + 16 + ix];
            double b0 = Bs[(kk + kr) * S + wx * 32 + ix];
            double b1 = Bs[(kk + kr) * S + wx * 32 + 16 + ix];
            c[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, c[0][0], 0, 0, 0);
            c[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, c[0][1], 0, 0, 0);
            c[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, c[1][0], 0, 0, 0);
            c[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, c[1][1], 0, 0, 0);
        }
    }
    static constexpr int NREG = 16;
    __device__ double get(int r) const { return c[r >> 3][(r >> 2) & 1][r & 3]; }
    __device__ void add(int r, double v) { c[r >> 3][(r >> 2) & 1][r & 3] += v; }
    static __device__ __forceinline__ int row(int r, int lane) { return 16 * (r >> 3) + (lane >> 4) + 4 * (r & 3); }
    static __device__ __forceinline__ int col(int r, int lane) { return 16 * ((r >> 2) & 1) + (lane & 15); }
};

// Operand access patterns.  Element (r, k) of the M x K operand A and element
// (k, c) of the K x N operand B.
//   A_KMAJ == false : A(r, k) = A[r * lda + k]   (row-major A)
//   A_KMAJ == true  : A(r, k) = A[k * lda + r]   (A stored transposed)
//   B_KMAJ == false : B(k, c) = B[k * ldb + c]   (row-major B)
//   B_KMAJ == true  : B(k, c) = B[c * ldb + k]   (B stored transposed)
// CHECK: rows >= mv, columns >= nv and k >= kv read as zero (any alignment);
// otherwise all reads are in range and 4-element vector aligned.
template <typename T, typename TIn, bool A_KMAJ, bool B_KMAJ, bool CHECK>
struct TileLoader {
    T ra[4], rb[4];
    __device__ __forceinline__ void fetch(const TIn* __restrict__ A, int64_t lda, const TIn* __restrict__ B,
                                          int64_t ldb, int k0, int mv, int nv, int kv, int t) {
        // A tile 64 x 16
        if (!A_KMAJ) {
            const int r = t >> 2, kq = (t & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = k0 + kq + e;
                ra[e] = (!CHECK || (r < mv && k < kv)) ? T(A[int64_t(r) * lda + k]) : T(0);
            }
        } else {
            const int k = t >> 4, rq = (t & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rq + e;
                ra[e] = (!CHECK || (r < mv && k0 + k < kv)) ? T(A[int64_t(k0 + k) * lda + r]) : T(0);
            }
        }
        if (!B_KMAJ) {
            const int k = t >> 4, cq = (t & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = cq + e;
                rb[e] = (!CHECK || (c < nv && k0 + k < kv)) ? T(B[int64_t(k0 + k) * ldb + c]) : T(0);
            }
        } else {
            const int c = t >> 2, kq = (t & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = k0 + kq + e;
                rb[e] = (!CHECK || (c < nv && k < kv)) ? T(B[int64_t(c) * ldb + k]) : T(0);
            }
        }
    }
    __device__ __forceinline__ void stash(T* As, T* Bs, int t) const {
        constexpr int S = LdsStride<T>::value;
        if (!A_KMAJ) {
            const int r = t >> 2, kq = (t & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) As[(kq + e) * S + r] = ra[e];
        } else {
            const int k = t >> 4, rq = (t & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) As[k * S + rq + e] = ra[e];
        }
        if (!B_KMAJ) {
            const int k = t >> 4, cq = (t & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) Bs[k * S + cq + e] = rb[e];
        } else {
            const int c = t >> 2, kq = (t & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) Bs[(kq + e) * S + c] = rb[e];
        }
    }
};

template <typename T>
struct GemmSmem {
    T a[2][KSTEP * LdsStride<T>::value];
    T b[2][KSTEP * LdsStride<T>::value];
};

// acc += A(64 x K) * B(K x 64) for one 64 x 64 output tile.  All 256 threads of
// the workgroup must call it (it contains barriers).  K is the number of K
// elements; without CHECK it must be a multiple of 16.
template <typename T, typename TIn, bool A_KMAJ, bool B_KMAJ, bool CHECK>
__device__ void tile_gemm(const TIn* __restrict__ A, int64_t lda, const TIn* __restrict__ B, int64_t ldb,
                          int mv, int nv, int K, GemmSmem<T>& sm, WaveAcc<T>& acc) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wy = w >> 1, wx = w & 1;
    TileLoader<T, TIn, A_KMAJ, B_KMAJ, CHECK> ld;
    const int nk = (K + KSTEP - 1) / KSTEP;
    if (nk == 0) return;
    ld.fetch(A, lda, B, ldb, 0, mv, nv, K, t);
    __syncthreads();  // previous users of sm are done
    ld.stash(sm.a[0], sm.b[0], t);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        if (s + 1 < nk) ld.fetch(A, lda, B, ldb, (s + 1) * KSTEP, mv, nv, K, t);
        acc.mma(sm.a[cur], sm.b[cur], wy, wx, lane);
        if (s + 1 < nk) {
            ld.stash(sm.a[cur ^ 1], sm.b[cur ^ 1], t);
            __syncthreads();
        }
    }
}

// Masked products over padded, in-range operands: element (r, k) of A is used
// only where ma(r, k) holds and element (k, c) of B only where mb(k, c) holds;
// elsewhere the operand reads as zero (a select, so non-finite stale values
// never reach the sum).  NoMask keeps every element.
struct NoMask {
    __device__ __forceinline__ bool operator()(int, int) const { return true; }
};

// live(wy, wx, kt): whether the wave owning the 32 x 32 quadrant (wy, wx) of the
// 64 x 64 output needs its product over the kt-th 32-deep tile of K.  A wave whose
// operands are masked to zero over that tile, or whose output is discarded, skips
// its matrix-core steps there (the sum is unchanged: it would add zeros).
struct AllLive {
    __device__ __forceinline__ bool operator()(int, int, int) const { return true; }
};

// K-slice depth as a parameter: KS = 16 R deep slices, each thread moving R
// groups of the 16-deep loader pattern.  Deeper slices carry more matrix-core
// work per global round trip, which matters when few blocks share a CU and the
// loads of the next slice are the only latency hiding.
template <typename T, bool A_KMAJ, bool B_KMAJ, int KS>
struct LoaderK {
    static constexpr int R = KS / KSTEP;
    TileLoader<T, T, A_KMAJ, B_KMAJ, false> g[R];
    __device__ __forceinline__ void fetch(const T* __restrict__ A, int64_t lda, const T* __restrict__ B, int64_t ldb,
                                          int k0, int t) {
#pragma unroll
        for (int q = 0; q < R; ++q) g[q].fetch(A, lda, B, ldb, k0 + KSTEP * q, TILE, TILE, 0, t);
    }
    __device__ __forceinline__ void stash(T* As, T* Bs, int t) const {
        constexpr int S = LdsStride<T>::value;
#pragma unroll
        for (int q = 0; q < R; ++q) g[q].stash(As + KSTEP * q * S, Bs + KSTEP * q * S, t);
    }
    template <typename MA, typename MB>
    __device__ __forceinline__ void apply(int k0, int t, MA ma, MB mb) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int kq0 = k0 + KSTEP * q;
            if (!A_KMAJ) {
                const int r = t >> 2, kq = (t & 3) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!ma(r, kq0 + kq + e)) g[q].ra[e] = T(0);
            } else {
                const int k = t >> 4, rq = (t & 15) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!ma(rq + e, kq0 + k)) g[q].ra[e] = T(0);
            }
            if (!B_KMAJ) {
                const int k = t >> 4, cq = (t & 15) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!mb(kq0 + k, cq + e)) g[q].rb[e] = T(0);
            } else {
                const int c = t >> 2, kq = (t & 3) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!mb(kq0 + kq + e, c)) g[q].rb[e] = T(0);
            }
        }
    }
};

template <typename T, int KS>
struct GemmSmemK {
    T a[2][KS * LdsStride<T>::value];
    T b[2][KS * LdsStride<T>::value];
};

// A masked tile product with KS-deep slices and two slices in flight: while the
// matrix cores work on slice s from LDS, the loads of slices s + 1 and s + 2 are
// both outstanding (two register sets used in turn), so a block whose K loop is
// bound by the latency of its own loads waits half as often.  K must be a
// multiple of KS.
template <typename T, int KS, bool A_KMAJ, bool B_KMAJ, typename MA, typename MB, typename LV = AllLive>
__device__ void tile_gemm_masked_k2(const T* __restrict__ A, int64_t lda, const T* __restrict__ B, int64_t ldb, int K,
                                    GemmSmemK<T, KS>& sm, WaveAcc<T>& acc, MA ma, MB mb, LV live = LV()) {
    static_assert(KS <= 32 && 32 % KS == 0, "a slice lies in one 32-deep tile of K");
    constexpr int S = LdsStride<T>::value;
    const int t = threadIdx.x & 255, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: scalar branches on live
    const int wy = w >> 1, wx = w & 1;
    LoaderK<T, A_KMAJ, B_KMAJ, KS> la, lb;
    const int nk = K / KS;
    if (nk == 0) return;
    auto mma = [&](int buf, int s) {
        if (!live(wy, wx, s * KS / 32)) return;
#pragma unroll
        for (int q = 0; q < KS / KSTEP; ++q) acc.mma(sm.a[buf] + KSTEP * q * S, sm.b[buf] + KSTEP * q * S, wy, wx, lane);
    };
    la.fetch(A, lda, B, ldb, 0, t);
    if (nk > 1) lb.fetch(A, lda, B, ldb, KS, t);
    la.apply(0, t, ma, mb);
    __syncthreads();
    la.stash(sm.a[0], sm.b[0], t);
    __syncthreads();
    for (int s = 0; s < nk; s += 2) {
        // LDS stage 0 holds slice s, lb carries slice s + 1
        if (s + 2 < nk) la.fetch(A, lda, B, ldb, (s + 2) * KS, t);
        mma(0, s);
        if (s + 1 < nk) {
            lb.apply((s + 1) * KS, t, ma, mb);
            lb.stash(sm.a[1], sm.b[1], t);
            __syncthreads();
            // LDS stage 1 holds slice s + 1, la carries slice s + 2
            if (s + 3 < nk) lb.fetch(A, lda, B, ldb, (s + 3) * KS, t);
            mma(1, s + 1);
            if (s + 2 < nk) {
                la.apply((s + 2) * KS, t, ma, mb);
                la.stash(sm.a[0], sm.b[0], t);
                __syncthreads();
            }
        }
    }
}

// Split-K variant for launch shapes with few blocks and long K ranges: G groups of
// four waves (blockDim = 256 G) share one 64 x 64 output.  Group g takes the
// K slices s = g, g + G, ... with its own double-buffered LDS stage, all groups
// step together (one workgroup barrier per step), and at the end groups 1..G-1
// hand their partial sums to group 0 through LDS, which adds them in group
// order, so the result does not depend on timing.  Only group 0's acc holds
// the product afterwards.
template <typename T, int G>
struct SplitSmem {
    GemmSmem<T> st[G];
};

template <typename T, int G, bool A_KMAJ, bool B_KMAJ, typename MA, typename MB, typename LV = AllLive>
__device__ void tile_gemm_masked_splitk(const T* __restrict__ A, int64_t lda, const T* __restrict__ B,
                                        int64_t ldb, int K, SplitSmem<T, G>& sm, WaveAcc<T>& acc, MA ma, MB mb,
                                        LV live = LV()) {
    const int tg = threadIdx.x, grp = tg >> 8, t = tg & 255, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: scalar branches on live
    const int wy = w >> 1, wx = w & 1;
    TileLoader<T, T, A_KMAJ, B_KMAJ, false> ld;
    GemmSmem<T>& my = sm.st[grp];
    const int nk = K / KSTEP;
    const int iters = (nk + G - 1) / G;
    auto apply = [&](int k0) {
        if (!A_KMAJ) {
            const int r = t >> 2, kq = (t & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!ma(r, k0 + kq + e)) ld.ra[e] = T(0);
        } else {
            const int k = t >> 4, rq = (t & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!ma(rq + e, k0 + k)) ld.ra[e] = T(0);
        }
        if (!B_KMAJ) {
            const int k = t >> 4, cq = (t & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!mb(k0 + k, cq + e)) ld.rb[e] = T(0);
        } else {
            const int c = t >> 2, kq = (t & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!mb(k0 + kq + e, c)) ld.rb[e] = T(0);
        }
    };
    if (iters > 0) {
        int s = grp;
        if (s < nk) {
            ld.fetch(A, lda, B, ldb, s * KSTEP, TILE, TILE, K, t);
            apply(s * KSTEP);
            ld.stash(my.a[0], my.b[0], t);
        }
        __syncthreads();
        for (int it = 0; it < iters; ++it) {
            const int cur = it & 1;
            const int sn = s + G;  // this group's next slice
            if (sn < nk) ld.fetch(A, lda, B, ldb, sn * KSTEP, TILE, TILE, K, t);
            if (s < nk && live(wy, wx, s * KSTEP / 32)) acc.mma(my.a[cur], my.b[cur], wy, wx, lane);
            if (sn < nk) {
                apply(sn * KSTEP);
                ld.stash(my.a[cur ^ 1], my.b[cur ^ 1], t);
            }
            __syncthreads();
            s = sn;
        }
    }
    // reduction: group g > 0 parks its partials in its own stage buffers
    constexpr int NR = WaveAcc<T>::NREG;
    static_assert(sizeof(GemmSmem<T>) >= sizeof(T) * NR * 256, "stage buffer too small for the partials");
    if (grp > 0) {
        T* park = reinterpret_cast<T*>(&sm.st[grp]);
#pragma unroll
        for (int r = 0; r < NR; ++r) park[r * 256 + t] = acc.get(r);
    }
    __syncthreads();
    if (grp == 0) {
        for (int g = 1; g < G; ++g) {
            const T* park = reinterpret_cast<const T*>(&sm.st[g]);
#pragma unroll
            for (int r = 0; r < NR; ++r) acc.add(r, park[r * 256 + t]);
        }
    }
}

// Visit the 16 accumulator registers of this thread with their tile coordinates.
template <typename T, typename F>
__device__ __forceinline__ void for_each_acc(const WaveAcc<T>& acc, F&& f) {
    const int t = threadIdx.x & 255, lane = t & 63, w = t >> 6;
    const int r0 = (w >> 1) * 32, c0 = (w & 1) * 32;
#pragma unroll
    for (int r = 0; r < WaveAcc<T>::NREG; ++r)
        f(r0 + WaveAcc<T>::row(r, lane), c0 + WaveAcc<T>::col(r, lane), acc.get(r));
}

// Fixed-order sum of the 256 per-thread values of a workgroup.
__device__ __forceinline__ double block_sum_256(double s, double* red) {
    __syncthreads();  // earlier readers of red are done
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (int(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    return red[0];
}

}  // namespace kq
