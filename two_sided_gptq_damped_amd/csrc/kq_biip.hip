// KronQ bidirectional incoherence processing (BiIP) for gfx950.
//
// What is computed (KronQ page, section "Kronecker-Factored Quantization": the
// diagonal rescale S = diag^{-1/4} of each Hessian factor, then orthogonal
// rotations on both sides; Theorem 1: the loss is invariant):
//   forward  W'' = Q_B S_B W S_A Q_A^T,  A'' = Q_A S_A^{-1} A S_A^{-1} Q_A^T,
//            B'' = Q_B S_B^{-1} B S_B^{-1} Q_B^T
//   inverse  V = S_B^{-1} Q_B^T V'' Q_A S_A^{-1}
// with s = diag(M)^{-1/4} (1 where the diagonal is not positive) and
// Q = (I (x) H_h / sqrt(h)) diag(signs): the Sylvester Walsh-Hadamard matrix on
// blocks of h = the largest power of two dividing the dimension, at most 4096,
// after caller-drawn random signs.
//
// Every step is a pass over rows: a row transform x -> post o (H (pre o x)) in
// LDS (fast Walsh-Hadamard butterflies, log2 h stages), and a tiled transpose
// that turns the left-hand transform into another row transform.  All passes
// are bound by HBM bandwidth (each reads and writes the matrix once).
#include <algorithm>
#include <cmath>

#include "kq_common.hpp"

namespace kq {

constexpr int BIIP_MAX_BLOCK = 4096;
constexpr int BIIP_SEG = 1024;  // entries per workgroup when the block is shorter

static int hadamard_block(int64_t d) {
    int64_t h = d & -d;
    return int(h < BIIP_MAX_BLOCK ? h : BIIP_MAX_BLOCK);
}

// pre / post vectors from the factor diagonals and the signs (fp64, rounded once):
//   mul[j] = sign_j * s_j      (W's side)
//   div[j] = sign_j / s_j      (the factor's side, and the inverse's post)
template <typename T>
__global__ void biip_vectors_kernel(const T* __restrict__ M, int64_t ldm, int d, const int8_t* __restrict__ signs,
                                    T* __restrict__ scale, T* __restrict__ mul, T* __restrict__ div) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= d) return;
    const double a = double(M[int64_t(j) * ldm + j]);
    const double s = a > 0.0 ? 1.0 / sqrt(sqrt(a)) : 1.0;
    const double g = signs[j] < 0 ? -1.0 : 1.0;
    scale[j] = T(s);
    mul[j] = T(g * s);
    div[j] = T(g / s);
}

// div[j] = sign_j / s_j from stored scales (the inverse transform's post).
template <typename T>
__global__ void biip_div_kernel(const T* __restrict__ scale, const int8_t* __restrict__ signs, int d,
                                T* __restrict__ div) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < d) div[j] = T((signs[j] < 0 ? -1.0 : 1.0) / double(scale[j]));
}

// out[r][j] = post_j * (H_h (pre o x))_j / sqrt(h) for every row r of M (rows x d),
// block by block; pre / post may be null (ones).  Workgroup = one segment of
// SEG = max(h, BIIP_SEG) entries of one row (whole blocks; entries past d are
// zero and belong to blocks past d, so they never mix into a real entry).
template <typename T>
__global__ __launch_bounds__(256) void fwht_rows_kernel(const T* __restrict__ M, int64_t ldm, int rows, int d, int h,
                                                        int seg, int nseg, const T* __restrict__ pre,
                                                        const T* __restrict__ post, T* __restrict__ out,
                                                        int64_t ldo) {
    __shared__ T x[BIIP_MAX_BLOCK > BIIP_SEG ? BIIP_MAX_BLOCK : BIIP_SEG];
    const int64_t bid = blockIdx.x;
    const int r = int(bid / nseg), c0 = int(bid % nseg) * seg;
    if (r >= rows) return;
    const T* src = M + int64_t(r) * ldm;
    for (int i = threadIdx.x; i < seg; i += 256) {
        const int j = c0 + i;
        x[i] = j < d ? (pre ? pre[j] * src[j] : src[j]) : T(0);
    }
    __syncthreads();
    for (int len = 1; len < h; len *= 2) {
        for (int p = threadIdx.x; p < seg / 2; p += 256) {
            const int i = (p / len) * 2 * len + p % len;
            const T a = x[i], b = x[i + len];
            x[i] = a + b;
            x[i + len] = a - b;
        }
        __syncthreads();
    }
    const T nrm = T(1.0 / sqrt(double(h)));
    T* dst = out + int64_t(r) * ldo;
    for (int i = threadIdx.x; i < seg; i += 256) {
        const int j = c0 + i;
        if (j < d) dst[j] = post ? post[j] * (x[i] * nrm) : x[i] * nrm;
    }
}

// out (cols x rows) = in^T (rows x cols), 32 x 32 tiles through LDS.
template <typename T>
__global__ void transpose_kernel(const T* __restrict__ in, int64_t ldi, int rows, int cols, T* __restrict__ out,
                                 int64_t ldo) {
    __shared__ T t[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    for (int k = threadIdx.y; k < 32; k += blockDim.y) {
        const int r = r0 + k, c = c0 + threadIdx.x;
        if (r < rows && c < cols) t[k][threadIdx.x] = in[int64_t(r) * ldi + c];
    }
    __syncthreads();
    for (int k = threadIdx.y; k < 32; k += blockDim.y) {
        const int c = c0 + k, r = r0 + threadIdx.x;
        if (r < rows && c < cols) out[int64_t(c) * ldo + r] = t[threadIdx.x][k];
    }
}

struct BiipLayout {
    size_t off_T1, off_T2, off_vec, bytes;
};

static BiipLayout biip_layout(kq_dtype dtype, int64_t m, int64_t n) {
    const size_t es = dtype == KQ_F64 ? 8 : 4;
    const int64_t big = std::max(m * n, std::max(m * m, n * n));
    BiipLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    L.off_T1 = take(size_t(big) * es);
    L.off_T2 = take(size_t(big) * es);
    L.off_vec = take(size_t(2 * (m + n)) * es);
    L.bytes = off;
    return L;
}

size_t biip_workspace_bytes(kq_dtype dtype, int64_t m, int64_t n) { return biip_layout(dtype, m, n).bytes; }

template <typename T>
struct BiipRun {
    hipStream_t st;

    kq_status rows(const T* M, int64_t ldm, int64_t nr, int64_t d, const T* pre, const T* post, T* out, int64_t ldo) {
        const int h = hadamard_block(d);
        const int seg = h > BIIP_SEG ? h : BIIP_SEG;
        const int nseg = int((d + seg - 1) / seg);
        hipLaunchKernelGGL(fwht_rows_kernel<T>, dim3(unsigned(nr * nseg)), dim3(256), 0, st, M, ldm, int(nr), int(d),
                           h, seg, nseg, pre, post, out, ldo);
        KQ_LAUNCHED("fwht_rows_kernel");
        return KQ_OK;
    }
    kq_status transpose(const T* in, int64_t ldi, int64_t nr, int64_t nc, T* out, int64_t ldo) {
        hipLaunchKernelGGL(transpose_kernel<T>, dim3(unsigned((nc + 31) / 32), unsigned((nr + 31) / 32)), dim3(32, 8),
                           0, st, in, ldi, int(nr), int(nc), out, ldo);
        KQ_LAUNCHED("transpose_kernel");
        return KQ_OK;
    }
    // out = Q_L diag(preL) (M diag(preR) Q_R^T) for the forward (pre) form, or
    // out = diag(postL) Q_L^T M Q_R diag(postR) for the inverse (post) form;
    // M is nr x nc, T1, T2 scratch of nr * nc.
    kq_status both_sides(const T* M, int64_t ldm, int64_t nr, int64_t nc, const T* preR, const T* preL,
                         const T* postR, const T* postL, T* T1, T* T2, T* out, int64_t ldo) {
        kq_status s = rows(M, ldm, nr, nc, preR, postR, T1, nc);
        if (s != KQ_OK) return s;
        if ((s = transpose(T1, nc, nr, nc, T2, nr)) != KQ_OK) return s;
        if ((s = rows(T2, nr, nc, nr, preL, postL, T1, nr)) != KQ_OK) return s;
        return transpose(T1, nr, nc, nr, out, ldo);
    }
};

template <typename T>
static kq_status biip_forward_typed(int64_t m, int64_t n, const T* W, int64_t ldw, const T* A, int64_t lda,
                                    const T* B, int64_t ldb, const int8_t* sn, const int8_t* sm, T* Wo, int64_t ldwo,
                                    T* Ao, int64_t ldao, T* Bo, int64_t ldbo, T* sa, T* sb, void* ws,
                                    hipStream_t st) {
    const BiipLayout L = biip_layout(sizeof(T) == 8 ? KQ_F64 : KQ_F32, m, n);
    char* base = static_cast<char*>(ws);
    T* T1 = reinterpret_cast<T*>(base + L.off_T1);
    T* T2 = reinterpret_cast<T*>(base + L.off_T2);
    T* mul_a = reinterpret_cast<T*>(base + L.off_vec);
    T* div_a = mul_a + n;
    T* mul_b = div_a + n;
    T* div_b = mul_b + m;
    hipLaunchKernelGGL(biip_vectors_kernel<T>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, A, lda, int(n), sn,
                       sa, mul_a, div_a);
    KQ_LAUNCHED("biip_vectors_kernel");
    hipLaunchKernelGGL(biip_vectors_kernel<T>, dim3(unsigned((m + 255) / 256)), dim3(256), 0, st, B, ldb, int(m), sm,
                       sb, mul_b, div_b);
    KQ_LAUNCHED("biip_vectors_kernel");
    BiipRun<T> run{st};
    kq_status s = run.both_sides(W, ldw, m, n, mul_a, mul_b, nullptr, nullptr, T1, T2, Wo, ldwo);
    if (s != KQ_OK) return s;
    if ((s = run.both_sides(A, lda, n, n, div_a, div_a, nullptr, nullptr, T1, T2, Ao, ldao)) != KQ_OK) return s;
    return run.both_sides(B, ldb, m, m, div_b, div_b, nullptr, nullptr, T1, T2, Bo, ldbo);
}

template <typename T>
static kq_status biip_inverse_typed(int64_t m, int64_t n, const T* V2, int64_t ldv2, const int8_t* sn,
                                    const int8_t* sm, const T* sa, const T* sb, T* V, int64_t ldv, void* ws,
                                    hipStream_t st) {
    const BiipLayout L = biip_layout(sizeof(T) == 8 ? KQ_F64 : KQ_F32, m, n);
    char* base = static_cast<char*>(ws);
    T* T1 = reinterpret_cast<T*>(base + L.off_T1);
    T* T2 = reinterpret_cast<T*>(base + L.off_T2);
    T* div_a = reinterpret_cast<T*>(base + L.off_vec);
    T* div_b = div_a + n;
    // sign_j / s_j from the stored scales (the forward call's s, rounded to T)
    auto fill = [&](const T* s, const int8_t* g, int64_t d, T* out) -> kq_status {
        hipLaunchKernelGGL(biip_div_kernel<T>, dim3(unsigned((d + 255) / 256)), dim3(256), 0, st, s, g, int(d), out);
        KQ_LAUNCHED("biip_div_kernel");
        return KQ_OK;
    };
    kq_status s = fill(sa, sn, n, div_a);
    if (s != KQ_OK) return s;
    if ((s = fill(sb, sm, m, div_b)) != KQ_OK) return s;
    BiipRun<T> run{st};
    return run.both_sides(V2, ldv2, m, n, nullptr, nullptr, div_a, div_b, T1, T2, V, ldv);
}

kq_status biip_forward_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* A,
                                int64_t lda, const void* B, int64_t ldb, const int8_t* sn, const int8_t* sm, void* Wo,
                                int64_t ldwo, void* Ao, int64_t ldao, void* Bo, int64_t ldbo, void* sa, void* sb,
                                void* ws, hipStream_t st) {
    if (dtype == KQ_F64)
        return biip_forward_typed<double>(m, n, static_cast<const double*>(W), ldw, static_cast<const double*>(A), lda,
                                          static_cast<const double*>(B), ldb, sn, sm, static_cast<double*>(Wo), ldwo,
                                          static_cast<double*>(Ao), ldao, static_cast<double*>(Bo), ldbo,
                                          static_cast<double*>(sa), static_cast<double*>(sb), ws, st);
    return biip_forward_typed<float>(m, n, static_cast<const float*>(W), ldw, static_cast<const float*>(A), lda,
                                     static_cast<const float*>(B), ldb, sn, sm, static_cast<float*>(Wo), ldwo,
                                     static_cast<float*>(Ao), ldao, static_cast<float*>(Bo), ldbo,
                                     static_cast<float*>(sa), static_cast<float*>(sb), ws, st);
}

kq_status biip_inverse_dispatch(kq_dtype dtype, int64_t m, int64_t n, const void* V2, int64_t ldv2, const int8_t* sn,
                                const int8_t* sm, const void* sa, const void* sb, void* V, int64_t ldv, void* ws,
                                hipStream_t st) {
    if (dtype == KQ_F64)
        return biip_inverse_typed<double>(m, n, static_cast<const double*>(V2), ldv2, sn, sm,
                                          static_cast<const double*>(sa), static_cast<const double*>(sb),
                                          static_cast<double*>(V), ldv, ws, st);
    return biip_inverse_typed<float>(m, n, static_cast<const float*>(V2), ldv2, sn, sm, static_cast<const float*>(sa),
                                     static_cast<const float*>(sb), static_cast<float*>(V), ldv, ws, st);
}

}  // namespace kq
