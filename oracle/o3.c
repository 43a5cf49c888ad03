/*
 * Tier O3 of the CPU oracle: the left-looking cubic two-sided GPTQ loop.
 * TEST INFRASTRUCTURE ONLY -- linked by the tests and the CPU-baseline leg of
 * the bench through oracle/o3.py; never by the HIP library.
 *
 * What it computes (FastKron page, sections 2.2-2.5): the same codes as GPTQ on
 * vecop(W) with Hessian A (x) B.  Entries are visited anti-diagonal by
 * anti-diagonal (k = i + j ascending; entries of one anti-diagonal do not
 * depend on each other, section 2.3), and each entry pulls the feedback of all
 * entries to its top-left when it is reached:
 *
 *   x_ij   = W_ij + sum_{i'<i} Lb[i][i'] R[i'][j] + sum_{j'<j} D[i][j'] La[j][j']
 *   z_ij   = clamp(rne(x_ij / s_i), -2^(b-1), 2^(b-1)-1),  v_ij = s_i z_ij
 *   D[i][j] = v_ij - x_ij
 *   R[i][j] = sum_{j'<=j} D[i][j'] La[j][j']
 *
 * Lb = L~_B and La = L~_A are the unit lower-triangular normalised factors
 * (L~[r][c] = U[c][r] / U[c][c]).  Expanding the outer-product feedback
 * X[i'][j'] += L~_B[i'][i] D_ij L~_A[j'][j] of section 2.4 and summing it over
 * all earlier entries gives exactly the two sums above, so this loop performs
 * m n (m + n - 2) / 2 multiply-adds in total.
 *
 * Grid step of entry (i, j): s_row[i], or s_row[i] * s_col[j] when column
 * scales are given (the per-entry steps beta_i alpha_j of the WaterKron page,
 * section 2.1).  Codes are clipped to [qmin, qmax] when `bounded` is nonzero;
 * otherwise they are unbounded integers (WaterKron page section 2.1).
 *
 * Build: compiled twice, with -DREAL=double (o3_f64) and -DREAL=float (o3_f32,
 * the fp32-arithmetic variant used to measure the oracle's own fp32 floor).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

#ifndef REAL
#define REAL double
#endif

#define NOT_FORCED INT32_MIN

static void quantize(REAL x, REAL s, int bounded, int qmin, int qmax, REAL* z, REAL* v, double* y) {
    if (s == (REAL)0) { *z = 0; *v = 0; *y = 0.0; return; }
    REAL t = x / s;                 /* IEEE division, no reciprocal */
    REAL r = rint(t);               /* default rounding mode: half to even */
    if (bounded) {
        if (r < (REAL)qmin) r = (REAL)qmin;
        if (r > (REAL)qmax) r = (REAL)qmax;
    }
    *z = r; *v = s * r; *y = (double)t;
}

/*
 * m x n problem, all matrices row-major and contiguous.
 *   W[m*n], Lb[m*m] (NULL means B = I), La[n*n], s_row[m], s_col[n] (NULL: none)
 *   force[m*n] (NULL, or NOT_FORCED except where the code is imposed)
 * Outputs: Z[m*n] codes (int32), V[m*n], Y[m*n] pre-rounding value in grid units,
 *          D[m*n] errors.  Returns 0, or -1 if the scratch row buffer cannot
 *          be allocated.
 */
int o3_solve(int64_t m, int64_t n, const REAL* W, const REAL* Lb, const REAL* La,
             const REAL* s_row, const REAL* s_col, int bits, const int32_t* force, int32_t* Z,
             REAL* V, double* Y, REAL* D, int threads) {
    const int bounded = bits > 0;
    const int qmin = bounded ? -(1 << (bits - 1)) : 0, qmax = bounded ? (1 << (bits - 1)) - 1 : 0;
    /* R stored transposed, Rt[j][i], so the column sum reads contiguously. */
    REAL* Rt = (REAL*)malloc(sizeof(REAL) * (size_t)m * (size_t)n);
    if (!Rt) return -1;
    if (threads > 0) omp_set_num_threads(threads);
    for (int64_t k = 0; k < m + n - 1; ++k) {
        const int64_t i0 = k - n + 1 > 0 ? k - n + 1 : 0;
        const int64_t i1 = k < m - 1 ? k : m - 1;
#pragma omp parallel for schedule(static)
        for (int64_t i = i0; i <= i1; ++i) {
            const int64_t j = k - i;
            REAL col = 0, row = 0;
            if (Lb) {
                const REAL* lb = Lb + i * m;
                const REAL* rt = Rt + j * m;
#pragma omp simd reduction(+ : col)
                for (int64_t a = 0; a < i; ++a) col += lb[a] * rt[a];
            }
            const REAL* d = D + i * n;
            const REAL* la = La + j * n;
#pragma omp simd reduction(+ : row)
            for (int64_t b = 0; b < j; ++b) row += d[b] * la[b];
            const REAL x = W[i * n + j] + col + row;
            REAL z, v; double y;
            const REAL sij = s_col ? s_row[i] * s_col[j] : s_row[i];
            quantize(x, sij, bounded, qmin, qmax, &z, &v, &y);
            if (force && force[i * n + j] != NOT_FORCED) { z = (REAL)force[i * n + j]; v = sij * z; }
            Z[i * n + j] = (int32_t)z;
            V[i * n + j] = v;
            Y[i * n + j] = y;
            D[i * n + j] = v - x;
            Rt[j * m + i] = row + D[i * n + j];
        }
    }
    free(Rt);
    return 0;
}
