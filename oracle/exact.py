"""Tier O0: two-sided GPTQ in exact rational arithmetic.  TEST INFRASTRUCTURE ONLY.

Every quantity is a ``fractions.Fraction``: the damped factors, their inverses,
the unit-diagonal LDL factor of the inverse (no square root is needed: the
feedback only uses L~ = U^T diag(U)^{-1}), the pre-rounding values and the
round-half-to-even decision.  The equivalence theorem of the FastKron page
(section 2.5: FastKron-naive, -antidiagonal, -recursive and FastKron give the
same outputs on the same inputs) holds exactly here, so every order below must
return identical codes.  Sizes are kept to a few entries per side.
"""
from __future__ import annotations

from fractions import Fraction as Fr

import numpy as np


def to_fr(M) -> list[list[Fr]]:
    return [[Fr(x) for x in row] for row in np.asarray(M, dtype=object).tolist()]


def eye(d):
    return [[Fr(int(i == j)) for j in range(d)] for i in range(d)]


def matmul(A, B):
    n, k, m = len(A), len(B), len(B[0])
    return [[sum((A[i][t] * B[t][j] for t in range(k)), Fr(0)) for j in range(m)] for i in range(n)]


def transpose(A):
    return [list(r) for r in zip(*A)]


def damp(A, delta: Fr):
    """A_d = A + delta * (tr A / d) * I (relative damping of each factor)."""
    d = len(A)
    lam = delta * sum((A[i][i] for i in range(d)), Fr(0)) / d
    return [[A[i][j] + (lam if i == j else 0) for j in range(d)] for i in range(d)]


def inverse(A):
    """Gauss-Jordan elimination with exact pivots."""
    d = len(A)
    M = [list(A[i]) + eye(d)[i] for i in range(d)]
    for c in range(d):
        p = next(r for r in range(c, d) if M[r][c] != 0)
        M[c], M[p] = M[p], M[c]
        piv = M[c][c]
        M[c] = [x / piv for x in M[c]]
        for r in range(d):
            if r != c and M[r][c] != 0:
                f = M[r][c]
                M[r] = [a - f * b for a, b in zip(M[r], M[c])]
    return [row[d:] for row in M]


def ldl(M):
    """M = L D L^T with L unit lower triangular and D diagonal (exact, no sqrt)."""
    d = len(M)
    L = eye(d)
    D = [Fr(0)] * d
    for j in range(d):
        D[j] = M[j][j] - sum((L[j][k] ** 2 * D[k] for k in range(j)), Fr(0))
        for i in range(j + 1, d):
            L[i][j] = (M[i][j] - sum((L[i][k] * L[j][k] * D[k] for k in range(j)), Fr(0))) / D[j]
    return L, D


def normalized_factor(Ad):
    """(N, u2): N = L~^T with L~ the unit LDL factor of Ad^{-1}, and u2[j] = U[j,j]^2.

    With U^T U = Ad^{-1} (U upper), Ad^{-1} = L~ diag(U_jj^2) L~^T, so N[j, j'] =
    U[j, j'] / U[j, j] exactly as in the floating-point tiers.
    """
    L, D = ldl(inverse(Ad))
    return transpose(L), D


def rne(y: Fr) -> int:
    """Round half to even on an exact rational."""
    f = y.numerator // y.denominator
    r = y - f
    if r > Fr(1, 2):
        return f + 1
    if r < Fr(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def quantize(x: Fr, s: Fr, qmin: int, qmax: int):
    if s == 0:
        return 0, Fr(0)
    z = min(max(rne(x / s), qmin), qmax)
    return z, s * z


def _orders(m, n, order):
    if order == "column":
        return [(i, j) for j in range(n) for i in range(m)]
    if order == "row":
        return [(i, j) for i in range(m) for j in range(n)]
    if order == "antidiagonal":
        return [(i, k - i) for k in range(m + n - 1) for i in range(max(0, k - n + 1), min(k, m - 1) + 1)]
    raise ValueError(order)


def naive(W, NA, NB, s, bits, order="column"):
    """Right-looking outer-product feedback, X[i',j'] += L~_B[i',i] Delta L~_A[j',j]."""
    m, n = len(W), len(W[0])
    qmin, qmax = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    X = [list(r) for r in W]
    Z = [[0] * n for _ in range(m)]
    D = [[Fr(0)] * n for _ in range(m)]
    for i, j in _orders(m, n, order):
        Z[i][j], v = quantize(X[i][j], s[i], qmin, qmax)
        D[i][j] = v - X[i][j]
        for a in range(i, m):
            for b in range(j, n):
                X[a][b] += NB[i][a] * D[i][j] * NA[j][b]
    return Z, D


def left_looking(W, NA, NB, s, bits):
    """Anti-diagonal order, each entry pulling its feedback when it is reached:
    x_ij = W_ij + sum_{i'<i} L~_B[i,i'] R[i',j] + sum_{j'<j} Delta[i,j'] L~_A[j,j'],
    R[i,j] = sum_{j'<=j} Delta[i,j'] L~_A[j,j'] (the row-accumulated error)."""
    m, n = len(W), len(W[0])
    qmin, qmax = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    Z = [[0] * n for _ in range(m)]
    D = [[Fr(0)] * n for _ in range(m)]
    R = [[Fr(0)] * n for _ in range(m)]
    for k in range(m + n - 1):
        for i in range(max(0, k - n + 1), min(k, m - 1) + 1):
            j = k - i
            row = sum((D[i][b] * NA[b][j] for b in range(j)), Fr(0))
            col = sum((NB[a][i] * R[a][j] for a in range(i)), Fr(0))
            x = W[i][j] + col + row
            Z[i][j], v = quantize(x, s[i], qmin, qmax)
            D[i][j] = v - x
            R[i][j] = row + D[i][j]
    return Z, D


def _band_update(X, D, NA, NB, src, tgt):
    """X[t] += (L~_B Delta_src L~_A^T)[t] for entries t in tgt."""
    m, n = len(X), len(X[0])
    S = [[D[i][j] if src(i, j) else Fr(0) for j in range(n)] for i in range(m)]
    LB = transpose(NB)
    U = matmul(matmul(LB, S), NA)
    for i in range(m):
        for j in range(n):
            if tgt(i, j):
                X[i][j] += U[i][j]


def recursive(W, NA, NB, s, bits, over="antidiagonal"):
    """Recursive halving of the processing sequence with batched propagation.

    over='antidiagonal' is FastKron (anti-diagonal ranges, FastKron page section
    2.5); over='vecop' halves the column-major entry sequence (the FastKron-recursive
    reading of section 2.4).
    """
    m, n = len(W), len(W[0])
    qmin, qmax = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    X = [list(r) for r in W]
    Z = [[0] * n for _ in range(m)]
    D = [[Fr(0)] * n for _ in range(m)]
    key = (lambda i, j: i + j) if over == "antidiagonal" else (lambda i, j: i + m * j)
    total = m + n - 1 if over == "antidiagonal" else m * n

    def solve(k0, k1):
        if k1 - k0 == 1:
            for i in range(m):
                for j in range(n):
                    if key(i, j) == k0:
                        Z[i][j], v = quantize(X[i][j], s[i], qmin, qmax)
                        D[i][j] = v - X[i][j]
            return
        mid = (k0 + k1) // 2
        solve(k0, mid)
        _band_update(X, D, NA, NB, lambda i, j: k0 <= key(i, j) < mid,
                     lambda i, j: mid <= key(i, j) < k1)
        solve(mid, k1)

    solve(0, total)
    return Z, D


def loss(W, V, Ad, Bd) -> Fr:
    """tr(B_d (V - W) A_d (V - W)^T) exactly."""
    E = [[V[i][j] - W[i][j] for j in range(len(W[0]))] for i in range(len(W))]
    P = matmul(matmul(matmul(Bd, E), Ad), transpose(E))
    return sum((P[i][i] for i in range(len(P))), Fr(0))
