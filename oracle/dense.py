"""numpy fp64 oracle tiers for two-sided GPTQ.  TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the bench's CPU-baseline leg may use this
module; the HIP library never does.  Nothing here is blocked, fused or
reordered beyond what the cited passage states: each function is the plain
definition, with numpy's matmul / inv / cholesky as library steps.

Notation (FastKron page, section 2.1): W is m x n (outputs x inputs), A is the
n x n input curvature, B the m x m output curvature, the Hessian of the loss
with respect to vecop(V) is A (x) B, and vecop is the column-major
vectorisation (WaterKron page, section 2 "Notation").  Entry (i, j) of W sits
at vecop index p = i + m*j.

U_A is the upper-triangular factor with positive diagonal and U_A^T U_A =
A_d^{-1}; its transpose is the lower Cholesky factor L^(A) of A_d^{-1} named in
the pith.science review of BaKron ("key_machinery").  The normalised factor
used in the feedback is L~_A[j', j] = U_A[j, j'] / U_A[j, j] (the unit-diagonal
LDL factor, FastKron page section 2.1 "LDL(A)").  This module stores it as
N_A = L~_A^T, i.e. row j of U_A divided by U_A[j, j].
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Factor preparation
# ----------------------------------------------------------------------------


def damp(A: np.ndarray, delta: float) -> np.ndarray:
    """A_d = A + delta * (tr A / d) * I.

    The WaterKron page (section 2, "Notation") assumes PSD factors invertible and
    adds a small damping kappa*I in practice; the reading adopted is kappa =
    delta times the mean diagonal, applied to each Kronecker factor separately.
    """
    A = np.asarray(A, dtype=np.float64)
    d = A.shape[0]
    return A + (delta * np.trace(A) / d) * np.eye(d)


def upper_factor_via_inverse(Ad: np.ndarray) -> np.ndarray:
    """Route (i): U = chol(Ad^{-1})^T, so U is upper with U^T U = Ad^{-1}.

    chol here is the lower Cholesky factor L with L L^T = M (WaterKron page,
    section 2 "Notation"); L^(A) = chol(A^{-1}) is the factor of the BaKron review.
    """
    L = np.linalg.cholesky(np.linalg.inv(np.asarray(Ad, dtype=np.float64)))
    return np.ascontiguousarray(L.T)


def upper_factor_via_reverse_cholesky(Ad: np.ndarray) -> np.ndarray:
    """Route (ii): U = RevCholesky(Ad)^{-T}, with RevCholesky(M) the lower L with
    L^T L = M (WaterKron page, section 2 "Notation").

    RevCholesky(Ad) = J C^T J where C = chol(J Ad J) and J reverses the index
    order; hence U = J C^{-1} J.
    """
    Ad = np.asarray(Ad, dtype=np.float64)
    d = Ad.shape[0]
    J = np.eye(d)[::-1]
    C = np.linalg.cholesky(J @ Ad @ J)
    return np.ascontiguousarray(J @ np.linalg.inv(C) @ J)


def normalized_factor(U: np.ndarray) -> np.ndarray:
    """N[j, j'] = U[j, j'] / U[j, j]: row j of U divided by its diagonal entry.

    N^T is the unit-diagonal LDL factor of Ad^{-1} (FastKron page section 2.1,
    "LDL(A)": the Cholesky factor with columns normalised by their diagonal).
    """
    U = np.asarray(U, dtype=np.float64)
    return U / np.diag(U)[:, None]


# ----------------------------------------------------------------------------
# Base quantizer
# ----------------------------------------------------------------------------


def grid(bits):
    """Symmetric b-bit integer grid [-2^(b-1), 2^(b-1)-1]; bits=None is the
    unbounded integer alphabet of the WaterKron page (section 2.1: the integers
    are not clipped), returned as infinite bounds."""
    if bits is None:
        return -np.inf, np.inf
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1


def scales(W: np.ndarray, bits: int, per_row: bool) -> np.ndarray:
    """s_i = max_j |W_ij| / (2^(b-1) - 1) per output row, or one value per tensor.

    Scales are chosen up front and handed to the algorithm (WaterKron page,
    section 2.4).  Returns an array of length m (per row) or 1 (per tensor).
    """
    W = np.asarray(W)
    _, qmax = grid(bits)
    if per_row:
        return np.max(np.abs(W), axis=1) / qmax
    return np.array([np.max(np.abs(W)) / qmax])


def row_scales(s: np.ndarray, m: int) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64).reshape(-1)
    return np.full(m, s[0]) if s.size == 1 else s.copy()


def entry_scale(s_row, alpha, i: int, j: int) -> float:
    """The grid step of entry (i, j): the row scale, times the column scale
    alpha_j when column scales are given (WaterKron page section 2.1: entry
    (i, j) of V is beta_i alpha_j Z_ij; beta plays the role of the row scale)."""
    return s_row[i] if alpha is None else s_row[i] * alpha[j]


def waterkron_scales(UA, UB, step: float, m: int | None = None):
    """WaterKron two-sided rate allocation (WaterKron page, section 3; section
    2.4 for the one-sided WaterSIC rule): alpha_j proportional to
    1 / L^(A)_jj and beta_i proportional to 1 / L^(B)_ii, with L the reverse
    Cholesky factor of the damped factor.  Since U = RevCholesky(A_d)^{-T} is
    upper triangular, 1 / L_jj = U_jj, so alpha = step * diag(U_A) and beta =
    diag(U_B) (all ones when B = I, which is WaterSIC).  ``step`` is the free
    proportionality constant: the grid step in the transformed geometry.
    Returns (alpha, beta) in fp64."""
    alpha = step * np.diag(np.asarray(UA, dtype=np.float64))
    if UB is None:
        return alpha, np.ones(int(m))
    return alpha, np.diag(np.asarray(UB, dtype=np.float64)).copy()


def empirical_entropy(Z) -> float:
    """Bits per entry of the empirical distribution of the integer codes:
    -sum_k p_k log2 p_k over the distinct values (the storage cost an entropy
    coder approaches, WaterKron page sections 1 and 2.1)."""
    _, counts = np.unique(np.asarray(Z).reshape(-1), return_counts=True)
    p = counts / counts.sum()
    return float(-np.sum(p * np.log2(p)))


def quantize(x: float, s: float, qmin: int, qmax: int) -> tuple[float, float, float]:
    """Closest grid point: z = clamp(rne(x / s)), v = s z.  Returns (z, v, y=x/s).

    The FastKron page (section 2.1) replaces 'round' by a map to the closest
    element of the alphabet; for a clipped uniform grid that is round-to-nearest
    (ties to even) followed by a clamp.  A zero scale (an all-zero row) maps to
    z = 0, v = 0.
    """
    if s == 0.0:
        return 0.0, 0.0, 0.0
    y = x / s
    z = min(max(float(np.rint(y)), qmin), qmax)
    return z, s * z, y


# ----------------------------------------------------------------------------
# Tier O1: literal vectorised GPTQ on the Kronecker Hessian
# ----------------------------------------------------------------------------


def vectorized_kron_gptq(W, Ad, Bd, s, bits, return_factor=False, alpha=None):
    """Standard GPTQ on w^ = vecop(W)^T with Hessian A_d (x) B_d.

    FastKron page, section 2.2: the two-sided extension is Algorithm 1 applied
    to the vectorised weight and 'input' curvature A (x) B.  The GPTQ recurrence
    (Frantar et al.): for p in order, q = quantize(w_p); err = (w_p - q)/U^_pp;
    w_{p+1:} -= err * U^_{p, p+1:}, with U^ the upper Cholesky factor of the
    inverse Hessian.  Equivalently Babai's nearest plane (BaKron / GPTQ-2D
    abstracts).  With column scales ``alpha`` the step of vecop entry p = i + m j
    is s_i alpha_j (WaterKron page section 3: the scale vector of the
    vectorised problem is alpha (x) beta); bits=None leaves the codes unclipped.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    H = np.kron(np.asarray(Ad, dtype=np.float64), np.asarray(Bd, dtype=np.float64))
    Uh = upper_factor_via_inverse(H)
    w = W.reshape(-1, order="F").copy()
    s_row = row_scales(s, m)
    qmin, qmax = grid(bits)
    z = np.zeros(m * n)
    v = np.zeros(m * n)
    y = np.zeros(m * n)
    for p in range(m * n):
        z[p], v[p], y[p] = quantize(w[p], entry_scale(s_row, alpha, p % m, p // m), qmin, qmax)
        err = (w[p] - v[p]) / Uh[p, p]
        w[p + 1:] -= err * Uh[p, p + 1:]
    out = (z.reshape((m, n), order="F"), v.reshape((m, n), order="F"),
           y.reshape((m, n), order="F"))
    return out + (Uh,) if return_factor else out


# ----------------------------------------------------------------------------
# Tier O2: the two-sided loop in matrix form
# ----------------------------------------------------------------------------


def entry_order(m: int, n: int, order: str):
    """Entry sequences that respect the componentwise partial order.

    'column' is vecop order (j outer, i inner); 'row' is i outer; 'antidiagonal'
    visits k = i + j ascending (FastKron page section 2.3, anti-diagonal k),
    rows ascending within a diagonal.
    """
    if order == "column":
        return [(i, j) for j in range(n) for i in range(m)]
    if order == "row":
        return [(i, j) for i in range(m) for j in range(n)]
    if order == "antidiagonal":
        return [(i, k - i) for k in range(m + n - 1)
                for i in range(max(0, k - n + 1), min(k, m - 1) + 1)]
    raise ValueError(order)


def two_sided_naive(W, UA, UB, s, bits, order="column", alpha=None):
    """FastKron-naive written in matrix space (FastKron page, sections 2.2-2.4).

    X := W; for each entry (i, j) in a valid order: quantize x = X[i, j], set
    Delta = v - x and apply the outer-product feedback
    X[i', j'] += L~_B[i', i] * Delta * L~_A[j', j] for i' >= i, j' >= j (the update
    W <- W + L_{:,i}^(B) Delta (L_{:,j}^(A))^T of section 2.4).  Only entries to the
    bottom-right change (section 2.3), so any order that visits (i', j') after
    every (i, j) <= (i', j') gives the same result.

    With column scales ``alpha`` entry (i, j) uses the step s_i alpha_j; with
    bits=None the codes are not clipped (the WaterKron alphabet).

    Returns (Z, V, Y, D): codes, dequantised values, pre-rounding value in grid
    units x/s, and the errors Delta.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    NA, NB = normalized_factor(UA), normalized_factor(UB)
    X = W.copy()
    s_row = row_scales(s, m)
    qmin, qmax = grid(bits)
    Z = np.zeros((m, n)); V = np.zeros((m, n)); Y = np.zeros((m, n)); D = np.zeros((m, n))
    for i, j in entry_order(m, n, order):
        x = X[i, j]
        Z[i, j], V[i, j], Y[i, j] = quantize(x, entry_scale(s_row, alpha, i, j), qmin, qmax)
        D[i, j] = V[i, j] - x
        X[i:, j:] += D[i, j] * np.outer(NB[i, i:], NA[j, j:])
    return Z, V, Y, D


def two_sided_recursive(W, UA, UB, s, bits):
    """FastKron (Algorithm 6 reading): recursion over anti-diagonal ranges.

    FastKron page section 2.5: solve the first half of the anti-diagonals, add
    the propagated errors L~_B antidiag_{k0..mid}(Delta) L~_A^T to the second half,
    solve the second half.  A leaf is a single anti-diagonal whose entries are
    independent (section 2.3).  Anti-diagonals here are 0-based, k = i + j.
    The propagation uses dense products of the full factors: it is the
    definition of the batched update, not an efficient schedule.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    LA, LB = normalized_factor(UA).T, normalized_factor(UB).T
    X = W.copy()
    s_row = row_scales(s, m)
    qmin, qmax = grid(bits)
    Z = np.zeros((m, n)); V = np.zeros((m, n)); Y = np.zeros((m, n)); D = np.zeros((m, n))
    kidx = np.add.outer(np.arange(m), np.arange(n))

    def solve(k0, k1):
        if k1 - k0 == 1:
            for i in range(max(0, k0 - n + 1), min(k0, m - 1) + 1):
                j = k0 - i
                Z[i, j], V[i, j], Y[i, j] = quantize(X[i, j], s_row[i], qmin, qmax)
                D[i, j] = V[i, j] - X[i, j]
            return
        mid = (k0 + k1) // 2
        solve(k0, mid)
        src = np.where((kidx >= k0) & (kidx < mid), D, 0.0)
        upd = LB @ src @ LA.T
        tgt = (kidx >= mid) & (kidx < k1)
        X[tgt] += upd[tgt]
        solve(mid, k1)

    solve(0, m + n - 1)
    return Z, V, Y, D


def two_sided_recursive_vecop(W, UA, UB, s, bits):
    """FastKron-recursive reading: lazy batched updates over the vecop sequence.

    FastKron page section 2.4: solve the first half of the entry sequence,
    propagate its errors to the second half with one batched update
    L~_B Delta L~_A^T, then solve the second half; no anti-diagonal batching.
    The sequence is vecop (column-major) order; block sizes halve recursively.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    LA, LB = normalized_factor(UA).T, normalized_factor(UB).T
    X = W.copy()
    s_row = row_scales(s, m)
    qmin, qmax = grid(bits)
    Z = np.zeros((m, n)); V = np.zeros((m, n)); Y = np.zeros((m, n)); D = np.zeros((m, n))
    pidx = np.add.outer(np.arange(m), m * np.arange(n))

    def solve(p0, p1):
        if p1 - p0 == 1:
            i, j = p0 % m, p0 // m
            Z[i, j], V[i, j], Y[i, j] = quantize(X[i, j], s_row[i], qmin, qmax)
            D[i, j] = V[i, j] - X[i, j]
            return
        mid = (p0 + p1) // 2
        solve(p0, mid)
        src = np.where((pidx >= p0) & (pidx < mid), D, 0.0)
        upd = LB @ src @ LA.T
        tgt = (pidx >= mid) & (pidx < p1)
        X[tgt] += upd[tgt]
        solve(mid, p1)

    solve(0, m * n)
    return Z, V, Y, D


def one_sided_gptq(W, UA, s, bits, alpha=None):
    """Standard one-sided GPTQ (Frantar et al.), Hessian A (x) I_m.

    Columns in order: q = quantize(W[:, j]) row-wise, err = (W[:, j] - q) / U[j, j],
    W[:, j+1:] -= err U[j, j+1:] (FastKron page section 2.2, Algorithm 1's
    recurrence; U the upper Cholesky factor of A^{-1}).  Column scales ``alpha``
    give entry (i, j) the step s_i alpha_j (WaterSIC, WaterKron page section 2.4,
    when alpha_j is proportional to U[j, j]); bits=None does not clip.
    """
    Wc = np.asarray(W, dtype=np.float64).copy()
    m, n = Wc.shape
    s_row = row_scales(s, m)
    qmin, qmax = grid(bits)
    Z = np.zeros((m, n)); V = np.zeros((m, n))
    for j in range(n):
        for i in range(m):
            Z[i, j], V[i, j], _ = quantize(Wc[i, j], entry_scale(s_row, alpha, i, j), qmin, qmax)
        err = (Wc[:, j] - V[:, j]) / UA[j, j]
        Wc[:, j + 1:] -= np.outer(err, UA[j, j + 1:])
    return Z, V


# ----------------------------------------------------------------------------
# Loss, factors, scores
# ----------------------------------------------------------------------------


def proxy_loss(W, V, Ad, Bd) -> float:
    """D_{A,B} = tr(B (V - W) A (V - W)^T) = ||(B^{1/2})^T (V-W) A^{1/2}||_F^2.

    WaterKron page section 1 item 1 (with S S^T = M for M^{1/2}); the FastKron
    page section 2.2 writes the same loss for symmetric roots.
    """
    E = np.asarray(V, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    return float(np.trace(np.asarray(Bd) @ E @ np.asarray(Ad) @ E.T))


def loss_from_errors(D, UA, UB) -> float:
    """sum_ij (Delta_ij / (U_B[i,i] U_A[j,j]))^2: the loss through the identity
    V - W = L~_B Delta L~_A^T and L~ = U^T diag(U)^{-1}."""
    dA = np.diag(np.asarray(UA, dtype=np.float64))
    dB = np.diag(np.asarray(UB, dtype=np.float64))
    return float(np.sum((np.asarray(D) / np.outer(dB, dA)) ** 2))


def factor_accumulate(X, S=None, alpha=1.0, beta=0.0):
    """S <- beta S + alpha X^T X for samples stored as rows of X.

    With alpha = 1/N this is the K-FAC / 'Marginal' factor A = E[a a^T] over N
    activation rows (FastKron page section 3.2 and section 2.6's accumulation of
    the Hessian from the calibration data); the same for gradient rows gives B.
    """
    X = np.asarray(X, dtype=np.float64)
    G = alpha * (X.T @ X)
    if S is None or beta == 0.0:
        return G
    return beta * np.asarray(S, dtype=np.float64) + G


def sensitivity(A, B) -> float:
    """KronQ sublayer score tr(A) * tr(B) (KronQ page, mixed-precision allocation)."""
    return float(np.trace(A) * np.trace(B))


def prepare(A, delta):
    """Damped factor and its upper factor: (A_d, U) with U^T U = A_d^{-1}."""
    Ad = damp(A, delta)
    return Ad, upper_factor_via_inverse(Ad)


# ----------------------------------------------------------------------------
# Kronecker approximations of H = E[a a^T (x) b b^T] from paired samples
# ----------------------------------------------------------------------------


def kronecker_hessian(Xa, Xb) -> np.ndarray:
    """H = (1/N) sum_s (a_s a_s^T) (x) (b_s b_s^T) for paired sample rows a_s of
    Xa (N x n) and b_s of Xb (N x m): the mn x mn Hessian that the Kronecker
    approximations target (WaterKron page Table 1; FastKron page section 3.2).
    Only for tiny n, m (it is formed explicitly)."""
    Xa = np.asarray(Xa, dtype=np.float64)
    Xb = np.asarray(Xb, dtype=np.float64)
    H = np.zeros((Xa.shape[1] * Xb.shape[1],) * 2)
    for a, b in zip(Xa, Xb):
        H += np.kron(np.outer(a, a), np.outer(b, b))
    return H / len(Xa)


def kronecker_factors(Xa, Xb, method: str, iters: int, delta: float = 0.0):
    """Alternating fixed-point iteration for H ~ A (x) B, from B_0 = I (WaterKron
    page section 5 and Table 1; FastKron page section 3.2).

    'flipflop' -- the flip-flop maximum-likelihood iteration for the matrix
      normal model (Dutilleul, cited on the WaterKron page) with the per-sample
      matrices G_s = b_s a_s^T, so that vecop(G_s) vecop(G_s)^T = a a^T (x) b b^T:
        A_{k+1} = (1/(N m)) sum_s (b_s^T B_k^{-1} b_s) a_s a_s^T
        B_{k+1} = (1/(N n)) sum_s (a_s^T A_{k+1}^{-1} a_s) b_s b_s^T
    'frobenius' -- the same iteration with A_{k+1}^{-1}, B_k^{-1} replaced by
      A_{k+1}, B_k, normalised so that each half-step is the exact minimiser of
      ||H - A (x) B||_F over one factor (the WaterKron page's power iteration):
        A_{k+1} = sum_s (b_s^T B_k b_s) a_s a_s^T / (N ||B_k||_F^2)
        B_{k+1} = sum_s (a_s^T A_{k+1} a_s) b_s b_s^T / (N ||A_{k+1}||_F^2)
    The inverses use the damped factors M + delta tr(M)/d I (delta = 0: none),
    the damping the WaterKron page adds to make PSD factors invertible.
    ``iters`` full updates (A, then B).  Returns (A, B) in fp64.
    """
    Xa = np.asarray(Xa, dtype=np.float64)
    Xb = np.asarray(Xb, dtype=np.float64)
    N, n = Xa.shape
    m = Xb.shape[1]
    B = np.eye(m)
    A = None
    def quad(X, M):  # x_s^T M x_s for every row x_s of X
        return np.sum((X @ M) * X, axis=1)

    for _ in range(iters):
        if method == "flipflop":
            w = quad(Xb, np.linalg.inv(damp(B, delta)))
            A = (Xa.T * w) @ Xa / (N * m)
            v = quad(Xa, np.linalg.inv(damp(A, delta)))
            B = (Xb.T * v) @ Xb / (N * n)
        elif method == "frobenius":
            w = quad(Xb, B)
            A = (Xa.T * w) @ Xa / (N * np.sum(B * B))
            v = quad(Xa, A)
            B = (Xb.T * v) @ Xb / (N * np.sum(A * A))
        else:
            raise ValueError(method)
    return A, B


def mismatch_factor(H, A, B) -> float:
    """Phi = tr(H (A (x) B)^{-1}) / (m n): the distortion penalty of the
    Kronecker approximation (WaterKron page, section 4)."""
    K = np.kron(np.asarray(A, dtype=np.float64), np.asarray(B, dtype=np.float64))
    return float(np.trace(np.linalg.solve(K, np.asarray(H, dtype=np.float64))) / len(K))


# ----------------------------------------------------------------------------
# KronQ bidirectional incoherence processing (BiIP)
# ----------------------------------------------------------------------------

BIIP_MAX_BLOCK = 4096


def hadamard_block(d: int, max_block: int = BIIP_MAX_BLOCK) -> int:
    """Walsh-Hadamard block size for dimension d: the largest power of two that
    divides d, at most max_block (a d that is not a power of two gets a
    block-diagonal transform, which is still orthogonal)."""
    return min(d & -d, max_block)


def biip_rotation(d: int, signs, max_block: int = BIIP_MAX_BLOCK) -> np.ndarray:
    """Q = (I_{d/h} (x) H_h / sqrt(h)) diag(signs), H_h the Sylvester
    Walsh-Hadamard matrix (H_2 = [[1, 1], [1, -1]], the KronQ page's 2 x 2
    example) and signs a +-1 vector (the randomised Hadamard transform)."""
    from scipy.linalg import hadamard
    h = hadamard_block(d, max_block)
    H = hadamard(h).astype(np.float64) / np.sqrt(h)
    return np.kron(np.eye(d // h), H) * np.asarray(signs, dtype=np.float64)[None, :]


def biip_scales(M) -> np.ndarray:
    """diag(M)^{-1/4} (KronQ page, BiIP: S_X = diag(H_X)^{-1/4}, S_G likewise);
    1 where a diagonal entry is not positive."""
    d = np.diag(np.asarray(M, dtype=np.float64))
    return np.where(d > 0, np.abs(d) ** -0.25, 1.0)


def biip_forward(W, A, B, signs_n, signs_m):
    """KronQ BiIP (KronQ page, section "Kronecker-Factored Quantization"):
    rescale W' = S_B W S_A with S = diag^{-1/4} of each factor, and the factors
    by the inverse scales (A' = S_A^{-1} A S_A^{-1}, B' likewise), so that the
    loss tr(B E A E^T) is unchanged; then rotate both sides, W'' = Q_B W' Q_A^T,
    A'' = Q_A A' Q_A^T, B'' = Q_B B' Q_B^T (Theorem 1: invariance under
    orthogonal Q_A, Q_B).  W is m x n, A n x n (H_X), B m x m (H_G).
    Returns (W'', A'', B'', s_A, s_B)."""
    W = np.asarray(W, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    m, n = W.shape
    sa, sb = biip_scales(A), biip_scales(B)
    Qa, Qb = biip_rotation(n, signs_n), biip_rotation(m, signs_m)
    W2 = Qb @ (sb[:, None] * W * sa[None, :]) @ Qa.T
    A2 = Qa @ (A / np.outer(sa, sa)) @ Qa.T
    B2 = Qb @ (B / np.outer(sb, sb)) @ Qb.T
    return W2, A2, B2, sa, sb


def biip_inverse(V2, signs_n, signs_m, sa, sb):
    """Back to the original coordinates: V = S_B^{-1} Q_B^T V'' Q_A S_A^{-1}."""
    V2 = np.asarray(V2, dtype=np.float64)
    m, n = V2.shape
    Qa, Qb = biip_rotation(n, signs_n), biip_rotation(m, signs_m)
    return (Qb.T @ V2 @ Qa) / np.asarray(sb)[:, None] / np.asarray(sa)[None, :]
