"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and arranges them into the shapes of the
workloads; it holds none of the quantization method's arithmetic (no factor
products, no damping, no Cholesky, no rounding).  Every generator uses numpy's
``Generator(PCG64(seed))`` with ``seed = 1000*config + role`` (and, for the
transformer-block workload, ``seed = 5000 + 100*sublayer + role``), so both the
CPU oracle and the GPU path receive bit-identical fp64 draws.

Roles: 1 = W, 2 = outlier mask, 3 = activation rows, 4 = activation channel
scales, 5 = gradient rows, 6 = gradient channel scales, 7 = Q_A, 8 = Q_B.

Workloads (weight matrix W is m x n = outputs x inputs; A is n x n built from
input activations, B is m x m built from output gradients):

* ``tiny``   32 x 32, W ~ N(0,1); activation samples 256 x n and gradient
  samples 256 x m, i.i.d. N(0,1); 4-bit grid with one scale for the tensor.
* ``spectral`` 256 x 256, W ~ N(0,1); A and B given directly as
  Q diag(k^-1.5) Q^T, k = 1..d, Q Haar-orthogonal (QR of a Gaussian matrix with
  the signs of R's diagonal folded into Q); 3-bit grid, one scale per row.
* ``llm`` m x n (4096 x 4096, 1024 x 4096, 14336 x 4096, 4096 x 14336):
  W = 0.02 N(0,1) with exactly round(0.001 m n) entries, drawn without
  replacement, multiplied by 10; 4096 activation rows x_rc = z_rc sigma_c and
  4096 gradient rows of the same recipe, sigma_c = exp(N(0,1)) per channel.
"""
from __future__ import annotations

import numpy as np

ROLE_W, ROLE_MASK, ROLE_ACT, ROLE_ACT_SCALE, ROLE_GRAD, ROLE_GRAD_SCALE, ROLE_QA, ROLE_QB = range(1, 9)

# Llama-3-8B block sublayers in the order used for seeding.
BLOCK_SUBLAYERS = (
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336),
)
# Sublayers that read the same hidden input share one activation factor A:
# the index of the sublayer whose seeds draw that shared A.
BLOCK_A_OWNER = {"q": 0, "k": 0, "v": 0, "o": 3, "gate": 4, "up": 4, "down": 6}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def gaussian(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    return rng(seed).standard_normal(shape) * scale


def haar_orthogonal(seed: int, d: int) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian, signs fixed by diag(R)."""
    g = rng(seed).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def spectral_spd(seed: int, d: int, power: float = -1.5) -> np.ndarray:
    """Q diag(k^power) Q^T for k = 1..d (an input recipe, not a step of the method)."""
    q = haar_orthogonal(seed, d)
    lam = np.arange(1, d + 1, dtype=np.float64) ** power
    a = (q * lam[None, :]) @ q.T
    return 0.5 * (a + a.T)


def heavy_weight(seed_w: int, seed_mask: int, m: int, n: int) -> np.ndarray:
    """0.02 N(0,1) with exactly round(0.001 m n) entries (no replacement) scaled by 10."""
    w = gaussian(seed_w, (m, n), 0.02)
    k = int(round(0.001 * m * n))
    idx = rng(seed_mask).choice(m * n, size=k, replace=False)
    w.reshape(-1)[idx] *= 10.0
    return w


def channel_scaled_rows(seed_rows: int, seed_scales: int, rows: int, dim: int) -> np.ndarray:
    """rows x dim samples x_rc = z_rc * sigma_c with sigma_c = exp(N(0,1))."""
    sigma = np.exp(rng(seed_scales).standard_normal(dim))
    return rng(seed_rows).standard_normal((rows, dim)) * sigma[None, :]


# ----------------------------------------------------------------------------
# Workload bundles.  Each returns a dict of fp64 numpy arrays plus metadata.
# 'act' / 'grad' are sample matrices whose Gram X^T X / rows gives A / B;
# 'A' / 'B' are given directly only by the spectral workload.
# ----------------------------------------------------------------------------

def tiny(m: int = 32, n: int = 32, samples: int = 256, config: int = 1) -> dict:
    base = 1000 * config
    return dict(
        name=f"tiny {m}x{n}", m=m, n=n, bits=4, per_row=False, damp=0.01,
        W=gaussian(base + ROLE_W, (m, n)),
        act=gaussian(base + ROLE_ACT, (samples, n)),
        grad=gaussian(base + ROLE_GRAD, (samples, m)),
    )


def spectral(m: int = 256, n: int = 256, config: int = 2) -> dict:
    base = 1000 * config
    return dict(
        name=f"spectral {m}x{n}", m=m, n=n, bits=3, per_row=True, damp=0.01,
        W=gaussian(base + ROLE_W, (m, n)),
        A=spectral_spd(base + ROLE_QA, n),
        B=spectral_spd(base + ROLE_QB, m),
    )


def llm(m: int, n: int, bits: int, config: int, rows: int = 4096) -> dict:
    base = 1000 * config
    return dict(
        name=f"llm {m}x{n}", m=m, n=n, bits=bits, per_row=True, damp=0.01,
        W=heavy_weight(base + ROLE_W, base + ROLE_MASK, m, n),
        act=channel_scaled_rows(base + ROLE_ACT, base + ROLE_ACT_SCALE, rows, n),
        grad=channel_scaled_rows(base + ROLE_GRAD, base + ROLE_GRAD_SCALE, rows, m),
    )


def block_sublayer(index: int, rows: int = 4096, bits: int = 2) -> dict:
    """One sublayer of the Llama-3-8B-shaped block (q, k, v, o, gate, up, down)."""
    name, m, n = BLOCK_SUBLAYERS[index]
    base = 5000 + 100 * index
    owner = 5000 + 100 * BLOCK_A_OWNER[name]
    return dict(
        name=f"block.{name} {m}x{n}", m=m, n=n, bits=bits, per_row=True, damp=0.01,
        W=heavy_weight(base + ROLE_W, base + ROLE_MASK, m, n),
        act=channel_scaled_rows(owner + ROLE_ACT, owner + ROLE_ACT_SCALE, rows, n),
        grad=channel_scaled_rows(base + ROLE_GRAD, base + ROLE_GRAD_SCALE, rows, m),
        a_owner=BLOCK_A_OWNER[name],
    )


def small_integer_problem(seed: int, m: int, n: int, samples: int = 4, span: int = 3) -> dict:
    """Integer-valued draws for exact rational runs: W entries in [-span*4, span*4],
    activation / gradient samples in [-span, span]."""
    g = rng(seed)
    return dict(
        m=m, n=n,
        W=g.integers(-4 * span, 4 * span + 1, size=(m, n)),
        act=g.integers(-span, span + 1, size=(samples + n, n)),
        grad=g.integers(-span, span + 1, size=(samples + m, m)),
    )
