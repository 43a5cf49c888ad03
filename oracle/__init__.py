"""CPU oracle for two-sided (Kronecker-factored) GPTQ -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or link anything in this package.  The product
path (the HIP library and its Python binding) never touches it, and this
package shares no code with the product path.

Contents, all in IEEE fp64 unless a function says otherwise:

* ``dense``  -- numpy tiers: damping, the two factor routes, the normalised
  factor, scales, the literal vectorised GPTQ on the Kronecker Hessian (tier
  O1), the entry-by-entry two-sided loop in two orders (tier O2), the
  recursive split over anti-diagonal ranges, one-sided GPTQ, the proxy loss
  and the K-FAC factor accumulation.
* ``exact``  -- tier O0: the same loops in exact rational arithmetic.
* ``o3``     -- tier O3: the left-looking cubic loop in plain C with OpenMP
  (``o3.c``), used for large shapes and as the timed CPU baseline.
* ``compare`` -- the parity comparator (code equality with the near-tie rule,
  mismatch fraction, loss relative error).

Sources are the pages on two-sided GPTQ: "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (section 2: notation, FastKron-naive,
FastKron-antidiagonal, FastKron-recursive, FastKron), "WaterKron and FlipFlop
Hessian" (section 2 notation; section 3's corollary proofs), the BaKron /
GPTQ-2D abstracts and the pith.science review of BaKron.

Parity pins: every function here is pinned by a test in ``tests/test_oracle_*.py``
against something other than itself (the printed Kronecker example, closed
forms, textbook special cases, exact rational agreement across orders).  The
absolute rounding output on general inputs is pinned only through those
cross-tier agreements and invariants: the pages print no worked two-sided
rounding example.
"""
