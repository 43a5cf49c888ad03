"""One layer through the whole path on the GPU: factor accumulation, damped
factors, scales, two-sided GPTQ and the proxy loss.  Every step is a call into
libkronq; this module only allocates device tensors and chains the calls.

Order of the steps (FastKron page, section 2.6: accumulate the Hessian factors
from the calibration data, factor them, run the core algorithm):
    A = E[a a^T] = X_a^T X_a / N,  B = E[g g^T] = X_g^T X_g / N
    U_A, U_B with U^T U = (factor + damp_rel tr/d I)^{-1}
    s = max |W_row| / (2^(bits-1) - 1)
    codes, V = two-sided GPTQ(W, U_A, U_B, s)
    loss = tr(B_d (V - W) A_d (V - W)^T)

The layer's loss comes from the solver's own rounding errors (kron_quantize's
loss output, the error-feedback form of the same trace); with check_loss=True
kron_loss also recomputes it from W and V alone, in fp64.

The two factor chains (accumulate, then prepare) are independent until the
solver needs both, and a prepare is a long chain of small dependent launches
(one diagonal block per step).  quantize_layer therefore runs the B chain on a
second stream, started once the A product is done, so that it fills the device
beside the A chain; the solver waits for both.

quantize_layers takes a sequence of layers (a model block, quantized one layer
after another) and pipelines them: the factor chains of layer k + 1 run on the
two side streams while layer k is solved on the caller's stream.  The solver's
leaves occupy at most one workgroup per tile of a tile-diagonal, so the
latency-bound prepare chains find free compute units beside them.
"""
from __future__ import annotations

import torch

from . import (KQ_OP_LOSS, KQ_OP_PREPARE, KQ_OP_QUANTIZE, KronError, kron_factor_accumulate, kron_loss,
               kron_prepare, kron_quantize, kron_row_scales, workspace)


def factor(X: torch.Tensor) -> torch.Tensor:
    """E[x x^T] over the rows of X."""
    S = torch.empty(X.shape[1], X.shape[1], dtype=X.dtype, device=X.device)
    return kron_factor_accumulate(X, S, 1.0 / X.shape[0], 0.0)


def prepare(A: torch.Tensor, damp_rel: float, info: torch.Tensor | None = None):
    """(U, trace, lambda) for the damped factor.  With info=None the call waits
    and raises KronError if the damped factor is not PD; otherwise it stays
    asynchronous and info[0] receives 0 or the failing pivot (1-based)."""
    d = A.shape[0]
    U = torch.empty_like(A)
    tr = torch.empty(1, dtype=torch.float64, device=A.device)
    lam = torch.empty(1, dtype=torch.float64, device=A.device)
    ws = workspace(KQ_OP_PREPARE, A.dtype, d, 0, A.device)
    kron_prepare(A, damp_rel, U, ws, trace_out=tr, lambda_out=lam, info=info)
    return U, tr, lam  # ws goes back to this stream's pool: stream-ordered reuse


def quantize(W, U_A, U_B, bits, per_row, scales=None, ws=None, loss_out=None, per_diagonal=False):
    """codes, V, scales; loss_out (a float64 device tensor), if given, receives
    the proxy loss of V from the rounding errors.  per_diagonal: the schedule
    that never waits inside a kernel (kron_quantize_per_diagonal)."""
    m, n = W.shape
    if scales is None:
        scales = torch.empty(m if per_row else 1, dtype=W.dtype, device=W.device)
        kron_row_scales(W, bits, per_row, scales)
    codes = torch.empty(m, n, dtype=torch.int8, device=W.device)
    V = torch.empty_like(W)
    if ws is None:
        ws = workspace(KQ_OP_QUANTIZE, W.dtype, m, n, W.device)
    kron_quantize(W, U_A, U_B, bits, per_row, scales, codes, V, ws, loss=loss_out, per_diagonal=per_diagonal)
    return codes, V, scales


def loss(W, V, A, B, damp_rel):
    m, n = W.shape
    out = torch.empty(1, dtype=torch.float64, device=W.device)
    ws = workspace(KQ_OP_LOSS, W.dtype, m, n, W.device)
    kron_loss(W, V, A, B, damp_rel, out, ws)
    return out


def quantize_layer(W, act, grad, bits, per_row=True, damp_rel=0.01, two_sided=True, check_loss=False):
    """Run the whole path for one layer.  act: N x n activation rows, grad: N x m gradient rows.
    Raises KronError if a damped factor is not positive definite.  The result's
    "loss" is the solver's; check_loss=True adds "loss_check" from kron_loss."""
    main = torch.cuda.current_stream(W.device)
    info = torch.zeros(2, dtype=torch.int32, device=W.device)
    A = factor(act)
    B = U_B = trB = None
    if two_sided:
        side = torch.cuda.Stream(W.device)
        side.wait_stream(main)  # the A product (and every input) is ready
        with torch.cuda.stream(side):
            B = factor(grad)
            U_B, trB, _ = prepare(B, damp_rel, info[1:])
        # blocks shared by the two streams are not reused before both are done with them
        for t in (grad, info):
            t.record_stream(side)
        for t in (B, U_B, trB):
            t.record_stream(main)
    U_A, trA, _ = prepare(A, damp_rel, info[:1])
    if two_sided:
        main.wait_stream(side)
    bad = info.cpu()
    for name, k in (("A", int(bad[0])), ("B", int(bad[1]))):
        if k != 0:
            raise KronError(2, f"kron_prepare: damped factor {name} is not positive definite (pivot step {k})")
    lo = torch.empty(1, dtype=torch.float64, device=W.device)
    codes, V, scales = quantize(W, U_A, U_B, bits, per_row, loss_out=lo)
    out = dict(A=A, B=B, U_A=U_A, U_B=U_B, trace_A=trA, trace_B=trB, codes=codes, V=V, scales=scales, loss=lo)
    if check_loss:
        out["loss_check"] = loss(W, V, A, B, damp_rel)
    return out


def _factor_chains(W, act, grad, bits, per_row, damp_rel, two_sided, sa, sb):
    """Issue one layer's factor chains: A (and the scales) on stream sa, B on
    stream sb once the A product is done.  Returns the layer's tensors and the
    events that mark the two chains done."""
    ea, eb = torch.cuda.Event(), torch.cuda.Event()
    with torch.cuda.stream(sa):
        info = torch.zeros(2, dtype=torch.int32, device=W.device)  # cleared on sa, before both chains
        A = factor(act)
        a_done = torch.cuda.Event()
        a_done.record(sa)
    out = dict(info=info, B=None, U_B=None, trace_B=None)
    if two_sided:
        sb.wait_event(a_done)
        with torch.cuda.stream(sb):
            B = factor(grad)
            U_B, trB, _ = prepare(B, damp_rel, info[1:])
            eb.record(sb)
        for t in (grad, info, B, U_B, trB):
            t.record_stream(sb)
        out.update(B=B, U_B=U_B, trace_B=trB)
    with torch.cuda.stream(sa):
        U_A, trA, _ = prepare(A, damp_rel, info[:1])
        scales = torch.empty(W.shape[0] if per_row else 1, dtype=W.dtype, device=W.device)
        kron_row_scales(W, bits, per_row, scales)
        ea.record(sa)
    for t in (act, W):
        t.record_stream(sa)
    out.update(A=A, U_A=U_A, trace_A=trA, scales=scales, events=(ea, eb) if two_sided else (ea,))
    return out


def quantize_layers(layers, bits, per_row=True, damp_rel=0.01, two_sided=True, check_loss=False):
    """Quantize a sequence of independent layers [(W, act, grad), ...].  The
    factor chains of layer k + 1 run beside the solve of layer k, and consecutive
    layers are solved on two alternate streams (the caller's and a second one),
    so two solves share the GPU: the tile sweeps of one solve occupy at most half
    of the CUs.  The solves use the per-diagonal schedule, whose workgroups never
    hold a compute unit while waiting for one another, so the work beside them
    gets the CUs that the sweeps leave free (the persistent schedule of
    kron_quantize is faster alone but slower shared).  Returns one dict per
    layer, as quantize_layer does, ready on the caller's stream.  The
    positive-definiteness of every damped factor is checked once, after the last
    layer has been issued (a host wait per layer would stop the pipeline);
    KronError names the first failing layer."""
    main = torch.cuda.current_stream()
    sa, sb, s2 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    for s in (sa, sb, s2):
        s.wait_stream(main)  # every input is ready
    solvers = (main, s2)
    results = []
    nxt = _factor_chains(*layers[0], bits, per_row, damp_rel, two_sided, sa, sb) if layers else None
    for k, (W, act, grad) in enumerate(layers):
        cur = nxt
        if k + 1 < len(layers):
            nxt = _factor_chains(*layers[k + 1], bits, per_row, damp_rel, two_sided, sa, sb)
        ss = solvers[k % 2]
        for e in cur["events"]:
            ss.wait_event(e)
        for key in ("A", "B", "U_A", "U_B", "trace_A", "trace_B", "scales", "info"):
            if cur[key] is not None:
                cur[key].record_stream(ss)
        with torch.cuda.stream(ss):
            lo = torch.empty(1, dtype=torch.float64, device=W.device)
            codes, V, scales = quantize(W, cur["U_A"], cur["U_B"], bits, per_row, scales=cur["scales"], loss_out=lo,
                                        per_diagonal=True)
            out = dict(A=cur["A"], B=cur["B"], U_A=cur["U_A"], U_B=cur["U_B"], trace_A=cur["trace_A"],
                       trace_B=cur["trace_B"], codes=codes, V=V, scales=scales, loss=lo, info=cur["info"])
            if check_loss:
                out["loss_check"] = loss(W, V, cur["A"], cur["B"], damp_rel)
        if ss is not main:
            W.record_stream(ss)
            # everything handed back was made on a side stream: the caller's
            # stream uses it from here on
            for key in ("A", "B", "U_A", "U_B", "trace_A", "trace_B", "scales", "codes", "V", "loss", "loss_check"):
                if out.get(key) is not None:
                    out[key].record_stream(main)
        results.append(out)
    main.wait_stream(s2)
    for k, out in enumerate(results):
        bad = out.pop("info").cpu()
        for name, piv in (("A", int(bad[0])), ("B", int(bad[1]))):
            if piv != 0:
                raise KronError(2, f"kron_prepare: layer {k}: damped factor {name} is not positive definite "
                                   f"(pivot step {piv})")
    return results
