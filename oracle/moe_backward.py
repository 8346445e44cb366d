"""Oracle for the backward pass of one Mixture-of-Experts layer (CPU, NumPy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's CPU-baseline leg
may import this module.  The HIP library never calls it, and it shares no
code, table or helper with the library.

The measured workloads of the FarSkip-Collective review (DeepSeek-V3 MoE
layers trained with expert parallelism: "What carries the argument", the
training speed-up of its abstract) and of the Luffy review (MoE models trained
on V100s: "Core claim", Fig. 8 caption) are training runs, so the layer's
gradients are part of the work those pages time.  The pages do not write the
gradients out; they follow from the forward pass (oracle/moe_oracle.py) by the
chain rule, with these readings where the forward is not differentiable or
rounds:
  * the top-k selection is piecewise constant: no gradient flows through the
    choice of experts, only through the kept weights;
  * the kept weights are the softmax over the kept logits (the renormalised
    softmax), so for a token with kept weights w and upstream gradient dw on
    them the logit gradient is  dL_i = w_i (dw_i - sum_j w_j dw_j)  on the
    kept experts and zero elsewhere;
  * the bias gradient is the sum over tokens of the logit gradient;
  * the bf16 rounding of the SwiGLU product A passes the gradient through
    unchanged (straight-through); the down-projection weight gradient uses
    the rounded A that the forward pass multiplied;
  * silu'(g) = s (1 + g (1 - s)) with s = 1 / (1 + exp(-g)).
All arithmetic is float64 on the given (bf16-valued or fp32) inputs.

Pins (tests/test_backward_oracle.py): central finite differences of the
brute-force dense forward (every input), exact k = 1 and k = E special cases
of the router gradient (zero; the full softmax Jacobian), exact power-of-two
scaling, and linearity in the upstream gradient.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import bf16_round, dispatch, gather_rows, router_logits, topk_route

__all__ = ["silu_grad", "renormalised_softmax_grad", "swiglu_expert_backward",
           "moe_layer_backward", "moe_layer_backward_parts"]


def _sigmoid(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu_grad(g) -> np.ndarray:
    """d/dg [g * sigmoid(g)] = s (1 + g (1 - s)), s = sigmoid(g), float64."""
    g = np.asarray(g, np.float64)
    s = _sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def renormalised_softmax_grad(w, dw) -> np.ndarray:
    """Logit gradient of the kept weights w = softmax over the kept logits.

    w, dw: [T, k] (kept weights and their upstream gradient).  Returns
    dL_kept [T, k] with dL_i = w_i (dw_i - sum_j w_j dw_j)."""
    w = np.asarray(w, np.float64)
    dw = np.asarray(dw, np.float64)
    return w * (dw - (w * dw).sum(axis=1, keepdims=True))


def swiglu_expert_backward(X, w_gate, w_up, w_down, dY, round_a: bool):
    """Gradients of one SwiGLU expert Y = bf16?(silu(X Wg^T) * (X Wu^T)) Wd^T.

    Returns dict(dX, dWg, dWu, dWd), float64."""
    X = np.asarray(X, np.float64)
    Wg = np.asarray(w_gate, np.float64)
    Wu = np.asarray(w_up, np.float64)
    Wd = np.asarray(w_down, np.float64)
    dY = np.asarray(dY, np.float64)
    G = X @ Wg.T
    U = X @ Wu.T
    s = _sigmoid(G)
    A = G * s * U
    if round_a:
        A = bf16_round(A)
    dA = dY @ Wd                 # [n, I]
    dWd = dY.T @ A               # [d, I]
    dG = dA * U * silu_grad(G)
    dU = dA * (G * s)
    dWg = dG.T @ X               # [I, d]
    dWu = dU.T @ X
    dX = dG @ Wg + dU @ Wu       # [n, d]
    return dict(dX=dX, dWg=dWg, dWu=dWu, dWd=dWd)


def moe_layer_backward(x, w_router, bias, w_gate, w_up, w_down, k: int, dout,
                       wsh_gate=None, wsh_up=None, wsh_down=None, round_a: bool = True,
                       logits=None) -> dict:
    """Gradients of the layer output with respect to every input, given the
    upstream gradient dout [T, d].

    The forward routing is taken on float32 logits (``router_logits``, or the
    ``logits`` given, as in the forward oracle), so the kept experts match
    the forward pass; the kept weights are recomputed in float64 from those
    logits.  Returns dict with dx [T,d], dw_router [E,d], dbias [E],
    dw_gate/dw_up [E,I,d], dw_down [E,d,I], dwsh_gate/dwsh_up [n_s,I_s,d],
    dwsh_down [n_s,d,I_s] (None without shared experts), and the
    intermediates ids, w (float64 kept weights), dw [T,k], dlogits_kept [T,k].
    """
    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    T, d = x.shape
    Wg = np.asarray(w_gate)
    E, I, _ = Wg.shape
    if logits is None:
        logits = router_logits(x, w_router, bias)
    ids, _ = topk_route(logits, k)
    L = np.asarray(logits, np.float64)
    kept = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    z = np.exp(kept - kept[:, :1])
    w = z / z.sum(axis=1, keepdims=True)          # renormalised softmax, float64

    counts, offsets, perm, inv_perm = dispatch(ids, E)
    perm = perm.astype(np.int64)
    inv = inv_perm.astype(np.int64).reshape(T, k)
    x_sorted = gather_rows(x, perm, k)
    tok = perm // k
    w_rows = w.reshape(-1)[perm]                   # gate weight of each sorted row
    dY_sorted = w_rows[:, None] * dout[tok]        # d out / d y_sorted

    dx = np.zeros((T, d), np.float64)
    dWg = np.zeros((E, I, d), np.float64)
    dWu = np.zeros((E, I, d), np.float64)
    dWd = np.zeros((E, d, I), np.float64)
    dX_sorted = np.zeros((perm.size, d), np.float64)
    y_sorted = np.zeros((perm.size, d), np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        Xe = x_sorted[r0:r1]
        g = swiglu_expert_backward(Xe, w_gate[e], w_up[e], w_down[e], dY_sorted[r0:r1], round_a)
        dWg[e], dWu[e], dWd[e] = g["dWg"], g["dWu"], g["dWd"]
        dX_sorted[r0:r1] = g["dX"]
        # the expert's output rows, for the gradient of the gate weights
        Gx = Xe @ np.asarray(w_gate[e], np.float64).T
        Ux = Xe @ np.asarray(w_up[e], np.float64).T
        A = Gx * _sigmoid(Gx) * Ux
        if round_a:
            A = bf16_round(A)
        y_sorted[r0:r1] = A @ np.asarray(w_down[e], np.float64).T
    # each token sums the input gradients of its k assignments, slot by slot
    for j in range(k):
        dx += dX_sorted[inv[:, j]]

    # gate: out[t] = sum_j w[t,j] y[t,j]  ->  dw[t,j] = dout[t] . y[t,j]
    dw = np.einsum("td,tjd->tj", dout, y_sorted[inv])
    dLk = renormalised_softmax_grad(w, dw)
    dL = np.zeros((T, E), np.float64)
    np.put_along_axis(dL, ids.astype(np.int64), dLk, axis=1)
    Wr = np.asarray(w_router, np.float64)
    dWr = dL.T @ x
    db = dL.sum(axis=0)
    dx += dL @ Wr

    dWsg = dWsu = dWsd = None
    if wsh_gate is not None and np.asarray(wsh_gate).shape[0] > 0:
        ns = np.asarray(wsh_gate).shape[0]
        dWsg = np.zeros(np.asarray(wsh_gate).shape, np.float64)
        dWsu = np.zeros_like(dWsg)
        dWsd = np.zeros(np.asarray(wsh_down).shape, np.float64)
        for s in range(ns):
            g = swiglu_expert_backward(x, wsh_gate[s], wsh_up[s], wsh_down[s], dout, round_a)
            dWsg[s], dWsu[s], dWsd[s] = g["dWg"], g["dWu"], g["dWd"]
            dx += g["dX"]
    return dict(dx=dx, dw_router=dWr, dbias=db, dw_gate=dWg, dw_up=dWu, dw_down=dWd,
                dwsh_gate=dWsg, dwsh_up=dWsu, dwsh_down=dWsd, ids=ids, w=w, dw=dw,
                dlogits_kept=dLk, perm=perm.astype(np.int32), offsets=offsets)


def moe_layer_backward_parts(x, w_router, bias, w_gate, w_up, w_down, k: int, dout,
                             wsh_gate=None, wsh_up=None, wsh_down=None, round_a: bool = True,
                             logits=None, experts=(), tokens=()) -> dict:
    """Parts of ``moe_layer_backward`` for layers too large for the whole of it:
    the same readings and the same steps, restricted to
      * the router gradients dw_router [E,d] and dbias [E] (whole: they need
        every token's gate-weight gradient, hence every expert's output rows);
      * the shared experts' weight gradients (whole);
      * the routed weight gradients of the experts listed in ``experts``;
      * dx of the tokens listed in ``tokens``: the input gradients of each
        token's own k rows (an expert's input gradient of a row depends on
        that row alone), summed in slot order, plus its router and shared
        terms.
    Returns dict(dw_router, dbias, dwsh_gate, dwsh_up, dwsh_down (None without
    shared experts), dw_gate/dw_up/dw_down: {e: array}, dx [len(tokens), d],
    tokens, ids, offsets), float64.  Pinned against moe_layer_backward on
    small layers."""
    from .moe_oracle import swiglu_expert

    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    T, d = x.shape
    E = np.asarray(w_gate).shape[0]
    if logits is None:
        logits = router_logits(x, w_router, bias)
    ids, _ = topk_route(logits, k)
    L = np.asarray(logits, np.float64)
    kept = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    z = np.exp(kept - kept[:, :1])
    w = z / z.sum(axis=1, keepdims=True)          # renormalised softmax, float64

    counts, offsets, perm, inv_perm = dispatch(ids, E)
    perm = perm.astype(np.int64)
    inv = inv_perm.astype(np.int64).reshape(T, k)
    x_sorted = gather_rows(x, perm, k)
    tok = perm // k
    w_rows = w.reshape(-1)[perm]
    dY_sorted = w_rows[:, None] * dout[tok]

    # every expert's output rows, for the gradient of the gate weights
    y_sorted = np.zeros((perm.size, d), np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            _, y_sorted[r0:r1] = swiglu_expert(x_sorted[r0:r1], w_gate[e], w_up[e], w_down[e],
                                               round_a)
    dw = np.einsum("td,tjd->tj", dout, y_sorted[inv])
    dLk = renormalised_softmax_grad(w, dw)
    dL = np.zeros((T, E), np.float64)
    np.put_along_axis(dL, ids.astype(np.int64), dLk, axis=1)
    Wr = np.asarray(w_router, np.float64)
    out = dict(dw_router=dL.T @ x, dbias=dL.sum(axis=0), ids=ids, offsets=offsets,
               dw_gate={}, dw_up={}, dw_down={})

    for e in experts:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            I = np.asarray(w_gate).shape[1]
            out["dw_gate"][e] = np.zeros((I, d))
            out["dw_up"][e] = np.zeros((I, d))
            out["dw_down"][e] = np.zeros((d, I))
            continue
        g = swiglu_expert_backward(x_sorted[r0:r1], w_gate[e], w_up[e], w_down[e],
                                   dY_sorted[r0:r1], round_a)
        out["dw_gate"][e], out["dw_up"][e], out["dw_down"][e] = g["dWg"], g["dWu"], g["dWd"]

    tokens = np.asarray(tokens, np.int64)
    rows = inv[tokens]                             # [n, k] sorted rows of the tokens
    dX_rows = np.zeros(rows.shape + (d,), np.float64)
    for e in np.unique(ids[tokens]):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        sel = np.nonzero((rows >= r0) & (rows < r1))
        rr = rows[sel]
        g = swiglu_expert_backward(x_sorted[rr], w_gate[e], w_up[e], w_down[e], dY_sorted[rr],
                                   round_a)
        dX_rows[sel] = g["dX"]
    dx = np.zeros((tokens.size, d), np.float64)
    for j in range(k):
        dx += dX_rows[:, j]
    dx += dL[tokens] @ Wr

    out["dwsh_gate"] = out["dwsh_up"] = out["dwsh_down"] = None
    if wsh_gate is not None and np.asarray(wsh_gate).shape[0] > 0:
        ns = np.asarray(wsh_gate).shape[0]
        out["dwsh_gate"] = np.zeros(np.asarray(wsh_gate).shape, np.float64)
        out["dwsh_up"] = np.zeros_like(out["dwsh_gate"])
        out["dwsh_down"] = np.zeros(np.asarray(wsh_down).shape, np.float64)
        for s in range(ns):
            g = swiglu_expert_backward(x, wsh_gate[s], wsh_up[s], wsh_down[s], dout, round_a)
            out["dwsh_gate"][s], out["dwsh_up"][s], out["dwsh_down"][s] = g["dWg"], g["dWu"], g["dWd"]
            dx += g["dX"][tokens]
    out["dx"] = dx
    out["tokens"] = tokens
    return out
