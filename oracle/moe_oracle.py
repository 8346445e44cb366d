"""Oracle for the forward pass of one Mixture-of-Experts layer (CPU, NumPy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it, and
it shares no code, table or helper with the library.

What it computes is the MoE sub-block as the pages name its operators: a gate
that picks experts per token, Dispatch of each token to its experts, the
routed experts, an always-on shared expert, and Combine back to token order
(FarSkip-Collective review: "Core claim" and "What carries the argument";
Fig. 2 caption, on the MoE layer's main operators; Fig. 11 caption, where
Combine is overlapped with the shared expert).  Top-k routing is named in the
expert-prototyping abstract of the "Daily Papers" search page (the count k of
experts a token activates), top-2 in the ScMoE abstract on the same page;
uneven routing with experts that receive few or no tokens in the LLEP
abstract there.  Grouping tokens by expert so that each
expert runs as a dense matrix product is the "Expert-Centric Scheduling" idea
of the OmniMoE abstract on that page.

The pages do not write out the layer's formulas.  Where they are silent this
module takes the plainest reading that the rest supports:
  * gate: softmax over all E router logits, keep the k largest, renormalise
    the kept probabilities to sum to one;
  * router logits  L = x W_r^T + b  (b optional);
  * ties between equal logits go to the lower expert index; slot j of a token
    holds its (j+1)-th largest logit;
  * dropless: no capacity limit, experts may receive zero tokens;
  * rows of an expert's segment are in ascending assignment order t*k + j;
  * expert FFN is SwiGLU without biases: (silu(X Wg^T) * (X Wu^T)) Wd^T with
    silu(z) = z / (1 + exp(-z));
  * shared experts are ungated, weight 1, applied to every token;
  * Combine: out[t] = sum_j w[t,j] * y[t, slot j] + shared[t].
Precision: all arithmetic here is float64.  The router logits are rounded to
float32 before the top-k decision, because float32 is the precision in which
the GPU takes it; for bf16 workloads the SwiGLU product A is rounded to bf16
(nearest even) before the down projection, as the GPU stores it in bf16.

Parity pins (tests/test_oracle_pins.py) tie every function here to closed
forms, library routines, invariants or brute force; see each docstring.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "silu",
    "router_logits",
    "router_logits_f32_lane_order",
    "topk_route",
    "dispatch",
    "gather_rows",
    "swiglu_expert",
    "grouped_ffn",
    "shared_ffn",
    "combine",
    "moe_layer",
    "moe_layer_dense",
    "token_outputs",
]


# ---------------------------------------------------------------------------
# Elementary pieces
# ---------------------------------------------------------------------------

_F32_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_STEP = 2.0 ** -133


def bf16_round(a) -> np.ndarray:
    """Round real values (given as float64) to the nearest bfloat16, ties to
    even; returns float64 holding the rounded values.

    bfloat16 keeps 8 significant bits and float32's exponent range.  For
    normal magnitudes the float64 significand is cut to its top 8 bits with
    round-half-even on the dropped 45 bits; below float32's smallest normal
    the grid is uniform with step 2^-133.
    Pinned against torch's float32->bfloat16 conversion and hand-made ties.
    """
    v = np.asarray(a, dtype=np.float64)
    out = np.empty_like(v)
    small = np.abs(v) < _F32_MIN_NORMAL
    big = ~small
    if big.any():
        u = v[big].view(np.uint64).copy()
        drop = np.uint64(45)
        lsb = (u >> drop) & np.uint64(1)
        u = u + (np.uint64((1 << 44) - 1) + lsb)
        u &= ~np.uint64((1 << 45) - 1)
        out[big] = u.view(np.float64)
    if small.any():
        out[small] = np.rint(v[small] / _BF16_SUBNORMAL_STEP) * _BF16_SUBNORMAL_STEP
    return out


def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64.
    Pinned: silu(0) = 0, silu(z) -> z for large z, -> 0- for very negative z,
    and against scipy's logistic function."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# Gate: logits, top-k, weights
# ---------------------------------------------------------------------------

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """L = x W_r^T + b, computed in float64 and rounded once to float32.

    For bf16 inputs and moderate d every product and partial sum is exact in
    float64, so the result is the correctly rounded float32 of the exact
    value (pinned against rational arithmetic on small inputs).
    """
    L = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L.astype(np.float32)


def router_logits_f32_lane_order(x, w_router, bias=None) -> np.ndarray:
    """Router logits for float32 workloads, in the float32 operation order of
    the library's float32 router, so that both sides take the top-k decision
    on bit-identical logits.

    Order: for each (token, expert), 64 partial sums, partial l adding the
    rounded products x[i]*w[i] for i = l, l+64, l+128, ... in ascending i
    (separate multiply and add, no fused multiply-add); then 6 butterfly
    rounds, partial l += partial (l xor m) for m = 32, 16, 8, 4, 2, 1; then
    the bias is added.  Every step is a float32 operation.
    """
    x = np.asarray(x, np.float32)
    w = np.asarray(w_router, np.float32)
    T, d = x.shape
    E = w.shape[0]
    part = np.zeros((T, E, 64), np.float32)
    for i0 in range(0, d, 64):
        n = min(64, d - i0)
        prod = x[:, None, i0:i0 + n] * w[None, :, i0:i0 + n]  # float32 products
        part[:, :, :n] = part[:, :, :n] + prod
    lanes = np.arange(64)
    for m in (32, 16, 8, 4, 2, 1):
        part = part + part[:, :, lanes ^ m]
    L = part[:, :, 0]
    if bias is not None:
        L = L + np.asarray(bias, np.float32)[None, :]
    return L.astype(np.float32)


def topk_route(logits, k: int):
    """Top-k gate with renormalised softmax weights.

    ids[t, j]: the expert with the (j+1)-th largest logit of token t; equal
    logits are ordered by ascending expert index (-0.0 equals +0.0).  This is
    a stable sort of the experts by descending logit.
    w[t, j]: p[ids[t, j]] / sum_j' p[ids[t, j']] with p = softmax over all E
    logits, in float64, rounded to float32 at the end.
    Pinned: weights sum to one; k = 1 gives exactly 1; k = E gives the full
    softmax (scipy); a constant shift changes nothing; duplicated router rows
    resolve to the lower index; brute-force rank counting agrees.
    """
    L = np.asarray(logits)
    L64 = L.astype(np.float64)
    L64 = np.where(L64 == 0.0, 0.0, L64)  # fold -0.0 into +0.0
    order = np.argsort(-L64, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    m = L64.max(axis=1, keepdims=True)
    p = np.exp(L64 - m)
    p = p / p.sum(axis=1, keepdims=True)  # softmax over all E
    kept = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = kept / kept.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)


# ---------------------------------------------------------------------------
# Dispatch
# ---------------------------------------------------------------------------

def dispatch(ids, E: int):
    """Group the T*k assignments a = t*k + j by expert, stably.

    Returns counts [E], offsets [E+1] (exclusive prefix sum, offsets[E] = T*k),
    perm [R] (perm[i] = assignment stored at sorted row i) and inv_perm [R]
    (inv_perm[a] = sorted row of assignment a).  Written as an explicit
    counting sort; pinned against numpy's stable argsort and bincount.
    """
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    R = flat.size
    counts = np.zeros(E, np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    perm = np.empty(R, np.int64)
    for a in range(R):
        e = flat[a]
        perm[cursor[e]] = a
        cursor[e] += 1
    inv_perm = np.empty(R, np.int64)
    inv_perm[perm] = np.arange(R)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv_perm.astype(np.int32))


def gather_rows(x, perm, k: int) -> np.ndarray:
    """x_sorted[i] = x[perm[i] // k]: the token row of each sorted assignment."""
    return np.asarray(x)[np.asarray(perm, np.int64) // k]


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------

def swiglu_expert(X, w_gate, w_up, w_down, round_a: bool):
    """One SwiGLU expert on rows X: A = silu(X Wg^T) * (X Wu^T), optionally
    rounded to bf16, then Y = A Wd^T.  float64.  Returns (A, Y)."""
    X = np.asarray(X, np.float64)
    G = X @ np.asarray(w_gate, np.float64).T
    U = X @ np.asarray(w_up, np.float64).T
    A = silu(G) * U
    if round_a:
        A = bf16_round(A)
    return A, A @ np.asarray(w_down, np.float64).T


def grouped_ffn(x_sorted, offsets, w_gate, w_up, w_down, round_a: bool,
                expert_fn=None):
    """Apply expert e to rows offsets[e]:offsets[e+1] of x_sorted.

    Returns (A [R, I], y_sorted [R, d]) in float64.  ``expert_fn(e, X)``
    replaces the SwiGLU expert when given (used by the identity-expert pin);
    it then returns (None, Y).
    """
    x_sorted = np.asarray(x_sorted)
    R, d = x_sorted.shape
    E = len(offsets) - 1
    y = np.zeros((R, d), np.float64)
    A = None if expert_fn is not None else np.zeros((R, np.asarray(w_gate).shape[1]), np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        if expert_fn is not None:
            y[r0:r1] = expert_fn(e, x_sorted[r0:r1])
        else:
            A[r0:r1], y[r0:r1] = swiglu_expert(x_sorted[r0:r1], w_gate[e], w_up[e],
                                               w_down[e], round_a)
    return A, y


def shared_ffn(x, wsh_gate, wsh_up, wsh_down, round_a: bool):
    """Sum of the ungated shared experts applied to every token, float64.
    Returns (A_shared [T, n_s*I_s], y_shared [T, d])."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    ns = np.asarray(wsh_gate).shape[0]
    A_all = []
    y = np.zeros((T, d), np.float64)
    for s in range(ns):
        A, Y = swiglu_expert(x, wsh_gate[s], wsh_up[s], wsh_down[s], round_a)
        A_all.append(A)
        y = y + Y
    return np.concatenate(A_all, axis=1), y


# ---------------------------------------------------------------------------
# Combine and the whole layer
# ---------------------------------------------------------------------------

def combine(y_sorted, inv_perm, w, y_shared, k: int) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y_sorted[inv_perm[t*k + j]]  (+ y_shared[t]), float64."""
    y_sorted = np.asarray(y_sorted, np.float64)
    w = np.asarray(w, np.float64)
    T = w.shape[0]
    inv = np.asarray(inv_perm, np.int64).reshape(T, k)
    out = np.zeros((T, y_sorted.shape[1]), np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y_sorted[inv[:, j]]
    if y_shared is not None:
        out += np.asarray(y_shared, np.float64)
    return out


def moe_layer(x, w_router, bias, w_gate, w_up, w_down, k: int,
              wsh_gate=None, wsh_up=None, wsh_down=None, round_a: bool = True,
              logits=None, expert_fn=None) -> dict:
    """The whole layer, step by step.  ``logits`` overrides the router
    (float32 logits given from outside, e.g. made by ``router_logits`` or
    ``router_logits_f32_lane_order``)."""
    E = np.asarray(w_router).shape[0] if w_router is not None else np.asarray(logits).shape[1]
    if logits is None:
        logits = router_logits(x, w_router, bias)
    ids, w = topk_route(logits, k)
    counts, offsets, perm, inv_perm = dispatch(ids, E)
    x_sorted = gather_rows(x, perm, k)
    A, y_sorted = grouped_ffn(x_sorted, offsets, w_gate, w_up, w_down, round_a,
                              expert_fn=expert_fn)
    A_shared, y_shared = (None, None)
    if wsh_gate is not None and np.asarray(wsh_gate).shape[0] > 0:
        A_shared, y_shared = shared_ffn(x, wsh_gate, wsh_up, wsh_down, round_a)
    out = combine(y_sorted, inv_perm, w, y_shared, k)
    return dict(logits=logits, ids=ids, w=w, counts=counts, offsets=offsets,
                perm=perm, inv_perm=inv_perm, x_sorted=x_sorted, A=A,
                y_sorted=y_sorted, A_shared=A_shared, y_shared=y_shared, out=out)


def moe_layer_dense(x, logits, w_gate, w_up, w_down, k: int,
                    wsh_gate=None, wsh_up=None, wsh_down=None,
                    round_a: bool = True, gate_f32: bool = True) -> np.ndarray:
    """Brute force: run every expert on every token and mask.

    mask[t, e] = 1 when fewer than k experts rank above e, where e' ranks
    above e if L[t,e'] > L[t,e], or L[t,e'] == L[t,e] and e' < e (an O(E^2)
    rank count, independent of any sort).  Weights are the softmax over all
    E restricted to the mask and renormalised.  float64 throughout.
    """
    x = np.asarray(x, np.float64)
    L = np.asarray(logits, np.float64)
    T, E = L.shape
    above = (L[:, None, :] > L[:, :, None]) | (
        (L[:, None, :] == L[:, :, None]) & (np.arange(E)[None, None, :] < np.arange(E)[None, :, None]))
    rank = above.sum(axis=2)  # rank[t, e] = number of experts ranked above e
    mask = rank < k
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    wt = np.where(mask, p, 0.0)
    wt = wt / wt.sum(axis=1, keepdims=True)
    if gate_f32:  # the gate weights are float32 values (False: kept in float64)
        wt = wt.astype(np.float32).astype(np.float64)
    out = np.zeros((T, x.shape[1]), np.float64)
    for e in range(E):
        _, Y = swiglu_expert(x, w_gate[e], w_up[e], w_down[e], round_a)
        out += wt[:, e:e + 1] * Y
    if wsh_gate is not None:
        for s in range(np.asarray(wsh_gate).shape[0]):
            _, Y = swiglu_expert(x, wsh_gate[s], wsh_up[s], wsh_down[s], round_a)
            out += Y
    return out


def token_outputs(tokens, x, logits, w_gate, w_up, w_down, k: int,
                  wsh_gate=None, wsh_up=None, wsh_down=None, round_a: bool = True):
    """Layer output rows for a few tokens only, one token at a time in effect:
    route each token on its logits row, run its k experts and the shared
    experts on it, combine.  Returns (ids, w, out) for those tokens, float64
    out.  Used to check full-size runs on sampled outputs."""
    tokens = np.asarray(tokens, np.int64)
    xs = np.asarray(x)[tokens].astype(np.float64)
    ids, w = topk_route(np.asarray(logits)[tokens], k)
    out = np.zeros((tokens.size, xs.shape[1]), np.float64)
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        _, Y = swiglu_expert(xs[rows], w_gate[e], w_up[e], w_down[e], round_a)
        out[rows] += w[rows, slots].astype(np.float64)[:, None] * Y
    if wsh_gate is not None:
        for s in range(np.asarray(wsh_gate).shape[0]):
            _, Y = swiglu_expert(xs, wsh_gate[s], wsh_up[s], wsh_down[s], round_a)
            out += Y
    return ids, w, out
