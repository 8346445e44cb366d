"""Oracle for token condensation in the MoE layer (CPU, NumPy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it, and
it shares no code, table or helper with the library.

The method is Luffy's token condensation (Luffy review, "Core claim" and
"What carries the argument"; the axiom ledger's domain assumptions that
condensing similar tokens to one representative is acceptable and that token
similarity survives the expert).  Tokens routed to the same expert that are
near-duplicates of an earlier token send no row of their own: the expert
output of the representative is reused for them.  The pages fix neither the
similarity measure's normalisation (the review's minor comment on §II-B) nor
how candidates are found in one forward pass (Luffy's fast measurement uses
training history, which a single forward pass does not have).  This module
takes these readings:

  * similarity: the plain cosine of two token rows, computed in float64; a
    threshold h on the [0, 1] "normalised" cosine is the threshold 2h - 1 on
    the plain one;
  * candidates: tokens whose 16-bit keys are equal, where bit b of a token's
    key is set when its projection onto caller-given hyperplane b is >= 0
    (sign random projections; the hyperplanes are an input, like any random
    draw of the method);
  * representative: the members of a key bucket in ascending token order
    m_0 < m_1 < ...; for t = m_i, c(t) is the first m_j with j < min(i, C)
    and cos(x_t, x_{m_j}) >= h (t itself when there is none), where C = 32
    bounds the similarity checks per token; then rep(t) = c(t) when
    c(c(t)) == c(t), else t, so that every condensed token maps to a token
    that is computed;
  * an assignment (t, j) is condensed when rep(t) != t and rep(t) is routed to
    the same expert; it then reuses the expert output of that assignment of
    rep(t).  Its own gate weight still applies, and the shared experts run on
    every token as before.

Parity pins: tests/test_condense_oracle.py (closed forms, exact duplicates,
brute force on hand-made cases, invariants of the condensed dispatch).
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as _m

KEY_BITS = 16
CANDIDATES = 32  # only the first CANDIDATES members of a key bucket can be representatives

__all__ = [
    "KEY_BITS",
    "CANDIDATES",
    "projections",
    "condense_keys",
    "cosine",
    "condense_reps",
    "condensed_sources",
    "dispatch_condensed",
    "condensed_layer",
]


def projections(x, hyperplanes) -> np.ndarray:
    """proj[t, b] = x_t . p_b in float64 (x and the hyperplanes as given)."""
    return np.asarray(x, np.float64) @ np.asarray(hyperplanes, np.float64).T


def condense_keys(proj) -> np.ndarray:
    """key[t] = sum_b [proj[t, b] >= 0] * 2^b over the KEY_BITS hyperplanes
    (-0.0 counts as >= 0, like +0.0)."""
    proj = np.asarray(proj)
    assert proj.shape[1] == KEY_BITS
    bits = (proj >= 0).astype(np.int64)
    return (bits << np.arange(KEY_BITS, dtype=np.int64)).sum(axis=1)


def cosine(a, b) -> float:
    """Plain cosine of two rows in float64; a zero row is similar to nothing
    (returns -inf) so that it is never condensed into another row."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    na, nb = np.sqrt(a @ a), np.sqrt(b @ b)
    if na == 0.0 or nb == 0.0:
        return -np.inf
    return float(a @ b / (na * nb))


def condense_reps(x, keys, cos_threshold: float, cos_fn=None,
                  candidates: int = CANDIDATES) -> np.ndarray:
    """rep[t] by the two-step rule of the module docstring.  ``cos_fn(t, t2)``
    overrides the cosine (for tests that fix similarities by hand)."""
    x = np.asarray(x)
    keys = np.asarray(keys, np.int64)
    T = keys.shape[0]
    if cos_fn is None:
        def cos_fn(t, t2):
            return cosine(x[t], x[t2])
    cand = np.arange(T)
    for t in range(T):
        earlier = [t2 for t2 in range(t) if keys[t2] == keys[t]]  # ascending
        for t2 in earlier[:candidates]:  # the first qualifying member wins
            if cos_fn(t, t2) >= cos_threshold:
                cand[t] = t2
                break
    rep = np.where(cand[cand] == cand, cand, np.arange(T))
    return rep


def condensed_sources(ids, rep):
    """For every assignment (t, j): the assignment index whose expert output it
    uses.  src[t*k + j] = rep(t)*k + j' when rep(t) != t and
    ids[rep(t), j'] == ids[t, j]; otherwise t*k + j itself.  Returns (src,
    condensed) as flat arrays of length T*k."""
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    src = np.arange(T * k)
    for t in range(T):
        r = rep[t]
        if r == t:
            continue
        for j in range(k):
            hit = np.nonzero(ids[r] == ids[t, j])[0]
            if hit.size:
                src[t * k + j] = r * k + hit[0]
    return src, src != np.arange(T * k)


def dispatch_condensed(ids, E: int, rep):
    """Stable counting sort by expert of the assignments that are not
    condensed; a condensed assignment gets the row of its source.

    Returns (counts, offsets, perm, inv_perm): counts/offsets over the rows
    that exist (offsets[E] = number of rows), perm[i] = the assignment stored
    in row i (ascending assignment index within an expert), inv_perm[a] = the
    row whose expert output assignment a uses."""
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    src, cond = condensed_sources(ids, rep)
    flat = ids.ravel()
    keep = np.nonzero(~cond)[0]
    counts = np.bincount(flat[keep], minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = keep[np.argsort(flat[keep], kind="stable")]
    inv_perm = np.full(T * k, -1, np.int64)
    inv_perm[perm] = np.arange(perm.size)
    inv_perm[cond] = inv_perm[src[cond]]
    return counts, offsets, perm, inv_perm


def condensed_layer(x, logits, w_gate, w_up, w_down, k: int, rep,
                    wsh_gate=None, wsh_up=None, wsh_down=None,
                    round_a: bool = True) -> dict:
    """The layer with condensation: route on ``logits``, dispatch the
    assignments that are not condensed, run the routed experts on those rows
    only, combine with each condensed assignment reading its source's row,
    add the shared experts (on every token).  float64."""
    E = np.asarray(logits).shape[1]
    ids, w = _m.topk_route(logits, k)
    counts, offsets, perm, inv_perm = dispatch_condensed(ids, E, rep)
    x_sorted = _m.gather_rows(x, perm, k)
    A, y_sorted = _m.grouped_ffn(x_sorted, offsets, w_gate, w_up, w_down, round_a)
    y_shared = None
    if wsh_gate is not None and np.asarray(wsh_gate).shape[0] > 0:
        _, y_shared = _m.shared_ffn(x, wsh_gate, wsh_up, wsh_down, round_a)
    out = _m.combine(y_sorted, inv_perm, w, y_shared, k)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm,
                inv_perm=inv_perm, y_sorted=y_sorted, y_shared=y_shared, out=out)
