"""Pins for the token-condensation oracle (oracle.condense): closed forms,
exact duplicates, hand-made cases with known cosines, brute force and
invariants.  CPU only.

The method is Luffy's token condensation (Luffy review, "Core claim"); the
readings the oracle takes where the pages are silent are listed in its module
docstring.  Each test ties a function to something other than itself, so that
a slip (a wrong key bit, a later instead of an earlier representative, a
missing chain cut, a condensed assignment of the wrong expert, a wrong row in
the combine) fails one of them."""
import math

import numpy as np
import pytest

import oracle
from oracle import condense as oc
from oracle import moe_oracle as mo


def _layer_inputs(seed, T=20, d=16, E=5, k=2, I=8, ns=1, Is=8):
    rng = np.random.default_rng(seed)
    sd = 1.0 / math.sqrt(d)
    f = lambda s, sc=1.0: (rng.standard_normal(s) * sc)  # noqa: E731
    p = dict(x=f((T, d)), w_router=f((E, d), sd), w_gate=f((E, I, d), sd), w_up=f((E, I, d), sd),
             w_down=f((E, d, I), sd))
    if ns:
        p.update(wsh_gate=f((ns, Is, d), sd), wsh_up=f((ns, Is, d), sd), wsh_down=f((ns, d, Is), sd))
    else:
        p.update(wsh_gate=None, wsh_up=None, wsh_down=None)
    return p


def _run(p, k, rep, round_a=False):
    L = mo.router_logits(p["x"], p["w_router"], None)
    return L, oc.condensed_layer(p["x"], L, p["w_gate"], p["w_up"], p["w_down"], k, rep,
                                 p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=round_a)


def test_key_bits_hand_example():
    proj = np.zeros((3, oc.KEY_BITS))
    proj[0] = -1.0                     # no bit set
    proj[1] = 1.0                      # all 16 bits
    proj[2] = -1.0
    proj[2, 0] = 0.5                   # bit 0
    proj[2, 3] = 0.0                   # bit 3 (zero counts as non-negative)
    proj[2, 15] = -0.0                 # bit 15 (negative zero too)
    assert oc.condense_keys(proj).tolist() == [0, 0xFFFF, 1 + 8 + 32768]


def test_projections_are_row_dot_products():
    rng = np.random.default_rng(1)
    x, P = rng.standard_normal((4, 6)), rng.standard_normal((oc.KEY_BITS, 6))
    pr = oc.projections(x, P)
    for t in range(4):
        for b in range(oc.KEY_BITS):
            assert pr[t, b] == pytest.approx(sum(x[t, i] * P[b, i] for i in range(6)), rel=1e-12)


def test_cosine_closed_forms():
    assert oc.cosine([1.0, 0.0], [2.0, 0.0]) == pytest.approx(1.0)
    assert oc.cosine([1.0, 0.0], [0.0, 3.0]) == pytest.approx(0.0)
    assert oc.cosine([1.0, 1.0], [-1.0, -1.0]) == pytest.approx(-1.0)
    assert oc.cosine([1.0, 0.0], [math.cos(0.3), math.sin(0.3)]) == pytest.approx(math.cos(0.3))
    assert oc.cosine([0.0, 0.0], [1.0, 0.0]) == -math.inf


def test_earliest_similar_token_is_the_representative():
    # four rows at 0, 10, 100 and 5 degrees, one key: 1 and 3 go to 0, 2 stays
    ang = np.radians([0.0, 10.0, 100.0, 5.0])
    x = np.stack([np.cos(ang), np.sin(ang)], axis=1)
    rep = oc.condense_reps(x, np.zeros(4, np.int64), math.cos(math.radians(20.0)))
    assert rep.tolist() == [0, 0, 2, 0]


def test_chain_is_cut():
    # 0, 30, 60 degrees with a 35-degree threshold: 1 -> 0, 2 -> 1, but 1 is
    # itself condensed, so 2 stays a representative
    ang = np.radians([0.0, 30.0, 60.0])
    x = np.stack([np.cos(ang), np.sin(ang)], axis=1)
    rep = oc.condense_reps(x, np.zeros(3, np.int64), math.cos(math.radians(35.0)))
    assert rep.tolist() == [0, 0, 2]


def test_only_the_first_32_bucket_members_can_be_representatives():
    # 34 mutually orthogonal rows share a key; row 34 copies member 33 (past
    # the first 32) and stays its own representative, row 35 copies member 31
    assert oc.CANDIDATES == 32
    d = 40
    x = np.zeros((36, d))
    x[np.arange(34), np.arange(34)] = 1.0
    x[34] = x[33]
    x[35] = x[31]
    rep = oc.condense_reps(x, np.zeros(36, np.int64), 0.9)
    assert rep[:34].tolist() == list(range(34))
    assert rep[34] == 34 and rep[35] == 31


def test_different_keys_never_condense_and_zero_rows_stay():
    x = np.ones((4, 3))
    x[3] = 0.0
    rep = oc.condense_reps(x, np.array([0, 1, 0, 0]), 0.5)
    assert rep.tolist() == [0, 1, 0, 3]  # 1 has its own key; the zero row 3 is similar to nothing


def test_threshold_above_one_condenses_nothing_and_layer_is_unchanged():
    p = _layer_inputs(2)
    T, k, E = p["x"].shape[0], 2, p["w_router"].shape[0]
    rep = oc.condense_reps(p["x"], np.zeros(T, np.int64), 1.5)
    assert rep.tolist() == list(range(T))
    L, got = _run(p, k, rep)
    ref = mo.moe_layer(p["x"], p["w_router"], None, p["w_gate"], p["w_up"], p["w_down"], k,
                       p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=False, logits=L)
    for key in ("counts", "offsets", "perm", "inv_perm"):
        np.testing.assert_array_equal(got[key], ref[key])
    np.testing.assert_array_equal(got["out"], ref["out"])


def test_exact_duplicates_reuse_the_first_copy_and_keep_the_output():
    p = _layer_inputs(3)
    x = p["x"]
    x[7] = x[2]
    x[11] = x[2]
    x[15] = x[4]
    k = 2
    rng = np.random.default_rng(4)
    keys = oc.condense_keys(oc.projections(x, rng.standard_normal((oc.KEY_BITS, x.shape[1]))))
    rep = oc.condense_reps(x, keys, 0.999)
    assert rep[7] == 2 and rep[11] == 2 and rep[15] == 4
    assert np.count_nonzero(rep != np.arange(x.shape[0])) == 3
    L, got = _run(p, k, rep)
    # the duplicates share their source's routing, so every one of their
    # assignments is condensed and the rows shrink by 3*k
    assert got["offsets"][-1] == x.shape[0] * k - 3 * k
    ref = mo.moe_layer(x, p["w_router"], None, p["w_gate"], p["w_up"], p["w_down"], k,
                       p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=False, logits=L)
    np.testing.assert_allclose(got["out"], ref["out"], rtol=1e-12, atol=1e-12)


def test_condensed_sources_only_for_a_shared_expert():
    ids = np.array([[0, 1, 2],
                    [2, 3, 4],    # token 1 -> rep 0: only expert 2 is shared (slot 0 of 1, slot 2 of 0)
                    [1, 0, 2]])   # token 2 -> rep 0: all three shared, in another slot order
    rep = np.array([0, 0, 0])
    src, cond = oc.condensed_sources(ids, rep)
    assert cond.tolist() == [False, False, False, True, False, False, True, True, True]
    assert src.tolist() == [0, 1, 2, 2, 4, 5, 1, 0, 2]


def _brute_dispatch(ids, E, rep):
    """Rows expert by expert, assignments in ascending index, skipping condensed ones."""
    T, k = ids.shape
    src, cond = oc.condensed_sources(ids, rep)
    perm, row_of = [], {}
    for e in range(E):
        for a in range(T * k):
            if ids.ravel()[a] == e and not cond[a]:
                row_of[a] = len(perm)
                perm.append(a)
    inv = [row_of[src[a]] for a in range(T * k)]
    return np.array(perm), np.array(inv)


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_condensed_dispatch_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 40, 7, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    cand = np.array([rng.integers(0, t + 1) for t in range(T)])
    rep = np.where(cand[cand] == cand, cand, np.arange(T))  # a valid map: representatives map to themselves
    counts, offsets, perm, inv = oc.dispatch_condensed(ids, E, rep)
    bperm, binv = _brute_dispatch(ids, E, rep)
    np.testing.assert_array_equal(perm, bperm)
    np.testing.assert_array_equal(inv, binv)
    assert offsets[-1] == perm.size == counts.sum()
    np.testing.assert_array_equal(np.diff(offsets), counts)


def test_condensed_layer_matches_token_by_token():
    p = _layer_inputs(8, T=12)
    x, k = p["x"], 2
    L = mo.router_logits(x, p["w_router"], None)
    ids, w = mo.topk_route(L, k)
    rep = np.arange(12)
    rep[5], rep[9] = 1, 3            # hand-made map (not from similarities)
    _, got = _run(p, k, rep)
    ref = np.zeros_like(got["out"])
    for t in range(12):
        for j in range(k):
            e = ids[t, j]
            srow = rep[t] if e in ids[rep[t]] else t
            _, Y = mo.swiglu_expert(x[srow:srow + 1], p["w_gate"][e], p["w_up"][e], p["w_down"][e], False)
            ref[t] += float(w[t, j]) * Y[0]
        _, S = mo.swiglu_expert(x[t:t + 1], p["wsh_gate"][0], p["wsh_up"][0], p["wsh_down"][0], False)
        ref[t] += S[0]
    np.testing.assert_allclose(got["out"], ref, rtol=1e-12, atol=1e-12)
