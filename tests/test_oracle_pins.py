"""Pins for the oracle: closed forms, library routines, invariants and brute force.

Each test ties an oracle function to something other than itself, chosen so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, a wrong tie rule) fails at least one of them.  CPU only.
"""
from fractions import Fraction

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe_oracle as mo




def _bf16_vals(rng, shape, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def _tiny(seed, T=24, d=16, E=6, k=2, I=8, ns=0, Is=8, bf16=True):
    rng = np.random.default_rng(seed)
    f = (lambda s, sc=1.0: _bf16_vals(rng, s, sc)) if bf16 else (
        lambda s, sc=1.0: (rng.standard_normal(s) * sc).astype(np.float32))
    sd = 1.0 / math.sqrt(d)
    p = dict(
        x=f((T, d)), w_router=f((E, d), sd), bias=rng.standard_normal(E).astype(np.float32) * 0.3,
        w_gate=f((E, I, d), sd), w_up=f((E, I, d), sd), w_down=f((E, d, I), sd))
    if ns:
        p.update(wsh_gate=f((ns, Is, d), sd), wsh_up=f((ns, Is, d), sd), wsh_down=f((ns, d, Is), sd))
    else:
        p.update(wsh_gate=None, wsh_up=None, wsh_down=None)
    return p


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        rng.standard_normal(2000) * 1e-39,  # float32 subnormals
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(v.astype(np.float64)), ref)


def test_bf16_round_ties_go_to_even():
    rng = np.random.default_rng(1)
    b = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    lo = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    hi = ((bits + 1).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2.0  # exact in float64
    even = np.where(bits % 2 == 0, lo, hi)
    np.testing.assert_array_equal(oracle.bf16_round(mid), even)
    # hand cases: spacing of bf16 next to 1.0 is 2^-7
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 1.0
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert oracle.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7  # above the tie
    assert oracle.bf16_round(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == -(1.0 + 2.0 ** -7)


# ---------------------------------------------------------------------------
# silu
# ---------------------------------------------------------------------------

def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    s = oracle.silu(-40.0)
    assert -1e-15 < s < 0.0
    z = np.linspace(-8, 8, 101)
    np.testing.assert_allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


# ---------------------------------------------------------------------------
# Router logits
# ---------------------------------------------------------------------------

def _f32_correct_round(fr: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even (search neighbours)."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda f: (abs(Fraction(float(f)) - fr),
                                      int(np.array(f).view(np.uint32)) & 1))
    return best


def test_router_logits_correctly_rounded():
    rng = np.random.default_rng(2)
    T, d, E = 5, 64, 7
    x = _bf16_vals(rng, (T, d))
    w = _bf16_vals(rng, (E, d), 1 / 8)
    b = rng.standard_normal(E).astype(np.float32)
    L = oracle.router_logits(x, w, b)
    assert L.dtype == np.float32
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, i])) * Fraction(float(w[e, i])) for i in range(d))
            exact += Fraction(float(b[e]))
            assert L[t, e] == _f32_correct_round(exact), (t, e)


def test_router_logits_orientation_and_bias():
    # x picks one coordinate; the logit must read W_r[e, that coordinate] + b[e]
    E, d = 4, 3
    w = np.arange(E * d, dtype=np.float32).reshape(E, d)
    b = np.array([10, 20, 30, 40], np.float32)
    x = np.eye(d, dtype=np.float32)
    L = oracle.router_logits(x, w, b)
    np.testing.assert_array_equal(L, (w.T + b[None, :]).astype(np.float32))
    np.testing.assert_array_equal(oracle.router_logits(x, w, None), w.T)


def test_lane_order_logits_exact_when_sums_are_exact():
    rng = np.random.default_rng(3)
    T, d, E = 6, 200, 5
    x = rng.integers(-8, 9, (T, d)).astype(np.float32)
    w = rng.integers(-8, 9, (E, d)).astype(np.float32)
    b = rng.integers(-8, 9, E).astype(np.float32)
    L = oracle.router_logits_f32_lane_order(x, w, b)
    np.testing.assert_array_equal(L, (x.astype(np.int64) @ w.T.astype(np.int64) + b).astype(np.float32))


def test_lane_order_logits_within_dot_product_bound():
    rng = np.random.default_rng(4)
    T, d, E = 16, 300, 9
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    L = oracle.router_logits_f32_lane_order(x, w, b).astype(np.float64)
    exact = x.astype(np.float64) @ w.T.astype(np.float64) + b
    u = 2.0 ** -24
    n = d + 1
    gamma = n * u / (1 - n * u)
    bound = gamma * (np.abs(x).astype(np.float64) @ np.abs(w).T.astype(np.float64) + np.abs(b)) + u * np.abs(exact)
    assert np.all(np.abs(L - exact) <= bound)
    assert np.any(L != exact.astype(np.float32))  # it is a genuinely different rounding order


def _one_logit(xv, d, bias=None):
    """Lane-order logit of one token against one all-ones router row, so that
    the products are the x values themselves (exact)."""
    x = np.zeros((1, d), np.float32)
    for i, v in xv.items():
        x[0, i] = v
    w = np.ones((1, d), np.float32)
    b = None if bias is None else np.array([bias], np.float32)
    return float(oracle.router_logits_f32_lane_order(x, w, b)[0, 0])


# Each case below is worked out by hand from the stated order (partial l
# takes i = l, l+64, ... ascending; separate multiply and add; butterfly over
# 32, 16, 8, 4, 2, 1; bias last) and chosen so that any other plausible order
# rounds to a different float32.  2^24 + 1 is a tie between 2^24 and 2^24 + 2
# and rounds to the even 2^24.
B24 = float(2 ** 24)


def test_lane_order_butterfly_runs_from_stride_32_down():
    # partials: p0 = 2^24, p1 = 1, p32 = -2^24.  Stride 32 first: p0 + p32 = 0
    # and p1 + p33 = 1; strides 16..2 add zeros; stride 1: 0 + 1 = 1.
    # From stride 1 up instead: p0 + p1 = 2^24 + 1 -> 2^24, then + (-2^24) = 0.
    got = _one_logit({0: B24, 1: 1.0, 32: -B24}, 64)
    assert got == 1.0
    exact = Fraction(int(B24)) + 1 - Fraction(int(B24))
    assert exact == 1  # here the stated order happens to be exact
    # a left-to-right sum loses the 1: (2^24 + 1) -> 2^24, minus 2^24
    seq = np.float32(0)
    for v in (B24, 1.0, -B24):
        seq = np.float32(seq + np.float32(v))
    assert float(seq) == 0.0


def test_lane_order_partials_take_every_64th_element():
    # d = 128.  Stated stride: partial 0 = p0 + p64 = 2^24 + 1 -> 2^24, partial
    # 1 = p1 = -2^24; butterfly: 2^24 + (-2^24) = 0 (the 1 was lost in lane 0).
    # Contiguous pairs (partial l = p_2l + p_2l+1) would give partial 0 =
    # 2^24 - 2^24 = 0 and partial 32 = p64 = 1, i.e. 1.
    got = _one_logit({0: B24, 64: 1.0, 1: -B24}, 128)
    assert got == 0.0


def test_lane_order_multiply_and_add_are_rounded_separately():
    # d = 128, one lane: partial 0 = p0 + p64 with p0 = (-1 - 2^-11) * 1 and
    # p64 = (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24 exactly, which rounds to
    # 1 + 2^-11 (a tie at half an ulp; 1 + 2^-11 is the even neighbour).  So
    # the partial is 0.  A fused multiply-add would keep the 2^-24.
    x = np.zeros((1, 128), np.float32)
    w = np.ones((1, 128), np.float32)
    x[0, 0] = -1.0 - 2.0 ** -11
    x[0, 64] = 1.0 + 2.0 ** -12
    w[0, 64] = 1.0 + 2.0 ** -12
    got = float(oracle.router_logits_f32_lane_order(x, w, None)[0, 0])
    assert got == 0.0
    exact = Fraction(x[0, 0].item()) + Fraction(x[0, 64].item()) * Fraction(w[0, 64].item())
    assert exact == Fraction(1, 2 ** 24)  # what a fused multiply-add would return


def test_lane_order_bias_is_added_after_the_butterfly():
    # partials p0 = p1 = 1: the butterfly gives 2, then + 2^24 = 2^24 + 2
    # (representable).  Adding the bias to partial 0 first would give
    # 2^24 + 1 -> 2^24, then + 1 -> 2^24.
    got = _one_logit({0: 1.0, 1: 1.0}, 64, bias=B24)
    assert got == B24 + 2.0


# ---------------------------------------------------------------------------
# Top-k gate
# ---------------------------------------------------------------------------

def _brute_topk(L, k):
    T, E = L.shape
    ids = np.empty((T, k), np.int64)
    for t in range(T):
        rank = []
        for e in range(E):
            r = sum(1 for f in range(E) if L[t, f] > L[t, e] or (L[t, f] == L[t, e] and f < e))
            rank.append(r)
        for e in range(E):
            if rank[e] < k:
                ids[t, rank[e]] = e
    return ids


@pytest.mark.parametrize("k", [1, 2, 3, 6])
def test_topk_matches_rank_count_with_ties(k):
    rng = np.random.default_rng(10 + k)
    L = (rng.integers(-3, 4, (200, 6)) / 2.0).astype(np.float32)  # heavy ties
    ids, w = oracle.topk_route(L, k)
    np.testing.assert_array_equal(ids, _brute_topk(L, k))
    for t in range(L.shape[0]):
        assert len(set(ids[t])) == k


def test_topk_negative_zero_ties_with_zero():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    ids, _ = oracle.topk_route(L, 2)
    np.testing.assert_array_equal(ids, [[0, 1], [0, 1]])


def test_topk_weights_sum_to_one_and_top1_is_one():
    rng = np.random.default_rng(5)
    L = (rng.standard_normal((500, 64)) * 3).astype(np.float32)
    for k in (1, 2, 6, 8, 16):
        _, w = oracle.topk_route(L, k)
        s = w.astype(np.float64).sum(axis=1)
        assert np.all(np.abs(s - 1.0) <= k * 2.0 ** -23)
        assert np.all(np.diff(w, axis=1) <= 0)  # descending logits -> descending weights
    _, w1 = oracle.topk_route(L, 1)
    assert np.all(w1 == 1.0)


def test_topk_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(6)
    L = (rng.standard_normal((100, 8)) * 2).astype(np.float32)
    ids, w = oracle.topk_route(L, 8)
    ref = scipy.special.softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=0, atol=1e-7)


def test_topk_shift_invariance():
    rng = np.random.default_rng(7)
    L = (rng.integers(-64, 64, (300, 16)) / 8.0).astype(np.float32)
    ids0, w0 = oracle.topk_route(L, 4)
    ids1, w1 = oracle.topk_route(L + np.float32(4.0), 4)  # exact shift
    np.testing.assert_array_equal(ids0, ids1)
    np.testing.assert_array_equal(w0, w1)


def test_topk_hand_example():
    # token 0: logits (2, 0, 1) -> experts (0, 2), weights e/(e+1), 1/(e+1)
    # token 1: logits (0, 1, 1) -> tie between 1 and 2: (1, 2), weights 1/2, 1/2
    L = np.array([[2, 0, 1], [0, 1, 1]], np.float32)
    ids, w = oracle.topk_route(L, 2)
    np.testing.assert_array_equal(ids, [[0, 2], [1, 2]])
    e = math.e
    np.testing.assert_allclose(w[0], [e / (e + 1), 1 / (e + 1)], rtol=0, atol=6e-8)
    np.testing.assert_array_equal(w[1], [0.5, 0.5])


def test_duplicated_router_row_resolves_to_lower_index():
    rng = np.random.default_rng(8)
    d, E = 32, 8
    x = _bf16_vals(rng, (400, d))
    w = _bf16_vals(rng, (E, d), 0.3)
    w[5] = w[2]  # expert 5 duplicates expert 2
    b = np.zeros(E, np.float32)
    L = oracle.router_logits(x, w, b)
    assert np.array_equal(L[:, 2], L[:, 5])
    ids, _ = oracle.topk_route(L, 3)
    both = [t for t in range(len(ids)) if 2 in ids[t] and 5 in ids[t]]
    assert both, "the duplicate pair never both made the top-k"
    for t in both:
        j2, j5 = list(ids[t]).index(2), list(ids[t]).index(5)
        assert j5 == j2 + 1
    # whenever 5 is chosen, 2 is chosen too
    assert all(2 in ids[t] for t in range(len(ids)) if 5 in ids[t])


# ---------------------------------------------------------------------------
# Dispatch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (37, 8, 2), (128, 16, 6), (64, 3, 3)])
def test_dispatch_is_a_stable_counting_sort(T, E, k):
    rng = np.random.default_rng(T * 131 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.dispatch(ids, E)
    flat = ids.ravel()
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)
    np.testing.assert_array_equal(np.sort(perm), np.arange(T * k))  # bijection
    np.testing.assert_array_equal(inv[perm], np.arange(T * k))
    np.testing.assert_array_equal(perm[inv], np.arange(T * k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_dispatch_edge_cases():
    counts, offsets, perm, inv = oracle.dispatch(np.zeros((0, 2), np.int32), 4)
    assert perm.size == 0 and np.all(counts == 0) and np.all(offsets == 0)
    ids = np.full((10, 1), 3, np.int32)  # everything to one expert
    counts, offsets, perm, inv = oracle.dispatch(ids, 5)
    np.testing.assert_array_equal(counts, [0, 0, 0, 10, 0])
    np.testing.assert_array_equal(offsets, [0, 0, 0, 0, 10, 10])
    np.testing.assert_array_equal(perm, np.arange(10))


def test_gather_rows_reads_token_of_each_assignment():
    rng = np.random.default_rng(9)
    T, E, k, d = 20, 5, 2, 4
    x = rng.standard_normal((T, d))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    _, _, perm, inv = oracle.dispatch(ids, E)
    xs = oracle.gather_rows(x, perm, k)
    for a in range(T * k):
        np.testing.assert_array_equal(xs[inv[a]], x[a // k])


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def test_identity_experts_top1_return_input_bitwise():
    p = _tiny(20, T=40, E=5, k=1)
    r = oracle.moe_layer(p["x"], p["w_router"], p["bias"], None, None, None, 1,
                         expert_fn=lambda e, X: np.asarray(X, np.float64))
    assert np.all(r["w"] == 1.0)
    np.testing.assert_array_equal(r["out"], p["x"].astype(np.float64))


@pytest.mark.parametrize("ns", [0, 2])
@pytest.mark.parametrize("k", [1, 2, 6])
def test_layer_matches_dense_bruteforce_unrounded(k, ns):
    p = _tiny(30 + k + ns, T=32, d=16, E=6, k=k, I=8, ns=ns, Is=8)
    r = oracle.moe_layer(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], k,
                         p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=False)
    dense = oracle.moe_layer_dense(p["x"], r["logits"], p["w_gate"], p["w_up"], p["w_down"], k,
                                   p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=False)
    np.testing.assert_allclose(r["out"], dense, rtol=1e-10, atol=1e-12)


def test_layer_matches_dense_bruteforce_bf16_a():
    k, ns = 2, 1
    p = _tiny(40, T=48, d=16, E=6, k=k, I=8, ns=ns, Is=16)
    r = oracle.moe_layer(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], k,
                         p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=True)
    dense = oracle.moe_layer_dense(p["x"], r["logits"], p["w_gate"], p["w_up"], p["w_down"], k,
                                   p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=True)
    close = np.isclose(r["out"], dense, rtol=1e-10, atol=1e-12)
    assert close.mean() > 0.99
    np.testing.assert_allclose(r["out"], dense, rtol=2e-2, atol=2e-2)
    # A really is rounded to bf16 and really differs from the unrounded product
    np.testing.assert_array_equal(r["A"], oracle.bf16_round(r["A"]))
    r32 = oracle.moe_layer(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], k,
                           p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=False)
    assert not np.array_equal(r32["A"], r["A"])


def test_down_projection_scaling_is_exact():
    k = 2
    p = _tiny(50, T=32, k=k, ns=1)
    args = (p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"])
    r1 = oracle.moe_layer(*args, p["w_down"], k, p["wsh_gate"], p["wsh_up"], p["wsh_down"])
    r2 = oracle.moe_layer(*args, 2 * p["w_down"], k, p["wsh_gate"], p["wsh_up"], 2 * p["wsh_down"])
    np.testing.assert_array_equal(r2["y_sorted"], 2 * r1["y_sorted"])
    np.testing.assert_array_equal(r2["out"], 2 * r1["out"])


def test_token_permutation_equivariance():
    k = 2
    p = _tiny(60, T=30, k=k, ns=1)
    r = oracle.moe_layer(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], k,
                         p["wsh_gate"], p["wsh_up"], p["wsh_down"])
    pi = np.random.default_rng(0).permutation(30)
    r2 = oracle.moe_layer(p["x"][pi], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], k,
                          p["wsh_gate"], p["wsh_up"], p["wsh_down"])
    np.testing.assert_array_equal(r2["ids"], r["ids"][pi])
    np.testing.assert_allclose(r2["out"], r["out"][pi], rtol=1e-12, atol=1e-12)


def test_expert_relabelling_invariance():
    k, E = 2, 6
    p = _tiny(70, T=40, E=E, k=k)
    r = oracle.moe_layer(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], k)
    sigma = np.array([3, 0, 5, 1, 4, 2])  # new expert sigma[e] is old expert e
    inv = np.argsort(sigma)
    r2 = oracle.moe_layer(p["x"], p["w_router"][inv], p["bias"][inv], p["w_gate"][inv],
                          p["w_up"][inv], p["w_down"][inv], k)
    np.testing.assert_array_equal(r2["ids"], sigma[r["ids"]])
    np.testing.assert_allclose(r2["out"], r["out"], rtol=1e-12, atol=1e-12)


def test_combine_hand_example():
    # two tokens, k = 2, d = 2; y_sorted rows placed by inv_perm
    y = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    inv = np.array([2, 0, 3, 1])  # token 0 -> rows 2, 0 ; token 1 -> rows 3, 1
    w = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    sh = np.array([[100.0, 200.0], [300.0, 400.0]])
    out = oracle.combine(y, inv, w, sh, 2)
    np.testing.assert_array_equal(out, [[0.75 * 5 + 0.25 * 1 + 100, 0.75 * 6 + 0.25 * 2 + 200],
                                        [0.5 * 7 + 0.5 * 3 + 300, 0.5 * 8 + 0.5 * 4 + 400]])


def test_token_outputs_agree_with_batched_layer():
    k = 3
    p = _tiny(80, T=50, E=7, k=k, ns=2)
    r = oracle.moe_layer(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"], p["w_down"], k,
                         p["wsh_gate"], p["wsh_up"], p["wsh_down"])
    toks = np.array([0, 7, 13, 49])
    ids, w, out = oracle.token_outputs(toks, p["x"], r["logits"], p["w_gate"], p["w_up"], p["w_down"], k,
                                       p["wsh_gate"], p["wsh_up"], p["wsh_down"])
    np.testing.assert_array_equal(ids, r["ids"][toks])
    np.testing.assert_array_equal(w, r["w"][toks])
    np.testing.assert_allclose(out, r["out"][toks], rtol=1e-9, atol=1e-12)


def test_swiglu_expert_hand_example():
    # one row x = (1, 2), I = 1: g = x.wg = 3, u = x.wu = -1, A = silu(3) * -1
    X = np.array([[1.0, 2.0]])
    wg = np.array([[1.0, 1.0]])
    wu = np.array([[1.0, -1.0]])
    wd = np.array([[2.0], [-3.0]])  # d = 2, I = 1
    A, Y = oracle.swiglu_expert(X, wg, wu, wd, round_a=False)
    a = -3.0 / (1.0 + math.exp(-3.0))
    assert A[0, 0] == pytest.approx(a, rel=1e-15)
    np.testing.assert_allclose(Y[0], [2 * a, -3 * a], rtol=1e-15)
