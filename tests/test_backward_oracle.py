"""Pins of the backward-pass oracle (oracle/moe_backward.py).

Each pin is independent of the oracle's own chain-rule code:
  * central finite differences of the brute-force dense forward pass
    (``moe_layer_dense``: every expert on every token, masked), in float64,
    for a random direction in every input;
  * k = 1: the kept weight is 1 whatever the logits, so the router gets no
    gradient (exactly zero);
  * k = E: the renormalised softmax is the full softmax, whose Jacobian is
    diag(p) - p p^T (p from scipy's softmax);
  * W_down x 2 scales every gradient but dW_down by exactly 2;
  * the gradients are linear in the upstream gradient;
  * silu'(g) against finite differences and silu'(0) = 1/2.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import moe_backward as mb


def _params(seed, T=5, d=8, E=4, k=2, I=6, ns=1, Is=4):
    rng = np.random.default_rng(seed)
    p = dict(
        x=rng.normal(size=(T, d)),
        w_router=rng.normal(size=(E, d)) / np.sqrt(d),
        bias=rng.normal(size=E) * 0.3,
        w_gate=rng.normal(size=(E, I, d)) / np.sqrt(d),
        w_up=rng.normal(size=(E, I, d)) / np.sqrt(d),
        w_down=rng.normal(size=(E, d, I)) / np.sqrt(I),
    )
    if ns:
        p.update(wsh_gate=rng.normal(size=(ns, Is, d)) / np.sqrt(d),
                 wsh_up=rng.normal(size=(ns, Is, d)) / np.sqrt(d),
                 wsh_down=rng.normal(size=(ns, d, Is)) / np.sqrt(Is))
    else:
        p.update(wsh_gate=None, wsh_up=None, wsh_down=None)
    return p


def _logits64(p):
    return p["x"] @ p["w_router"].T + p["bias"][None, :]


def _min_gap(L, k):
    s = -np.sort(-L, axis=1)
    return (s[:, k - 1] - s[:, k]).min() if k < L.shape[1] else np.inf


def _loss(p, dout, k):
    out = oracle.moe_layer_dense(p["x"], _logits64(p), p["w_gate"], p["w_up"], p["w_down"], k,
                                 p["wsh_gate"], p["wsh_up"], p["wsh_down"], round_a=False,
                                 gate_f32=False)
    return float((dout * out).sum())


def _backward(p, dout, k, round_a=False):
    return mb.moe_layer_backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"],
                                 p["w_down"], k, dout, p["wsh_gate"], p["wsh_up"],
                                 p["wsh_down"], round_a=round_a, logits=_logits64(p))


GRAD_OF = {"x": "dx", "w_router": "dw_router", "bias": "dbias", "w_gate": "dw_gate",
           "w_up": "dw_up", "w_down": "dw_down", "wsh_gate": "dwsh_gate",
           "wsh_up": "dwsh_up", "wsh_down": "dwsh_down"}


@pytest.mark.parametrize("k,ns", [(2, 1), (1, 0), (3, 2), (4, 1)])
def test_gradients_match_finite_differences_of_dense_forward(k, ns):
    seed = 0
    while True:  # a tie-free case: the kept set does not change under the perturbation
        p = _params(seed, k=k, ns=ns)
        if _min_gap(_logits64(p), k) > 1e-2:
            break
        seed += 1
    rng = np.random.default_rng(100 + seed)
    dout = rng.normal(size=p["x"].shape)
    g = _backward(p, dout, k)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if p[name] is None:
            assert g[gname] is None
            continue
        v = rng.normal(size=p[name].shape)
        pp = dict(p)
        pm = dict(p)
        pp[name] = p[name] + eps * v
        pm[name] = p[name] - eps * v
        fd = (_loss(pp, dout, k) - _loss(pm, dout, k)) / (2 * eps)
        an = float((g[gname] * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_top1_router_gets_no_gradient():
    p = _params(3, k=1)
    dout = np.random.default_rng(4).normal(size=p["x"].shape)
    g = _backward(p, dout, 1)
    assert np.all(g["dlogits_kept"] == 0.0)
    assert np.all(g["dw_router"] == 0.0) and np.all(g["dbias"] == 0.0)


def test_k_equals_E_router_gradient_is_the_softmax_jacobian():
    E = 4
    p = _params(5, E=E, k=E)
    dout = np.random.default_rng(6).normal(size=p["x"].shape)
    g = _backward(p, dout, E)
    L = _logits64(p)
    P = softmax(L, axis=1)
    # dw on each expert (slot order -> expert order)
    dw_e = np.zeros_like(L)
    np.put_along_axis(dw_e, g["ids"].astype(np.int64), g["dw"], axis=1)
    dL_ref = np.stack([(np.diag(P[t]) - np.outer(P[t], P[t])) @ dw_e[t] for t in range(L.shape[0])])
    np.testing.assert_allclose(g["dlogits_kept"],
                               np.take_along_axis(dL_ref, g["ids"].astype(np.int64), axis=1),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dbias"], dL_ref.sum(axis=0), rtol=1e-12, atol=1e-14)


def test_down_projection_scaling_is_exact():
    p = _params(7, ns=0)
    dout = np.random.default_rng(8).normal(size=p["x"].shape)
    g1 = _backward(p, dout, 2, round_a=True)
    p2 = dict(p)
    p2["w_down"] = p["w_down"] * 2.0
    g2 = _backward(p2, dout, 2, round_a=True)
    for n in ("dx", "dw_router", "dbias", "dw_gate", "dw_up"):
        assert np.array_equal(g2[n], 2.0 * g1[n]), n
    assert np.array_equal(g2["dw_down"], g1["dw_down"])


def test_gradients_are_linear_in_dout():
    p = _params(9, k=2, ns=1)
    rng = np.random.default_rng(10)
    a = rng.normal(size=p["x"].shape)
    b = rng.normal(size=p["x"].shape)
    ga, gb, gab = _backward(p, a, 2), _backward(p, b, 2), _backward(p, a + 2 * b, 2)
    for n in GRAD_OF.values():
        np.testing.assert_allclose(gab[n], ga[n] + 2 * gb[n], rtol=1e-10, atol=1e-12)


def test_silu_grad_closed_form_and_finite_differences():
    assert mb.silu_grad(0.0) == 0.5
    z = np.linspace(-8, 8, 41)
    eps = 1e-6
    fd = (oracle.silu(z + eps) - oracle.silu(z - eps)) / (2 * eps)
    np.testing.assert_allclose(mb.silu_grad(z), fd, rtol=1e-7, atol=1e-9)


@pytest.mark.parametrize("k,ns,round_a", [(2, 1, True), (1, 0, False), (3, 2, True)])
def test_backward_parts_agree_with_whole_backward(k, ns, round_a):
    """moe_layer_backward_parts (the restriction used at full size) returns,
    for the experts and tokens asked for, what the whole backward returns:
    the router and shared gradients whole, the listed experts' weight
    gradients (zero for an expert without tokens) and dx of the listed tokens
    (a token twice, in any order).  Pinned through the whole backward, which
    the finite-difference pins above tie to the dense forward."""
    p = _params(40 + k, T=14, d=8, E=6, k=k, I=6, ns=ns)
    p["bias"] = np.array([2.0, 1.5, 1.0, -1.0, -6.0, -9.0])  # experts 4, 5 get few or none
    dout = np.random.default_rng(7).normal(size=(14, 8))
    whole = mb.moe_layer_backward(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"],
                                  p["w_down"], k, dout, p["wsh_gate"], p["wsh_up"], p["wsh_down"],
                                  round_a=round_a)
    counts = np.diff(np.asarray(whole["offsets"]))
    empty = [int(e) for e in np.nonzero(counts == 0)[0]]
    assert empty, "the case should leave an expert without tokens"
    experts = [int(np.argmax(counts)), empty[0], 2]
    tokens = [13, 0, 5, 5, 9]
    part = mb.moe_layer_backward_parts(p["x"], p["w_router"], p["bias"], p["w_gate"], p["w_up"],
                                       p["w_down"], k, dout, p["wsh_gate"], p["wsh_up"],
                                       p["wsh_down"], round_a=round_a, experts=experts,
                                       tokens=tokens)
    close = dict(rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(part["dx"], whole["dx"][tokens], **close)
    np.testing.assert_allclose(part["dw_router"], whole["dw_router"], **close)
    np.testing.assert_allclose(part["dbias"], whole["dbias"], **close)
    for e in experts:
        for n in ("dw_gate", "dw_up", "dw_down"):
            np.testing.assert_allclose(part[n][e], whole[n][e], **close)
    assert np.all(part["dw_gate"][empty[0]] == 0.0)
    for n in ("dwsh_gate", "dwsh_up", "dwsh_down"):
        if ns:
            np.testing.assert_allclose(part[n], whole[n], **close)
        else:
            assert part[n] is None and whole[n] is None
