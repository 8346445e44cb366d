"""The seeded input recipes: determinism, representability and workload shape."""
import math

import numpy as np
import pytest

import moe_synth
import oracle


def test_generation_is_deterministic_and_per_tensor():
    cfg = moe_synth.MoEShape("t", T=100, d=64, E=8, k=2, I=64, n_shared=1, I_shared=64, seed=5)
    a = moe_synth.generate(cfg)
    b = moe_synth.generate(cfg, names=["w_up", "x"])  # a subset, in another order
    np.testing.assert_array_equal(a["x"], b["x"])
    np.testing.assert_array_equal(a["w_up"], b["w_up"])
    c = moe_synth.generate(cfg.replace(seed=6), names=["x"])
    assert not np.array_equal(a["x"], c["x"])


def test_bf16_inputs_are_representable_and_f32_inputs_are_not_rounded():
    cfg = moe_synth.MoEShape("t", T=64, d=64, E=4, k=2, I=64, n_shared=1, I_shared=64, seed=1)
    a = moe_synth.generate(cfg)
    for name in ("x", "w_router", "w_gate", "w_up", "w_down", "wsh_gate", "wsh_up", "wsh_down"):
        np.testing.assert_array_equal(oracle.bf16_round(a[name].astype(np.float64)), a[name])
    f = moe_synth.generate(cfg.replace(dtype="f32"), names=["x"])
    assert not np.array_equal(oracle.bf16_round(f["x"].astype(np.float64)), f["x"])


def test_weight_scale_is_one_over_d_variance():
    cfg = moe_synth.MoEShape("t", T=8, d=256, E=4, k=1, I=512, seed=2)
    a = moe_synth.generate(cfg, names=["w_gate", "w_down", "w_router"])
    for name in ("w_gate", "w_down", "w_router"):
        v = a[name].astype(np.float64).var()
        assert v == pytest.approx(1.0 / cfg.d, rel=0.05), name


def test_zipf_bias_leaves_an_expert_without_tokens():
    cfg = moe_synth.CONFIGS["qwen3_30b_a3b"]
    a = moe_synth.generate(cfg, names=["x", "w_router", "bias"])
    ids, _ = oracle.topk_route(oracle.router_logits(a["x"], a["w_router"], a["bias"]), cfg.k)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    assert (counts == 0).sum() >= 1
    assert counts.max() > 0.9 * cfg.T  # one very hot expert


def test_normal_bias_skews_load_mildly():
    cfg = moe_synth.CONFIGS["deepseek_v2_lite"]
    a = moe_synth.generate(cfg, names=["x", "w_router", "bias"])
    assert a["bias"].std() == pytest.approx(math.sqrt(0.5), rel=0.3)
    ids, _ = oracle.topk_route(oracle.router_logits(a["x"], a["w_router"], a["bias"]), cfg.k)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    assert counts.min() > 0 and 2.0 < counts.max() / counts.mean() < 12.0


def test_duplicated_rows_recipe():
    cfg = moe_synth.CONFIGS["prefill_stress"].replace(T=1024)
    a = moe_synth.generate(cfg, names=["x"])
    x = a["x"].astype(np.float64)
    # a duplicated row sits within the noise of some earlier row
    n = x.shape[0]
    sq = (x ** 2).sum(1)
    near = 0
    for i in range(1, n):
        d2 = sq[:i] + sq[i] - 2 * x[:i] @ x[i]
        if d2.min() < 0.01 * cfg.d:  # noise variance 1e-3 per element -> ~2 units over d=2048
            near += 1
    assert near == pytest.approx(math.floor(0.3 * n), abs=5)
