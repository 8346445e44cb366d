"""GPU parity: every entry point of the C ABI against the oracle, on seeded
inputs sized so the oracle finishes in seconds while the GPU path still spans
several tiles and ragged tails, plus edge cases (one token, one expert, the
maximum expert count and top-k, empty experts, T = 0)."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_synth import MoEShape

pytestmark = pytest.mark.gpu

CASES = {
    # about 175 rows per expert (one ragged 256-row tile each), 3 column tiles,
    # one shared expert
    "med_bf16_shared": MoEShape("med_bf16_shared", T=700, d=256, E=16, k=4, I=384, n_shared=1,
                                I_shared=256, seed=11, bias="normal"),
    # column counts that end half way through a 128-wide tile, two shared experts
    "med_bf16_ragged": MoEShape("med_bf16_ragged", T=333, d=192, E=8, k=2, I=320, n_shared=2,
                                I_shared=192, seed=12),
    # skewed load with experts that receive no token
    "med_bf16_zipf": MoEShape("med_bf16_zipf", T=512, d=128, E=32, k=4, I=128, seed=13, bias="zipf",
                             zipf_alpha=1.5),
    "tiny_fp32": moe_synth.CONFIGS["tiny_fp32"],
    "fp32_ragged": MoEShape("fp32_ragged", T=150, d=64, E=6, k=3, I=192, n_shared=1, I_shared=64,
                            dtype="f32", seed=14),
    "max_experts": MoEShape("max_experts", T=100, d=64, E=256, k=16, I=64, seed=15),
    "one_expert": MoEShape("one_expert", T=300, d=128, E=1, k=1, I=128, n_shared=1, I_shared=64,
                           seed=16),
    "one_token": MoEShape("one_token", T=1, d=128, E=8, k=2, I=128, n_shared=1, I_shared=128, seed=17),
}

_cache = {}


def case(name):
    if name not in _cache:
        import gpu_helpers as gh
        cfg = CASES[name]
        arrays = moe_synth.generate(cfg)
        if cfg.dtype == "f32":
            L = oracle.router_logits_f32_lane_order(arrays["x"], arrays["w_router"], arrays["bias"])
        else:
            L = oracle.router_logits(arrays["x"], arrays["w_router"], arrays["bias"])
        ref = oracle.moe_layer(arrays["x"], arrays["w_router"], arrays["bias"], arrays["w_gate"],
                               arrays["w_up"], arrays["w_down"], cfg.k, arrays["wsh_gate"],
                               arrays["wsh_up"], arrays["wsh_down"], round_a=cfg.dtype == "bf16",
                               logits=L)
        print(f"[case {name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} I={cfg.I} "
              f"shared={cfg.n_shared}x{cfg.I_shared} {cfg.dtype}", flush=True)
        _cache[name] = (cfg, arrays, ref, gh.Layer(cfg, arrays))
    return _cache[name]


ALL = list(CASES)
BF16 = [n for n in ALL if CASES[n].dtype == "bf16"]


@pytest.mark.parametrize("name", ALL)
def test_route_from_given_logits(name):
    cfg, arrays, ref, lay = case(name)
    ids, w, L = lay.route(logits_in=ref["logits"])
    np.testing.assert_array_equal(L, ref["logits"])
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.abs(w.astype(np.float64) - ref["w"]).max() <= 2e-6


def test_route_from_given_logits_with_ties():
    cfg = CASES["med_bf16_zipf"]
    import gpu_helpers as gh
    rng = np.random.default_rng(99)
    L = (rng.integers(-3, 4, (cfg.T, cfg.E)) / 2.0).astype(np.float32)
    L[::7] = -0.0
    L[1::7, ::2] = 0.0
    ids_ref, w_ref = oracle.topk_route(L, cfg.k)
    ids, w, L_out = case("med_bf16_zipf")[3].route(logits_in=L)
    np.testing.assert_array_equal(ids, ids_ref)
    assert np.abs(w.astype(np.float64) - w_ref).max() <= 2e-6


@pytest.mark.parametrize("name", ALL)
def test_route_computed_logits(name):
    import gpu_helpers as gh
    cfg, arrays, ref, lay = case(name)
    ids, w, L = lay.route()
    gh.check_topk_of_own_logits(L, ids, cfg.k)
    if cfg.dtype == "f32":
        # the float32 router's operation order is replayed exactly by the oracle
        np.testing.assert_array_equal(L, ref["logits"])
        np.testing.assert_array_equal(ids, ref["ids"])
        assert np.abs(w.astype(np.float64) - ref["w"]).max() <= 2e-6
        return
    bound = gh.logits_bound(arrays["x"], arrays["w_router"], arrays["bias"], ref["logits"])
    dL = np.abs(L.astype(np.float64) - ref["logits"])
    assert np.all(dL <= bound), f"logits outside the dot-product bound: {(dL / bound).max():.2f}x"
    differ = gh.certify_routing(ids, ref["ids"], ref["logits"], bound)
    same = np.setdiff1d(np.arange(cfg.T), differ)
    tol = 2e-6 + 2.0 * dL.max()
    assert np.abs(w[same].astype(np.float64) - ref["w"][same]).max() <= tol


# Shapes for the router that holds W_r in registers (bf16, E <= 64, d one of
# 256, 512, 1024, 2048), each with more 16-token groups than the GPU has CUs,
# so that blocks walk several groups and the last group is ragged.
RESIDENT_ROUTE = {
    "res_e40_d512": MoEShape("res_e40_d512", T=4500, d=512, E=40, k=4, I=64, seed=31,
                             bias="normal"),
    "res_e16_d1024": MoEShape("res_e16_d1024", T=9001, d=1024, E=16, k=2, I=64, seed=32),
    "res_e32_d256": MoEShape("res_e32_d256", T=4205, d=256, E=32, k=3, I=64, seed=33,
                             bias="normal"),
    "res_e64_d2048": MoEShape("res_e64_d2048", T=8200, d=2048, E=64, k=6, I=64, seed=34),
}


@pytest.mark.parametrize("name", list(RESIDENT_ROUTE))
def test_route_register_resident(name):
    """Logits within the dot-product bound of the oracle's, ids the oracle's
    top-k up to certified near ties, weights within tolerance elsewhere."""
    import gpu_helpers as gh
    cfg = RESIDENT_ROUTE[name]
    print(f"[route {name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k}", flush=True)
    arrays = moe_synth.generate(cfg, workers=16)
    lay = gh.Layer(cfg, arrays)
    ids, w, L = lay.route()
    gh.check_topk_of_own_logits(L, ids, cfg.k)
    L_ref = oracle.router_logits(arrays["x"], arrays["w_router"], arrays["bias"])
    ids_ref, w_ref = oracle.topk_route(L_ref, cfg.k)
    bound = gh.logits_bound(arrays["x"], arrays["w_router"], arrays["bias"], L_ref)
    dL = np.abs(L.astype(np.float64) - L_ref)
    assert np.all(dL <= bound), f"logits outside the dot-product bound: {(dL / bound).max():.2f}x"
    differ = gh.certify_routing(ids, ids_ref, L_ref, bound)
    same = np.setdiff1d(np.arange(cfg.T), differ)
    assert np.abs(w[same].astype(np.float64) - w_ref[same]).max() <= 2e-6 + 2.0 * dL.max()


@pytest.mark.parametrize("name", ALL)
def test_dispatch_bit_exact(name):
    cfg, arrays, ref, lay = case(name)
    got = lay.dispatch(ref["ids"])
    for key in ("counts", "offsets", "perm", "inv_perm"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    xs = got["x_sorted"].float().cpu().numpy()
    np.testing.assert_array_equal(xs, ref["x_sorted"].astype(np.float32))


def test_dispatch_everything_to_one_expert():
    cfg, arrays, ref, lay = case("med_bf16_shared")
    ids = np.tile(np.array([5, 2, 9, 0], np.int32), (cfg.T, 1))
    got = lay.dispatch(ids)
    counts, offsets, perm, inv = oracle.dispatch(ids, cfg.E)
    np.testing.assert_array_equal(got["counts"], counts)
    np.testing.assert_array_equal(got["offsets"], offsets)
    np.testing.assert_array_equal(got["perm"], perm)
    np.testing.assert_array_equal(got["inv_perm"], inv)


@pytest.mark.parametrize("name", ALL)
def test_grouped_ffn(name):
    import gpu_helpers as gh
    cfg, arrays, ref, lay = case(name)
    got = lay.ffn(ref["x_sorted"], ref["offsets"])
    if cfg.dtype == "bf16":
        gh.check_swiglu_a(got["A"], ref["A"], ref["x_sorted"], ref["offsets"], arrays["w_gate"],
                          arrays["w_up"])
        gh.assert_fp_close(got["y_sorted"], ref["y_sorted"], "y_sorted")
        if cfg.n_shared:
            Is = cfg.I_shared
            for s_ in range(cfg.n_shared):
                cols = slice(s_ * Is, (s_ + 1) * Is)
                gh.check_swiglu_a(got["A_shared"][:, cols], ref["A_shared"][:, cols], arrays["x"],
                                  [0, cfg.T], arrays["wsh_gate"][s_:s_ + 1],
                                  arrays["wsh_up"][s_:s_ + 1], what=f"A_shared[{s_}]")
            gh.assert_fp_close(got["y_shared"], ref["y_shared"], "y_shared")
    else:
        gh.assert_fp_close(got["A"], ref["A"], "A", mean_abs=1e-5, max_rel=1e-4)
        gh.assert_fp_close(got["y_sorted"], ref["y_sorted"], "y_sorted", mean_abs=1e-5, max_rel=1e-4)
        if cfg.n_shared:
            gh.assert_fp_close(got["y_shared"], ref["y_shared"], "y_shared", mean_abs=1e-5, max_rel=1e-4)


@pytest.mark.parametrize("name", ALL)
def test_combine(name):
    import gpu_helpers as gh
    cfg, arrays, ref, lay = case(name)
    ysh = ref["y_shared"].astype(np.float32) if ref["y_shared"] is not None else None
    y32 = ref["y_sorted"].astype(np.float32)
    out = lay.combine(y32, ref["inv_perm"], ref["w"], ysh)
    exp = oracle.combine(y32, ref["inv_perm"], ref["w"], ysh, cfg.k)
    gh.assert_fp_close(out, exp, "out", mean_abs=1e-6, max_rel=1e-5)


def test_dispatch_then_combine_identity_round_trip():
    """Top-1, weight 1, expert output := the dispatched row: out == x bitwise."""
    cfg = CASES["med_bf16_ragged"].replace(k=1, n_shared=0, I_shared=0)
    import gpu_helpers as gh
    arrays = moe_synth.generate(cfg)
    lay = gh.Layer(cfg, arrays)
    ids = np.random.default_rng(5).integers(0, cfg.E, (cfg.T, 1)).astype(np.int32)
    got = lay.dispatch(ids)
    y = got["x_sorted"].float().cpu().numpy()
    out = lay.combine(y, got["inv_perm"], np.ones((cfg.T, 1), np.float32), None)
    np.testing.assert_array_equal(out, arrays["x"])


@pytest.mark.parametrize("name", ALL)
def test_layer(name):
    import gpu_helpers as gh
    cfg, arrays, ref, lay = case(name)
    got = lay.layer()
    if cfg.dtype == "f32":
        np.testing.assert_array_equal(got["ids"], ref["ids"])
        same = np.arange(cfg.T)
    else:
        bound = gh.logits_bound(arrays["x"], arrays["w_router"], arrays["bias"], ref["logits"])
        differ = gh.certify_routing(got["ids"], ref["ids"], ref["logits"], bound)
        same = np.setdiff1d(np.arange(cfg.T), differ)
        if differ.size:
            print(f"[case {name}] {differ.size} certified near-tie tokens routed differently")
    if same.size == cfg.T:
        for key in ("counts", "offsets", "perm"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    tol = dict(mean_abs=1e-5, max_rel=1e-4) if cfg.dtype == "f32" else {}
    gh.assert_fp_close(got["out"][same], ref["out"][same], "out", **tol)


@pytest.mark.parametrize("name", ["med_bf16_shared", "tiny_fp32", "max_experts"])
def test_layer_is_deterministic(name):
    cfg, arrays, ref, lay = case(name)
    a = lay.layer()
    b = lay.layer()
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


@pytest.mark.parametrize("name", ["med_bf16_shared", "med_bf16_zipf", "one_expert"])
def test_gemm_load_variants_agree(name):
    """The bf16 grouped GEMMs have two operand-load variants: buffer loads with
    32-bit offsets (used whenever every offset fits) and 64-bit global loads
    (otherwise; asked for here through moe_layer_fwd_variant with
    MOE_VARIANT_GLOBAL_LOADS).  Both give the same layer outputs bit for bit
    (test_layer holds the default call to the oracle)."""
    import expert_routing_grouped_route_amd as moe
    cfg, arrays, ref, lay = case(name)
    a = lay.layer()
    b = lay.layer(variant=moe.MOE_VARIANT_GLOBAL_LOADS)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


@pytest.mark.parametrize("name", ALL)
def test_layer_overlap_matches_single_stream(name):
    """The shared experts on a second stream give bit-identical results (same
    kernels and tiles, only the launch streams differ), on two calls in a row."""
    cfg, arrays, ref, lay = case(name)
    a = lay.layer()
    for _ in range(2):
        b = lay.layer_overlap()
        for key in a:
            np.testing.assert_array_equal(b[key], a[key], err_msg=key)


def test_down_projection_scaling_is_exact():
    cfg, arrays, ref, lay = case("med_bf16_shared")
    a = lay.layer()
    b = lay.layer(w_down_scale=2.0)
    np.testing.assert_array_equal(b["ids"], a["ids"])
    np.testing.assert_array_equal(b["out"], 2.0 * a["out"])


def test_zero_tokens_layer_writes_zero_counts():
    import expert_routing_grouped_route_amd as moe
    cfg, arrays, ref, lay = case("med_bf16_shared")
    t = lay.t
    d = moe.dims(0, cfg.d, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.I_shared, cfg.dtype)
    ws_bytes = moe.moe_workspace_bytes(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    counts = torch.full((cfg.E,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((cfg.E + 1,), 7, dtype=torch.int32, device="cuda")
    moe.moe_layer_fwd(d, None, t["w_router"], t["bias"], t["w_gate"], t["w_up"], t["w_down"],
                      t["wsh_gate"], t["wsh_up"], t["wsh_down"], None, None, None, counts, offsets,
                      None, ws, ws_bytes)
    torch.cuda.synchronize()
    assert torch.all(counts == 0) and torch.all(offsets == 0)
