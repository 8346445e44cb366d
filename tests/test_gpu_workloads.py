"""GPU parity at the full sizes of the five model-shaped workloads, in the
launch configuration the benchmark times (one moe_layer_fwd call on one
stream), compared with the oracle element by element.

On every workload:
  * logits: moe_route's logits (the router kernel the layer runs) lie within
    the float32 dot-product bound of the oracle's (bf16 layers), or equal the
    oracle's replay of the float32 lane order bit for bit (fp32 layer);
  * routing: the layer's ids are the oracle's top-k of those same logits bit
    for bit, with weights within 2e-6; against the oracle's own logits a token
    may differ only where it is a certified near tie;
  * dispatch: counts, offsets and perm equal the oracle's counting sort of the
    same ids bit for bit;
  * output: every element of out against the oracle's layer routed on the
    GPU's logits (so a certified tie cannot become a whole-row mismatch);
  * layers with shared experts: the two-stream entry point gives the one-stream
    output bit for bit, and is checked against the oracle directly too.
On the DeepSeek-V2-Lite- and Qwen3-30B-A3B-shaped workloads also the
standalone entry points at full size: moe_dispatch (x_sorted bit-exact) and
moe_grouped_ffn (the SwiGLU products A within their rounding bound, y_sorted
and the shared experts' output within tolerance).
The oracle runs the whole layer in fp64 on the host: about 1 s for the
DeepSeek-V2-Lite shape and 10-20 s for the Llama-4-Scout and prefill shapes on
16 cores."""
import time

import numpy as np
import pytest

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

FFN_FULL = ("deepseek_v2_lite", "qwen3_30b_a3b")


def _say(name, msg, t0):
    print(f"[workload {name}] {msg} ({time.time() - t0:.1f} s)", flush=True)


@pytest.mark.parametrize("name", moe_synth.CONFIG_ORDER)
def test_workload(name):
    import gpu_helpers as gh
    t0 = time.time()
    cfg = moe_synth.CONFIGS[name]
    print(f"[workload {name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} I={cfg.I} "
          f"shared={cfg.n_shared}x{cfg.I_shared} {cfg.dtype}", flush=True)
    a = moe_synth.generate(cfg, workers=16)
    lay = gh.Layer(cfg, a)
    got = lay.layer()
    ids_r, w_r, L_gpu = lay.route()
    _say(name, "GPU layer and router done", t0)
    np.testing.assert_array_equal(got["ids"], ids_r)   # the layer routes as moe_route
    np.testing.assert_array_equal(got["w"], w_r)

    # logits and routing against the oracle's own logits
    if cfg.dtype == "f32":
        L_ref = oracle.router_logits_f32_lane_order(a["x"], a["w_router"], a["bias"])
        np.testing.assert_array_equal(L_gpu, L_ref)
        differ = np.array([], np.int64)
    else:
        L_ref = oracle.router_logits(a["x"], a["w_router"], a["bias"])
        bound = gh.logits_bound(a["x"], a["w_router"], a["bias"], L_ref)
        dL = np.abs(L_gpu.astype(np.float64) - L_ref)
        assert np.all(dL <= bound), f"logits outside the dot-product bound: {(dL / bound).max():.2f}x"
        ids_own, _ = oracle.topk_route(L_ref, cfg.k)
        differ = gh.certify_routing(got["ids"], ids_own, L_ref, bound)
    _say(name, f"logits within bound; {differ.size} certified near-tie tokens differ from "
               "the oracle's own routing", t0)

    # the whole layer in the oracle, routed on the GPU's logits
    round_a = cfg.dtype == "bf16"
    ref = oracle.moe_layer(a["x"], a["w_router"], a["bias"], a["w_gate"], a["w_up"], a["w_down"],
                           cfg.k, a["wsh_gate"], a["wsh_up"], a["wsh_down"], round_a=round_a,
                           logits=L_gpu)
    _say(name, "oracle layer done", t0)
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    assert np.abs(got["w"].astype(np.float64) - ref["w"]).max() <= 2e-6
    for key in ("counts", "offsets", "perm"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    tol = dict(mean_abs=1e-5, max_rel=1e-4) if cfg.dtype == "f32" else {}
    ma, mr = gh.assert_fp_close(got["out"], ref["out"], f"{name} out", **tol)
    _say(name, f"all {cfg.T} x {cfg.d} outputs: mean_abs={ma:.2e} max_rel={mr:.2e}", t0)

    if cfg.n_shared:
        got2 = lay.layer_overlap()
        np.testing.assert_array_equal(got2["out"], got["out"])
        np.testing.assert_array_equal(got2["ids"], got["ids"])
        gh.assert_fp_close(got2["out"], ref["out"], f"{name} out (two streams)", **tol)
        _say(name, "two-stream output identical and within tolerance", t0)

    if name in FFN_FULL:
        # the standalone dispatch and grouped FFN on the same ids
        disp = lay.dispatch(got["ids"])
        for key in ("counts", "offsets", "perm", "inv_perm"):
            np.testing.assert_array_equal(disp[key], ref[key], err_msg=key)
        xs = disp["x_sorted"].float().cpu().numpy()
        np.testing.assert_array_equal(xs, ref["x_sorted"].astype(np.float32))
        ffn = lay.ffn(disp["x_sorted"], disp["offsets"])
        flips = gh.check_swiglu_a(ffn["A"], ref["A"], ref["x_sorted"], ref["offsets"],
                                  a["w_gate"], a["w_up"])
        ma, mr = gh.assert_fp_close(ffn["y_sorted"], ref["y_sorted"], f"{name} y_sorted")
        msg = f"moe_dispatch exact; A: {flips:.3%} one-ulp flips; y_sorted mean_abs={ma:.2e} max_rel={mr:.2e}"
        if cfg.n_shared:
            Is = cfg.I_shared
            for s_ in range(cfg.n_shared):
                cols = slice(s_ * Is, (s_ + 1) * Is)
                gh.check_swiglu_a(ffn["A_shared"][:, cols], ref["A_shared"][:, cols], a["x"],
                                  [0, cfg.T], a["wsh_gate"][s_:s_ + 1], a["wsh_up"][s_:s_ + 1],
                                  what=f"A_shared[{s_}]")
            ma, mr = gh.assert_fp_close(ffn["y_shared"], ref["y_shared"], f"{name} y_shared")
            msg += f"; y_shared mean_abs={ma:.2e} max_rel={mr:.2e}"
        _say(name, msg, t0)
