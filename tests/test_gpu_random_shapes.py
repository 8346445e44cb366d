"""GPU parity on seeded random layer shapes, drawn within the C ABI's limits
(T >= 1, 1 <= k <= min(E, 16), E <= 256, d, I, I_shared multiples of 64), so
that tile edges, ragged experts, shared-expert widths and both dtypes are hit
in combinations the named cases do not cover.  Each shape checks the whole
layer against the oracle (routing bit-exact on these sizes, dispatch
bit-exact, outputs within tolerance) and that the condensed entry point with a
threshold above 1 is the same layer bit for bit."""
import numpy as np
import pytest

import moe_synth
import oracle
from moe_synth import MoEShape

pytestmark = pytest.mark.gpu


def draw_shape(i):
    rng = np.random.default_rng(1000 + i)
    E = int(rng.choice([1, 3, 8, 17, 40, 64, 100]))
    k = int(rng.integers(1, min(E, 8) + 1))
    ns = int(rng.choice([0, 0, 1, 2]))
    dtype = "f32" if i % 4 == 3 else "bf16"
    return MoEShape(f"rand{i}", T=int(rng.integers(1, 1500)), d=64 * int(rng.integers(1, 7)),
                    E=E, k=k, I=64 * int(rng.integers(1, 9)), n_shared=ns,
                    I_shared=64 * int(rng.integers(1, 5)) if ns else 0, dtype=dtype,
                    seed=2000 + i, bias=str(rng.choice(["none", "normal"])))


@pytest.mark.parametrize("i", range(8))
def test_random_shape_layer(i):
    import gpu_helpers as gh
    from test_gpu_condense import run_condensed
    cfg = draw_shape(i)
    print(f"[random {i}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} I={cfg.I} "
          f"shared={cfg.n_shared}x{cfg.I_shared} {cfg.dtype} bias={cfg.bias}", flush=True)
    a = moe_synth.generate(cfg)
    lay = gh.Layer(cfg, a)
    got = lay.layer()
    if cfg.dtype == "f32":
        L = oracle.router_logits_f32_lane_order(a["x"], a["w_router"], a["bias"])
    else:
        L = oracle.router_logits(a["x"], a["w_router"], a["bias"])
    ref = oracle.moe_layer(a["x"], a["w_router"], a["bias"], a["w_gate"], a["w_up"], a["w_down"],
                           cfg.k, a["wsh_gate"], a["wsh_up"], a["wsh_down"],
                           round_a=cfg.dtype == "bf16", logits=L)
    if cfg.dtype == "f32":
        np.testing.assert_array_equal(got["ids"], ref["ids"])
    else:
        bound = gh.logits_bound(a["x"], a["w_router"], a["bias"], L)
        differ = gh.certify_routing(got["ids"], ref["ids"], L, bound)
        assert differ.size == 0, f"{differ.size} certified near ties; this shape needs a new seed"
    for key in ("counts", "offsets", "perm"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    tol = dict(mean_abs=1e-5, max_rel=1e-4) if cfg.dtype == "f32" else {}
    gh.assert_fp_close(got["out"], ref["out"], f"rand{i} out", **tol)

    hyper = moe_synth.condense_hyperplanes(cfg)
    cond = run_condensed(lay, hyper, 1.5)
    for key in ("out", "ids", "w", "counts", "offsets", "perm"):
        np.testing.assert_array_equal(cond[key], got[key], err_msg=f"condensed {key}")
