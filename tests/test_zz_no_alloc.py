"""moe_layer_fwd_static, the layer on the library's static device scratch (no
workspace argument, no allocation), through the C ABI: on two calls in a row,
the second with fewer tokens, its outputs equal moe_layer_fwd's with a
caller-given workspace bit for bit (the same kernels on the same inputs).
Sizes whose workspace exceeds the scratch are refused before anything is
enqueued."""
import numpy as np
import pytest
import torch

import expert_routing_grouped_route_amd as moe
import moe_synth
from moe_synth import MoEShape

pytestmark = pytest.mark.gpu

KEYS = ("out", "ids", "w", "counts", "offsets", "perm")


def _run(cfg, static):
    a = moe_synth.generate(cfg)
    t = {n: (None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(
        torch.float32 if n == "bias" else torch.bfloat16).cuda()) for n, v in a.items()}
    d = moe.dims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.I_shared, cfg.dtype)
    R = cfg.T * cfg.k
    res = dict(out=torch.full((cfg.T, cfg.d), 7.0, device="cuda"),
               ids=torch.full((cfg.T, cfg.k), -1, dtype=torch.int32, device="cuda"),
               w=torch.full((cfg.T, cfg.k), 7.0, device="cuda"),
               counts=torch.full((cfg.E,), -1, dtype=torch.int32, device="cuda"),
               offsets=torch.full((cfg.E + 1,), -1, dtype=torch.int32, device="cuda"),
               perm=torch.full((R,), -1, dtype=torch.int32, device="cuda"))
    args = (d, t["x"], t["w_router"], t["bias"], t["w_gate"], t["w_up"], t["w_down"],
            t["wsh_gate"], t["wsh_up"], t["wsh_down"], res["out"], res["ids"], res["w"],
            res["counts"], res["offsets"], res["perm"])
    print(f"[no-alloc] {cfg.name} T={cfg.T} {'static scratch' if static else 'workspace'}",
          flush=True)
    if static:
        moe.moe_layer_fwd_static(*args)
    else:
        wsb = moe.moe_workspace_bytes(d)
        assert wsb <= moe.MOE_STATIC_SCRATCH_BYTES
        ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")
        moe.moe_layer_fwd(*args, ws, wsb)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def test_static_scratch_matches_workspace_call_twice():
    big = MoEShape("no_alloc_a", T=700, d=256, E=16, k=4, I=320, n_shared=1, I_shared=128,
                   seed=31, bias="normal")
    small = big.replace(name="no_alloc_b", T=90, seed=32)
    for cfg in (big, small):  # the second call leaves a larger call's contents behind it
        ref = _run(cfg, static=False)
        got = _run(cfg, static=True)
        for k in KEYS:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{cfg.name} {k}")
        assert np.all(got["perm"] >= 0) and np.isfinite(got["out"]).all()


def test_static_scratch_refuses_sizes_beyond_it():
    cfg = moe_synth.CONFIGS["deepseek_v2_lite"]
    d = moe.dims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.I_shared, cfg.dtype)
    assert moe.moe_workspace_bytes(d) > moe.MOE_STATIC_SCRATCH_BYTES
    out = torch.full((4, 4), 7.0, device="cuda")
    with pytest.raises(moe.MoeError) as err:
        moe.moe_layer_fwd_static(d, 16, 16, None, 16, 16, 16, 16, 16, 16, out, None, None, None,
                                 None, None)
    assert err.value.status == moe.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was enqueued
