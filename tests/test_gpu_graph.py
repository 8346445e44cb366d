"""The layer under HIP graph capture: moe_layer_fwd (and the condensed entry
point) recorded once into a graph and replayed several times, with eager
calls and synchronisations between the replays, give the eager result bit
for bit on every replay.  The library issues no memset and no host
synchronisation inside a call, so the whole layer is capturable."""
import numpy as np
import pytest
import torch

import moe_synth
from test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


def _outputs(lay):
    c = lay.cfg
    return dict(out=lay._f32(c.T, c.d), ids=lay._i32(c.T, c.k), w=lay._f32(c.T, c.k),
                counts=lay._i32(c.E), offsets=lay._i32(c.E + 1), perm=lay._i32(lay.R))


def _call(lay, o, stream):
    import expert_routing_grouped_route_amd as moe
    t = lay.t
    moe.moe_layer_fwd(lay.dims, t["x"], t["w_router"], t.get("bias"), t["w_gate"], t["w_up"],
                      t["w_down"], t.get("wsh_gate"), t.get("wsh_up"), t.get("wsh_down"), o["out"],
                      o["ids"], o["w"], o["counts"], o["offsets"], o["perm"], lay.ws, lay.ws_bytes,
                      stream)


@pytest.mark.parametrize("name", ["med_bf16_shared", "med_bf16_zipf", "tiny_fp32"])
def test_layer_graph_replays_match_eager(name):
    import gpu_helpers as gh
    cfg = CASES[name]
    print(f"[graph {name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} {cfg.dtype}", flush=True)
    lay = gh.Layer(cfg, moe_synth.generate(cfg))
    eager = _outputs(lay)
    _call(lay, eager, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = {k: gh.to_np(v) for k, v in eager.items()}

    static = _outputs(lay)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call before capture, as torch recommends
        _call(lay, static, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(lay, static, torch.cuda.current_stream())
    for rep in range(3):
        for v in static.values():
            v.fill_(-7)  # the replay must rewrite every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, v in static.items():
            np.testing.assert_array_equal(gh.to_np(v), ref[key], err_msg=f"replay {rep}: {key}")
        _call(lay, eager, torch.cuda.current_stream())  # eager work between replays
        torch.cuda.synchronize()
