"""GPU parity at the full sizes of the five model-shaped workloads, in the
launch configuration the benchmark times (one moe_layer_fwd call).

Checked on every workload:
  * routing: each token's ids are the top-k of the GPU's own logits, and
    agree with the oracle's except at certified near ties;
  * dispatch: counts, offsets and perm are a stable counting sort of the
    GPU's ids (bit-exact against the oracle whenever routing agrees fully);
  * output: sampled token rows (random ones, the first and last token, tokens
    of the rarest experts, and rows of the busiest expert's ragged last
    256-row GEMM tile: its first rows, the rows around its 128-row half and
    its last 32-row group, and its last rows) against the oracle computed one
    token at a time;
  * the two-stream entry point gives the same output bit for bit (layers with
    shared experts).
The fp32 workload is small enough for a full comparison."""
import numpy as np
import pytest

import moe_synth
import oracle

pytestmark = pytest.mark.gpu


M_TILE = 256  # rows per M-tile of the bf16 grouped GEMM


def sample_tokens(ids_ref, E, k, rng, n_random=40):
    T = ids_ref.shape[0]
    counts = np.bincount(ids_ref.ravel(), minlength=E)
    toks = set(rng.choice(T, size=min(n_random, T), replace=False).tolist()) | {0, T - 1}
    nz = np.nonzero(counts)[0]
    for e in nz[np.argsort(counts[nz])][:3]:  # rarest non-empty experts
        toks |= set(np.nonzero(np.any(ids_ref == e, axis=1))[0][:2].tolist())
    hot = int(np.argmax(counts))
    rows = np.nonzero(np.any(ids_ref == hot, axis=1))[0]  # the expert's rows, in order
    n = len(rows)
    tail = (n - 1) // M_TILE * M_TILE  # first row of its last (ragged) M-tile
    picks = list(range(tail, min(n, tail + 3)))          # first rows of the last tile
    picks += [tail + 127, tail + 128]                    # around the 128-row half
    last32 = (n - 1) // 32 * 32
    picks += [last32 - 1, last32]                        # around the last 32-row group
    picks += [n - 2, n - 1]                              # its last rows
    toks |= {int(rows[i]) for i in picks if 0 <= i < n}
    return np.array(sorted(toks))


@pytest.mark.parametrize("name", moe_synth.CONFIG_ORDER)
def test_workload(name):
    import gpu_helpers as gh
    cfg = moe_synth.CONFIGS[name]
    print(f"[workload {name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} I={cfg.I} "
          f"shared={cfg.n_shared}x{cfg.I_shared} {cfg.dtype}", flush=True)
    arrays = moe_synth.generate(cfg, workers=16)
    lay = gh.Layer(cfg, arrays)
    got = lay.layer()
    print(f"[workload {name}] layer done", flush=True)

    a = arrays
    if cfg.dtype == "f32":
        L_ref = oracle.router_logits_f32_lane_order(a["x"], a["w_router"], a["bias"])
    else:
        L_ref = oracle.router_logits(a["x"], a["w_router"], a["bias"])
    ids_ref, w_ref = oracle.topk_route(L_ref, cfg.k)

    # routing
    if cfg.dtype == "f32":
        np.testing.assert_array_equal(got["ids"], ids_ref)
        differ = np.array([], np.int64)
    else:
        bound = gh.logits_bound(a["x"], a["w_router"], a["bias"], L_ref)
        differ = gh.certify_routing(got["ids"], ids_ref, L_ref, bound)
    print(f"[workload {name}] routing: {differ.size} certified near-tie tokens differ", flush=True)

    # dispatch: a stable counting sort of the GPU's own ids
    flat = got["ids"].ravel().astype(np.int64)
    np.testing.assert_array_equal(got["counts"], np.bincount(flat, minlength=cfg.E))
    np.testing.assert_array_equal(got["offsets"][1:], np.cumsum(got["counts"]))
    assert got["offsets"][0] == 0
    np.testing.assert_array_equal(got["perm"], np.argsort(flat, kind="stable"))
    if differ.size == 0:
        counts, offsets, perm, _ = oracle.dispatch(ids_ref, cfg.E)
        np.testing.assert_array_equal(got["counts"], counts)
        np.testing.assert_array_equal(got["offsets"], offsets)
        np.testing.assert_array_equal(got["perm"], perm)

    # outputs
    same = np.setdiff1d(np.arange(cfg.T), differ)
    round_a = cfg.dtype == "bf16"
    if cfg.T <= 512:
        ref = oracle.moe_layer(a["x"], a["w_router"], a["bias"], a["w_gate"], a["w_up"], a["w_down"],
                               cfg.k, a["wsh_gate"], a["wsh_up"], a["wsh_down"], round_a=round_a,
                               logits=L_ref)
        toks, ref_out = same, ref["out"][same]
    else:
        toks = np.intersect1d(sample_tokens(ids_ref, cfg.E, cfg.k, np.random.default_rng(cfg.seed)), same)
        _, w_s, ref_out = oracle.token_outputs(toks, a["x"], L_ref, a["w_gate"], a["w_up"], a["w_down"],
                                               cfg.k, a["wsh_gate"], a["wsh_up"], a["wsh_down"],
                                               round_a=round_a)
        # weights from the GPU's logits: off by at most twice the logits' error
        w_tol = 2e-6 if cfg.dtype == "f32" else 2e-6 + 2.0 * bound[toks].max()
        np.testing.assert_allclose(got["w"][toks], w_s, rtol=0, atol=w_tol)
    tol = dict(mean_abs=1e-5, max_rel=1e-4) if cfg.dtype == "f32" else {}
    ma, mr = gh.assert_fp_close(got["out"][toks], ref_out, f"{name} out", **tol)
    print(f"[workload {name}] {toks.size} rows: mean_abs={ma:.2e} max_rel={mr:.2e}", flush=True)

    if cfg.n_shared:
        got2 = lay.layer_overlap()
        np.testing.assert_array_equal(got2["out"], got["out"])
        np.testing.assert_array_equal(got2["ids"], got["ids"])
        print(f"[workload {name}] two-stream output identical", flush=True)
