"""GPU parity of the token-condensed layer (moe_layer_fwd_condensed) against
the condensation oracle (oracle.condense; Luffy review, "Core claim").

The keys are a decision taken on fp32 projections: the test gets the GPU's
own projections through moe_route with the hyperplanes as the router's
weights (the same kernel and launch the condensed layer runs, so the same
values), checks them against the fp64 projections within the dot-product
bound, and takes the keys from them, as the GPU does.  Representatives are
then compared with the oracle's rule applied to those keys with fp64
cosines: bit-exact, except at certified near-threshold cosines.  Counts,
offsets, perm and the rows each assignment reads are compared bit for bit
with the oracle's condensed dispatch of the GPU's own routing; outputs within
the usual tolerance.  At the prefill-stress workload's full size: validity of
every representative, the condensed dispatch, and sampled output rows."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_synth import MoEShape
from oracle import condense as oc

pytestmark = pytest.mark.gpu

CASES = {
    # 30% near-duplicate rows, one shared expert, several 256-row tiles
    "dup_bf16": MoEShape("dup_bf16", T=900, d=256, E=8, k=2, I=256, n_shared=1, I_shared=128,
                         seed=21, dup_frac=0.3, dup_noise_var=1e-4),
    # skewed routing with empty experts, top-4, no shared expert
    "dup_bf16_zipf": MoEShape("dup_bf16_zipf", T=600, d=192, E=16, k=4, I=128, seed=22,
                              bias="zipf", zipf_alpha=1.5, dup_frac=0.4, dup_noise_var=1e-4),
    "dup_f32": MoEShape("dup_f32", T=300, d=128, E=6, k=2, I=128, n_shared=1, I_shared=64,
                        dtype="f32", seed=23, dup_frac=0.3, dup_noise_var=1e-4),
    "one_token": MoEShape("one_token_c", T=1, d=128, E=8, k=2, I=128, seed=24),
}
THRESHOLD = 0.9


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()


def run_condensed(lay, hyper, thr):
    import expert_routing_grouped_route_amd as moe
    import gpu_helpers as gh
    c, t = lay.cfg, lay.t
    out = lay._f32(c.T, c.d)
    ids, w = lay._i32(c.T, c.k), lay._f32(c.T, c.k)
    counts, offsets, perm = lay._i32(c.E), lay._i32(c.E + 1), lay._i32(lay.R)
    rep = lay._i32(c.T)
    perm.fill_(-1)
    ws_bytes = moe.moe_condensed_workspace_bytes(lay.dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    moe.moe_layer_fwd_condensed(lay.dims, t["x"], t["w_router"], t.get("bias"), t["w_gate"],
                                t["w_up"], t["w_down"], t.get("wsh_gate"), t.get("wsh_up"),
                                t.get("wsh_down"), _dev(hyper, lay.dt), thr, out, ids, w, counts,
                                offsets, perm, rep, ws, ws_bytes)
    torch.cuda.synchronize()
    return {k_: gh.to_np(v) for k_, v in dict(out=out, ids=ids, w=w, counts=counts,
                                               offsets=offsets, perm=perm, rep=rep).items()}


def gpu_projections(lay, hyper):
    """The GPU's fp32 projections: moe_route with the hyperplanes as 16 experts, top-1."""
    import expert_routing_grouped_route_amd as moe
    import gpu_helpers as gh
    c = lay.cfg
    d16 = moe.dims(c.T, c.d, oc.KEY_BITS, 1, c.I, 0, 0, c.dtype)
    proj = lay._f32(c.T, oc.KEY_BITS)
    moe.moe_route(d16, lay.t["x"], _dev(hyper, lay.dt), None, None, proj, lay._i32(c.T),
                  lay._f32(c.T))
    torch.cuda.synchronize()
    return gh.to_np(proj)


def check_projections(x, hyper, proj):
    import gpu_helpers as gh
    ref = oc.projections(x, hyper)
    bound = gh.logits_bound(x, hyper, None, ref.astype(np.float32))
    assert np.all(np.abs(proj - ref) <= bound + 1e-30), "projections outside the dot-product bound"


def near_threshold_tokens(x, keys, thr, eps):
    """Tokens with a cosine within eps of the threshold against one of the
    first CANDIDATES earlier members of their key bucket."""
    out = set()
    for t in range(x.shape[0]):
        earlier = [t2 for t2 in range(t) if keys[t2] == keys[t]][: oc.CANDIDATES]
        for t2 in earlier:
            if abs(oc.cosine(x[t], x[t2]) - thr) <= eps:
                out.add(t)
    return out


def case(name):
    import gpu_helpers as gh
    cfg = CASES[name]
    arrays = moe_synth.generate(cfg)
    hyper = moe_synth.condense_hyperplanes(cfg)
    print(f"[condense {name}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} dup={cfg.dup_frac} {cfg.dtype}",
          flush=True)
    return cfg, arrays, hyper, gh.Layer(cfg, arrays)


@pytest.mark.parametrize("name", list(CASES))
def test_condensed_layer_matches_oracle(name):
    import gpu_helpers as gh
    cfg, a, hyper, lay = case(name)
    got = run_condensed(lay, hyper, THRESHOLD)
    x = a["x"].astype(np.float64)

    proj = gpu_projections(lay, hyper)
    check_projections(a["x"], hyper, proj)
    keys = oc.condense_keys(proj)
    rep_ref = oc.condense_reps(x, keys, THRESHOLD)
    fuzzy = near_threshold_tokens(x, keys, THRESHOLD, 1e-4)
    diff = np.nonzero(got["rep"] != rep_ref)[0]
    assert set(diff.tolist()) <= fuzzy, f"representatives differ at {diff[:10]}"
    if cfg.dup_frac:
        assert np.count_nonzero(got["rep"] != np.arange(cfg.T)) > 0.5 * cfg.dup_frac * cfg.T

    # routing as in the plain layer; then the condensed dispatch of the GPU's routing, bit for bit
    if cfg.dtype == "f32":
        L = oracle.router_logits_f32_lane_order(a["x"], a["w_router"], a["bias"])
    else:
        L = oracle.router_logits(a["x"], a["w_router"], a["bias"])
    ids_ref, w_ref = oracle.topk_route(L, cfg.k)
    np.testing.assert_array_equal(got["ids"], ids_ref)
    counts, offsets, perm, inv = oc.dispatch_condensed(got["ids"], cfg.E, got["rep"])
    np.testing.assert_array_equal(got["counts"], counts)
    np.testing.assert_array_equal(got["offsets"], offsets)
    np.testing.assert_array_equal(got["perm"][: offsets[-1]], perm)

    ref = oc.condensed_layer(a["x"], L, a["w_gate"], a["w_up"], a["w_down"], cfg.k, got["rep"],
                             a["wsh_gate"], a["wsh_up"], a["wsh_down"], round_a=cfg.dtype == "bf16")
    tol = dict(mean_abs=1e-5, max_rel=1e-4) if cfg.dtype == "f32" else {}
    ma, mr = gh.assert_fp_close(got["out"], ref["out"], f"{name} out", **tol)
    print(f"[condense {name}] {np.count_nonzero(got['rep'] != np.arange(cfg.T))} tokens condensed, "
          f"rows {offsets[-1]} of {cfg.T * cfg.k}; out mean_abs={ma:.2e} max_rel={mr:.2e}", flush=True)


@pytest.mark.parametrize("name", ["dup_bf16", "dup_f32"])
def test_threshold_above_one_is_the_plain_layer(name):
    cfg, a, hyper, lay = case(name)
    got = run_condensed(lay, hyper, 1.5)
    plain = lay.layer()
    np.testing.assert_array_equal(got["rep"], np.arange(cfg.T))
    for key in ("out", "ids", "w", "counts", "offsets", "perm"):
        np.testing.assert_array_equal(got[key], plain[key], err_msg=key)


def test_one_large_bucket_condenses_to_the_first_token():
    """300 identical rows: one key bucket far larger than the 32 candidates
    (its first position is found by the binary-search path).  Every token
    condenses to token 0, only token 0's assignments keep rows, and the output
    equals the plain layer's bit for bit (identical rows give identical
    expert outputs)."""
    cfg = MoEShape("same_rows", T=300, d=128, E=8, k=2, I=128, n_shared=1, I_shared=64, seed=25)
    import gpu_helpers as gh
    a = moe_synth.generate(cfg)
    a["x"][:] = a["x"][0]
    hyper = moe_synth.condense_hyperplanes(cfg)
    lay = gh.Layer(cfg, a)
    got = run_condensed(lay, hyper, THRESHOLD)
    np.testing.assert_array_equal(got["rep"], np.zeros(cfg.T, np.int32))
    assert got["offsets"][-1] == cfg.k
    plain = lay.layer()
    np.testing.assert_array_equal(got["out"], plain["out"])


def test_condensed_layer_is_deterministic():
    cfg, a, hyper, lay = case("dup_bf16")
    g1 = run_condensed(lay, hyper, THRESHOLD)
    g2 = run_condensed(lay, hyper, THRESHOLD)
    for key in g1:
        np.testing.assert_array_equal(g1[key], g2[key], err_msg=key)


def test_condensed_prefill_stress_full_size():
    """The 32768-token workload with 30% near-duplicate rows, in the launch
    configuration the benchmark times: every representative is valid, the
    dispatch is the condensed counting sort of the GPU's routing, and sampled
    output rows match the oracle computed token by token."""
    import gpu_helpers as gh
    cfg = moe_synth.CONFIGS["prefill_stress"]
    print(f"[condense prefill_stress] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k}", flush=True)
    a = moe_synth.generate(cfg, workers=16)
    hyper = moe_synth.condense_hyperplanes(cfg)
    lay = gh.Layer(cfg, a)
    got = run_condensed(lay, hyper, THRESHOLD)
    rep, T = got["rep"], cfg.T
    cond = np.nonzero(rep != np.arange(T))[0]
    print(f"[condense prefill_stress] {cond.size} tokens condensed, rows {got['offsets'][-1]} "
          f"of {T * cfg.k}", flush=True)
    assert cond.size > 0.15 * T  # 30% of the rows are near-duplicates

    # validity: earlier, itself a representative, same key, similar
    proj = gpu_projections(lay, hyper)
    keys = oc.condense_keys(proj)
    assert np.all(rep[cond] < cond)
    assert np.all(rep[rep] == rep)
    assert np.all(keys[rep[cond]] == keys[cond])
    x = a["x"]
    rng = np.random.default_rng(5)
    for t in rng.choice(cond, size=min(300, cond.size), replace=False):
        assert oc.cosine(x[t], x[rep[t]]) >= THRESHOLD - 1e-4, f"token {t}"

    counts, offsets, perm, inv = oc.dispatch_condensed(got["ids"], cfg.E, rep)
    np.testing.assert_array_equal(got["counts"], counts)
    np.testing.assert_array_equal(got["offsets"], offsets)
    np.testing.assert_array_equal(got["perm"][: offsets[-1]], perm)

    # sampled outputs: condensed and plain tokens, each from its own routing
    L = oracle.router_logits(a["x"], a["w_router"], a["bias"])
    toks = np.unique(np.concatenate([rng.choice(cond, 20, replace=False),
                                     rng.choice(np.setdiff1d(np.arange(T), cond), 10, replace=False),
                                     [0, T - 1]]))
    ids_s, w_s = oracle.topk_route(L[toks], cfg.k)
    np.testing.assert_array_equal(got["ids"][toks], ids_s)
    ref = np.zeros((toks.size, cfg.d))
    for n, t in enumerate(toks):
        r = rep[t]
        for j in range(cfg.k):
            e = ids_s[n, j]
            src = r if e in got["ids"][r] else t
            _, Y = oracle.swiglu_expert(x[src:src + 1], a["w_gate"][e], a["w_up"][e], a["w_down"][e], True)
            ref[n] += float(w_s[n, j]) * Y[0]
        for s_ in range(cfg.n_shared):
            _, S = oracle.swiglu_expert(x[t:t + 1], a["wsh_gate"][s_], a["wsh_up"][s_], a["wsh_down"][s_], True)
            ref[n] += S[0]
    ma, mr = gh.assert_fp_close(got["out"][toks], ref, "prefill_stress condensed out")
    print(f"[condense prefill_stress] {toks.size} rows: mean_abs={ma:.2e} max_rel={mr:.2e}", flush=True)
