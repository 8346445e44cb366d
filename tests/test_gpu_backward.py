"""GPU parity of the layer's backward pass (moe_layer_bwd, through the C ABI)
against the fp64 backward oracle, on seeded inputs: bf16 and fp32 layers,
shared experts, skewed routing with experts that receive no token, top-1
(no router gradient), k = E, one token.

The oracle routes on the GPU's own router logits (moe_route's logits_out,
the kernel moe_layer_bwd runs too), so both sides keep the same experts.
Gradients are compared with the layer's rules scaled to each tensor's size:
mean |g - r| <= 1e-3 rms(r) and max_i |g_i - r_i| / max(|r_i|, rms(r)) <=
2e-2.  Experts without tokens must get exactly zero weight gradients; two
calls must agree bit for bit.  The products run on the matrix cores (each
fp32 operand as bf16 hi + lo parts); for fp32 layers the vector-ALU variant
(moe_layer_bwd_variant with MOE_VARIANT_BWD_VALU) is held to the same bar."""
import numpy as np
import pytest
import torch

import expert_routing_grouped_route_amd as moe
import moe_synth
import oracle
from moe_synth import MoEShape
from oracle import moe_backward as mb

pytestmark = pytest.mark.gpu

CASES = {
    "bwd_bf16_shared": MoEShape("bwd_bf16_shared", T=300, d=128, E=8, k=2, I=192, n_shared=1,
                                I_shared=64, seed=21, bias="normal"),
    "bwd_bf16_zipf": MoEShape("bwd_bf16_zipf", T=256, d=128, E=16, k=4, I=128, seed=22,
                              bias="zipf", zipf_alpha=1.5),
    "bwd_fp32_two_shared": MoEShape("bwd_fp32_two_shared", T=150, d=64, E=6, k=3, I=192,
                                    n_shared=2, I_shared=64, dtype="f32", seed=23),
    "bwd_top1": MoEShape("bwd_top1", T=200, d=64, E=4, k=1, I=64, n_shared=1, I_shared=64,
                         seed=24),
    "bwd_one_token": MoEShape("bwd_one_token", T=1, d=64, E=8, k=2, I=64, seed=25),
    "bwd_k_equals_E": MoEShape("bwd_k_equals_E", T=70, d=64, E=4, k=4, I=64, seed=26),
    "bwd_fp32_zipf": MoEShape("bwd_fp32_zipf", T=256, d=128, E=16, k=4, I=128, dtype="f32",
                              seed=29, bias="zipf", zipf_alpha=2.0),  # 2 experts get no token
}

GRADS = ("dx", "dw_router", "dbias", "dw_gate", "dw_up", "dw_down", "dwsh_gate", "dwsh_up",
         "dwsh_down")


def _np(t):
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


class Case:
    def __init__(self, cfg):
        self.cfg = cfg
        self.a = moe_synth.generate(cfg, workers=16)
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.t = {n: (None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(
            torch.float32 if n == "bias" else dt).cuda()) for n, v in self.a.items()}
        self.dims = moe.dims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.I_shared,
                             cfg.dtype)
        rng = np.random.default_rng(1000 + cfg.seed)
        self.dout = rng.normal(size=(cfg.T, cfg.d)).astype(np.float32)

    def logits(self):
        c = self.cfg
        ids = torch.empty(c.T, c.k, dtype=torch.int32, device="cuda")
        w = torch.empty(c.T, c.k, dtype=torch.float32, device="cuda")
        L = torch.empty(c.T, c.E, dtype=torch.float32, device="cuda")
        moe.moe_route(self.dims, self.t["x"], self.t["w_router"], self.t.get("bias"), None, L,
                      ids, w)
        torch.cuda.synchronize()
        return _np(L)

    def backward(self, variant=0):
        """moe_layer_bwd (moe_layer_bwd_variant for a nonzero variant)."""
        c, t = self.cfg, self.t
        f = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
        g = dict(dx=f(c.T, c.d), dw_router=f(c.E, c.d), dbias=f(c.E), dw_gate=f(c.E, c.I, c.d),
                 dw_up=f(c.E, c.I, c.d), dw_down=f(c.E, c.d, c.I))
        if c.n_shared:
            g.update(dwsh_gate=f(c.n_shared, c.I_shared, c.d),
                     dwsh_up=f(c.n_shared, c.I_shared, c.d),
                     dwsh_down=f(c.n_shared, c.d, c.I_shared))
        else:
            g.update(dwsh_gate=None, dwsh_up=None, dwsh_down=None)
        wsb = moe.moe_backward_workspace_bytes(self.dims)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        dout = torch.from_numpy(self.dout).cuda()
        print(f"[bwd {c.name}] T={c.T} d={c.d} E={c.E} k={c.k} I={c.I} "
              f"shared={c.n_shared}x{c.I_shared} {c.dtype}", flush=True)
        args = (self.dims, t["x"], t["w_router"], t.get("bias"), t["w_gate"], t["w_up"],
                t["w_down"], t.get("wsh_gate"), t.get("wsh_up"), t.get("wsh_down"), dout,
                g["dx"], g["dw_router"], g["dbias"], g["dw_gate"], g["dw_up"], g["dw_down"],
                g["dwsh_gate"], g["dwsh_up"], g["dwsh_down"], ws, wsb)
        if variant:
            moe.moe_layer_bwd_variant(*args, variant)
        else:
            moe.moe_layer_bwd(*args)
        torch.cuda.synchronize()
        return {n: (None if v is None else _np(v)) for n, v in g.items()}

    def reference(self, L):
        c, a = self.cfg, self.a
        return mb.moe_layer_backward(a["x"], a["w_router"], a["bias"], a["w_gate"], a["w_up"],
                                     a["w_down"], c.k, self.dout, a["wsh_gate"], a["wsh_up"],
                                     a["wsh_down"], round_a=c.dtype == "bf16", logits=L)


def assert_grad_close(g, r, what):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    scale = rms if rms > 0 else 1.0
    diff = np.abs(g - r)
    mean_rel = float(diff.mean()) / scale
    max_rel = float((diff / np.maximum(np.abs(r), scale)).max()) if r.size else 0.0
    assert mean_rel <= 1e-3 and max_rel <= 2e-2, f"{what}: mean|g-r|/rms={mean_rel:.3e} max_rel={max_rel:.3e}"


_cases = {}


def get(name):
    if name not in _cases:
        _cases[name] = Case(CASES[name])
    return _cases[name]


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    c = get(name)
    L = c.logits()
    got = c.backward()
    ref = c.reference(L)
    for n in GRADS:
        if ref[n] is None:
            assert got[n] is None
            continue
        assert_grad_close(got[n], ref[n], f"{name}.{n}")
    # experts that receive no token get exactly zero weight gradients
    empty = np.nonzero(np.diff(np.asarray(ref["offsets"])) == 0)[0]
    for e in empty:
        for n in ("dw_gate", "dw_up", "dw_down", "dw_router"):
            assert np.all(got[n][e] == 0.0), (name, n, e)
    if c.cfg.k == 1:  # the kept weight is 1 whatever the logits
        assert np.all(got["dw_router"] == 0.0) and np.all(got["dbias"] == 0.0)


@pytest.mark.parametrize("name", ["bwd_fp32_two_shared", "bwd_fp32_zipf"])
def test_backward_vector_alu_variant_matches_oracle(name):
    """fp32 layers with every gradient product on the VALU in fp32
    (MOE_VARIANT_BWD_VALU) instead of the matrix cores' bf16 hi/lo parts: the
    same bar against the oracle, with two shared experts, and with Zipf-skewed
    routing that leaves experts without tokens (their weight gradients must
    be exactly zero).  bf16 layers ignore the variant."""
    c = get(name)
    L = c.logits()
    got = c.backward(variant=moe.MOE_VARIANT_BWD_VALU)
    ref = c.reference(L)
    empty = np.nonzero(np.diff(np.asarray(ref["offsets"])) == 0)[0]
    for e in empty:
        for n in ("dw_gate", "dw_up", "dw_down", "dw_router"):
            assert np.all(got[n][e] == 0.0), (name, n, e)
    for n in GRADS:
        if ref[n] is not None:
            assert_grad_close(got[n], ref[n], f"{name}.{n} (VALU)")


@pytest.mark.parametrize("name", ["bwd_bf16_shared", "bwd_bf16_zipf"])
def test_backward_global_load_variant(name):
    """The GEMM operands through 64-bit global loads instead of buffer loads
    (the variant taken when a product's offsets exceed 32 bits; asked for here
    with MOE_VARIANT_GLOBAL_LOADS): the same bar against the oracle, and the
    same gradients bit for bit as the buffer-load call (same data in LDS, same
    MFMA order)."""
    c = get(name)
    L = c.logits()
    base = c.backward()
    got = c.backward(variant=moe.MOE_VARIANT_GLOBAL_LOADS)
    ref = c.reference(L)
    for n in GRADS:
        if ref[n] is None:
            continue
        assert_grad_close(got[n], ref[n], f"{name}.{n} (global loads)")
        assert np.array_equal(got[n], base[n]), n


@pytest.mark.parametrize("name", ["bwd_bf16_zipf", "bwd_fp32_zipf"])
def test_backward_has_empty_experts_in_skewed_case(name):
    c = get(name)
    ref = c.reference(c.logits())
    assert np.any(np.diff(np.asarray(ref["offsets"])) == 0)


@pytest.mark.parametrize("name", ["bwd_bf16_shared", "bwd_fp32_two_shared"])
def test_backward_is_deterministic(name):
    c = get(name)
    g1, g2 = c.backward(), c.backward()
    for n in GRADS:
        if g1[n] is not None:
            assert np.array_equal(g1[n], g2[n]), n


@pytest.mark.parametrize("name", ["tiny_fp32", "deepseek_v2_lite", "qwen3_30b_a3b"])
def test_backward_full_size(name):
    """Full-size layers in the configuration bench.py times: the tiny fp32
    layer, the DeepSeek-V2-Lite shape (4096 tokens, 64 experts top-6, two shared
    experts) and the Qwen3-30B-A3B shape (8192 tokens, 128 experts top-8,
    Zipf-skewed routing with empty experts).  Every gradient against the full
    fp64 oracle (10-30 s of host time each)."""
    cfg = moe_synth.CONFIGS[name]
    c = Case(cfg)
    L = c.logits()
    got = c.backward()
    print(f"[bwd {cfg.name}] GPU done; running the oracle", flush=True)
    ref = c.reference(L)
    for n in GRADS:
        if ref[n] is None:
            assert got[n] is None
            continue
        assert_grad_close(got[n], ref[n], f"{cfg.name}.{n}")
    empty = np.nonzero(np.diff(np.asarray(ref["offsets"])) == 0)[0]
    for e in empty:
        assert np.all(got["dw_gate"][e] == 0.0) and np.all(got["dw_down"][e] == 0.0), e


def test_backward_zero_tokens_is_a_no_op():
    """T = 0: the call returns MOE_OK and enqueues nothing (outputs untouched)."""
    cfg = MoEShape("bwd_empty", T=0, d=64, E=4, k=2, I=64, seed=27)
    d = moe.dims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, 0, 0, "bf16")
    f = lambda *s: torch.full(s, 7.0, dtype=torch.float32, device="cuda")
    x = torch.empty(1, cfg.d, dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros(cfg.E, cfg.d, dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros(cfg.E, cfg.I, cfg.d, dtype=torch.bfloat16, device="cuda")
    wu = torch.zeros_like(wg)
    wd = torch.zeros(cfg.E, cfg.d, cfg.I, dtype=torch.bfloat16, device="cuda")
    dout = torch.empty(1, cfg.d, dtype=torch.float32, device="cuda")
    dx = f(1, cfg.d)
    dwr, dwg, dwu, dwd = f(cfg.E, cfg.d), f(cfg.E, cfg.I, cfg.d), f(cfg.E, cfg.I, cfg.d), f(cfg.E, cfg.d, cfg.I)
    wsb = moe.moe_backward_workspace_bytes(d)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    moe.moe_layer_bwd(d, x, wr, None, wg, wu, wd, None, None, None, dout, dx, dwr, None, dwg, dwu,
                      dwd, None, None, None, ws, wsb)
    torch.cuda.synchronize()
    for t in (dx, dwr, dwg, dwu, dwd):
        assert torch.all(t == 7.0)


@pytest.mark.parametrize("name", ["llama4_scout", "prefill_stress"])
def test_backward_full_size_parts(name):
    """The two largest layers at full size, in the configuration bench.py
    times: the Llama-4-Scout shape (8192 tokens, d = 5120, 16 experts top-1 of
    I = 8192 plus a shared expert; its W_u^T block sits about 1.3 GB past
    W_g^T) and the prefill shape (32768 tokens, 64 experts top-6, two shared
    experts; the weight-gradient products reduce over about 400 k columns and
    the shared ones are split over K).  The whole fp64 backward would take
    minutes of host time here, so the oracle computes parts of it
    (moe_layer_backward_parts, pinned against the whole backward): the router
    gradients and the shared experts' weight gradients whole, the weight
    gradients of the busiest, the least busy and one random expert (and zeros
    for an expert without tokens), and dx of 64 random tokens, the first and
    last token and the least busy expert's tokens."""
    cfg = moe_synth.CONFIGS[name]
    c = Case(cfg)
    L = c.logits()
    got = c.backward()
    print(f"[bwd {cfg.name}] GPU done; running the oracle's parts", flush=True)
    ids, _ = oracle.topk_route(L, cfg.k)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    nz = np.nonzero(counts)[0]
    rng = np.random.default_rng(cfg.seed)
    busiest, least = int(np.argmax(counts)), int(nz[np.argmin(counts[nz])])
    experts = sorted({busiest, least, int(rng.integers(cfg.E))})
    least_toks = np.nonzero(np.any(ids == least, axis=1))[0][:8]
    tokens = np.unique(np.concatenate([rng.choice(cfg.T, 64, replace=False), [0, cfg.T - 1],
                                       least_toks]))
    a = c.a
    ref = mb.moe_layer_backward_parts(a["x"], a["w_router"], a["bias"], a["w_gate"], a["w_up"],
                                      a["w_down"], cfg.k, c.dout, a["wsh_gate"], a["wsh_up"],
                                      a["wsh_down"], round_a=True, logits=L, experts=experts,
                                      tokens=tokens)
    assert_grad_close(got["dx"][tokens], ref["dx"], f"{name}.dx[{tokens.size} tokens]")
    if cfg.k > 1:
        assert_grad_close(got["dw_router"], ref["dw_router"], f"{name}.dw_router")
        assert_grad_close(got["dbias"], ref["dbias"], f"{name}.dbias")
    else:  # the kept weight is 1 whatever the logits
        assert np.all(got["dw_router"] == 0.0) and np.all(got["dbias"] == 0.0)
    for e in experts:
        for n in ("dw_gate", "dw_up", "dw_down"):
            assert_grad_close(got[n][e], ref[n][e], f"{name}.{n}[{e}]")
    for n in ("dwsh_gate", "dwsh_up", "dwsh_down"):
        assert_grad_close(got[n], ref[n], f"{name}.{n}")
    for e in np.nonzero(counts == 0)[0]:
        for n in ("dw_gate", "dw_up", "dw_down"):
            assert np.all(got[n][e] == 0.0), (name, n, e)
    print(f"[bwd {cfg.name}] experts {experts}, {tokens.size} tokens: all within tolerance",
          flush=True)
