"""Seeded synthetic inputs for the Mixture-of-Experts layer forward pass.

This module holds random draws and the recipes that shape them (sizes, value
distributions, router-bias skew, duplicated token rows) and nothing else: no
step of the layer itself (routing, dispatch, expert FFN, combine) lives here.
Both the oracle and the HIP library are fed from it; neither is imported.

Every tensor comes from its own counter-keyed PCG64 stream
(``SeedSequence(seed, spawn_key=(tag, index))``), so a tensor, or one expert's
slice of a stacked tensor, can be drawn on its own and in parallel, and the
result does not depend on which other tensors were drawn.

Distributions (``N(mean, var)`` takes a variance as its second argument):
  x            ~ N(0, 1)                        [T, d]
  w_router     ~ N(0, 1/d)                      [E, d]
  w_gate, w_up ~ N(0, 1/d)                      [E, I, d]
  w_down       ~ N(0, 1/d)                      [E, d, I]
  shared       the same, with n_shared experts of width I_shared
  bias         "normal": N(0, bias_var) per expert
               "zipf":   ln p_e with p_e proportional to rank_e ** -s, ranks a
                         seeded permutation of 1..E (skews load; some experts
                         receive no token)
  duplicates   floor(dup_frac * T) destination rows, drawn without
               replacement from [1, T) and visited in ascending order; each
               becomes a copy of a uniformly drawn earlier row plus
               N(0, dup_noise_var) noise (an earlier row may itself be a copy)

For bf16 workloads every tensor except the bias is rounded to bfloat16
(round to nearest even, through torch's conversion) after drawing, and is
returned as float32 holding exactly those bf16 values, so both sides see the
same numbers.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_TAGS = {
    "x": 1,
    "dup": 2,
    "w_router": 3,
    "bias": 4,
    "w_gate": 5,
    "w_up": 6,
    "w_down": 7,
    "wsh_gate": 8,
    "wsh_up": 9,
    "wsh_down": 10,
    "condense_hyperplanes": 11,
}

WEIGHT_NAMES = ("w_gate", "w_up", "w_down")
SHARED_NAMES = ("wsh_gate", "wsh_up", "wsh_down")
ALL_NAMES = ("x", "w_router", "bias") + WEIGHT_NAMES + SHARED_NAMES

_X_ROWS_PER_STREAM = 1024


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """One MoE-layer workload: sizes, precision and the input recipe."""

    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    n_shared: int = 0
    I_shared: int = 0
    dtype: str = "bf16"  # "bf16" (bf16 inputs, fp32 accumulate) or "f32"
    seed: int = 0
    bias: str = "none"  # "none" | "normal" | "zipf"
    bias_var: float = 0.5
    zipf_s: float = 1.1
    zipf_alpha: float = 1.0
    dup_frac: float = 0.0
    dup_noise_var: float = 1e-3

    @property
    def R(self) -> int:
        """Number of (token, slot) assignments."""
        return self.T * self.k

    def replace(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)

    def shape_of(self, name: str) -> tuple:
        s = {
            "x": (self.T, self.d),
            "w_router": (self.E, self.d),
            "bias": (self.E,),
            "w_gate": (self.E, self.I, self.d),
            "w_up": (self.E, self.I, self.d),
            "w_down": (self.E, self.d, self.I),
            "wsh_gate": (self.n_shared, self.I_shared, self.d),
            "wsh_up": (self.n_shared, self.I_shared, self.d),
            "wsh_down": (self.n_shared, self.d, self.I_shared),
        }
        return s[name]


# The five workloads, named by the model whose MoE layer they are shaped like.
CONFIGS = {
    "tiny_fp32": MoEShape("tiny_fp32", T=256, d=128, E=8, k=2, I=256,
                          dtype="f32", seed=0),
    "deepseek_v2_lite": MoEShape("deepseek_v2_lite", T=4096, d=2048, E=64, k=6,
                                 I=1408, n_shared=2, I_shared=1408, seed=1,
                                 bias="normal", bias_var=0.5),
    "qwen3_30b_a3b": MoEShape("qwen3_30b_a3b", T=8192, d=2048, E=128, k=8,
                              I=768, seed=2, bias="zipf", zipf_s=1.1),
    "llama4_scout": MoEShape("llama4_scout", T=8192, d=5120, E=16, k=1, I=8192,
                             n_shared=1, I_shared=8192, seed=3),
    "prefill_stress": MoEShape("prefill_stress", T=32768, d=2048, E=64, k=6,
                               I=1408, n_shared=2, I_shared=1408, seed=4,
                               dup_frac=0.3, dup_noise_var=1e-3),
}
CONFIG_ORDER = ("tiny_fp32", "deepseek_v2_lite", "qwen3_30b_a3b",
                "llama4_scout", "prefill_stress")


def _rng(seed: int, name: str, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(_TAGS[name], index))
    return np.random.Generator(np.random.PCG64(ss))


def _round_bf16_inplace(a: np.ndarray) -> None:
    """Round float32 values to bf16 (nearest even) in place, via torch."""
    import torch

    t = torch.from_numpy(a.reshape(-1))
    chunk = 1 << 26
    for s in range(0, t.numel(), chunk):
        seg = t[s:s + chunk]
        seg.copy_(seg.to(torch.bfloat16).to(torch.float32))


def _normal_into(out: np.ndarray, rng: np.random.Generator, std: float) -> None:
    rng.standard_normal(out=out, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)


def _gen_x(cfg: MoEShape, workers: int) -> np.ndarray:
    x = np.empty((cfg.T, cfg.d), np.float32)
    n_chunks = max(1, -(-cfg.T // _X_ROWS_PER_STREAM))

    def fill(c):
        r0 = c * _X_ROWS_PER_STREAM
        r1 = min(cfg.T, r0 + _X_ROWS_PER_STREAM)
        _normal_into(x[r0:r1], _rng(cfg.seed, "x", c), 1.0)

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(n_chunks)))
    if cfg.dup_frac > 0.0 and cfg.T > 1:
        rng = _rng(cfg.seed, "dup")
        n_dup = int(math.floor(cfg.dup_frac * cfg.T))
        n_dup = min(n_dup, cfg.T - 1)
        dest = np.sort(rng.choice(np.arange(1, cfg.T), size=n_dup, replace=False))
        u = rng.random(n_dup)
        src = np.minimum((u * dest).astype(np.int64), dest - 1)
        noise = rng.standard_normal((n_dup, cfg.d), dtype=np.float32)
        noise *= np.float32(math.sqrt(cfg.dup_noise_var))
        for j in range(n_dup):  # ascending: a source row is final when copied
            x[dest[j]] = x[src[j]] + noise[j]
    return x


def _gen_bias(cfg: MoEShape):
    if cfg.bias == "none":
        return None
    rng = _rng(cfg.seed, "bias")
    if cfg.bias == "normal":
        return (rng.standard_normal(cfg.E) * math.sqrt(cfg.bias_var)).astype(np.float32)
    if cfg.bias == "zipf":
        rank = rng.permutation(cfg.E).astype(np.float64) + 1.0
        p = rank ** (-cfg.zipf_s)
        p /= p.sum()
        return (cfg.zipf_alpha * np.log(p)).astype(np.float32)
    raise ValueError(f"unknown bias recipe {cfg.bias!r}")


def _gen_stack(cfg: MoEShape, name: str, workers: int) -> np.ndarray:
    shape = cfg.shape_of(name)
    out = np.empty(shape, np.float32)
    std = math.sqrt(1.0 / cfg.d)

    def fill(e):
        _normal_into(out[e], _rng(cfg.seed, name, e), std)
        if cfg.dtype == "bf16":
            _round_bf16_inplace(out[e])

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(shape[0])))
    return out


def generate(cfg: MoEShape, names=None, workers: int = 8) -> dict:
    """Draw the inputs of ``cfg``; returns float32 numpy arrays (bias may be None).

    ``names`` restricts the draw to a subset of ``ALL_NAMES``.
    """
    names = ALL_NAMES if names is None else tuple(names)
    out = {}
    for name in names:
        if name == "x":
            x = _gen_x(cfg, workers)
            if cfg.dtype == "bf16":
                _round_bf16_inplace(x)
            out["x"] = x
        elif name == "w_router":
            w = np.empty(cfg.shape_of("w_router"), np.float32)
            _normal_into(w, _rng(cfg.seed, "w_router"), math.sqrt(1.0 / cfg.d))
            if cfg.dtype == "bf16":
                _round_bf16_inplace(w)
            out["w_router"] = w
        elif name == "bias":
            out["bias"] = _gen_bias(cfg)
        elif name in WEIGHT_NAMES:
            out[name] = _gen_stack(cfg, name, workers)
        elif name in SHARED_NAMES:
            out[name] = _gen_stack(cfg, name, workers) if cfg.n_shared > 0 else None
        else:
            raise KeyError(name)
    return out


def condense_hyperplanes(cfg: MoEShape, bits: int = 16) -> np.ndarray:
    """The random hyperplanes of token condensation's keys: [bits, d] float32
    draws of N(0, 1), rounded to bf16 for bf16 workloads, from a stream of
    their own (the other inputs of ``cfg`` are unchanged by drawing them)."""
    p = np.empty((bits, cfg.d), np.float32)
    _normal_into(p, _rng(cfg.seed, "condense_hyperplanes"), 1.0)
    if cfg.dtype == "bf16":
        _round_bf16_inplace(p)
    return p


def to_device(arrays: dict, cfg: MoEShape, device="cuda"):
    """Move generated arrays to torch tensors: x and weights in the workload's
    dtype (exact, the values are already representable), bias in float32."""
    import torch

    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = {}
    for name, a in arrays.items():
        if a is None:
            out[name] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(a))
        if name != "bias":
            t = t.to(dt)
        out[name] = t.to(device)
    return out
