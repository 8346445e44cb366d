"""The C ABI on the host: the library loads without a GPU, exports every entry
point include/moe.h declares (and nothing else of its own), and rejects
invalid arguments with the documented status before any HIP call.

Every call here fails validation, so no kernel is ever launched."""
import ctypes
import os
import re
import subprocess

import pytest

import expert_routing_grouped_route_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_entry_points():
    text = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


def test_header_and_binding_agree():
    names = declared_entry_points()
    assert sorted(names) == sorted(moe.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for name in declared_entry_points():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    ours = {s for s in exported if s.startswith("moe") or "moe" in s}
    assert ours == set(declared_entry_points())


def test_status_strings():
    names = ["MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
             "MOE_ERR_HIP", "MOE_ERR_SCRATCH"]
    for code, name in enumerate(names):
        assert moe.moe_status_str(code).startswith(name)
    assert moe.moe_status_str(99) == "unknown moe_status_t"


GOOD = dict(T=1000, d=256, E=16, k=4, I=384, n_shared=1, I_shared=256, dtype="bf16")


def dims(**kw):
    p = dict(GOOD)
    p.update(kw)
    return moe.dims(**p)


def test_workspace_bytes():
    d = dims()
    ws = moe.moe_workspace_bytes(d)
    R = 1000 * 4
    # at least A (bf16) and y_sorted (fp32)
    assert ws >= R * 384 * 2 + R * 256 * 4
    assert moe.moe_workspace_bytes(dims(T=2000)) > ws
    assert moe.moe_workspace_bytes(dims(dtype="f32")) > ws
    assert moe.moe_workspace_bytes(dims(T=0)) > 0
    for bad in (dict(E=300), dict(k=17, E=20), dict(d=100), dict(T=-1), dict(n_shared=1, I_shared=0)):
        assert moe.moe_workspace_bytes(dims(**bad)) == 0, bad


@pytest.mark.parametrize("bad,code", [
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(d=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=2, I_shared=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=0, I_shared=64), moe.MOE_ERR_INVALID_ARG),
    (dict(E=257), moe.MOE_ERR_UNSUPPORTED),
    (dict(k=17, E=32), moe.MOE_ERR_UNSUPPORTED),
    (dict(k=5, E=4), moe.MOE_ERR_UNSUPPORTED),
    (dict(d=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(I=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(I_shared=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 29, k=4), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_dims_rejected_by_every_entry_point(bad, code):
    d = dims(**bad)
    P = 1 << 40  # never dereferenced: validation fails first
    lib = moe.lib()
    assert lib.moe_route(ctypes.byref(d), P, P, None, None, None, P, P, 0) == code
    assert lib.moe_dispatch(ctypes.byref(d), P, P, P, P, P, P, P, P, 1 << 40, 0) == code
    assert lib.moe_grouped_ffn(ctypes.byref(d), P, P, P, P, P, P, P, P, P, P, P, P, 1 << 40, 0) == code
    assert lib.moe_combine(ctypes.byref(d), P, P, P, None, P, 0) == code
    assert lib.moe_layer_fwd(ctypes.byref(d), P, P, None, P, P, P, P, P, P, P, None, None, None,
                             None, None, P, 1 << 40, 0) == code
    assert lib.moe_layer_fwd_overlap(ctypes.byref(d), P, P, None, P, P, P, P, P, P, P, None, None,
                                     None, None, None, P, 1 << 40, 0, P, P, P) == code


def test_null_dims_rejected():
    lib = moe.lib()
    assert lib.moe_route(None, 0, 0, None, None, None, 0, 0, 0) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_bytes(None) == 0


class Bufs:
    """Distinct, 256-byte aligned fake device addresses, 4 GiB apart."""

    def __init__(self):
        self.n = 0

    def __call__(self):
        self.n += 1
        return (1 << 40) + (self.n << 32)


def layer_args(d, **override):
    b = Bufs()
    a = dict(x=b(), w_router=b(), bias=None, w_gate=b(), w_up=b(), w_down=b(), wsh_gate=b(),
             wsh_up=b(), wsh_down=b(), out=b(), ids=None, w=None, counts=None, offsets=None,
             perm=None, ws=b(), ws_bytes=moe.moe_workspace_bytes(d))
    a.update(override)
    return a


def call_layer(d, a):
    return moe.lib().moe_layer_fwd(ctypes.byref(d), a["x"], a["w_router"], a["bias"], a["w_gate"],
                                   a["w_up"], a["w_down"], a["wsh_gate"], a["wsh_up"],
                                   a["wsh_down"], a["out"], a["ids"], a["w"], a["counts"],
                                   a["offsets"], a["perm"], a["ws"], a["ws_bytes"], 0)


@pytest.mark.parametrize("override,code", [
    (dict(x=None), moe.MOE_ERR_INVALID_ARG),
    (dict(out=None), moe.MOE_ERR_INVALID_ARG),
    (dict(ws=None), moe.MOE_ERR_INVALID_ARG),
    (dict(wsh_down=None), moe.MOE_ERR_INVALID_ARG),
    (dict(w_gate=(1 << 40) + 8), moe.MOE_ERR_INVALID_ARG),  # misaligned
    (dict(bias=(1 << 41) + 4), moe.MOE_ERR_INVALID_ARG),    # misaligned optional input
    (dict(ws_bytes=1024), moe.MOE_ERR_WORKSPACE),
])
def test_layer_rejects_bad_buffers(override, code):
    d = dims()
    a = layer_args(d)
    if "w_gate" in override:
        override = dict(w_gate=a["w_gate"] + 8)
    a.update(override)
    assert call_layer(d, a) == code


def test_layer_rejects_output_overlapping_input():
    d = dims()
    a = layer_args(d)
    a["out"] = a["x"] + 4096  # inside x [T, d] bf16
    assert call_layer(d, a) == moe.MOE_ERR_INVALID_ARG
    a = layer_args(d)
    a["ids"] = a["ws"] + 256  # an optional output inside the workspace
    assert call_layer(d, a) == moe.MOE_ERR_INVALID_ARG


def test_inputs_may_alias_each_other():
    d = dims()
    a = layer_args(d)
    a["w_up"] = a["w_gate"]  # read-only buffers may be shared
    a["ws_bytes"] = 1024     # stop at the workspace check, before any launch
    assert call_layer(d, a) == moe.MOE_ERR_WORKSPACE


def test_route_requires_x_only_without_given_logits():
    d = dims()
    lib = moe.lib()
    b = Bufs()
    ids, w = b(), b()
    assert lib.moe_route(ctypes.byref(d), None, b(), None, None, None, ids, w, 0) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(d), b(), b(), None, None, None, None, w, 0) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(d), b(), b(), None, None, b() + 4, ids, w, 0) == moe.MOE_ERR_INVALID_ARG


def test_overlap_layer_requires_side_stream_and_events():
    d = dims()
    a = layer_args(d)
    lib = moe.lib()
    args = [ctypes.byref(d), a["x"], a["w_router"], None, a["w_gate"], a["w_up"], a["w_down"],
            a["wsh_gate"], a["wsh_up"], a["wsh_down"], a["out"], None, None, None, None, None,
            a["ws"], a["ws_bytes"], 0]
    b = Bufs()
    side, fork, join = b(), b(), b()  # never dereferenced: validation fails first
    assert lib.moe_layer_fwd_overlap(*args, None, fork, join) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_fwd_overlap(*args, side, None, join) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_fwd_overlap(*args, side, fork, None) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[-2] = 1024  # workspace too small: rejected before any event or launch
    assert lib.moe_layer_fwd_overlap(*bad, side, fork, join) == moe.MOE_ERR_WORKSPACE


def test_timed_layer_rejects_bad_event_list():
    d = dims()
    a = layer_args(d)
    lib = moe.lib()
    arr = (ctypes.c_void_p * 7)(*([1] * 7))
    args = [ctypes.byref(d), a["x"], a["w_router"], None, a["w_gate"], a["w_up"], a["w_down"],
            a["wsh_gate"], a["wsh_up"], a["wsh_down"], a["out"], None, None, None, None, None,
            a["ws"], a["ws_bytes"]]
    assert lib.moe_layer_fwd_timed(*args, arr, 7, 0) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_fwd_timed(*args, None, 3, 0) == moe.MOE_ERR_INVALID_ARG
    zero = (ctypes.c_void_p * 2)(None, None)
    assert lib.moe_layer_fwd_timed(*args, zero, 2, 0) == moe.MOE_ERR_INVALID_ARG


def _call_condensed(d, a, hyper, thr, rep, ws_bytes):
    return moe.lib().moe_layer_fwd_condensed(
        ctypes.byref(d), a["x"], a["w_router"], None, a["w_gate"], a["w_up"], a["w_down"],
        a["wsh_gate"], a["wsh_up"], a["wsh_down"], hyper, thr, a["out"], None, None, None, None,
        None, rep, a["ws"], ws_bytes, 0)


def test_condensed_workspace_is_larger_and_covers_the_layer():
    d = dims()
    assert moe.moe_condensed_workspace_bytes(d) > moe.moe_workspace_bytes(d)
    assert moe.lib().moe_condensed_workspace_bytes(None) == 0


def test_condensed_layer_validation():
    d = dims()
    a = layer_args(d)
    hyper, rep = (1 << 44), (1 << 44) + (1 << 32)  # apart from layer_args' buffers
    need = moe.moe_condensed_workspace_bytes(d)
    # hyperplanes are required; the threshold must not be NaN
    assert _call_condensed(d, a, None, 0.9, None, need) == moe.MOE_ERR_INVALID_ARG
    assert _call_condensed(d, a, hyper, float("nan"), None, need) == moe.MOE_ERR_INVALID_ARG
    # the plain layer's workspace is not enough
    assert _call_condensed(d, a, hyper, 0.9, rep, moe.moe_workspace_bytes(d)) == moe.MOE_ERR_WORKSPACE
    # rep_out must not overlap another buffer, hyperplanes must be aligned
    assert _call_condensed(d, a, hyper, 0.9, a["x"] + 256, need) == moe.MOE_ERR_INVALID_ARG
    assert _call_condensed(d, a, hyper + 8, 0.9, None, need) == moe.MOE_ERR_INVALID_ARG


def _bwd_call(d, ptrs, ws_bytes, **over):
    names = ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "wsh_gate", "wsh_up",
             "wsh_down", "dout", "dx", "dw_router", "dbias", "dw_gate", "dw_up", "dw_down",
             "dwsh_gate", "dwsh_up", "dwsh_down", "ws")
    p = dict(ptrs)
    p.update(over)
    return moe.lib().moe_layer_bwd(ctypes.byref(d), *[p[n] for n in names], ws_bytes, 0)


def _bwd_ptrs():
    # distinct, 1 TiB apart, never dereferenced (every case fails validation)
    names = ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "wsh_gate", "wsh_up",
             "wsh_down", "dout", "dx", "dw_router", "dbias", "dw_gate", "dw_up", "dw_down",
             "dwsh_gate", "dwsh_up", "dwsh_down", "ws")
    return {n: (i + 1) << 40 for i, n in enumerate(names)}


def test_backward_workspace_covers_the_layer_workspace():
    d = dims(n_shared=1, I_shared=128)
    assert moe.moe_backward_workspace_bytes(d) > moe.moe_workspace_bytes(d)
    assert moe.lib().moe_backward_workspace_bytes(None) == 0
    assert moe.moe_backward_workspace_bytes(dims(E=300)) == 0


def test_backward_validation():
    d = dims(n_shared=1, I_shared=128)
    need = moe.moe_backward_workspace_bytes(d)
    p = _bwd_ptrs()
    assert _bwd_call(dims(E=300), p, need) == moe.MOE_ERR_UNSUPPORTED
    assert _bwd_call(d, p, need - 1) == moe.MOE_ERR_WORKSPACE
    assert _bwd_call(d, p, moe.moe_workspace_bytes(d)) == moe.MOE_ERR_WORKSPACE
    for req in ("x", "dout", "dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dwsh_gate", "ws"):
        assert _bwd_call(d, p, need, **{req: None}) == moe.MOE_ERR_INVALID_ARG, req
    assert _bwd_call(d, p, need, dx=p["x"] + 16) == moe.MOE_ERR_INVALID_ARG  # output overlaps x
    assert _bwd_call(d, p, need, dw_gate=p["dw_gate"] + 4) == moe.MOE_ERR_INVALID_ARG  # misaligned
    # without shared experts their gradients may be NULL
    d0 = dims()
    assert _bwd_call(d0, p, need, wsh_gate=None, wsh_up=None, wsh_down=None, dwsh_gate=None,
                     dwsh_up=None, dwsh_down=None, ws=None) == moe.MOE_ERR_INVALID_ARG


def test_variant_entry_points_reject_unknown_bits():
    """Only the documented variant bits are accepted (checked before any launch)."""
    d = dims()
    a = layer_args(d)
    lib = moe.lib()
    fwd = [ctypes.byref(d), a["x"], a["w_router"], None, a["w_gate"], a["w_up"], a["w_down"],
           a["wsh_gate"], a["wsh_up"], a["wsh_down"], a["out"], None, None, None, None, None,
           a["ws"], a["ws_bytes"]]
    assert lib.moe_layer_fwd_variant(*fwd, moe.MOE_VARIANT_BWD_VALU, 0) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_fwd_variant(*fwd, 8, 0) == moe.MOE_ERR_INVALID_ARG
    b = Bufs()
    bwd = [ctypes.byref(d)] + [b() for _ in range(20)] + [1 << 40]
    assert lib.moe_layer_bwd_variant(*bwd, 4, 0) == moe.MOE_ERR_INVALID_ARG


def test_static_layer_refuses_sizes_beyond_its_scratch():
    """moe_layer_fwd_static checks the workspace its sizes need against the
    static scratch before touching the device (no GPU needed to refuse)."""
    lib = moe.lib()
    big = moe.dims(4096, 2048, 64, 6, 1408, 2, 1408, "bf16")
    assert moe.moe_workspace_bytes(big) > moe.MOE_STATIC_SCRATCH_BYTES
    b = Bufs()
    args = [ctypes.byref(big)] + [b() for _ in range(15)] + [0]
    assert lib.moe_layer_fwd_static(*args) == moe.MOE_ERR_SCRATCH
    bad = moe.dims(16, 100, 4, 2, 64)  # d not a multiple of 64
    assert lib.moe_layer_fwd_static(ctypes.byref(bad), *args[1:]) == moe.MOE_ERR_UNSUPPORTED
