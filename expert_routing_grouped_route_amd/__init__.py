"""Python binding of the MoE-layer C ABI (``libmoe.so``, built for gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are passed as device pointers (``tensor.data_ptr()``) and the
stream as a raw ``hipStream_t`` handle; torch is not otherwise involved.  The
functions carry the names of the C entry points (see include/moe.h for the
contract of each) and raise ``MoeError`` when the library returns a status
other than MOE_OK.  There is no fallback: when the library has not been built
every call raises ``MoeLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_ERR_SCRATCH = 5
MOE_STATIC_SCRATCH_BYTES = 64 << 20

MOE_VARIANT_GLOBAL_LOADS = 1
MOE_VARIANT_BWD_VALU = 2

ENTRY_POINTS = ("moe_workspace_bytes", "moe_status_str", "moe_route", "moe_dispatch",
                "moe_grouped_ffn", "moe_combine", "moe_layer_fwd", "moe_layer_fwd_timed",
                "moe_layer_fwd_overlap", "moe_condensed_workspace_bytes",
                "moe_layer_fwd_condensed", "moe_backward_workspace_bytes", "moe_layer_bwd",
                "moe_layer_fwd_variant", "moe_layer_bwd_variant", "moe_layer_fwd_static")


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message}")
        self.status = status


class moe_dims_t(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("I_shared", ctypes.c_int32), ("dtype", ctypes.c_int)]


def dims(T, d, E, k, I, n_shared=0, I_shared=0, dtype="bf16") -> moe_dims_t:
    """Build a moe_dims_t; dtype is "bf16", "f32" or the integer code."""
    code = {"bf16": MOE_BF16, "f32": MOE_F32}.get(dtype, dtype)
    return moe_dims_t(int(T), int(d), int(E), int(k), int(I), int(n_shared), int(I_shared), int(code))


_lib = None
_P = ctypes.c_void_p
_DIMS = ctypes.POINTER(moe_dims_t)
_SIGS = {
    "moe_workspace_bytes": (ctypes.c_size_t, [_DIMS]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_grouped_ffn": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P]),
    "moe_layer_fwd": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_layer_fwd_timed": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P, ctypes.c_size_t,
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, _P]),
    "moe_layer_fwd_overlap": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P, _P]),
    "moe_condensed_workspace_bytes": (ctypes.c_size_t, [_DIMS]),
    "moe_layer_fwd_condensed": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_size_t, _P]),
    "moe_backward_workspace_bytes": (ctypes.c_size_t, [_DIMS]),
    "moe_layer_bwd": (ctypes.c_int, [_DIMS] + [_P] * 20 + [ctypes.c_size_t, _P]),
    "moe_layer_fwd_variant": (ctypes.c_int, [_DIMS] + [_P] * 16 + [ctypes.c_size_t, ctypes.c_int,
                                                                   _P]),
    "moe_layer_bwd_variant": (ctypes.c_int, [_DIMS] + [_P] * 20 + [ctypes.c_size_t, ctypes.c_int,
                                                                   _P]),
    "moe_layer_fwd_static": (ctypes.c_int, [_DIMS] + [_P] * 16),
}


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeLibraryMissing(
                f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoeError(fn, st, moe_status_str(st))


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def moe_workspace_bytes(d: moe_dims_t) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(d)))


def moe_route(d: moe_dims_t, x, w_router, bias, logits_in, logits_out, topk_ids, topk_w,
              stream=None):
    st = lib().moe_route(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits_in),
                         _ptr(logits_out), _ptr(topk_ids), _ptr(topk_w), _stream(stream))
    _check("moe_route", st)


def moe_dispatch(d: moe_dims_t, x, topk_ids, counts, offsets, perm, inv_perm, x_sorted, ws,
                 ws_bytes, stream=None):
    st = lib().moe_dispatch(ctypes.byref(d), _ptr(x), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                            _ptr(perm), _ptr(inv_perm), _ptr(x_sorted), _ptr(ws), int(ws_bytes),
                            _stream(stream))
    _check("moe_dispatch", st)


def moe_grouped_ffn(d: moe_dims_t, x_sorted, offsets, w_gate, w_up, w_down, x, wsh_gate, wsh_up,
                    wsh_down, y_sorted, y_shared, ws, ws_bytes, stream=None):
    st = lib().moe_grouped_ffn(ctypes.byref(d), _ptr(x_sorted), _ptr(offsets), _ptr(w_gate),
                               _ptr(w_up), _ptr(w_down), _ptr(x), _ptr(wsh_gate), _ptr(wsh_up),
                               _ptr(wsh_down), _ptr(y_sorted), _ptr(y_shared), _ptr(ws),
                               int(ws_bytes), _stream(stream))
    _check("moe_grouped_ffn", st)


def moe_combine(d: moe_dims_t, y_sorted, inv_perm, topk_w, y_shared, out, stream=None):
    st = lib().moe_combine(ctypes.byref(d), _ptr(y_sorted), _ptr(inv_perm), _ptr(topk_w),
                           _ptr(y_shared), _ptr(out), _stream(stream))
    _check("moe_combine", st)


def moe_layer_fwd(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up,
                  wsh_down, out, topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out, ws,
                  ws_bytes, stream=None):
    st = lib().moe_layer_fwd(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
                             _ptr(w_up), _ptr(w_down), _ptr(wsh_gate), _ptr(wsh_up),
                             _ptr(wsh_down), _ptr(out), _ptr(topk_ids_out), _ptr(topk_w_out),
                             _ptr(counts_out), _ptr(offsets_out), _ptr(perm_out), _ptr(ws),
                             int(ws_bytes), _stream(stream))
    _check("moe_layer_fwd", st)


def moe_layer_fwd_timed(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up,
                        wsh_down, out, topk_ids_out, topk_w_out, counts_out, offsets_out, perm_out,
                        ws, ws_bytes, events, stream=None):
    """``events``: raw hipEvent_t handles (ints), e.g. ``torch.cuda.Event.cuda_event``."""
    arr = (ctypes.c_void_p * max(1, len(events)))(*[int(e) for e in events])
    st = lib().moe_layer_fwd_timed(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias),
                                   _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wsh_gate),
                                   _ptr(wsh_up), _ptr(wsh_down), _ptr(out), _ptr(topk_ids_out),
                                   _ptr(topk_w_out), _ptr(counts_out), _ptr(offsets_out),
                                   _ptr(perm_out), _ptr(ws), int(ws_bytes), arr, len(events),
                                   _stream(stream))
    _check("moe_layer_fwd_timed", st)


def moe_layer_fwd_overlap(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate,
                          wsh_up, wsh_down, out, topk_ids_out, topk_w_out, counts_out, offsets_out,
                          perm_out, ws, ws_bytes, side, fork, join, stream=None):
    """Shared experts on ``side`` (a torch.cuda.Stream or raw handle); ``fork`` and
    ``join`` are torch.cuda.Event objects or raw hipEvent_t handles."""
    ev = lambda e: int(e) if isinstance(e, int) else int(e.cuda_event)
    st = lib().moe_layer_fwd_overlap(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias),
                                     _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wsh_gate),
                                     _ptr(wsh_up), _ptr(wsh_down), _ptr(out), _ptr(topk_ids_out),
                                     _ptr(topk_w_out), _ptr(counts_out), _ptr(offsets_out),
                                     _ptr(perm_out), _ptr(ws), int(ws_bytes), _stream(stream),
                                     _stream(side), ev(fork), ev(join))
    _check("moe_layer_fwd_overlap", st)


def moe_condensed_workspace_bytes(d: moe_dims_t) -> int:
    return int(lib().moe_condensed_workspace_bytes(ctypes.byref(d)))


def moe_layer_fwd_condensed(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate,
                            wsh_up, wsh_down, hyperplanes, cos_threshold, out, topk_ids_out,
                            topk_w_out, counts_out, offsets_out, perm_out, rep_out, ws, ws_bytes,
                            stream=None):
    """The layer with token condensation; ``hyperplanes`` is [16, d] in the dtype of x."""
    st = lib().moe_layer_fwd_condensed(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias),
                                       _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wsh_gate),
                                       _ptr(wsh_up), _ptr(wsh_down), _ptr(hyperplanes),
                                       float(cos_threshold), _ptr(out), _ptr(topk_ids_out),
                                       _ptr(topk_w_out), _ptr(counts_out), _ptr(offsets_out),
                                       _ptr(perm_out), _ptr(rep_out), _ptr(ws), int(ws_bytes),
                                       _stream(stream))
    _check("moe_layer_fwd_condensed", st)


def moe_backward_workspace_bytes(d: moe_dims_t) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(d)))


def moe_layer_bwd(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate, wsh_up,
                  wsh_down, dout, dx, dw_router, dbias, dw_gate, dw_up, dw_down, dwsh_gate,
                  dwsh_up, dwsh_down, ws, ws_bytes, stream=None):
    st = lib().moe_layer_bwd(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
                             _ptr(w_up), _ptr(w_down), _ptr(wsh_gate), _ptr(wsh_up),
                             _ptr(wsh_down), _ptr(dout), _ptr(dx), _ptr(dw_router), _ptr(dbias),
                             _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(dwsh_gate),
                             _ptr(dwsh_up), _ptr(dwsh_down), _ptr(ws), int(ws_bytes),
                             _stream(stream))
    _check("moe_layer_bwd", st)


def moe_layer_fwd_variant(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate,
                          wsh_up, wsh_down, out, topk_ids_out, topk_w_out, counts_out,
                          offsets_out, perm_out, ws, ws_bytes, variant, stream=None):
    st = lib().moe_layer_fwd_variant(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias),
                                     _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wsh_gate),
                                     _ptr(wsh_up), _ptr(wsh_down), _ptr(out), _ptr(topk_ids_out),
                                     _ptr(topk_w_out), _ptr(counts_out), _ptr(offsets_out),
                                     _ptr(perm_out), _ptr(ws), int(ws_bytes), int(variant),
                                     _stream(stream))
    _check("moe_layer_fwd_variant", st)


def moe_layer_bwd_variant(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate,
                          wsh_up, wsh_down, dout, dx, dw_router, dbias, dw_gate, dw_up, dw_down,
                          dwsh_gate, dwsh_up, dwsh_down, ws, ws_bytes, variant, stream=None):
    st = lib().moe_layer_bwd_variant(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias),
                                     _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wsh_gate),
                                     _ptr(wsh_up), _ptr(wsh_down), _ptr(dout), _ptr(dx),
                                     _ptr(dw_router), _ptr(dbias), _ptr(dw_gate), _ptr(dw_up),
                                     _ptr(dw_down), _ptr(dwsh_gate), _ptr(dwsh_up),
                                     _ptr(dwsh_down), _ptr(ws), int(ws_bytes), int(variant),
                                     _stream(stream))
    _check("moe_layer_bwd_variant", st)


def moe_layer_fwd_static(d: moe_dims_t, x, w_router, bias, w_gate, w_up, w_down, wsh_gate,
                         wsh_up, wsh_down, out, topk_ids_out, topk_w_out, counts_out, offsets_out,
                         perm_out, stream=None):
    """moe_layer_fwd on the library's static device scratch (no workspace)."""
    st = lib().moe_layer_fwd_static(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias),
                                    _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wsh_gate),
                                    _ptr(wsh_up), _ptr(wsh_down), _ptr(out), _ptr(topk_ids_out),
                                    _ptr(topk_w_out), _ptr(counts_out), _ptr(offsets_out),
                                    _ptr(perm_out), _stream(stream))
    _check("moe_layer_fwd_static", st)
