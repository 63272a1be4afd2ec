"""Python binding of libmoe.so, the routed mixture-of-experts FFN layer for MI355X (gfx950).

Argument marshalling only: every function here forwards to the C entry point of the same
name in ``include/moe.h``; all arithmetic happens in the library's HIP kernels.  Tensors
are torch tensors on the GPU (torch provides device memory and streams); any argument may
also be passed as a raw integer device pointer.  A non-OK status raises ``MoeError``.

The library must have been built (``python -m routed_expert_ffn_router_amd.build`` or
``__graft_entry__.build()``); importing this package without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_WF_MXFP4, MOE_WF_NVFP4 = 0, 1
MOE_AQ_EXACT, MOE_AQ_MXFP8 = 0, 1
MOE_WS_STATUS_OFFSET = 0
MOE_WS_ROUTE_TIMEOUT, MOE_WS_BAD_EXPERT_ID = 0x1, 0x2


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_lib.moe_status_string(status).decode()} (status {status})")


class moe_shape(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("wformat", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("renorm_skip", ctypes.c_float), ("n_shared", ctypes.c_int32),
                ("act_quant", ctypes.c_int32)]


class moe_expert(ctypes.Structure):
    _fields_ = [("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("gate_ts", ctypes.c_float), ("up_ts", ctypes.c_float), ("down_ts", ctypes.c_float),
                ("reserved", ctypes.c_float)]


EXPERT_BYTES = ctypes.sizeof(moe_expert)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                      f"python -m routed_expert_ffn_router_amd.build")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_SP = ctypes.POINTER(moe_shape)
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
TRACE_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int, ctypes.c_void_p)
EVENT_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_char_p, ctypes.POINTER(ctypes.c_void_p),
                              ctypes.POINTER(ctypes.c_void_p))


class moe_observer(ctypes.Structure):
    _fields_ = [("trace_hook", ctypes.c_void_p), ("trace_user", ctypes.c_void_p),
                ("event_hook", ctypes.c_void_p), ("event_user", ctypes.c_void_p)]


_SIGS = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_blob_stride": (_sz, [_SP]),
    "moe_workspace_bytes": (_sz, [_SP, _i32]),
    "moe_workspace_init": (ctypes.c_int, [_SP, _i32, _P, _sz, _i32, _P]),
    "moe_fill_table": (ctypes.c_int, [_SP, _P, _sz, _P, _P]),
    "moe_route": (ctypes.c_int, [_SP, _P, _i32, _P, _P, _P, _P, _P, _sz, _P]),
    "moe_permute": (ctypes.c_int, [_SP, _P, _i32, _P, _P, _P, _P, _sz, _P]),
    "moe_gather_experts": (ctypes.c_int, [_SP, _P, _P, _i32, _P, _P, _P]),
    "moe_expert_ffn": (ctypes.c_int, [_SP, _P, _P, _i32, _P, _P, _P, _P, _sz, _P]),
    "moe_combine": (ctypes.c_int, [_SP, _P, _P, _P, _i32, _P, _P, _P]),
    "moe_layer": (ctypes.c_int, [_SP, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P]),
    "moe_layer_observed": (ctypes.c_int, [_SP, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P,
                                          ctypes.POINTER(moe_observer)]),
    "moe_layer_noalloc": (ctypes.c_int, [_SP, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def make_observer(trace=None, events=None):
    """An observer for moe_layer_observed: trace(kernel: str, phase: int, stream: int) is called
    before (phase 0) and after (phase 1) each kernel is enqueued; events(kernel: str) may return a
    pair of raw hipEvent_t handles (ints) that the kernel's own dispatch records at its start and
    end, or None.  Returns the structure; keep it alive for the duration of the call."""
    obs = moe_observer()
    refs = []
    if trace is not None:
        cb = TRACE_HOOK(lambda user, name, phase, stream: trace(name.decode(), phase, stream or 0))
        refs.append(cb)
        obs.trace_hook = ctypes.cast(cb, ctypes.c_void_p)
    if events is not None:
        def _ev(user, name, start, stop):
            pair = events(name.decode())
            if pair is not None:
                start[0], stop[0] = pair
        cb = EVENT_HOOK(_ev)
        refs.append(cb)
        obs.event_hook = ctypes.cast(cb, ctypes.c_void_p)
    obs._refs = refs         # the callbacks live as long as the structure
    return obs


def header_functions() -> list:
    """Names of the functions declared in include/moe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(moe_\w+)\s*\(", text, re.M)))


def library() -> ctypes.CDLL:
    return _lib


# ---------------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def make_shape(d_model: int, d_ff: int, n_experts: int, top_k: int, wformat: int = MOE_WF_MXFP4,
               act_dtype: int = MOE_DT_BF16, routed_scaling: float = 1.0, renorm_skip: float = 0.0,
               n_shared: int = 0, act_quant: int = MOE_AQ_EXACT) -> moe_shape:
    return moe_shape(d_model, d_ff, n_experts, top_k, wformat, act_dtype, routed_scaling, renorm_skip, n_shared,
                     act_quant)


def abi_version() -> int:
    return _lib.moe_abi_version()


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_blob_stride(shape: moe_shape) -> int:
    return _lib.moe_blob_stride(ctypes.byref(shape))


def moe_workspace_bytes(shape: moe_shape, T: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(shape), T)


def workspace(shape: moe_shape, T: int, device="cuda"):
    """A zero-filled uint8 device tensor of moe_workspace_bytes(shape, T) bytes (at least 256): a
    prepared workspace (status 0, default poll limit).

    The zero fill runs on torch's current stream: a caller that launches on another stream makes
    that stream wait for it first (torch.cuda.synchronize() or Stream.wait_stream), as for any input.
    """
    import torch
    n = max(moe_workspace_bytes(shape, T), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_workspace_init(shape, T: int, ws, poll_limit: int = 0, ws_bytes=None, stream=None):
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("moe_workspace_init", _lib.moe_workspace_init(ctypes.byref(shape), T, _ptr(ws), ws_bytes, poll_limit,
                                                         _stream(stream)))


def workspace_status(ws) -> int:
    """The workspace's status word (MOE_WS_* bits); reads 4 bytes back, so it synchronises."""
    import torch
    return int(ws[MOE_WS_STATUS_OFFSET:MOE_WS_STATUS_OFFSET + 4].cpu().view(torch.int32)[0]) & 0xFFFFFFFF


def moe_fill_table(shape, base, stride: int, table, stream=None):
    _check("moe_fill_table", _lib.moe_fill_table(ctypes.byref(shape), _ptr(base), stride, _ptr(table),
                                                 _stream(stream)))


def moe_route(shape, x, T: int, w_router, logit_bias, topk_idx, topk_w, ws, ws_bytes=None, stream=None):
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("moe_route", _lib.moe_route(ctypes.byref(shape), _ptr(x), T, _ptr(w_router), _ptr(logit_bias),
                                       _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)))


def moe_permute(shape, topk_idx, T: int, expert_offsets, sorted_pick, pick_pos, ws=None, ws_bytes=0,
                stream=None):
    _check("moe_permute", _lib.moe_permute(ctypes.byref(shape), _ptr(topk_idx), T, _ptr(expert_offsets),
                                           _ptr(sorted_pick), _ptr(pick_pos), _ptr(ws), ws_bytes,
                                           _stream(stream)))


def moe_gather_experts(shape, d_table, d_list, n: int, staging, d_staged_table, stream=None):
    _check("moe_gather_experts", _lib.moe_gather_experts(ctypes.byref(shape), _ptr(d_table), _ptr(d_list), n,
                                                         _ptr(staging), _ptr(d_staged_table), _stream(stream)))


def moe_expert_ffn(shape, d_table, x, T: int, expert_offsets, sorted_pick, o, ws, ws_bytes=None, stream=None):
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("moe_expert_ffn", _lib.moe_expert_ffn(ctypes.byref(shape), _ptr(d_table), _ptr(x), T,
                                                 _ptr(expert_offsets), _ptr(sorted_pick), _ptr(o), _ptr(ws),
                                                 ws_bytes, _stream(stream)))


def moe_combine(shape, o, topk_w, pick_pos, T: int, residual, y, stream=None):
    _check("moe_combine", _lib.moe_combine(ctypes.byref(shape), _ptr(o), _ptr(topk_w), _ptr(pick_pos), T,
                                           _ptr(residual), _ptr(y), _stream(stream)))


def moe_layer(shape, x, T: int, w_router, logit_bias, d_table, staging, residual, y, topk_idx_out=None,
              topk_w_out=None, ws=None, ws_bytes=None, stream=None, observer=None):
    """moe_layer, or moe_layer_observed when an observer (make_observer) is given."""
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    args = (ctypes.byref(shape), _ptr(x), T, _ptr(w_router), _ptr(logit_bias), _ptr(d_table), _ptr(staging),
            _ptr(residual), _ptr(y), _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), ws_bytes, _stream(stream))
    if observer is None:
        _check("moe_layer", _lib.moe_layer(*args))
    else:
        _check("moe_layer_observed", _lib.moe_layer_observed(*args, ctypes.byref(observer)))


def moe_layer_noalloc(shape, x, T: int, w_router, logit_bias, d_table, residual, y, topk_idx_out=None,
                      topk_w_out=None, stream=None):
    """moe_layer with the library's own per-GPU scratch array instead of a workspace (no allocation)."""
    _check("moe_layer_noalloc", _lib.moe_layer_noalloc(ctypes.byref(shape), _ptr(x), T, _ptr(w_router),
                                                       _ptr(logit_bias), _ptr(d_table), _ptr(residual), _ptr(y),
                                                       _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream)))
