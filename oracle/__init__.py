"""Python face of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It never imports
the HIP library's package and the HIP library never imports it; the two share
only the seeded input generators in ``synth``.

Every array handed to the C code is a numpy array; activations are converted to
float64 exactly (bf16 and fp32 values are all representable in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

MXFP4 = 0
NVFP4 = 1


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP, IEEE fp64, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_e2m1.restype = dbl
        L.oracle_e2m1.argtypes = [ctypes.c_uint]
        L.oracle_e8m0.restype = dbl
        L.oracle_e8m0.argtypes = [ctypes.c_uint]
        L.oracle_e4m3.restype = dbl
        L.oracle_e4m3.argtypes = [ctypes.c_uint]
        L.oracle_num_threads.restype = i32
        L.oracle_blob_stride.restype = i64
        L.oracle_blob_stride.argtypes = [i32, i32, i32]
        L.oracle_dequant.restype = i32
        L.oracle_dequant.argtypes = [P, P, dbl, i64, i64, i32, P]
        L.oracle_route.restype = i32
        L.oracle_route.argtypes = [P, i32, i32, P, P, i32, i32, dbl, P, P, P]
        L.oracle_permute.restype = i32
        L.oracle_permute.argtypes = [P, i32, i32, i32, P, P, P]
        L.oracle_expert_ffn.restype = i32
        L.oracle_expert_ffn.argtypes = [P, i32, i32, i32, i32, i32, P, i32, i32, P, P, P]
        L.oracle_e4m3_round.restype = dbl
        L.oracle_e4m3_round.argtypes = [dbl]
        L.oracle_quant_mxfp8.restype = None
        L.oracle_quant_mxfp8.argtypes = [P, i64]
        L.oracle_combine.restype = i32
        L.oracle_combine.argtypes = [P, P, P, i32, i32, i32, dbl, P, P, P]
        L.oracle_layer.restype = i32
        L.oracle_layer.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, dbl, dbl, P, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(v: float) -> float:
    """A parameter as the fp32 value the C ABI carries, widened exactly to fp64."""
    return float(np.float32(v))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# ---------------------------------------------------------------------------------------------
# conversions
# ---------------------------------------------------------------------------------------------


def to_f64(x) -> np.ndarray:
    """Exact fp64 copy of a bf16 / fp32 / fp64 torch tensor or numpy array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                bits = x.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
                return np.ascontiguousarray(bits.view(np.float32).astype(np.float64))
            return np.ascontiguousarray(x.numpy().astype(np.float64))
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e8m0(b: int) -> float:
    return lib().oracle_e8m0(b)


def e4m3(b: int) -> float:
    return lib().oracle_e4m3(b)


def num_threads() -> int:
    return lib().oracle_num_threads()


def blob_stride(d: int, f: int, wformat: int) -> int:
    return lib().oracle_blob_stride(d, f, wformat)


def dequant(q: np.ndarray, s: np.ndarray, rows: int, K: int, wformat: int, ts: float = 1.0) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    out = np.empty((rows, K), dtype=np.float64)
    _check(lib().oracle_dequant(_p(q), _p(s), ts, rows, K, wformat, _p(out)), "dequant")
    return out


# ---------------------------------------------------------------------------------------------
# layer steps
# ---------------------------------------------------------------------------------------------


def route(x64: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray], k: int, renorm_skip: float = 0.0):
    """Returns (logits [T,E] f64, idx [T,k] i32, w [T,k] f64); with renorm_skip, dropped picks have
    idx -1 and w 0.  renorm_skip is taken as the fp32 value the C ABI's moe_shape carries."""
    T, d = x64.shape
    E = w_router.shape[0]
    wr = np.ascontiguousarray(w_router, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    logits = np.empty((T, E), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _check(lib().oracle_route(_p(x64), T, d, _p(wr), _p(b), E, k, _f32(renorm_skip), _p(logits), _p(idx), _p(w)),
           "route")
    return logits, idx, w


def permute(idx: np.ndarray, E: int):
    """Returns (offsets [E+1], sorted_pick [T*k], pick_pos [T*k]) as int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    offsets = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(T * k, dtype=np.int32)
    pp = np.empty(T * k, dtype=np.int32)
    _check(lib().oracle_permute(_p(idx), T, k, E, _p(offsets), _p(sp), _p(pp)), "permute")
    return offsets, sp, pp


def _blob_ptrs(blobs: Sequence[Optional[np.ndarray]]):
    arr = (ctypes.c_void_p * len(blobs))()
    for i, b in enumerate(blobs):
        arr[i] = None if b is None else _p(b).value
    return arr


def e4m3_round(v: float) -> float:
    return lib().oracle_e4m3_round(v)


def quant_mxfp8(v: np.ndarray) -> np.ndarray:
    """The opt-in activation quantiser on a copy of v (length a multiple of 32, blocks of 32)."""
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    lib().oracle_quant_mxfp8(_p(out), out.size)
    return out


def expert_ffn(blobs, d: int, f: int, wformat: int, x64: np.ndarray, k: int,
               offsets: np.ndarray, sorted_pick: np.ndarray, act_quant: int = 0) -> np.ndarray:
    """o [T*k, d]; row i belongs to pick sorted_pick[i]."""
    T = x64.shape[0]
    E = len(blobs)
    o = np.empty((T * k, d), dtype=np.float64)
    ptrs = _blob_ptrs(blobs)
    _check(lib().oracle_expert_ffn(ctypes.cast(ptrs, ctypes.c_void_p), d, f, E, wformat, act_quant, _p(x64), T, k,
                                   _p(np.ascontiguousarray(offsets, dtype=np.int32)),
                                   _p(np.ascontiguousarray(sorted_pick, dtype=np.int32)), _p(o)),
           "expert_ffn")
    return o


def combine(o: np.ndarray, w: np.ndarray, pick_pos: np.ndarray, scaling: float = 1.0,
            residual: Optional[np.ndarray] = None, o_shared: Optional[np.ndarray] = None) -> np.ndarray:
    T, k = w.shape
    d = o.shape[1]
    y = np.empty((T, d), dtype=np.float64)
    _check(lib().oracle_combine(_p(np.ascontiguousarray(o)), _p(np.ascontiguousarray(w)),
                                _p(np.ascontiguousarray(pick_pos, dtype=np.int32)), T, k, d, scaling,
                                _p(o_shared), _p(residual), _p(y)), "combine")
    return y


def layer(x64: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray], blobs, d: int, f: int,
          k: int, wformat: int, scaling: float = 1.0, residual: Optional[np.ndarray] = None,
          renorm_skip: float = 0.0, shared_blob: Optional[np.ndarray] = None, act_quant: int = 0):
    """Whole layer (with the shared expert's blob, if given).  Returns (y [T,d] f64, idx [T,k] i32,
    w [T,k] f64, logits [T,E] f64)."""
    T = x64.shape[0]
    E = len(blobs)
    y = np.empty((T, d), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64)
    wr = np.ascontiguousarray(w_router, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ptrs = _blob_ptrs(blobs)
    _check(lib().oracle_layer(_p(x64), T, d, f, E, k, wformat, act_quant, scaling, _f32(renorm_skip), _p(wr), _p(b),
                              ctypes.cast(ptrs, ctypes.c_void_p),
                              None if shared_blob is None else _p(np.ascontiguousarray(shared_blob)),
                              _p(residual), _p(y), _p(idx), _p(w), _p(logits)), "layer")
    return y, idx, w, logits
