"""ctypes front end of the fp64 oracle in attn_ref.c.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Inputs are numpy arrays or
CPU torch tensors of any float dtype; they are widened to float64 here, so a
bf16 tensor is read as exactly the values it holds.
"""
import ctypes
import os

import numpy as np

from . import LIB_PATH, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i, d = ctypes.c_int, ctypes.c_double
        lib.oracle_attn_fwd.argtypes = [i, i, i, i, dp, dp, dp, d, i, dp, dp, i]
        lib.oracle_attn_fwd.restype = None
        lib.oracle_attn_bwd.argtypes = [i, i, i, i, dp, dp, dp, dp, d, i, dp, dp, dp, dp, dp, i]
        lib.oracle_attn_bwd.restype = None
        lib.oracle_attn_bwd_sampled.argtypes = [i, i, dp, dp, dp, dp, d, i, i, ip, i, ip, dp, dp, dp, dp, dp, i]
        lib.oracle_attn_bwd_sampled.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return _load().oracle_max_threads()


def attn_fwd(q, k, v, scale, causal, nthreads=0):
    """o [B,H,S,D] and lse [B,H,S] (natural log) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, S, D = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, H, S), dtype=np.float64)
    _load().oracle_attn_fwd(B, H, S, D, _p(q), _p(k), _p(v), float(scale), int(bool(causal)), _p(o), _p(lse),
                            int(nthreads))
    return o, lse


def attn_bwd(q, k, v, dout, scale, causal, nthreads=0):
    """dq, dk, dv [B,H,S,D], lse and delta [B,H,S], all fp64."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, S, D = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    lse = np.zeros((B, H, S), dtype=np.float64)
    delta = np.zeros((B, H, S), dtype=np.float64)
    _load().oracle_attn_bwd(B, H, S, D, _p(q), _p(k), _p(v), _p(dout), float(scale), int(bool(causal)), _p(dq),
                            _p(dk), _p(dv), _p(lse), _p(delta), int(nthreads))
    return dq, dk, dv, lse, delta


def attn_bwd_sampled(q, k, v, dout, scale, causal, rows, cols, nthreads=0):
    """One head ([S,D] tensors): dq at `rows`, dk/dv at `cols`, plus lse and delta for every row."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    S, D = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int32))
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < S)
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < S)
    dq = np.zeros((rows.size, D))
    dk = np.zeros((cols.size, D))
    dv = np.zeros((cols.size, D))
    lse = np.zeros(S)
    delta = np.zeros(S)
    ip = ctypes.POINTER(ctypes.c_int32)
    _load().oracle_attn_bwd_sampled(S, D, _p(q), _p(k), _p(v), _p(dout), float(scale), int(bool(causal)),
                                    rows.size, rows.ctypes.data_as(ip), cols.size, cols.ctypes.data_as(ip), _p(dq),
                                    _p(dk), _p(dv), _p(lse), _p(delta), int(nthreads))
    return dq, dk, dv, lse, delta
