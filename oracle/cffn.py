"""Binding of ffn_ref.c: the oracle's expert FFN as plain C loops (double precision).

Test infrastructure only (see oracle/__init__.py)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ffn_ref.c")
_SO = os.path.join(_HERE, "liboracle_ffn.so")


def build(force: bool = False) -> str:
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Job(ctypes.Structure):
    _fields_ = [("rec", ctypes.c_void_p), ("ts3", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("nt", ctypes.c_int)]


_lib = None


def _l():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        L.oracle_expert_ffn_batch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int]
        L.oracle_expert_ffn_batch.restype = ctypes.c_int
        _lib = L
    return _lib


def expert_ffn_batch(jobs, fmt: int, H: int, I: int, nthreads: int = 8):
    """jobs: list of (record uint8[R], ts float32[3], x float64[nt, H]); returns list of y float64[nt, H]."""
    keep, outs = [], []
    arr = (_Job * max(1, len(jobs)))()
    for j, (rec, ts, x) in enumerate(jobs):
        rec = np.ascontiguousarray(rec, np.uint8)
        ts = np.ascontiguousarray(ts, np.float32)
        x = np.ascontiguousarray(x, np.float64)
        y = np.zeros_like(x)
        keep += [rec, ts, x]
        outs.append(y)
        arr[j] = _Job(rec.ctypes.data, ts.ctypes.data, x.ctypes.data, y.ctypes.data, x.shape[0])
    if jobs:
        _l().oracle_expert_ffn_batch(ctypes.addressof(arr), len(jobs), fmt, H, I, nthreads)
    return outs
