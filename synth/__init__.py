"""Seeded synthetic inputs, shared by the CPU oracle and the GPU tests/bench.

Holds no arithmetic of the method (no routing, dequantization or FFN).  The
heavy lifting (weights, records) is in ``synth.c``; this wrapper only
marshals arrays.  See ``synth.c`` for the generator and record byte layout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")

FMT_INT4 = 0
FMT_NVFP4 = 1

TAG_WEIGHT = 1
TAG_X = 2
TAG_ROUTER = 3
TAG_PREFILL_X = 4

WEIGHT_SIGMA = 0.02


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (plain C, no GPU code)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-mavx2", "-mfma", "-ffp-contract=off", "-fno-math-errno", "-fPIC",
                               "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64, u64, u64]
        L.synth_normal_f32.argtypes = [u64, u64, u64, u64, i64, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, u64, i64, dbl, vp]
        L.synth_uniform_f64.argtypes = [u64, u64, u64, u64, i64, vp]
        L.synth_record_bytes.restype = i64
        L.synth_record_bytes.argtypes = [i64, i64]
        L.synth_weights_f32.argtypes = [u64, i64, i64, i64, i32, i64, i64, dbl, vp]
        L.synth_record.argtypes = [u64, i64, i64, i64, i64, i64, i32, dbl, vp, vp, vp]
        L.synth_fill_records.restype = i32
        L.synth_fill_records.argtypes = [u64, i64, i64, i64, i32, dbl, i64, i64, vp, vp, i32]
        L.synth_zipf_logp.argtypes = [u64, i64, i64, dbl, vp]
        L.synth_trace_logits.argtypes = [u64, i64, i64, dbl, i64, i64, vp]
        L.synth_spec_ids.argtypes = [u64, i64, i64, dbl, i64, vp, i32, dbl, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def record_bytes(H: int, I: int) -> int:
    return int(lib().synth_record_bytes(H, I))


def weights_f32(seed: int, E: int, l: int, e: int, m: int, H: int, I: int, sigma: float = WEIGHT_SIGMA) -> np.ndarray:
    """Float weights (before quantization) of matrix m (0 gate [I,H], 1 up [I,H], 2 down [H,I])."""
    N, Kd = (H, I) if m == 2 else (I, H)
    out = np.empty((N, Kd), np.float32)
    lib().synth_weights_f32(seed, E, l, e, m, H, I, sigma, _ptr(out))
    return out


def record(seed: int, E: int, l: int, e: int, H: int, I: int, fmt: int, sigma: float = WEIGHT_SIGMA):
    """(record bytes uint8[R], tensor scales float32[3]) of expert (l, e)."""
    R = record_bytes(H, I)
    rec = np.empty(R, np.uint8)
    ts = np.empty(3, np.float32)
    scratch = np.empty(H * I, np.float32)
    lib().synth_record(seed, E, l, e, H, I, fmt, sigma, _ptr(rec), _ptr(ts), _ptr(scratch))
    return rec, ts


def fill_records(seed: int, E: int, H: int, I: int, fmt: int, first: int, count: int, dst_ptr: int,
                 ts_out: np.ndarray, nthreads: int = 8, sigma: float = WEIGHT_SIGMA) -> None:
    """Write `count` records (flat ids first..first+count-1) to raw memory at dst_ptr.

    ts_out: float32[count*3] receives the tensor scales."""
    assert ts_out.dtype == np.float32 and ts_out.size >= 3 * count and ts_out.flags.c_contiguous
    rc = lib().synth_fill_records(seed, E, H, I, fmt, sigma, first, count, ctypes.c_void_p(dst_ptr),
                                  _ptr(ts_out), nthreads)
    if rc != 0:
        raise RuntimeError("synth_fill_records failed: %d" % rc)


def pool_numpy(seed: int, L: int, E: int, H: int, I: int, fmt: int, nthreads: int = 8):
    """Whole pool as a numpy array (small configs only): (pool uint8[L*E, R], ts float32[L*E, 3])."""
    R = record_bytes(H, I)
    pool = np.empty((L * E, R), np.uint8)
    ts = np.empty((L * E, 3), np.float32)
    fill_records(seed, E, H, I, fmt, 0, L * E, _ptr(pool), ts.reshape(-1), nthreads)
    return pool, ts


def normal_bf16(seed: int, tag: int, a: int, b: int, n: int, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(seed, tag, a, b, n, scale, _ptr(out))
    return out


def activations(seed: int, layer: int, t0: int, n: int, H: int, tag: int = TAG_X) -> np.ndarray:
    """bf16 bits [n, H] of ~N(0,1) activations for tokens t0..t0+n-1 at `layer`."""
    out = np.empty((n, H), np.uint16)
    for t in range(n):
        out[t] = normal_bf16(seed, tag, layer, t0 + t, H)
    return out


def router_weights(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    """bf16 bits [E, H] of router weights ~N(0, 1/H)."""
    return normal_bf16(seed, TAG_ROUTER, layer, 0, E * H, 1.0 / np.sqrt(H)).reshape(E, H)


def zipf_logp(seed: int, layer: int, E: int, s: float) -> np.ndarray:
    out = np.empty(E, np.float64)
    lib().synth_zipf_logp(seed, layer, E, s, _ptr(out))
    return out


def trace_logits(seed: int, layer: int, E: int, s: float, t0: int, n: int) -> np.ndarray:
    """fp32 [n, E] trace logits: log p (Zipf(s) over a seeded permutation) + Gumbel noise."""
    out = np.empty((n, E), np.float32)
    lib().synth_trace_logits(seed, layer, E, s, t0, n, _ptr(out))
    return out


def gumbel_topk_sets(logits: np.ndarray, K: int) -> np.ndarray:
    """The K experts each trace row draws (largest perturbed log-probabilities), int32 [n, K].

    Generator-side only: used to build speculative predictions from the true draw."""
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def spec_ids(seed: int, layer: int, E: int, s: float, t: int, truth: np.ndarray, keep: float) -> np.ndarray:
    truth = np.ascontiguousarray(truth, np.int32)
    out = np.empty(truth.size, np.int32)
    lib().synth_spec_ids(seed, layer, E, s, t, _ptr(truth), truth.size, keep, _ptr(out))
    return out


def uniform(seed: int, tag: int, a: int, b: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform_f64(seed, tag, a, b, n, _ptr(out))
    return out
