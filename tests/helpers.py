"""Shared helpers for the GPU parity tests: pinned pools filled by the seeded
generator, engine construction, tolerance checks.  The oracle reads the same
pinned bytes the library copies from (written by the generator, never by the GPU)."""
from __future__ import annotations

import ctypes

import os

import numpy as np

import synth

REL_L2 = 5e-3
MAX_ABS = 2e-2


class PinnedPool:
    """L*E records in pinned host memory (eff_host_alloc), filled by synth."""

    def __init__(self, eff, seed, L, E, H, I, fmt, nthreads=16, layers=None, flats=None):
        self.eff = eff
        self.L, self.E, self.H, self.I, self.fmt = L, E, H, I, fmt
        self.R = synth.record_bytes(H, I)
        self.nbytes = L * E * self.R
        self.ptr = eff.host_alloc(self.nbytes)
        self.ts = np.ones(L * E * 3, np.float32)
        if flats is not None:   # only these records (the generator keys each record by its flat id)
            fl = sorted(set(int(f) for f in flats))
            i = 0
            while i < len(fl):
                j = i
                while j + 1 < len(fl) and fl[j + 1] == fl[j] + 1:
                    j += 1
                n = j - i + 1
                ts = np.empty(n * 3, np.float32)
                synth.fill_records(seed, E, H, I, fmt, fl[i], n, self.ptr + fl[i] * self.R, ts, nthreads)
                self.ts[fl[i] * 3:(fl[i] + n) * 3] = ts
                i = j + 1
            return
        layers = range(L) if layers is None else layers
        for l in layers:   # layers not listed stay unfilled (never routed to in that test)
            ts = np.empty(E * 3, np.float32)
            synth.fill_records(seed, E, H, I, fmt, l * E, E, self.ptr + l * E * self.R, ts, nthreads)
            self.ts[l * E * 3:(l + 1) * E * 3] = ts

    def record(self, flat: int) -> np.ndarray:
        buf = (ctypes.c_uint8 * self.R).from_address(self.ptr + flat * self.R)
        return np.frombuffer(buf, np.uint8)

    def tensor_scales(self, flat: int) -> np.ndarray:
        return self.ts[flat * 3:flat * 3 + 3]

    def free(self):
        if self.ptr:
            self.eff.host_free(self.ptr)
            self.ptr = 0


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# worst rel-L2 / max-abs seen per test, printed at the end of the session (tests/conftest.py)
OBSERVED = {}


def record_error(err, mx):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    e0, m0, n0 = OBSERVED.get(test, (0.0, 0.0, 0))
    OBSERVED[test] = (max(e0, err), max(m0, mx), n0 + 1)


def assert_close_bf16(got_bits, ref_bits, rel=REL_L2, mabs=MAX_ABS, what=""):
    g, r = bf16_to_f64(got_bits), bf16_to_f64(ref_bits)
    err = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    mx = float(np.max(np.abs(g - r))) if g.size else 0.0
    record_error(err, mx)
    assert err <= rel and mx <= mabs, "%s rel-L2 %.3e (<= %.1e) max-abs %.3e (<= %.1e)" % (what, err, rel, mx, mabs)
    return err, mx


def rel_l2(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def make_engine(eff, pool: PinnedPool, K, S, max_tokens, f_q16, max_prefill_tokens=0, host_threads=8, flags=0):
    cfg = eff.make_config(pool.L, pool.E, K, pool.H, pool.I, pool.fmt, S, max_tokens, max_prefill_tokens,
                          f_q16, host_threads, flags)
    ts = pool.ts if pool.fmt == synth.FMT_NVFP4 else None
    return eff.Engine(cfg, pool.ptr, ts)


def oracle_engine(pool: PinnedPool, K, S, f_q16, use_c=None):
    from oracle.engine import OracleEngine
    return OracleEngine(pool.L, pool.E, K, pool.H, pool.I, pool.fmt, S, f_q16, pool.record, pool.tensor_scales,
                        use_c=use_c, nthreads=16)
