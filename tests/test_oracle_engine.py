"""Pins of the oracle's composed decode and prefill layers (tiny workload).

* Cache-size invariance: outputs are bit-identical for every cache size and
  every f ([FT-deep] §4: GPU memory changes speed, never the result; [FT-blog]
  §四 "GPU 显存只影响性能，永远不影响正确性").  GPU entries are evaluated from the
  copied slot bytes, so a wrong table entry or copy would show.
* Negative control: copying the wrong record into a slot must change the output.
* Prefill equals T independent decodes; the on-demand fallback (S < 2E)
  equals the double-buffered path; streamed slot bytes equal the host records.
"""
import numpy as np
import pytest

import synth
from synth.configs import TINY
from oracle.engine import OracleEngine

W = TINY


@pytest.fixture(scope="module")
def pool():
    return synth.pool_numpy(W.seed, W.L, W.E, W.H, W.I, W.fmt)


def make(pool, S, f):
    P, TS = pool
    return OracleEngine(W.L, W.E, W.K, W.H, W.I, W.fmt, S, f, lambda i: P[i], lambda i: TS[i])


def run_decode(eng, ntok, start=0):
    outs = []
    for t in range(start, start + ntok):
        for l in range(W.L):
            x = synth.activations(W.seed, l, t, 1, W.H)
            wr = synth.router_weights(W.seed, l, W.E, W.H)
            r = eng.decode_layer(l, x, router_bits=wr)
            eng.cache.check_bijection()
            outs.append(r["out_bits"].copy())
    return np.stack(outs)


def test_cache_size_invariance(pool):
    ref = run_decode(make(pool, W.L * W.E, 65536), 24)
    fetched_any, host_any = False, False
    for S in (0, 1, 2, 4, W.L * W.E):
        for f in W.f_sweep:
            eng = make(pool, S, f)
            got = run_decode(eng, 24)
            assert np.array_equal(got, ref), (S, f)
            fetched_any |= any(eng.cache.owner[v] >= 0 for v in range(S))
    assert fetched_any


def test_partition_mixes_sides(pool):
    eng = make(pool, 4, 32768)
    gpu = host = 0
    for t in range(32):
        for l in range(W.L):
            r = eng.decode_layer(l, synth.activations(W.seed, l, t, 1, W.H),
                                 router_bits=synth.router_weights(W.seed, l, W.E, W.H))
            gpu += sum(s >= 0 for s in r["slots"])
            host += sum(c >= 0 for c in r["cpu_ids"])
    assert gpu > 0 and host > 0


def test_negative_control_wrong_copy_fails(pool):
    P, TS = pool
    eng = make(pool, 4, 65536)
    orig = eng._copy

    def bad_copy(fetch):
        orig([(fl ^ 1, v) for fl, v in fetch])   # copy a neighbour's record
    eng._copy = bad_copy
    ref = run_decode(make(pool, 4, 65536), 4)
    assert not np.array_equal(run_decode(eng, 4), ref)


def test_prefill_equals_decodes_and_fallback(pool):
    T = 12
    S_big = 2 * W.E + 3
    outs_stream, outs_fallback, outs_decode = [], [], []
    eng_s = make(pool, S_big, 65536)
    eng_f = make(pool, W.S, 65536)          # S = 4 < 2E: on-demand fallback
    eng_d = make(pool, W.L * W.E, 65536)
    P, _ = pool
    for l in range(W.L):
        X = synth.activations(W.seed, l, 0, T, W.H, tag=synth.TAG_PREFILL_X)
        wr = synth.router_weights(W.seed, l, W.E, W.H)
        rs = eng_s.prefill_layer(l, X, wr)
        b = l % 2
        for e in range(W.E):    # streamed slot bytes are the host records
            assert np.array_equal(eng_s.arena[b * W.E + e], P[l * W.E + e])
        outs_stream.append(rs["out_bits"])
        outs_fallback.append(eng_f.prefill_layer(l, X, wr)["out_bits"])
        outs_decode.append(np.concatenate([eng_d.decode_layer(l, X[t:t + 1], router_bits=wr)["out_bits"]
                                           for t in range(T)]))
    for a, b_, c in zip(outs_stream, outs_fallback, outs_decode):
        assert np.array_equal(a, b_)
        assert np.array_equal(a, c)


def test_prefill_token_subset(pool):
    eng = make(pool, 2 * W.E, 65536)
    X = synth.activations(W.seed, 0, 0, 10, W.H, tag=synth.TAG_PREFILL_X)
    wr = synth.router_weights(W.seed, 0, W.E, W.H)
    full = eng.prefill_layer(0, X, wr)["out_bits"]
    eng2 = make(pool, 2 * W.E, 65536)
    sub = eng2.prefill_layer(0, X, wr, tokens=[2, 7])["out_bits"]
    assert np.array_equal(sub, full[[2, 7]])
