"""Pins of the oracle SwiGLU expert and combine.

* silu against its closed form at special points.
* one-hot probes: x = e_j makes the gate/up projections the j-th columns of the
  (generator's) weight matrices, with no summation -- pins row/column roles.
* the routed mixture equals the dense brute force over all experts with the
  non-selected ones weighted by zero (the textbook dense mixture).
* x = 0 gives 0; the C restatement agrees with the numpy one on both formats.
"""
import math

import numpy as np
import pytest

import synth
from oracle import cffn
from oracle import formats as F
from oracle.ffn import combine, expert_ffn, silu
from oracle.router import topk_softmax


def test_silu_points():
    assert silu(np.array(0.0)) == 0.0
    assert abs(silu(np.array(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(silu(np.array(40.0)) - 40.0) < 1e-12
    assert abs(silu(np.array(-40.0))) < 1e-15
    z = np.linspace(-5, 5, 11)
    assert np.allclose(silu(z), z * 1.0 / (1.0 + np.exp(-z)))


@pytest.mark.parametrize("fmt", [F.INT4, F.NVFP4])
def test_one_hot_probe(fmt):
    H, I, E = 64, 128, 8
    rec, ts = synth.record(17, E, 0, 5, H, I, fmt)
    Wg, Wu, Wd = F.dequant_record(rec, fmt, H, I, ts)
    wg_f = synth.weights_f32(17, E, 0, 5, 0, H, I).astype(np.float64)
    wu_f = synth.weights_f32(17, E, 0, 5, 1, H, I).astype(np.float64)
    for j in (0, 1, 7, 31, 32, 63):
        x = np.zeros((1, H))
        x[0, j] = 1.0
        g = x @ Wg.T
        assert np.array_equal(g[0], Wg[:, j])
        # and that column is the generator's column j within the quantization error
        assert np.linalg.norm(g[0] - wg_f[:, j]) / np.linalg.norm(wg_f[:, j]) < 0.25
        y = expert_ffn(Wg, Wu, Wd, x)
        a = silu(Wg[:, j]) * Wu[:, j]
        assert np.allclose(y[0], Wd @ a, rtol=0, atol=1e-15)
    assert np.linalg.norm(Wu[:, 3] - wu_f[:, 3]) / np.linalg.norm(wu_f[:, 3]) < 0.25


def test_zero_input_gives_zero():
    rec, ts = synth.record(1, 8, 0, 0, 64, 128, F.INT4)
    Wg, Wu, Wd = F.dequant_record(rec, F.INT4, 64, 128, ts)
    assert np.array_equal(expert_ffn(Wg, Wu, Wd, np.zeros((2, 64))), np.zeros((2, 64)))


def test_routed_equals_dense_mixture():
    E, K, H, I = 8, 3, 64, 128
    mats = []
    for e in range(E):
        rec, ts = synth.record(23, E, 0, e, H, I, F.INT4)
        mats.append(F.dequant_record(rec, F.INT4, H, I, ts))
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, H))
    logits = rng.standard_normal((5, E)).astype(np.float32)
    ids, w = topk_softmax(logits, K)
    y = np.zeros((5, K, H))
    for t in range(5):
        for k in range(K):
            y[t, k] = expert_ffn(*mats[ids[t, k]], x[t:t + 1])[0]
    routed = combine(y, w)
    dense = np.zeros((5, H))
    for t in range(5):
        gate = np.zeros(E)
        gate[ids[t]] = w[t]
        for e in range(E):
            dense[t] += gate[e] * expert_ffn(*mats[e], x[t:t + 1])[0]
    assert np.allclose(routed, dense, rtol=1e-13, atol=1e-15)


def test_negative_control_dropped_expert_fails():
    E, K, H, I = 8, 2, 64, 128
    rec, ts = synth.record(2, E, 0, 1, H, I, F.INT4)
    W = F.dequant_record(rec, F.INT4, H, I, ts)
    x = np.random.default_rng(2).standard_normal((1, H))
    y = expert_ffn(*W, x)
    full = combine(np.stack([y, y], axis=1), np.array([[0.6, 0.4]]))
    dropped = combine(np.stack([y, np.zeros_like(y)], axis=1), np.array([[0.6, 0.4]]))
    assert np.linalg.norm(full - dropped) / np.linalg.norm(full) > 0.3


@pytest.mark.parametrize("fmt", [F.INT4, F.NVFP4])
def test_c_oracle_matches_numpy(fmt):
    H, I = 128, 192
    jobs, refs = [], []
    rng = np.random.default_rng(9)
    for e in range(3):
        rec, ts = synth.record(31, 8, 1, e, H, I, fmt)
        x = rng.standard_normal((2, H))
        jobs.append((rec, ts, x))
        refs.append(expert_ffn(*F.dequant_record(rec, fmt, H, I, ts), x))
    outs = cffn.expert_ffn_batch(jobs, fmt, H, I, nthreads=2)
    for y, r in zip(outs, refs):
        assert np.allclose(y, r, rtol=1e-11, atol=1e-14)
