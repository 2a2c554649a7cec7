"""Pins of the oracle router: the fixed-order fp32 logits stay within the fp32
error bound of the exact sum; top-k is the brute-force ordering (logit desc,
id asc); ties go to the lower id; the selection is permutation-equivariant;
softmax weights have their closed form."""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle.router import lane_width, logits_fixed_order, topk_softmax


@pytest.mark.parametrize("H", [64, 128, 256, 512, 2560])
def test_logits_within_fp32_bound(H):
    E, B = 24, 3
    x = synth.activations(5, 0, 0, B, H)
    w = synth.normal_bf16(5, synth.TAG_ROUTER, 0, 0, E * H, 1 / math.sqrt(H)).reshape(E, H)
    lg = logits_fixed_order(x, w)
    xf, wf = F.bf16_bits_to_f64(x), F.bf16_bits_to_f64(w)
    eps = 2.0 ** -24
    for b in range(B):
        for e in range(E):
            prods = [float(a) * float(c) for a, c in zip(xf[b], wf[e])]
            exact = math.fsum(prods)
            bound = (H + 6) * eps * math.fsum(abs(p) for p in prods)
            assert abs(float(lg[b, e]) - exact) <= bound


def test_lane_width():
    assert lane_width(64) == 1 and lane_width(128) == 2 and lane_width(256) == 4
    assert lane_width(512) == 8 and lane_width(2048) == 8 and lane_width(2560) == 8 and lane_width(192) == 1


def test_order_is_the_documented_one():
    """H = 64: one product per lane, so the result is exactly the pairwise fold of lanes
    (l, l+32), then (l, l+16), ... ; construct values where another order gives another answer."""
    H = 64
    p = np.zeros(H, np.float32)
    p[0], p[32], p[16], p[48] = 1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24
    # fold: s0 = 1 + 2^-24 -> 1 (tie to even); s16 = 2^-23; then 1 + 2^-23 (exact)
    x = F.f64_to_bf16_bits(np.where(p != 0, 1.0, 0.0))[None, :]
    w = F.f64_to_bf16_bits(p.astype(np.float64))[None, :]
    assert float(logits_fixed_order(x, w)[0, 0]) == 1.0 + 2.0 ** -23
    # a left-to-right sum would give 1.0: (1 + 2^-24) + 2^-24 + 2^-24 with each step rounding back to 1
    seq = np.float32(0)
    for v in p:
        seq = np.float32(seq + v)
    assert float(seq) == 1.0


def brute_topk(row, K):
    best = None
    for comb in itertools.combinations(range(len(row)), K):
        key = (sum(row[list(comb)]), [-c for c in comb])
        if best is None or key > best[0]:
            best = (key, comb)
    return sorted(best[1], key=lambda e: (-row[e], e))


def test_topk_bruteforce_small():
    rng = np.random.default_rng(0)
    for _ in range(50):
        E, K = 7, 3
        row = rng.standard_normal(E).astype(np.float32)
        ids, w = topk_softmax(row[None], K)
        assert list(ids[0]) == brute_topk(row.astype(np.float64), K)


def test_ties_go_to_lower_id():
    row = np.array([0.5, 1.0, 1.0, 0.2, 1.0], np.float32)
    ids, _ = topk_softmax(row[None], 2)
    assert list(ids[0]) == [1, 2]
    row = np.array([0.0, -0.0, 0.0], np.float32)
    ids, _ = topk_softmax(row[None], 2)
    assert list(ids[0]) == [0, 1]


def test_permutation_equivariance():
    rng = np.random.default_rng(1)
    row = rng.standard_normal(32).astype(np.float32)
    perm = rng.permutation(32)
    ids, w = topk_softmax(row[None], 5)
    ids2, w2 = topk_softmax(row[perm][None], 5)
    inv = np.argsort(perm)
    assert list(perm[ids2[0]]) == list(ids[0])
    assert np.allclose(w, w2)
    assert list(inv[ids[0]]) == list(ids2[0])


def test_softmax_closed_form():
    row = np.array([0.3, 2.0, -1.0, 1.25], np.float32)
    ids, w = topk_softmax(row[None], 2)
    assert list(ids[0]) == [1, 3]
    d = float(row[3]) - float(row[1])
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(d))) < 1e-15
    assert abs(w.sum() - 1.0) < 1e-15
    ids, w = topk_softmax(row[None], 1)
    assert w[0, 0] == 1.0
