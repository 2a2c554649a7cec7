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


# Order-sensitive products for V > 1.  Each case lists (input index j, product x_j * w_j) with every
# other product zero; the expected fp32 logit is derived by hand from the documented order (lane l
# adds j = 64*V*c + V*l + i, blocks c outer, i inner, then the pairwise fold (l, l+o) for o = 32..1)
# and fp32 round-to-nearest-even.  The alternative orders a plausible mistake would use give the other
# value named in each comment.  All products are exact: x_j = 1 and w_j is a power of two or 1.
ORDER_CASES = [
    # H = 512: V = 8, one block.  Lane 0 adds j = 0..7 in turn: 2^25 + 1 rounds back to 2^25 (spacing 4),
    # then - 2^25 gives 0.  One input per lane (V = 1) would leave the 1 alone in lane 1: result 1.
    (512, [(0, 2.0 ** 25), (1, 1.0), (2, -2.0 ** 25)], 0.0),
    # H = 2048: V = 8, four blocks of 512.  c outer, i inner: lane 0 adds j = 0 (2^24), 1 (+1: the tie
    # rounds to even, 2^24), then j = 512 (-2^24): 0.  With i outer the cancellation comes first: 1.
    (2048, [(0, 2.0 ** 24), (1, 1.0), (512, -2.0 ** 24)], 0.0),
    # H = 2048: the lanes fold (l, l+32) first.  Lane 0 holds 2^25 (j = 0), lane 32 holds -2^25
    # (j = 256) and lane 1 holds 1 (j = 8): (2^25 - 2^25) + 1 = 1.  Folding (l, l+1) first gives
    # 2^25 + 1 = 2^25 and then 0; a left-to-right sum of the lanes also gives 0.
    (2048, [(0, 2.0 ** 25), (256, -2.0 ** 25), (8, 1.0)], 1.0),
    # H = 2560: V = 8 (2560 = 64 * 8 * 5).  Lane 0 adds j = 0 (2^24), 4 (+1, rounds to 2^24), 7 (-2^24):
    # 0.  With V = 4 the 1 would sit in lane 1 with -2^24 (exact -16777215): 2^24 - 16777215 = 1.
    (2560, [(0, 2.0 ** 24), (4, 1.0), (7, -2.0 ** 24)], 0.0),
    # H = 2560: the last of five blocks (j = 2048) comes after the whole first block: 0 as above; with
    # the blocks inner the 1 comes after the cancellation: 1.
    (2560, [(0, 2.0 ** 24), (1, 1.0), (2048, -2.0 ** 24)], 0.0),
    # H = 4096: V = 8, eight blocks; lanes 16 and 48 cancel at the first fold, lane 0's 1 survives:
    # lane 0 (j = 0) 1, lane 16 (j = 128) 2^25, lane 48 (j = 384) -2^25, lane 32 (j = 256) 2^-20.
    # Fold o=32: s0 = 1 + 2^-20, s16 = 0.  o=16: s0 += s16.  Result 1 + 2^-20 (exact).  Folding o=16
    # first adds 2^25 to 1 (lost), then 2^-20 is lost against 2^25 too: 0 after the cancellation.
    (4096, [(0, 1.0), (128, 2.0 ** 25), (384, -2.0 ** 25), (256, 2.0 ** -20)], 1.0 + 2.0 ** -20),
]


def order_case_inputs(H, prods):
    """bf16 bit arrays x [1, H] (ones) and w [1, H] (the products) for one order case."""
    w = np.zeros(H, np.float64)
    for j, v in prods:
        w[j] = v
    x = F.f64_to_bf16_bits(np.ones(H))[None, :]
    return x, F.f64_to_bf16_bits(w)[None, :]


@pytest.mark.parametrize("case", range(len(ORDER_CASES)))
def test_order_v_gt_1(case):
    """The documented order for V > 1 (blocks of V consecutive inputs per lane, blocks outer), against
    values derived by hand; each case fails under the nearest alternative order."""
    H, prods, want = ORDER_CASES[case]
    assert lane_width(H) == 8
    x, w = order_case_inputs(H, prods)
    assert float(logits_fixed_order(x, w)[0, 0]) == want


def _alt_order_sum(H, prods, V, blocks_outer=True, fold_down=True):
    """A deliberately different summation order (negative control): V inputs per lane block, blocks
    outer or inner, lanes folded from o = 32 down or from o = 1 up."""
    p = np.zeros(H, np.float32)
    for j, v in prods:
        p[j] = v
    R = H // (64 * V)
    acc = np.zeros(64, np.float32)
    order = [(c, i) for c in range(R) for i in range(V)] if blocks_outer else \
        [(c, i) for i in range(V) for c in range(R)]
    for c, i in order:
        acc = (acc + p[64 * V * c + V * np.arange(64) + i]).astype(np.float32)
    offs = [32, 16, 8, 4, 2, 1] if fold_down else [1, 2, 4, 8, 16, 32]
    for o in offs:
        if fold_down:
            acc[:o] = (acc[:o] + acc[o:2 * o]).astype(np.float32)
        else:   # pairs (2m, 2m+1) first: s[l] += s[l + o] for l a multiple of 2o
            idx = np.arange(0, 64, 2 * o)
            acc[idx] = (acc[idx] + acc[idx + o]).astype(np.float32)
    return float(acc[0])


def test_order_cases_fail_under_other_orders():
    """Negative control: each plausible wrong order (one input per lane, a smaller V, blocks inner,
    lanes folded from o = 1 up) misses the hand-derived value of at least one case, and the documented
    order, written this second way, meets all of them."""
    for H, prods, want in ORDER_CASES:
        assert _alt_order_sum(H, prods, 8) == want
    for kw in (dict(V=1), dict(V=4), dict(V=8, blocks_outer=False), dict(V=8, fold_down=False)):
        assert any(_alt_order_sum(H, prods, **kw) != want for H, prods, want in ORDER_CASES), kw


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
