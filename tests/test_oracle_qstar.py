"""Pins of the oracle's q* rule ([FT-deep] §4 design pattern ②; [FT-blog] §六).

The rule is checked against its plain definition (brute force over every F),
the closed form q* ~ m * B_P / B_H, and invariants that follow from the cost
being the max of a non-decreasing and a non-increasing function of F."""
import os
import random

import numpy as np
import pytest

from oracle.qstar import Q16, qstar_bruteforce, qstar_rule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qstar_table.txt")


def brute_all_f(m: int) -> np.ndarray:
    """Vectorised brute force over all 65537 f for one m (lowest minimiser)."""
    F = np.arange(m + 1, dtype=np.int64)[:, None]
    f = np.arange(Q16 + 1, dtype=np.int64)[None, :]
    cost = np.maximum(F * (Q16 - f), (m - F) * f)
    return np.argmin(cost, axis=0)


@pytest.mark.parametrize("m", list(range(0, 21)))
def test_rule_equals_bruteforce_every_f(m):
    ref = brute_all_f(m)
    got = np.array([qstar_rule(m, f) for f in range(Q16 + 1)])
    assert np.array_equal(got, ref)


def test_rule_equals_bruteforce_random_large_m():
    rng = random.Random(7)
    for _ in range(3000):
        m = rng.randint(0, 4096)
        f = rng.randint(0, Q16)
        assert qstar_rule(m, f) == qstar_bruteforce(m, f)


def test_closed_form_within_one():
    rng = random.Random(11)
    for _ in range(20000):
        m = rng.randint(0, 5000)
        f = rng.randint(1, Q16 - 1)
        assert abs(qstar_rule(m, f) - m * f / Q16) < 1.0


def test_bounds_and_monotone():
    for m in range(0, 60):
        prev = -1
        for f in range(0, Q16 + 1, 97):
            q = qstar_rule(m, f)
            assert 0 <= q <= m
            assert q >= prev
            prev = q
    for f in (1, 16384, 26214, 32768, 45875, 65535):
        qs = [qstar_rule(m, f) for m in range(300)]
        assert all(b >= a for a, b in zip(qs, qs[1:]))


def test_symmetry_ties_to_lower():
    # q*(m, f) + q*(m, 65536 - f) is m, or m - 1 exactly when the balance point is a tie
    fs = sorted(set(range(0, Q16 + 1, 61)) | set(range(0, Q16 + 1, 2048)))
    ties = 0
    for m in range(0, 40):
        for f in fs:
            a, b = qstar_rule(m, f), qstar_rule(m, Q16 - f)
            # costs of floor and ceil of the balance point are equal iff (m + 1) * f = (floor + 1) * 65536
            tie = 0 < f < Q16 and ((m + 1) * f) % Q16 == 0
            assert a + b == (m - 1 if tie else m), (m, f, a, b)
            ties += tie
    assert ties > 50


def test_worked_ties():
    assert qstar_rule(1, 32768) == 0
    assert qstar_rule(3, 32768) == 1
    assert qstar_rule(3, 16384) == 0
    assert qstar_rule(3, 49152) == 2
    for m in range(1, 200, 2):
        assert qstar_rule(m, 32768) == (m - 1) // 2


def test_endpoints():
    for m in range(0, 500):
        assert qstar_rule(m, 0) == 0
        assert qstar_rule(m, Q16) == m
        if m <= 65534:
            assert qstar_rule(m, 65535) == m


def test_golden_table():
    rows = [ln.split() for ln in open(GOLDEN) if not ln.startswith("#")]
    fs = [int(x) for x in open(GOLDEN).read().splitlines()[1].split()[2:]]
    for row in rows:
        m = int(row[0])
        for f, q in zip(fs, row[1:]):
            assert qstar_rule(m, f) == int(q)


def test_negative_control_wrong_tie_break_fails():
    """A rule that breaks ties upward must disagree with the definition somewhere."""
    def upward(m, f):
        lo = (m * f) >> 16
        c = lambda F: max(F * (Q16 - f), (m - F) * f)
        return min(m, lo if c(lo) < c(lo + 1) else lo + 1)
    assert any(upward(m, 32768) != qstar_bruteforce(m, 32768) for m in range(1, 10))


def test_invalid_inputs():
    with pytest.raises(ValueError):
        qstar_rule(3, Q16 + 1)
    with pytest.raises(ValueError):
        qstar_rule(-1, 5)


# f from measured rates ([FT-deep] §4 design pattern ②: B_P / B_H times 65536, an integer)
def test_frac_q16_matches_the_configs_values():
    from oracle.qstar import frac_q16
    # the 35b-a3b and dsv4 decode configs quote f = 0.4 and 0.7 as 26214 and 45875
    assert frac_q16(0.4, 1.0) == 26214 and frac_q16(0.7, 1.0) == 45875
    assert frac_q16(4e9, 10e9) == 26214 and frac_q16(7.0, 10.0) == 45875


def test_frac_q16_ends_and_edges():
    from oracle.qstar import frac_q16
    assert frac_q16(1.0, 1.0) == 65536          # link as fast as host memory: fetch every miss
    assert frac_q16(3.0, 1.0) == 65536          # faster link: capped
    assert frac_q16(0.0, 5.0) == 0              # no link: everything on the host
    assert frac_q16(5.0, 0.0) == 65536          # no host bandwidth: everything fetched
    assert frac_q16(1.0, 65536.0) == 1 and frac_q16(1.0, 65537.0) == 0   # the integer part, not rounding
    assert frac_q16(65535.0, 65536.0) == 65535
    for bad in ((-1.0, 1.0), (1.0, -1.0), (float("nan"), 1.0)):
        with pytest.raises(ValueError):
            frac_q16(*bad)


def test_frac_q16_monotone_and_consistent_with_qstar():
    import random
    from oracle.qstar import frac_q16, qstar_rule
    rnd = random.Random(7)
    for _ in range(2000):
        bh = rnd.uniform(1e9, 500e9)
        bp, bp2 = sorted(rnd.uniform(0, 1.2 * bh) for _ in range(2))
        f, f2 = frac_q16(bp, bh), frac_q16(bp2, bh)
        assert 0 <= f <= f2 <= 65536                   # more link bandwidth never fetches less
        r = min(1.0, bp / bh)
        assert abs(f - 65536 * r) < 1.0 + 1e-9          # within one unit of the exact ratio
        for m in (1, 7, 16, 160):
            assert abs(qstar_rule(m, f) - m * r) <= 1.0 + m / 65536   # q* ~ m B_P / B_H ([FT-blog] §六)
