"""The bandwidth-matched split q* (how many of m misses to fetch).

[FT-blog] §六 derives it: fetching q experts of S bytes over the link takes
T_fill = q*S/B_P, computing the other m-q on the host with the bandwidth left
over takes T_cpu = (m-q)*S/(B_H - B_P); balancing the two gives q* ~ m*B_P/B_H.
[FT-deep] §4 design pattern ② states the same in Q16 fixed point: f = B_P/B_H
as an integer in [0, 65536]; the fetch time is proportional to F*(65536 - f) and
the host time to (m - F)*f; of the two integers around the balance point it
keeps the one whose slower branch is faster.

Definition used as the plain answer (the thing the method reaches exactly):
    q*(m, f) = argmin_{F in [0, m]} max(F*(65536 - f), (m - F)*f), ties to the lower F.
Readings (pages silent): f = 0 gives 0 (the page's code only enters its rule
for f > 0); f = 65536 means the link is as fast as host memory, so all misses
are fetched.
"""
from __future__ import annotations

Q16 = 1 << 16


def qstar_rule(m: int, f: int) -> int:
    """Two-candidate rule in the order [FT-deep] §4 ② describes: floor of the balance point,
    compare the max-cost of it and the next integer, keep the cheaper (lower on a tie), cap at m."""
    if not (0 <= f <= Q16) or m < 0:
        raise ValueError("m >= 0 and 0 <= f <= 65536 required")
    if f == 0:
        return 0
    lo = (m * f) >> 16

    def cost(F: int) -> int:
        return max(F * (Q16 - f), (m - F) * f)

    best = lo if cost(lo) <= cost(lo + 1) else lo + 1
    return min(m, best)


def qstar_bruteforce(m: int, f: int) -> int:
    """argmin over every F in [0, m] of max(F*(65536-f), (m-F)*f); the first (lowest) minimiser."""
    best_F, best_c = 0, None
    for F in range(m + 1):
        c = max(F * (Q16 - f), (m - F) * f)
        if best_c is None or c < best_c:
            best_F, best_c = F, c
    return best_F


def frac_q16(pcie_bytes_per_s: float, host_bytes_per_s: float) -> int:
    """f from the two measured rates, as [FT-deep] §4 design pattern ② defines it: B_P / B_H
    times 65536, an integer.  Readings (the pages give no rounding or range rule): the integer
    part (floor), which also turns the configs' 0.4 and 0.7 into their 26214 and 45875; capped
    at 65536, the value that fetches every miss, which is where B_P >= B_H leaves the method
    ([FT-blog] §六: q* -> m as B_H approaches B_P); a host rate of zero with a nonzero link rate
    also gives 65536, and no link (B_P = 0) gives 0.  Negative or NaN rates are rejected.
    Exact rational arithmetic on the two floats, so the floor is taken of the true quotient."""
    from fractions import Fraction
    import math
    bp, bh = pcie_bytes_per_s, host_bytes_per_s
    if math.isnan(bp) or math.isnan(bh) or bp < 0 or bh < 0:
        raise ValueError("rates must be non-negative numbers")
    if bp == 0:
        return 0
    if bh == 0 or math.isinf(bp):
        return Q16
    if math.isinf(bh):
        return 0
    return min(Q16, math.floor(Fraction(bp) * Q16 / Fraction(bh)))
