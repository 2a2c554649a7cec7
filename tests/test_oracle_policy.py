"""Pins of the oracle slot-cache policy.

* Textbook LRU: with f = 65536 (fetch every miss), one id per call and no
  speculation the policy is plain LRU over the flat-id stream; its miss
  sequence must equal an independent move-to-front list ([FT-deep] §4 ⑤ says
  the slot victim is argmin(usage), i.e. least recently used).
* S >= L*E: fetches = distinct ids seen; S = 0: every expert goes to the host.
* table/owner stay a bijection; hits are never evicted in their own call;
  |fetch| <= q*; the fetched misses are the q' most recent ones.
* exactly-once partition ([FT-deep] §4 ③) with a drop-an-expert negative control.
* speculative calls keep the in-flight layer's slots and leave recency alone.
* prefill install leaves the last two layers in the double buffer ([FT-blog] §五).
"""
import random
from collections import OrderedDict

import pytest

from oracle.policy import SlotCache, check_partition
from oracle.qstar import qstar_rule


def mtf_lru_misses(stream, S):
    lru = OrderedDict()
    misses = []
    for x in stream:
        if x in lru:
            lru.move_to_end(x)
            misses.append(False)
        else:
            misses.append(True)
            if S == 0:
                continue
            if len(lru) >= S:
                lru.popitem(last=False)
            lru[x] = True
    return misses


@pytest.mark.parametrize("S", [1, 2, 3, 5, 9])
def test_textbook_lru(S):
    rng = random.Random(S)
    L, E = 2, 8
    c = SlotCache(L, E, S, 65536)
    stream, got = [], []
    for _ in range(400):
        l, e = rng.randrange(L), rng.randrange(E)
        r = c.ensure_split(l, [e])
        stream.append(l * E + e)
        got.append(r.m == 1)
        assert r.q == r.m  # every miss fetched while victims exist
        c.check_bijection()
    assert got == mtf_lru_misses(stream, S)


def test_full_cache_fetches_distinct():
    rng = random.Random(1)
    L, E, K = 2, 8, 3
    c = SlotCache(L, E, L * E, 65536)
    seen, fetched = set(), 0
    for _ in range(200):
        l = rng.randrange(L)
        ids = rng.sample(range(E), K)
        r = c.ensure_split(l, ids)
        fetched += len(r.fetch)
        seen |= {l * E + e for e in ids}
        assert all(s >= 0 for s in r.slots)
    assert fetched == len(seen)


def test_zero_slots_all_host():
    c = SlotCache(2, 8, 0, 65536)
    r = c.ensure_split(1, [3, 5, 3])
    assert r.slots == [-1, -1, -1] and r.cpu_ids == [3, 5, 3] and r.fetch == [] and r.m == 2 and r.host == 2


def test_random_invariants():
    rng = random.Random(5)
    for trial in range(40):
        L, E, S = 3, 16, rng.randint(0, 20)
        f = rng.choice([0, 1, 16384, 26214, 32768, 45875, 65535, 65536])
        c = SlotCache(L, E, S, f)
        for step in range(60):
            l = rng.randrange(L)
            B, K = rng.randint(1, 3), rng.randint(1, 4)
            ids = [e for _ in range(B) for e in rng.sample(range(E), K)]
            rec_before = list(c.recency)
            hits_before = {e: c.table[l * E + e] for e in set(ids) if c.table[l * E + e] >= 0}
            r = c.ensure_split(l, ids)
            c.check_bijection()
            check_partition(ids, r.slots, r.cpu_ids)
            # hits keep their slot
            for e, v in hits_before.items():
                assert c.table[l * E + e] == v
            # m counts unique misses; q' <= q*(m, f)
            assert r.m == len(set(ids)) - len(hits_before)
            assert r.q <= qstar_rule(r.m, f) and r.q + r.host == r.m
            # the fetched misses are the q' highest-recency ones (ties: lower id)
            misses = sorted(set(ids) - set(hits_before), key=lambda e: (-rec_before[l * E + e], e))
            assert [fl - l * E for fl, _ in r.fetch] == misses[:r.q]
            # recency of every routed expert is now this step
            assert all(c.recency[l * E + e] == c.step for e in set(ids))


def test_negative_control_dropped_entry_fails():
    c = SlotCache(1, 8, 2, 32768)
    ids = [1, 2, 3, 4]
    r = c.ensure_split(0, ids)
    check_partition(ids, r.slots, r.cpu_ids)
    host = [p for p, v in enumerate(r.cpu_ids) if v >= 0]
    assert host
    bad = list(r.cpu_ids)
    bad[host[0]] = -1
    with pytest.raises(AssertionError):
        check_partition(ids, r.slots, bad)
    gpu = [p for p, v in enumerate(r.slots) if v >= 0]
    if gpu:
        both = list(r.cpu_ids)
        both[gpu[0]] = ids[gpu[0]]
        with pytest.raises(AssertionError):
            check_partition(ids, r.slots, both)


def test_speculative_keeps_inflight_layer_and_recency():
    L, E, S = 3, 8, 6
    c = SlotCache(L, E, S, 65536)
    r0 = c.ensure_split(0, [0, 1, 2, 3, 4, 5])   # fills all six slots
    used = set(r0.slots)
    rec = list(c.recency)
    spec = c.ensure_split(1, [0, 1, 2], speculative=True)
    assert spec.q == 0 and spec.fetch == []         # every slot belongs to the in-flight layer
    assert spec.cpu_ids == [-1, -1, -1]
    assert c.recency == rec
    r1 = c.ensure_split(1, [6])                      # a real call may evict layer 0's slots now
    assert r1.q == 1 and r1.fetch[0][1] in used


def test_speculative_then_real_hits():
    L, E, S = 2, 8, 8
    c = SlotCache(L, E, S, 65536)
    c.ensure_split(0, [0, 1])
    spec = c.ensure_split(1, [4, 5, 6], speculative=True)
    assert spec.q == 3
    r = c.ensure_split(1, [4, 7])
    assert r.m == 1 and r.slots[0] == spec.slots[0]


def test_speculative_budget_takes_the_ranked_prefix():
    """A speculative call under a budget fetches exactly the first `budget` (miss, victim) pairs of what the
    same call without one would, from the same state; hits are stamped alike, every entry maps to a slot
    holding its expert or to -1, and a real call from that state is unaffected by the budget."""
    import copy
    import random
    rng = random.Random(5)
    L, E, S = 3, 16, 10
    checked = 0
    for _ in range(300):
        base = SlotCache(L, E, S, 65535)
        for _ in range(rng.randint(0, 6)):   # a random history of real and speculative calls
            base.ensure_split(rng.randrange(L), rng.sample(range(E), rng.randint(1, 5)),
                              speculative=rng.random() < 0.3)
        layer, ids = rng.randrange(L), rng.sample(range(E), rng.randint(1, 8))
        ref_cache = copy.deepcopy(base)
        ref = ref_cache.ensure_split(layer, ids, speculative=True)
        for budget in (0, 1, 2, 5):
            c = copy.deepcopy(base)
            c.spec_budget = budget
            r = c.ensure_split(layer, ids, speculative=True)
            assert r.q == min(ref.q, budget) and r.m == ref.m
            assert r.fetch == ref.fetch[:budget]
            assert r.cpu_ids == [-1] * len(ids)
            for e, v in zip(ids, r.slots):
                assert v == -1 or c.owner[v] == layer * E + e
                if v >= 0:
                    assert c.usage[v] == c.step          # hit or installed: stamped with this call
            assert c.recency == base.recency             # speculation leaves recency alone
            c.check_bijection()
            real_a, real_b = copy.deepcopy(base), copy.deepcopy(base)
            real_b.spec_budget = budget
            assert real_a.ensure_split(layer, ids) == real_b.ensure_split(layer, ids)
            checked += ref.q > budget
    assert checked > 50   # the budget bound often


def test_speculative_gap_is_capacity_left_by_the_real_fetches():
    """With a link gap of G records per layer, a speculative call fetches exactly the first
    max(0, G - q) pairs the unbudgeted call would, q the fetch count of the latest real call of the
    history (tracked here from the returned results, not read from the cache); real calls are
    unaffected; with a budget too, the smaller cap wins."""
    import copy
    import random
    rng = random.Random(9)
    L, E, S = 3, 16, 10
    checked = 0
    for _ in range(300):
        base = SlotCache(L, E, S, 65535)
        q_real = 0
        for _ in range(rng.randint(0, 6)):
            spec = rng.random() < 0.3
            r = base.ensure_split(rng.randrange(L), rng.sample(range(E), rng.randint(1, 5)), speculative=spec)
            if not spec:
                q_real = r.q
        layer, ids = rng.randrange(L), rng.sample(range(E), rng.randint(1, 8))
        ref = copy.deepcopy(base).ensure_split(layer, ids, speculative=True)
        for G in (0, 1, 3, 6):
            for budget in (None, 1):
                c = copy.deepcopy(base)
                c.spec_link, c.spec_budget = G, budget
                r = c.ensure_split(layer, ids, speculative=True)
                cap = max(0, G - q_real) if budget is None else min(budget, max(0, G - q_real))
                assert r.q == min(ref.q, cap) and r.fetch == ref.fetch[:cap]
                checked += ref.q > cap
            real_a, real_b = copy.deepcopy(base), copy.deepcopy(base)
            real_b.spec_link = G
            assert real_a.ensure_split(layer, ids) == real_b.ensure_split(layer, ids)
    assert checked > 100


def test_speculative_gap_follows_the_latest_real_call():
    """Worked case: the cap is G minus the fetches of the real call just before the speculative one."""
    L, E, S = 2, 8, 8
    c = SlotCache(L, E, S, 65536, spec_link=3)
    r = c.ensure_split(0, [0, 1])                  # two misses, both fetched
    assert r.q == 2
    spec = c.ensure_split(1, [4, 5, 6], speculative=True)
    assert spec.q == 1 and spec.m == 3             # 3 - 2 = 1 guess
    r = c.ensure_split(0, [0, 1])                  # both hit: nothing fetched
    assert r.q == 0
    spec = c.ensure_split(1, [4, 5, 6, 7], speculative=True)
    assert spec.q == 3                             # 3 - 0 = 3 guesses (4 was fetched before)


def test_speculative_budget_zero_only_protects_hits():
    L, E, S = 2, 8, 4
    c = SlotCache(L, E, S, 65536, spec_budget=0)
    c.ensure_split(0, [0, 1])
    c.ensure_split(1, [2])
    spec = c.ensure_split(0, [1, 5, 6], speculative=True)
    assert spec.q == 0 and spec.fetch == [] and spec.m == 2
    assert spec.slots[1:] == [-1, -1]
    assert c.usage[spec.slots[0]] == c.step            # the predicted resident is protected


def test_prefill_install_leaves_last_two_layers():
    L, E = 5, 8
    c = SlotCache(L, E, 2 * E + 3, 65536)
    c.ensure_split(0, [1, 2])                        # a decode fetch somewhere in the cache
    total = 0
    for l in range(L):
        copies = c.prefill_install(l)
        total += len(copies)
        b = l % 2
        assert all(c.table[l * E + e] == b * E + e for e in range(E))
        c.check_bijection()
    assert total == L * E
    for l in range(L):
        expect = l >= L - 2
        assert all((c.table[l * E + e] >= 0) == expect for e in range(E))
    with pytest.raises(ValueError):
        SlotCache(2, 8, 15, 65536).prefill_install(0)


def test_prefill_moves_expert_out_of_other_slot():
    L, E = 2, 4
    c = SlotCache(L, E, 2 * E + 2, 65536)
    r = c.ensure_split(1, [2])
    old = r.slots[0]
    c.prefill_install(1)
    assert c.table[1 * E + 2] == E + 2
    if old != E + 2:
        assert c.owner[old] == -1 and c.usage[old] == -1
    c.check_bijection()


# ---------------------------------------------------------------------- runtime rebuild
@pytest.mark.parametrize("S,S2", [(3, 5), (5, 2), (4, 0), (0, 3), (2, 9)])
def test_rebuild_then_textbook_lru(S, S2):
    """After a rebuild to S2 slots ([FT-blog] §七 item 1) the cache starts empty: with f = 65536 and
    one id per call the misses from there on are an independent move-to-front list of capacity S2
    started empty, whatever the cache held before."""
    rng = random.Random(10 * S + S2)
    L, E = 2, 8
    c = SlotCache(L, E, S, 65536)
    before = []
    for _ in range(150):
        l, e = rng.randrange(L), rng.randrange(E)
        c.ensure_split(l, [e])
        before.append(l * E + e)
    c.rebuild(S2)
    assert c.table == [-1] * (L * E) and c.owner == [-1] * S2 and c.usage == [-1] * S2
    stream, got = [], []
    for _ in range(300):
        l, e = rng.randrange(L), rng.randrange(E)
        r = c.ensure_split(l, [e])
        stream.append(l * E + e)
        got.append(r.m == 1)
        c.check_bijection()
        assert all(0 <= v < S2 for _, v in r.fetch)
    assert got == mtf_lru_misses(stream, S2)


def test_rebuild_keeps_clock_and_recency_and_refuses_a_pending_ensure():
    rng = random.Random(5)
    L, E, K = 2, 8, 3
    c = SlotCache(L, E, 6, 26214)
    for _ in range(40):
        c.ensure_split(rng.randrange(L), rng.sample(range(E), K))
    step, last, rec = c.step, c.last_real, list(c.recency)
    c.rebuild(4)
    assert (c.step, c.last_real, c.recency) == (step, last, rec)
    # the first call after the rebuild: every unique id misses, and the q* misses ranked by the
    # recency carried over are the ones fetched
    ids = [1, 4, 6]
    r = c.ensure_split(0, ids)
    assert r.m == 3 and r.q == qstar_rule(3, 26214)
    order = sorted(ids, key=lambda e: (-rec[e], e))
    assert [f for f, _ in r.fetch] == order[:r.q]
    c.ensure(1, [2])
    with pytest.raises(RuntimeError):
        c.rebuild(8)
    with pytest.raises(ValueError):
        SlotCache(L, E, 2, 65536).rebuild(-1)
