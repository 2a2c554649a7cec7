"""Slot cache state machine, step by step, in plain integers.

What the pages fix:
* The GPU holds a cache of slots, one (layer, expert) record per slot, shared
  by all layers; the full expert pool stays in host memory as the source of
  truth ([FT-blog] §四; [FT-deep] §4 overview).
* Expert ids are one flat space layer * E + expert ([FT-deep] §4 design
  pattern ⑤; [FT-blog] §七 item 3).
* Slot LRU: int64 `usage` timestamps and a global step counter; the victim is
  argmin(usage).  A second LRU, `expert_recency`, decides which misses are
  fetched, q* decides how many ([FT-deep] §4 design pattern ⑤).
* One device kernel deduplicates, checks residency, computes q, picks victims
  (the K least recently used in one scan) and rewrites logical ids to a slot
  or to the host marker ([FT-blog] §六).
* ensure rewrites the routed ids in place to a slot or -1; the host branch
  gets the original id where the GPU does not own the entry and -1 elsewhere
  ([FT-deep] §4 design pattern ③).
* Prefill streams whole layers into two buffers picked by layer_id % 2, which
  are the first 2*E slots of the same cache; what is left there seeds decode;
  with fewer than 2*E slots the overlap is off and experts load on demand
  ([FT-deep] §4 design pattern ①; [FT-blog] §五).

Readings where the pages are silent (each listed in the design doc):
* step += 1 per ensure call (real or speculative) and per prefill install.
* m counts the *unique* missing experts of the call.
* Misses are ranked by (recency desc, expert id asc); victims are slots with
  usage below a floor, ordered by (usage asc, slot asc); empty slots have usage
  -1 and come first.  floor = this step for a real call (so this call's hits
  are never evicted); floor = the last real step for a speculative call (so
  the layer whose expert compute may still be running keeps its slots).
* q' = min(q*, number of victims); the i-th ranked miss takes the i-th victim.
* A speculative call fetches only (no host share) and leaves recency alone.
* Optional speculative budget ([NVMe-8GB] "엔진" item 3: guesses for the next
  layer are few, two of them there, and read in the gap left by the real reads):
  a speculative call fetches at most `spec_budget` records, the first of its
  ranked misses; None leaves q' as above.  Real calls ignore the budget.
* Optional link gap (the same passage: guesses use only the transfer time the
  real reads leave): with `spec_link` = G records the link can carry in one
  layer's time, a speculative call fetches at most max(0, G - q_real), q_real the
  q' of the latest real split (the layer's own fetches), again the first of its
  ranked misses.  Both caps may apply at once (the smaller wins).
* A runtime rebuild to S' slots ([FT-blog] §七 item 1: the GPU expert cache is
  repartitioned for a new budget at a safe point, without touching the host pool;
  since the pool is the source of truth, losing the cache only costs speed) starts
  from an empty cache of S' slots.  The step counter, last_real and the expert
  recency are statistics of the routing, not of the cache, and carry over.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

from .qstar import qstar_rule


@dataclass
class SplitResult:
    slots: List[int]                    # per entry: slot >= 0 (GPU computes) or -1
    cpu_ids: List[int]                  # per entry: expert id (host computes) or -1
    fetch: List[Tuple[int, int]]        # (flat id, slot) copies to issue, in order
    m: int
    q: int                              # q' actually fetched
    host: int                           # unique experts left to the host


@dataclass
class _Pending:
    layer: int
    ids: List[int]
    uniq: List[int]
    miss: List[int]
    s: int
    floor: int
    speculative: bool


class SlotCache:
    def __init__(self, L: int, E: int, S: int, f_q16: int, spec_budget: int | None = None,
                 spec_link: int | None = None):
        self.L, self.E, self.S, self.f = L, E, S, f_q16
        self.spec_budget = spec_budget
        self.spec_link = spec_link
        self.last_real_q = 0      # q' of the latest real split
        self.table = [-1] * (L * E)
        self.owner = [-1] * S
        self.usage = [-1] * S
        self.recency = [-1] * (L * E)
        self.step = 0
        self.last_real = 0
        self.pending: _Pending | None = None

    # ------------------------------------------------------------------ decode
    def ensure(self, layer: int, ids: List[int], speculative: bool = False) -> List[int]:
        """Steps 1-4: stamp hits, collect misses; returns slot-or--1 per entry."""
        E = self.E
        if any(not (0 <= e < E) for e in ids):
            raise ValueError("expert id out of range")
        self.step += 1
        s = self.step
        floor = self.last_real if speculative else s
        uniq = sorted(set(ids))
        for e in uniq:
            v = self.table[layer * E + e]
            if v >= 0:
                self.usage[v] = s
        miss = [e for e in uniq if self.table[layer * E + e] < 0]
        self.pending = _Pending(layer, list(ids), uniq, miss, s, floor, speculative)
        return [self.table[layer * E + e] for e in ids]

    def split(self) -> SplitResult:
        """Steps 5-10: q*, ranking, victims, installs, the -1 partition."""
        p = self.pending
        if p is None:
            raise RuntimeError("split without a pending ensure")
        self.pending = None
        E, l = self.E, p.layer
        m = len(p.miss)
        q = qstar_rule(m, self.f)
        ranked = sorted(p.miss, key=lambda e: (-self.recency[l * E + e], e))
        victims = sorted((v for v in range(self.S) if self.usage[v] < p.floor),
                         key=lambda v: (self.usage[v], v))
        qq = min(q, len(victims))
        if p.speculative and self.spec_budget is not None:
            qq = min(qq, self.spec_budget)
        if p.speculative and self.spec_link is not None:
            qq = min(qq, max(0, self.spec_link - self.last_real_q))
        fetch = []
        for i in range(qq):
            v, e = victims[i], ranked[i]
            if self.owner[v] >= 0:
                self.table[self.owner[v]] = -1
            self.owner[v] = l * E + e
            self.table[l * E + e] = v
            self.usage[v] = p.s
            fetch.append((l * E + e, v))
        slots = [self.table[l * E + e] for e in p.ids]
        if p.speculative:
            cpu_ids = [-1] * len(p.ids)
            host = 0
        else:
            cpu_ids = [e if sl < 0 else -1 for e, sl in zip(p.ids, slots)]
            host = m - qq
            for e in p.uniq:
                self.recency[l * E + e] = p.s
            self.last_real = p.s
            self.last_real_q = qq
        return SplitResult(slots, cpu_ids, fetch, m, qq, host)

    def ensure_split(self, layer: int, ids: List[int], speculative: bool = False) -> SplitResult:
        self.ensure(layer, ids, speculative)
        return self.split()

    # ------------------------------------------------------------------ prefill
    def _install(self, flat: int, v: int, s: int) -> bool:
        """Put flat id into slot v (evicting v's owner, freeing its old slot). True if bytes must move."""
        w = self.table[flat]
        if w == v:
            self.usage[v] = s
            return False
        if self.owner[v] >= 0:
            self.table[self.owner[v]] = -1
        if w >= 0:
            self.owner[w] = -1
            self.usage[w] = -1
        self.owner[v] = flat
        self.table[flat] = v
        self.usage[v] = s
        return True

    def prefill_install(self, layer: int) -> List[Tuple[int, int]]:
        """Whole layer into buffer layer % 2 (slots b*E .. b*E+E-1).  Needs S >= 2E."""
        E = self.E
        if self.S < 2 * E:
            raise ValueError("double buffering needs S >= 2E")
        self.step += 1
        s = self.step
        b = layer % 2
        copies = []
        for e in range(E):
            if self._install(layer * E + e, b * E + e, s):
                copies.append((layer * E + e, b * E + e))
        self.last_real = s
        return copies

    def prefill_fallback_group(self, layer: int, experts: List[int]) -> List[Tuple[int, int]]:
        """On-demand fallback: install up to min(S, E) experts into slots 0.. in the order given."""
        if len(experts) > min(self.S, self.E) or len(experts) == 0:
            raise ValueError("group size must be in [1, min(S, E)]")
        self.step += 1
        s = self.step
        copies = []
        for i, e in enumerate(experts):
            if self._install(layer * self.E + e, i, s):
                copies.append((layer * self.E + e, i))
        self.last_real = s
        return copies

    # ------------------------------------------------------------------ checks
    # ------------------------------------------------------------------ rebuild
    def rebuild(self, S_new: int) -> None:
        """The cache rebuilt with S_new slots: every slot empty, nothing resident; step,
        last_real and recency kept.  Only at a safe point: no ensure waiting for its split."""
        if S_new < 0:
            raise ValueError("S_new >= 0 required")
        if self.pending is not None:
            raise RuntimeError("rebuild with an ensure pending its split")
        self.S = S_new
        self.table = [-1] * (self.L * self.E)
        self.owner = [-1] * S_new
        self.usage = [-1] * S_new

    def check_bijection(self) -> None:
        for v, o in enumerate(self.owner):
            if o >= 0 and self.table[o] != v:
                raise AssertionError("owner/table mismatch at slot %d" % v)
        for flat, v in enumerate(self.table):
            if v >= 0 and self.owner[v] != flat:
                raise AssertionError("table/owner mismatch at flat id %d" % flat)


def check_partition(ids: List[int], slots: List[int], cpu_ids: List[int]) -> None:
    """Exactly-once: each entry is owned by exactly one side, consistently per unique expert."""
    side = {}
    for e, sl, c in zip(ids, slots, cpu_ids):
        gpu, host = sl >= 0, c >= 0
        if gpu == host:
            raise AssertionError("entry of expert %d owned by %s" % (e, "both" if gpu else "neither"))
        if host and c != e:
            raise AssertionError("host id %d != routed id %d" % (c, e))
        key = ("gpu", sl) if gpu else ("host", e)
        if side.setdefault(e, key) != key:
            raise AssertionError("expert %d split across sides/slots" % e)
