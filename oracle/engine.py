"""One decode MoE layer and one prefill MoE layer, put together from the oracle parts.

Decode ([FT-deep] §4 design pattern ③): route -> ensure (slot or -1) -> split
(q*, victims, fetch list, host ids) -> copy the fetched records into their
slots -> GPU entries are evaluated from the *slot copy*, host entries from the
host pool -> top-k-weighted combine.  Evaluating GPU entries from the copied
bytes makes cache-size invariance a real check of the policy: a wrong slot or
a wrong copy changes the output.

Prefill ([FT-deep] §4 design pattern ①, [FT-blog] §五): the whole layer is
streamed into buffer layer % 2 (the first 2E slots), then every routed (token,
k) is evaluated from that buffer.  With S < 2E the oracle follows the on-demand
fallback: the routed experts of the layer, ascending, in groups of min(S, E),
each group copied into slots 0.. and then evaluated.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional

import numpy as np

from . import cffn
from .ffn import combine, expert_ffn, x_f64
from .formats import dequant_record, f64_to_bf16_bits
from .policy import SlotCache, check_partition
from .router import logits_fixed_order, topk_softmax


class OracleEngine:
    def __init__(self, L: int, E: int, K: int, H: int, I: int, fmt: int, S: int, f_q16: int,
                 get_record: Callable[[int], np.ndarray], get_ts: Callable[[int], np.ndarray],
                 use_c: Optional[bool] = None, nthreads: int = 8):
        self.L, self.E, self.K, self.H, self.I, self.fmt, self.S = L, E, K, H, I, fmt, S
        self.cache = SlotCache(L, E, S, f_q16)
        self.get_record, self.get_ts = get_record, get_ts
        self.arena: Dict[int, np.ndarray] = {}      # slot -> copied record bytes
        self.use_c = (H * I > 64 * 1024) if use_c is None else use_c
        self.nthreads = nthreads

    def rebuild(self, S_new: int) -> None:
        """Runtime cache rebuild ([FT-blog] §七 item 1): the slot contents go with the old cache."""
        self.cache.rebuild(S_new)
        self.S = S_new
        self.arena = {}

    # ------------------------------------------------------------------ helpers
    def _copy(self, fetch) -> None:
        for flat, v in fetch:
            self.arena[v] = np.array(self.get_record(flat), np.uint8, copy=True)

    def _evaluate(self, groups) -> List[np.ndarray]:
        """groups: list of (record bytes, ts3, x float64 [n, H]) -> list of y [n, H]."""
        if self.use_c:
            return cffn.expert_ffn_batch(groups, self.fmt, self.H, self.I, self.nthreads)
        out = []
        for rec, ts, x in groups:
            Wg, Wu, Wd = dequant_record(rec, self.fmt, self.H, self.I, ts)
            out.append(expert_ffn(Wg, Wu, Wd, x))
        return out

    # ------------------------------------------------------------------ decode
    def decode_layer(self, layer: int, x_bits: np.ndarray, logits: Optional[np.ndarray] = None,
                     router_bits: Optional[np.ndarray] = None,
                     spec_next: Optional[np.ndarray] = None) -> dict:
        E, K = self.E, self.K
        B = x_bits.shape[0]
        if logits is None:
            logits = logits_fixed_order(x_bits, router_bits)
        ids, w = topk_softmax(logits, K)
        flat_ids = [int(e) for e in ids.reshape(-1)]
        ensured = self.cache.ensure(layer, flat_ids)
        res = self.cache.split()
        check_partition(flat_ids, res.slots, res.cpu_ids)
        self._copy(res.fetch)
        spec = None
        if spec_next is not None and layer + 1 < self.L:
            self.cache.ensure(layer + 1, [int(e) for e in np.asarray(spec_next).reshape(-1)], speculative=True)
            spec = self.cache.split()
            self._copy(spec.fetch)
        x = x_f64(x_bits)
        # group entries: GPU by slot, host by expert id; each expert evaluated once for its tokens
        groups, members = {}, {}
        for p, e in enumerate(flat_ids):
            t = p // K
            key = ("gpu", res.slots[p]) if res.slots[p] >= 0 else ("host", e)
            members.setdefault(key, []).append(p)
            groups.setdefault(key, e)
        keys = sorted(members)
        jobs = []
        for key in keys:
            e = groups[key]
            rec = self.arena[key[1]] if key[0] == "gpu" else self.get_record(layer * E + e)
            toks = [p // K for p in members[key]]
            jobs.append((rec, self.get_ts(layer * E + e), x[toks]))
        ys = self._evaluate(jobs)
        y = np.zeros((B, K, self.H), np.float64)
        for key, yk in zip(keys, ys):
            for row, p in enumerate(members[key]):
                y[p // K, p % K] = yk[row]
        out = combine(y, w)
        return dict(ids=ids, w=w, logits=logits, ensured=ensured, slots=res.slots, cpu_ids=res.cpu_ids,
                    fetch=res.fetch, m=res.m, q=res.q, host=res.host, spec=spec, y=y, out=out,
                    out_bits=f64_to_bf16_bits(out))

    # ------------------------------------------------------------------ prefill
    def prefill_layer(self, layer: int, x_bits: np.ndarray, router_bits: np.ndarray,
                      tokens: Optional[List[int]] = None) -> dict:
        """Outputs for `tokens` (all by default) of one prefill chunk through one MoE layer."""
        E, K = self.E, self.K
        T = x_bits.shape[0]
        tokens = list(range(T)) if tokens is None else list(tokens)
        xs = x_bits[tokens]
        logits = logits_fixed_order(xs, router_bits)
        ids, w = topk_softmax(logits, K)
        x = x_f64(xs)
        y = np.zeros((len(tokens), K, self.H), np.float64)
        copies_all = []
        if self.S >= 2 * E:
            copies = self.cache.prefill_install(layer)
            self._copy(copies)
            copies_all += copies
            b = layer % 2
            batches = [list(range(E))]
            slot_of = lambda e, grp: b * E + e
        else:
            routed = sorted(set(int(e) for e in ids.reshape(-1)))
            G = min(self.S, E)
            batches = [routed[i:i + G] for i in range(0, len(routed), G)]
            slot_of = lambda e, grp: grp.index(e)
        for grp in batches:
            if self.S < 2 * E:
                copies = self.cache.prefill_fallback_group(layer, grp)
                self._copy(copies)
                copies_all += copies
            jobs, mem = [], []
            for e in grp:
                rows = [(i, k) for i in range(len(tokens)) for k in range(K) if ids[i, k] == e]
                if not rows:
                    continue
                v = slot_of(e, grp)
                jobs.append((self.arena[v], self.get_ts(layer * E + e), x[[i for i, _ in rows]]))
                mem.append(rows)
            for rows, yk in zip(mem, self._evaluate(jobs)):
                for r, (i, k) in enumerate(rows):
                    y[i, k] = yk[r]
        out = combine(y, w)
        return dict(ids=ids, w=w, logits=logits, y=y, out=out, out_bits=f64_to_bf16_bits(out),
                    copies=copies_all, tokens=tokens)
