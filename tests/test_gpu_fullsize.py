"""GPU parity at the full sizes of the timed workloads, in the launch configuration the bench times.

Decode, 35b-a3b (40 layers x 256 int4 experts in pinned host memory, 5120 slots, f = 0.4, B = 1):
32 tokens x 40 layers of eff_decode_layer with trace logits, issued back to back (no host
synchronization between calls: asynchronous host share, in-kernel fetches), then
  * the final table, owner, usage, recency and clock, bit for bit, against the oracle policy
    replayed over the same routing (plain LRU code, every call in order);
  * the per-call hit / fetch / host totals against the replay;
  * sampled outputs (layers and tokens spread over the run, the first and the last call included)
    against the oracle's routed MoE of the dequantized records (fp64), rel-L2 <= 5e-3 and
    max-abs <= 2e-2.  The output does not depend on the cache, so the pool record is the reference.
Decode, qwen3.8-flash-next (48 layers x 512 NVFP4 experts of 2560 x 640 in pinned host memory,
top-10, 2457 slots, f = 65535, B = 16, speculative next-layer requests keeping 65 % of the true
top-10): 4 steps x 48 layers issued back to back, 160 entries per call (the control kernel's
paths for more than 64 entries, the 8-token decode kernels with two token chunks per unit); the
final tables and the hit / fetch / host / speculative totals bit for bit against the oracle policy,
and sampled outputs against the oracle.
Decode, dsv4-flash (256 NVFP4 experts of 4096 x 2048 per layer, top-6, 2201 slots, f = 45875,
Zipf(1.0), B = 4): the whole 43-layer pool (155.8 GB) cannot be pinned on a machine whose pinned
allocations stop near 70 GB, so 16 of its layers are (58 GB, past 32-bit record offsets); 3 steps x
16 layers issued back to back; only the records the routing trace reaches are generated (the
generator keys each record by its flat id, so they are the full pool's), the rest is allocated but
never read.  Final tables and totals against the oracle policy, sampled outputs against the oracle.
Prefill, dsv4-flash (256 NVFP4 experts of 4096 x 2048, top-6, 2201 slots, T = 2048 tokens): two
layers streamed into the double buffer and the grouped GEMMs, 64 sampled tokens per layer against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from oracle import cffn  # noqa: E402
from oracle.ffn import combine, x_f64  # noqa: E402
from oracle.formats import f64_to_bf16_bits  # noqa: E402
from oracle.policy import SlotCache  # noqa: E402
from oracle.router import topk_softmax  # noqa: E402
from synth.configs import A3B, DSV4_DECODE, DSV4_PREFILL, QWEN_NEXT  # noqa: E402
from tests.helpers import PinnedPool, assert_close_bf16  # noqa: E402
from tests.test_gpu_prefill import run_prefill  # noqa: E402

TOKENS = 32


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    assert torch.cuda.is_available()
    return e


def test_decode_35b_a3b_full_size(eff):
    W = A3B
    L, E, K, H, I = W.L, W.E, W.K, W.H, W.I
    print("full-size decode %s: L=%d E=%d K=%d H=%d I=%d S=%d f=%d tokens=%d" % (
        W.name, L, E, K, H, I, W.S, W.f_q16, TOKENS), flush=True)
    pool = PinnedPool(eff, W.seed, L, E, H, I, W.fmt)
    eng = None
    try:
        cfg = eff.make_config(L, E, K, H, I, W.fmt, W.S, 1, 0, W.f_q16, 12)
        eng = eff.Engine(cfg, pool.ptr, None)
        X = [synth.activations(W.seed, l, 0, TOKENS, H) for l in range(L)]
        LG = [synth.trace_logits(W.seed, l, E, W.zipf_s, 0, TOKENS) for l in range(L)]
        Xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in X]
        LGd = [torch.from_numpy(lg).cuda() for lg in LG]
        OUT = torch.empty((TOKENS, L, H), dtype=torch.int16, device="cuda")
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        for t in range(TOKENS):
            for l in range(L):
                eng.decode_layer(l, Xd[l][t:t + 1], OUT[t, l:l + 1], logits=LGd[l][t:t + 1], side=side)
        torch.cuda.synchronize()
        st = eng.stats()
        snap = eng.snapshot_tables()
        out = OUT.cpu().numpy().view(np.uint16)

        # the oracle policy over the same calls, in the same order
        cache = SlotCache(L, E, W.S, W.f_q16)
        hits = fetched = host = 0
        for t in range(TOKENS):
            for l in range(L):
                ids, _ = topk_softmax(LG[l][t:t + 1], K)
                cache.ensure(l, [int(e) for e in ids.reshape(-1)])
                res = cache.split()
                hits += len(set(int(e) for e in ids.reshape(-1))) - res.m
                fetched += res.q
                host += res.host
        assert list(snap["table"]) == cache.table
        assert list(snap["owner"]) == cache.owner
        assert list(snap["usage"]) == cache.usage
        assert list(snap["recency"]) == cache.recency
        assert (st["hits"], st["fetched"], st["host"]) == (hits, fetched, host)
        assert fetched > 0 and host > 0 and hits > 0   # every branch of the split was taken

        # sampled outputs: the routed MoE of the dequantized records, in fp64
        samples = [(0, 0), (TOKENS - 1, L - 1)] + [((7 * i) % TOKENS, (13 * i + 5) % L) for i in range(10)]
        for t, l in samples:
            ids, w = topk_softmax(LG[l][t:t + 1], K)
            x = x_f64(X[l][t:t + 1])
            jobs = [(pool.record(l * E + int(e)), pool.tensor_scales(l * E + int(e)), x) for e in ids[0]]
            ys = cffn.expert_ffn_batch(jobs, W.fmt, H, I, 16)
            y = np.stack([yk[0] for yk in ys])[None]          # [1, K, H]
            ref = f64_to_bf16_bits(combine(y, w))
            assert_close_bf16(out[t, l:l + 1], ref, what="token %d layer %d" % (t, l))
    finally:
        if eng is not None:
            eng.close()
        pool.free()


def test_decode_qwen_next_full_size_batch16(eff):
    W, B, steps = QWEN_NEXT, 16, 4
    L, E, K, H, I = W.L, W.E, W.K, W.H, W.I
    print("full-size decode %s: L=%d E=%d K=%d H=%d I=%d S=%d f=%d B=%d steps=%d spec=%.2f" % (
        W.name, L, E, K, H, I, W.S, W.f_q16, B, steps, W.spec_keep), flush=True)
    pool = PinnedPool(eff, W.seed, L, E, H, I, W.fmt)
    eng = None
    try:
        cfg = eff.make_config(L, E, K, H, I, W.fmt, W.S, B, 0, W.f_q16, 12)
        eng = eff.Engine(cfg, pool.ptr, pool.ts)
        n_rows = steps * B
        X = [synth.activations(W.seed, l, 0, n_rows, H) for l in range(L)]
        LG = [synth.trace_logits(W.seed, l, E, W.zipf_s, 0, n_rows) for l in range(L)]
        SP = []  # SP[l]: the speculative ids for layer l + 1 issued with layer l's call
        for l in range(L - 1):
            truth = synth.gumbel_topk_sets(LG[l + 1], K)
            SP.append(np.stack([synth.spec_ids(W.seed, l + 1, E, W.zipf_s, r, truth[r], W.spec_keep)
                                for r in range(n_rows)]).astype(np.int32))
        Xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in X]
        LGd = [torch.from_numpy(lg).cuda() for lg in LG]
        SPd = [torch.from_numpy(sp.reshape(-1)).cuda() for sp in SP]
        OUT = torch.empty((steps, L, B, H), dtype=torch.int16, device="cuda")
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        for t in range(steps):
            rows = slice(t * B, (t + 1) * B)
            for l in range(L):
                spec = SPd[l][t * B * K:(t + 1) * B * K] if l + 1 < L else None
                eng.decode_layer(l, Xd[l][rows], OUT[t, l], logits=LGd[l][rows], spec_ids=spec, side=side)
        torch.cuda.synchronize()
        st = eng.stats()
        snap = eng.snapshot_tables()
        out = OUT.cpu().numpy().view(np.uint16)

        # the oracle policy over the same calls, in the same order (real, then the speculative one)
        cache = SlotCache(L, E, W.S, W.f_q16)
        hits = fetched = host = spec_fetched = 0
        for t in range(steps):
            rows = slice(t * B, (t + 1) * B)
            for l in range(L):
                ids, _ = topk_softmax(LG[l][rows], K)
                flat = [int(e) for e in ids.reshape(-1)]
                cache.ensure(l, flat)
                res = cache.split()
                hits += len(set(flat)) - res.m
                fetched += res.q
                host += res.host
                if l + 1 < L:
                    cache.ensure(l + 1, [int(e) for e in SP[l][rows].reshape(-1)], speculative=True)
                    spec_fetched += cache.split().q
        assert list(snap["table"]) == cache.table
        assert list(snap["owner"]) == cache.owner
        assert list(snap["usage"]) == cache.usage
        assert list(snap["recency"]) == cache.recency
        assert (snap["step"], snap["last_real"]) == (cache.step, cache.last_real)
        assert (st["hits"], st["fetched"], st["host"], st["spec_fetched"]) == (hits, fetched, host, spec_fetched)
        assert fetched > 0 and spec_fetched > 0 and hits > 0

        # sampled outputs (tokens 0, 5, 10, 15 of a few calls): the routed MoE of the pool records, fp64
        for t, l in [(0, 0), (steps - 1, L - 1), (1, 17), (2, 30)]:
            rows = slice(t * B, (t + 1) * B)
            ids, w = topk_softmax(LG[l][rows], K)
            for b in (0, 5, 10, 15):
                x = x_f64(X[l][t * B + b:t * B + b + 1])
                jobs = [(pool.record(l * E + int(e)), pool.tensor_scales(l * E + int(e)), x) for e in ids[b]]
                ys = cffn.expert_ffn_batch(jobs, W.fmt, H, I, 16)
                y = np.stack([yk[0] for yk in ys])[None]
                ref = f64_to_bf16_bits(combine(y, w[b:b + 1]))
                assert_close_bf16(out[t, l, b:b + 1], ref, what="step %d layer %d token %d" % (t, l, b))
    finally:
        if eng is not None:
            eng.close()
        pool.free()


def test_decode_dsv4_full_size_batch4(eff):
    W, B, steps = DSV4_DECODE, 4, 3
    L, E, K, H, I = 16, W.E, W.K, W.H, W.I   # 16 of the 43 layers: the pinned pool must fit
    print("full-size decode %s: L=%d E=%d K=%d H=%d I=%d S=%d f=%d B=%d steps=%d" % (
        W.name, L, E, K, H, I, W.S, W.f_q16, B, steps), flush=True)
    n_rows = steps * B
    LG = [synth.trace_logits(W.seed, l, E, W.zipf_s, 0, n_rows) for l in range(L)]
    IDS = [topk_softmax(lg, K) for lg in LG]
    touched = {l * E + int(e) for l in range(L) for e in IDS[l][0].reshape(-1)}
    pool = PinnedPool(eff, W.seed, L, E, H, I, W.fmt, flats=touched)
    eng = None
    try:
        cfg = eff.make_config(L, E, K, H, I, W.fmt, W.S, B, 0, W.f_q16, 12)
        eng = eff.Engine(cfg, pool.ptr, pool.ts)
        X = [synth.activations(W.seed, l, 0, n_rows, H) for l in range(L)]
        Xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in X]
        LGd = [torch.from_numpy(lg).cuda() for lg in LG]
        OUT = torch.empty((steps, L, B, H), dtype=torch.int16, device="cuda")
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        for t in range(steps):
            rows = slice(t * B, (t + 1) * B)
            for l in range(L):
                eng.decode_layer(l, Xd[l][rows], OUT[t, l], logits=LGd[l][rows], side=side)
        torch.cuda.synchronize()
        st = eng.stats()
        snap = eng.snapshot_tables()
        out = OUT.cpu().numpy().view(np.uint16)

        cache = SlotCache(L, E, W.S, W.f_q16)
        hits = fetched = host = 0
        for t in range(steps):
            rows = slice(t * B, (t + 1) * B)
            for l in range(L):
                flat = [int(e) for e in IDS[l][0][rows].reshape(-1)]
                cache.ensure(l, flat)
                res = cache.split()
                hits += len(set(flat)) - res.m
                fetched += res.q
                host += res.host
        assert list(snap["table"]) == cache.table
        assert list(snap["owner"]) == cache.owner
        assert list(snap["usage"]) == cache.usage
        assert list(snap["recency"]) == cache.recency
        assert (snap["step"], snap["last_real"]) == (cache.step, cache.last_real)
        assert (st["hits"], st["fetched"], st["host"]) == (hits, fetched, host)
        assert fetched > 0 and host > 0 and hits > 0

        for t, l in [(0, 0), (steps - 1, L - 1), (1, 9)]:
            rows = slice(t * B, (t + 1) * B)
            ids, w = IDS[l][0][rows], IDS[l][1][rows]
            for b in (0, 3):
                x = x_f64(X[l][t * B + b:t * B + b + 1])
                jobs = [(pool.record(l * E + int(e)), pool.tensor_scales(l * E + int(e)), x) for e in ids[b]]
                ys = cffn.expert_ffn_batch(jobs, W.fmt, H, I, 16)
                y = np.stack([yk[0] for yk in ys])[None]
                ref = f64_to_bf16_bits(combine(y, w[b:b + 1]))
                assert_close_bf16(out[t, l, b:b + 1], ref, what="step %d layer %d token %d" % (t, l, b))
    finally:
        if eng is not None:
            eng.close()
        pool.free()


def test_prefill_dsv4_full_size(eff):
    W = DSV4_PREFILL
    T = W.prefill_T
    print("full-size prefill %s: E=%d K=%d H=%d I=%d S=%d T=%d, 2 layers" % (W.name, W.E, W.K, W.H, W.I, W.S, T),
          flush=True)
    pool = PinnedPool(eff, W.seed, 2, W.E, W.H, W.I, W.fmt)
    try:
        # 64 sampled tokens per layer: the ends, tile edges, and a stride over the chunk
        fixed = [0, 1, 63, 64, 511, 1024, 1500, 2046, T - 1]
        toks = sorted(fixed + [t for t in range(5, T, 37) if t not in fixed][:64 - len(fixed)])
        assert len(toks) == 64
        run_prefill(eff, pool, W.K, W.S, T, [0, 1], W.seed, tokens_checked=toks)
    finally:
        pool.free()
