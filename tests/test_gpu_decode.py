"""GPU parity of decode layers against the oracle.

Per call: routing ids, slots, host ids and counts bit for bit; expert outputs y
and the combined bf16 output within rel-L2 <= 5e-3 and max-abs <= 2e-2.  Covers
both weight formats, batch 1 and ragged batches (tokens per expert up to 16,
more than one token chunk), every f of the tiny sweep, all-host (S = 0) and
all-GPU partitions, speculative requests (with budget and link caps), and cache-size invariance on the GPU
(bit-identical outputs for every S >= B*K when f = 65536)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from synth.configs import TINY  # noqa: E402
from tests.helpers import MAX_ABS, PinnedPool, assert_close_bf16, make_engine, oracle_engine, rel_l2  # noqa: E402


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    assert torch.cuda.is_available()
    return e


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def run_decode(eff, pool, K, S, f, B, tokens, router=True, zipf=1.1, spec_keep=-1.0, seed=11,
               compare_y=True, flags=0, spec_budget=None, spec_gap=False, spec_link=None):
    """Decode `tokens` steps through all layers on the GPU (eff_decode_layer) and the oracle."""
    L, E, H = pool.L, pool.E, pool.H
    eng = make_engine(eff, pool, K, S, B, f, flags=flags)
    orc = oracle_engine(pool, K, S, f)
    set_spec(eng, orc, spec_budget, spec_gap, spec_link)
    side = torch.cuda.Stream()
    outs = []
    try:
        wrs = [synth.router_weights(seed, l, E, H) for l in range(L)]
        wrs_d = [dev_bf16(w) for w in wrs]
        for t in range(tokens):
            for l in range(L):
                x = synth.activations(seed, l, t * B, B, H)
                xd = dev_bf16(x)
                out = torch.empty((B, H), dtype=torch.int16, device="cuda")
                spec_ids = None
                spec_np = None
                if router:
                    lg = None
                else:
                    lg = synth.trace_logits(seed, l, E, zipf, t * B, B)
                if spec_keep >= 0 and l + 1 < L:
                    nxt = synth.trace_logits(seed, l + 1, E, zipf, t * B, B)
                    truth = synth.gumbel_topk_sets(nxt, K)
                    spec_np = np.stack([synth.spec_ids(seed, l + 1, E, zipf, t * B + b, truth[b], spec_keep)
                                        for b in range(B)])
                    spec_ids = torch.from_numpy(spec_np.reshape(-1)).cuda()
                eng.decode_layer(l, xd, out, w_router=wrs_d[l] if router else None,
                                 logits=None if router else torch.from_numpy(lg).cuda(), spec_ids=spec_ids,
                                 side=side)
                torch.cuda.synchronize()
                got = eng.last_layer_arrays(B)
                r = orc.decode_layer(l, x, logits=lg, router_bits=wrs[l] if router else None, spec_next=spec_np)
                assert np.array_equal(got["ids"], r["ids"].reshape(-1)), ("ids", t, l)
                assert list(got["slots"]) == r["slots"], ("slots", t, l)
                assert list(got["cpu"]) == r["cpu_ids"], ("cpu", t, l)
                assert list(got["counts"][:3]) == [r["m"], r["q"], r["host"]], ("counts", t, l)
                if r["spec"] is not None:
                    assert list(got["counts"][3:5]) == [r["spec"].m, r["spec"].q], ("spec counts", t, l)
                o = out.cpu().numpy().view(np.uint16)
                assert_close_bf16(o, r["out_bits"], what="out t=%d l=%d" % (t, l))
                outs.append(o.copy())
        snap = eng.snapshot_tables()
        assert list(snap["table"]) == orc.cache.table
        assert list(snap["usage"]) == orc.cache.usage
        return np.stack(outs), eng.stats()
    finally:
        eng.close()


@pytest.fixture(scope="module")
def tiny_pool(eff):
    p = PinnedPool(eff, TINY.seed, TINY.L, TINY.E, TINY.H, TINY.I, TINY.fmt)
    yield p
    p.free()


@pytest.mark.parametrize("f", list(TINY.f_sweep))
def test_tiny_decode_every_f(eff, tiny_pool, f):
    outs, st = run_decode(eff, tiny_pool, TINY.K, TINY.S, f, 1, 16, seed=TINY.seed)
    assert outs.shape[0] == 16 * TINY.L


@pytest.mark.parametrize("f", [0, 32768, 65536])
def test_tiny_decode_sync_host(eff, tiny_pool, f):
    """The host share on the calling thread (EFF_CFG_SYNC_HOST) gives the same results."""
    a, _ = run_decode(eff, tiny_pool, TINY.K, TINY.S, f, 1, 8, seed=TINY.seed)
    b, _ = run_decode(eff, tiny_pool, TINY.K, TINY.S, f, 1, 8, seed=TINY.seed, flags=eff.CFG_SYNC_HOST)
    assert np.array_equal(a, b)


def set_spec(eng, orc, spec_budget, spec_gap, spec_link):
    """The same speculative caps on the engine and the oracle policy (None: the defaults)."""
    if spec_budget is not None or spec_gap:
        eng.set_speculation(-1 if spec_budget is None else spec_budget, spec_gap)
        orc.cache.spec_budget = spec_budget
    if spec_link is not None:
        eng.set_speculation_link(spec_link)
        orc.cache.spec_link = spec_link


def run_ahead(eff, pool, K, S, f, B, tokens, zipf, seed, spec_keep=-1.0, flags=0, spec_budget=None,
              spec_gap=False, spec_link=None):
    """Every layer of every token enqueued before a single synchronize (the host runs ahead of
    the device; host shares and speculative copies are ordered on the device only); all outputs
    and the final tables against the oracle (with the same speculative caps, if any)."""
    L, E, H = pool.L, pool.E, pool.H
    eng = make_engine(eff, pool, K, S, B, f, flags=flags)
    orc = oracle_engine(pool, K, S, f)
    set_spec(eng, orc, spec_budget, spec_gap, spec_link)
    side = torch.cuda.Stream()
    try:
        xs, lgs, specs, outs = {}, {}, {}, {}
        for t in range(tokens):
            for l in range(L):
                xs[t, l] = synth.activations(seed, l, t * B, B, H)
                lgs[t, l] = synth.trace_logits(seed, l, E, zipf, t * B, B)
                specs[t, l] = None
                if spec_keep >= 0 and l + 1 < L:
                    nxt = synth.trace_logits(seed, l + 1, E, zipf, t * B, B)
                    truth = synth.gumbel_topk_sets(nxt, K)
                    specs[t, l] = np.stack([synth.spec_ids(seed, l + 1, E, zipf, t * B + b, truth[b], spec_keep)
                                            for b in range(B)])
        dev = {k: (dev_bf16(xs[k]), torch.from_numpy(lgs[k]).cuda(),
                   None if specs[k] is None else torch.from_numpy(specs[k].reshape(-1)).cuda()) for k in xs}
        torch.cuda.synchronize()
        for t in range(tokens):
            for l in range(L):
                xd, lg, sp = dev[t, l]
                outs[t, l] = torch.empty((B, H), dtype=torch.int16, device="cuda")
                eng.decode_layer(l, xd, outs[t, l], logits=lg, spec_ids=sp, side=side)
        torch.cuda.synchronize()
        tot = dict(fetched=0, host=0, spec_fetched=0)
        for t in range(tokens):
            for l in range(L):
                r = orc.decode_layer(l, xs[t, l], logits=lgs[t, l], spec_next=specs[t, l])
                assert_close_bf16(outs[t, l].cpu().numpy().view(np.uint16), r["out_bits"],
                                  what="run-ahead t=%d l=%d" % (t, l))
                tot["fetched"] += r["q"]
                tot["host"] += r["host"]
                tot["spec_fetched"] += r["spec"].q if r["spec"] is not None else 0
        snap = eng.snapshot_tables()
        assert list(snap["table"]) == orc.cache.table
        assert list(snap["owner"]) == orc.cache.owner
        assert list(snap["usage"]) == orc.cache.usage
        assert list(snap["recency"]) == orc.cache.recency
        st = eng.stats()
        assert {k: st[k] for k in tot} == tot
        return st
    finally:
        eng.close()


@pytest.mark.parametrize("B,budget,gap", [(8, 2, True), (8, 2, False), (16, 2, True), (16, None, True),
                                          (16, 3, False)])
def test_decode_run_ahead_speculative_budget_gap(eff, B, budget, gap):
    """Speculative requests with a budget, copied right after the control kernel or in the gap after
    the gate/up kernel, every layer enqueued without a host synchronization, so that a layer's
    speculative copy overlaps the next layer's control kernel: at the qwen3.8-flash-next expert shape
    (2560 x 640 NVFP4, top-10) with several records per request.  Every output and the final tables
    against the oracle policy with the same budget."""
    print("run-ahead speculative: B=%d budget=%s gap=%s" % (B, budget, gap), flush=True)
    pool = PinnedPool(eff, 31, 4, 64, 2560, 640, synth.FMT_NVFP4)
    try:
        st = run_ahead(eff, pool, 10, 3 * B * 10 // 2, 65535, B, 4, 1.2, 31, spec_keep=0.65, spec_budget=budget,
                       spec_gap=gap)
        assert st["spec_fetched"] > 0 and st["fetched"] > 0
    finally:
        pool.free()


@pytest.mark.parametrize("B,link,budget,gap", [(16, 24, None, False), (16, 12, 3, True), (8, 0, None, True),
                                               (8, 40, None, False)])
def test_decode_run_ahead_speculative_link_cap(eff, B, link, budget, gap):
    """The link cap on speculative fetches (the records one layer's link time carries, less the layer's
    own real fetches), alone and with a budget, copied in either place, every layer enqueued before one
    synchronize: outputs, counts and the final tables against the oracle policy with the same caps."""
    print("run-ahead speculative link cap: B=%d link=%d budget=%s gap=%s" % (B, link, budget, gap), flush=True)
    pool = PinnedPool(eff, 33, 4, 64, 2560, 640, synth.FMT_NVFP4)
    try:
        st = run_ahead(eff, pool, 10, 3 * B * 10 // 2, 65535, B, 4, 1.2, 33, spec_keep=0.65, spec_budget=budget,
                       spec_gap=gap, spec_link=link)
        assert st["fetched"] > 0
        if link == 0:
            assert st["spec_fetched"] == 0, st
    finally:
        pool.free()


def test_speculation_link_cap_limits_guesses(eff):
    """A link cap no smaller than any layer's real plus speculative fetches changes nothing; a small one
    fetches fewer guesses; the outputs are the same every time (the pool is the source of truth)."""
    pool = PinnedPool(eff, 22, 3, 32, 2560, 640, synth.FMT_NVFP4)
    try:
        kw = dict(router=False, zipf=1.2, spec_keep=0.65, seed=22)
        ref, st0 = run_decode(eff, pool, 10, 40, 65535, 2, 4, **kw)
        big, st1 = run_decode(eff, pool, 10, 40, 65535, 2, 4, spec_link=1000, **kw)
        small, st2 = run_decode(eff, pool, 10, 40, 65535, 2, 4, spec_link=6, **kw)
        assert np.array_equal(big, ref) and np.array_equal(small, ref)
        keys = ("calls", "hits", "fetched", "host", "spec_fetched", "bytes_fetched")
        assert {k: st1[k] for k in keys} == {k: st0[k] for k in keys}
        assert st2["spec_fetched"] < st0["spec_fetched"]
    finally:
        pool.free()


def test_set_speculation_link_rejects_bad_values(eff, tiny_pool):
    eng = make_engine(eff, tiny_pool, TINY.K, TINY.S, 1, 32768)
    try:
        assert eff.lib().eff_set_speculation_link(eng.h, -2) == eff.EFF_EINVAL
        assert eff.lib().eff_set_speculation_link(eng.h, -1) == 0
        eng.set_speculation_link(5)
    finally:
        eng.close()


@pytest.mark.parametrize("fmt,H,I,E,K,B,S,f,spec", [
    (synth.FMT_INT4, 2048, 512, 64, 8, 1, 96, 26214, -1.0),
    (synth.FMT_NVFP4, 2560, 640, 48, 10, 2, 60, 65535, 0.65),
    (synth.FMT_INT4, 256, 128, 16, 4, 3, 6, 16384, -1.0),
])
def test_decode_run_ahead(eff, fmt, H, I, E, K, B, S, f, spec):
    pool = PinnedPool(eff, 23, 4, E, H, I, fmt)
    try:
        st = run_ahead(eff, pool, K, S, f, B, 6, 1.1, 23, spec_keep=spec)
        assert st["fetched"] > 0
        if spec >= 0:
            assert st["spec_fetched"] > 0
        else:
            assert st["host"] > 0
    finally:
        pool.free()


def test_tiny_all_host_and_invariance(eff, tiny_pool):
    ref, _ = run_decode(eff, tiny_pool, TINY.K, 16, 65536, 1, 12, seed=TINY.seed)
    same, _ = run_decode(eff, tiny_pool, TINY.K, 4, 65536, 1, 12, seed=TINY.seed)
    assert np.array_equal(ref, same)        # S >= B*K with f = 65536: all on the GPU, bit-identical
    host, st = run_decode(eff, tiny_pool, TINY.K, 0, 65536, 1, 12, seed=TINY.seed)
    assert st["fetched"] == 0 and st["host"] > 0
    assert_close_bf16(host, ref, what="all-host vs all-GPU")


@pytest.mark.parametrize("fmt,H,I,E,K,B,S,f", [
    (synth.FMT_INT4, 2048, 512, 16, 8, 1, 24, 26214),
    (synth.FMT_INT4, 2048, 512, 16, 8, 3, 40, 45875),
    (synth.FMT_NVFP4, 4096, 2048, 12, 6, 1, 8, 45875),
    (synth.FMT_NVFP4, 4096, 2048, 12, 6, 4, 20, 65535),
    (synth.FMT_NVFP4, 2560, 640, 24, 10, 16, 60, 65535),
    (synth.FMT_NVFP4, 2560, 640, 64, 10, 1, 40, 65535),
    (synth.FMT_NVFP4, 2560, 640, 64, 10, 8, 120, 65535),
    (synth.FMT_NVFP4, 2560, 640, 64, 10, 12, 100, 65535),   # 4-token chunks, three per unit
    (synth.FMT_INT4, 2048, 512, 64, 8, 8, 100, 45875),      # int4, 4-token chunks
    (synth.FMT_INT4, 2048, 512, 64, 8, 16, 100, 65535),     # int4, 8-token chunks
    # units with more tokens than the down kernel stages in one pass (38 KiB of LDS): a second pass
    (synth.FMT_NVFP4, 2560, 640, 16, 10, 32, 16, 65535),   # 16 of 32 tokens per pass, weights kept
    (synth.FMT_INT4, 2048, 512, 16, 8, 32, 16, 65535),     # 24 of 32 per pass, weights kept
    (synth.FMT_NVFP4, 4096, 2048, 8, 6, 8, 8, 65535),      # 4 of 8 per pass, runs streamed again
])
def test_decode_shapes(eff, fmt, H, I, E, K, B, S, f):
    pool = PinnedPool(eff, 21, 2, E, H, I, fmt)
    try:
        run_decode(eff, pool, K, S, f, B, 3, router=False, zipf=1.1, seed=21)
    finally:
        pool.free()


def test_decode_speculative(eff):
    pool = PinnedPool(eff, 22, 3, 32, 2560, 640, synth.FMT_NVFP4)
    try:
        _, st = run_decode(eff, pool, 10, 40, 65535, 2, 4, router=False, zipf=1.2, spec_keep=0.65, seed=22)
        assert st["spec_fetched"] > 0
    finally:
        pool.free()


@pytest.mark.parametrize("budget,gap", [(2, True), (0, False), (None, True), (3, False)])
def test_decode_speculative_budget_and_gap(eff, budget, gap):
    """A budget on speculative fetches and copies started after the gate/up kernel: ids, slots, split and
    speculative counts, outputs and the final tables match the oracle's policy with the same budget; the
    outputs equal those of the unbudgeted run (the pool is the source of truth)."""
    pool = PinnedPool(eff, 22, 3, 32, 2560, 640, synth.FMT_NVFP4)
    try:
        ref, st0 = run_decode(eff, pool, 10, 40, 65535, 2, 4, router=False, zipf=1.2, spec_keep=0.65, seed=22)
        outs, st = run_decode(eff, pool, 10, 40, 65535, 2, 4, router=False, zipf=1.2, spec_keep=0.65, seed=22,
                              spec_budget=budget, spec_gap=gap)
        assert np.array_equal(outs, ref)
        if budget is None:
            assert st["spec_fetched"] == st0["spec_fetched"]
        else:
            assert st["spec_fetched"] <= budget * 4 * 2   # at most `budget` per speculative request
            assert st["spec_fetched"] < st0["spec_fetched"]
    finally:
        pool.free()


def test_set_speculation_rejects_bad_values(eff, tiny_pool):
    eng = make_engine(eff, tiny_pool, TINY.K, TINY.S, 1, 32768)
    try:
        for a, b in ((-2, 0), (1, 2), (0, -1)):
            assert eff.lib().eff_set_speculation(eng.h, a, b) == eff.EFF_EINVAL
        assert eff.lib().eff_set_speculation(eng.h, -1, 0) == 0
        eng.set_speculation(2, True)
    finally:
        eng.close()


@pytest.mark.parametrize("fmt,H,I", [(synth.FMT_INT4, 2048, 512), (synth.FMT_NVFP4, 4096, 2048),
                                     (synth.FMT_NVFP4, 2560, 640), (synth.FMT_INT4, 64, 128)])
def test_expert_ffn_outputs(eff, fmt, H, I):
    """eff_expert_ffn_decode alone: y of every GPU entry against the oracle's fp64 y."""
    from oracle.cffn import expert_ffn_batch
    E, K, B = 8, 4, 5
    pool = PinnedPool(eff, 23, 1, E, H, I, fmt)
    eng = make_engine(eff, pool, K, E, B, 65536)
    try:
        ids = np.array([[0, 1, 2, 3], [1, 2, 3, 4], [2, 5, 6, 7], [0, 1, 6, 3], [7, 6, 5, 4]], np.int32)
        d = torch.from_numpy(ids.reshape(-1).copy()).cuda()
        eng.ensure_experts(0, d)
        eng.split_misses(d, torch.empty_like(d), torch.empty(3, dtype=torch.int32, device="cuda"))
        eng.copy_missing()
        x = synth.activations(23, 0, 0, B, H)
        y = torch.full((B, K, H), 7.0, dtype=torch.float32, device="cuda")
        eng.expert_ffn_decode(0, dev_bf16(x), d, y)
        torch.cuda.synchronize()
        yg = y.cpu().numpy()
        xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        jobs = [(pool.record(int(ids[b, k])), pool.tensor_scales(int(ids[b, k])), xf[b:b + 1])
                for b in range(B) for k in range(K)]
        refs = expert_ffn_batch(jobs, fmt, H, I, nthreads=16)
        for j, (b, k) in enumerate([(b, k) for b in range(B) for k in range(K)]):
            assert rel_l2(yg[b, k], refs[j][0]) < 2e-3, (b, k)
            assert float(np.max(np.abs(yg[b, k] - refs[j][0]))) <= MAX_ABS, (b, k)
    finally:
        eng.close()
        pool.free()


def test_bad_speculative_id_reported(eff, tiny_pool):
    """A speculative id outside [0, E) is skipped on the device and reported by the next call."""
    eng = make_engine(eff, tiny_pool, TINY.K, TINY.S, 1, 65536)
    side = torch.cuda.Stream()
    try:
        x = dev_bf16(synth.activations(5, 0, 0, 1, TINY.H))
        lg = torch.from_numpy(synth.trace_logits(5, 0, TINY.E, 1.1, 0, 1)).cuda()
        out = torch.empty((1, TINY.H), dtype=torch.int16, device="cuda")
        bad = torch.tensor([1, TINY.E], dtype=torch.int32, device="cuda")
        eng.decode_layer(0, x, out, logits=lg, spec_ids=bad, side=side)
        torch.cuda.synchronize()
        with pytest.raises(eff.EffError) as ei:
            eng.decode_layer(1, x, out, logits=lg, side=side)
        assert ei.value.code == eff.EFF_EDEVICE
    finally:
        eng.close()
