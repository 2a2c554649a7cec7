"""Runtime cache rebuild with validation before anything is freed ([FT-blog] §七 item 1;
[FT-deep] §4 design pattern ⑦).

* Accepted rebuilds (shrink, to zero slots, grow past the size the engine was created with) in the
  middle of a decode run: every later output against the oracle (rel-L2 <= 5e-3, max-abs <= 2e-2)
  and the table, usage and recency bit for bit against the oracle policy with the same rebuild.
* Rejected requests (too many slots, over the byte budget, an ensure waiting for its split) return
  EFF_EREJECTED and leave the engine unchanged: its tables are bit-identical and it goes on
  decoding exactly like the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests.helpers import PinnedPool, assert_close_bf16, make_engine, oracle_engine  # noqa: E402


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    assert torch.cuda.is_available()
    return e


def test_rebuild_accepts_and_rejects(eff):
    fmt, H, I, L, E, K, S, f = synth.FMT_INT4, 2048, 512, 4, 64, 8, 40, 26214
    print("rebuild: fmt=%d H=%d I=%d L=%d E=%d K=%d S=%d f=%d" % (fmt, H, I, L, E, K, S, f), flush=True)
    seed, zipf = 29, 1.1
    pool = PinnedPool(eff, seed, L, E, H, I, fmt)
    eng = None
    try:
        eng = make_engine(eff, pool, K, S, 1, f)
        orc = oracle_engine(pool, K, S, f)
        side = torch.cuda.Stream()
        out = torch.empty((1, H), dtype=torch.int16, device="cuda")
        t_next = [0]

        def run(tokens):
            fetched0, host0 = eng.stats()["fetched"], eng.stats()["host"]
            for _ in range(tokens):
                t = t_next[0]
                t_next[0] += 1
                for l in range(L):
                    x = synth.activations(seed, l, t, 1, H)
                    lg = synth.trace_logits(seed, l, E, zipf, t, 1)
                    eng.decode_layer(l, torch.from_numpy(x.view(np.int16)).cuda(), out,
                                     logits=torch.from_numpy(lg).cuda(), side=side)
                    torch.cuda.synchronize()
                    r = orc.decode_layer(l, x, logits=lg)
                    assert_close_bf16(out.cpu().numpy().view(np.uint16), r["out_bits"], what="t=%d l=%d" % (t, l))
            snap = eng.snapshot_tables()
            assert list(snap["table"]) == orc.cache.table
            assert list(snap["owner"]) == orc.cache.owner and list(snap["usage"]) == orc.cache.usage
            assert list(snap["recency"]) == orc.cache.recency
            assert (snap["step"], snap["last_real"]) == (orc.cache.step, orc.cache.last_real)
            st = eng.stats()
            return st["fetched"] - fetched0, st["host"] - host0

        run(4)

        def rejected(call):
            before = eng.snapshot_tables()
            with pytest.raises(eff.EffError) as ei:
                call()
            assert ei.value.code == eff.EFF_EREJECTED, ei.value
            after = eng.snapshot_tables()
            for k in ("table", "owner", "usage", "recency"):
                assert np.array_equal(before[k], after[k]), k

        rejected(lambda: eng.rebuild_cache(20000))
        rejected(lambda: eng.rebuild_cache(24, max_arena_bytes=24 * pool.R - 1))
        # an ensure waiting for its split is not a safe point
        ids = torch.tensor([1, 2, 3, 4, 5, 6, 7, 8], dtype=torch.int32, device="cuda")
        eng.ensure_experts(0, ids)
        torch.cuda.synchronize()
        rejected(lambda: eng.rebuild_cache(24))
        # finish that call as the oracle does, then go on
        ids_h = [1, 2, 3, 4, 5, 6, 7, 8]
        cpu = torch.empty(8, dtype=torch.int32, device="cuda")
        counts = torch.empty(3, dtype=torch.int32, device="cuda")
        eng.split_misses(ids, cpu, counts)
        eng.copy_missing(side=side)
        torch.cuda.synchronize()
        orc.cache.ensure(0, ids_h)
        orc._copy(orc.cache.split().fetch)
        assert eng.cfg.num_slots == S
        run(2)

        eng.rebuild_cache(16, max_arena_bytes=16 * pool.R)   # shrink, exactly at the budget
        orc.rebuild(16)
        fetched, host = run(4)
        assert fetched > 0 and host > 0
        eng.rebuild_cache(0)                                 # no cache: every expert on the host
        orc.rebuild(0)
        fetched, host = run(2)
        assert fetched == 0 and host > 0
        eng.rebuild_cache(96)                                # grow past the created size
        orc.rebuild(96)
        fetched, host = run(4)
        assert fetched > 0
    finally:
        if eng is not None:
            eng.close()
        pool.free()
