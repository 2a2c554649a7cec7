"""A decode step captured into a HIP graph and replayed equals the same calls made eagerly, and the oracle.

Two engines with one configuration see the same tokens: one through eager eff_decode_layer calls,
the other by replaying a graph that holds every layer of one decode step (captured once; each
token's inputs are copied into the captured buffers before its replay, with a synchronization and
a table snapshot between replays).  Per token, the outputs are bit-identical and so are the slot
tables, usage and recency.  Cases: int4 without and NVFP4 with speculative requests (the side
stream joins the capture through the call's events), batch 1 and 4; the cache is small enough
that hits, fetches and host shares all occur.  Every replayed token is also checked against the oracle
engine over the same trace: each layer's bf16 output within rel-L2 <= 5e-3 / max-abs <= 2e-2, and the
table, owner, usage and recency after the token bit for bit against the oracle policy (the third case
with a speculative budget of 2 copied in the gap after the gate/up kernel)."""
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


CASES = [  # fmt, H, I, L, E, K, B, S, f, spec, spec budget (None: none), copies in the gap
    (synth.FMT_INT4, 2048, 512, 4, 64, 8, 1, 40, 26214, False, None, False),
    (synth.FMT_NVFP4, 2560, 640, 3, 64, 10, 4, 60, 45875, True, None, False),
    (synth.FMT_NVFP4, 2560, 640, 4, 64, 10, 8, 120, 52428, True, 2, True),
]


@pytest.mark.parametrize("fmt,H,I,L,E,K,B,S,f,spec,budget,gap", CASES)
def test_decode_step_graph_replay(eff, fmt, H, I, L, E, K, B, S, f, spec, budget, gap):
    print("graph replay: fmt=%d H=%d I=%d L=%d E=%d K=%d B=%d S=%d f=%d spec=%s budget=%s gap=%s" % (
        fmt, H, I, L, E, K, B, S, f, spec, budget, gap), flush=True)
    seed, T, zipf = 21, 6, 1.1
    pool = PinnedPool(eff, seed, L, E, H, I, fmt)
    eager = graph_eng = None
    try:
        eager = make_engine(eff, pool, K, S, B, f)
        graph_eng = make_engine(eff, pool, K, S, B, f)
        orc = oracle_engine(pool, K, S, f)
        if budget is not None or gap:
            for e in (eager, graph_eng):
                e.set_speculation(-1 if budget is None else budget, gap)
            orc.cache.spec_budget = budget
        X = [synth.activations(seed, l, 0, T * B, H) for l in range(L)]
        LG = [synth.trace_logits(seed, l, E, zipf, 0, T * B) for l in range(L)]
        SP = None
        if spec:
            SP = []
            for l in range(L):
                rows = []
                for t in range(T * B):
                    if l + 1 < L:
                        truth = synth.gumbel_topk_sets(LG[l + 1][t:t + 1], K)[0]
                        rows.append(synth.spec_ids(seed, l + 1, E, zipf, t, truth, 0.65))
                    else:
                        rows.append(np.zeros(K, np.int32))
                SP.append(np.stack(rows).astype(np.int32))
        Xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in X]
        LGd = [torch.from_numpy(lg).cuda() for lg in LG]
        SPd = [torch.from_numpy(sp.reshape(-1)).cuda() for sp in SP] if spec else None

        # eager reference
        side_a = torch.cuda.Stream()
        ref = []
        for t in range(T):
            outs = []
            for l in range(L):
                o = torch.empty((B, H), dtype=torch.int16, device="cuda")
                eager.decode_layer(l, Xd[l][t * B:(t + 1) * B], o, logits=LGd[l][t * B:(t + 1) * B],
                                   spec_ids=SPd[l][t * B * K:(t + 1) * B * K] if spec else None, side=side_a)
                outs.append(o)
            torch.cuda.synchronize()
            ref.append((np.stack([o.cpu().numpy() for o in outs]), eager.snapshot_tables()))

        # one decode step captured once, replayed per token
        xb = torch.empty((L, B, H), dtype=torch.int16, device="cuda")
        lb = torch.empty((L, B, E), dtype=torch.float32, device="cuda")
        sb = torch.empty((L, B * K), dtype=torch.int32, device="cuda")
        ob = torch.empty((L, B, H), dtype=torch.int16, device="cuda")
        cap, side_b = torch.cuda.Stream(), torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for l in range(L):
                graph_eng.decode_layer(l, xb[l], ob[l], logits=lb[l], spec_ids=sb[l] if spec else None,
                                       compute=cap, side=side_b)
        for t in range(T):
            for l in range(L):
                xb[l].copy_(Xd[l][t * B:(t + 1) * B])
                lb[l].copy_(LGd[l][t * B:(t + 1) * B])
                if spec:
                    sb[l].copy_(SPd[l][t * B * K:(t + 1) * B * K])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = ob.cpu().numpy()
            want, snap_a = ref[t]
            assert np.array_equal(got, want), ("outputs differ from the eager calls", t)
            snap_b = graph_eng.snapshot_tables()
            for k in ("table", "owner", "usage", "recency"):
                assert np.array_equal(snap_b[k], snap_a[k]), (k, t)
            # the replayed token against the oracle engine over the same trace
            for l in range(L):
                r = orc.decode_layer(l, X[l][t * B:(t + 1) * B], logits=LG[l][t * B:(t + 1) * B],
                                     spec_next=SP[l][t * B:(t + 1) * B] if spec and l + 1 < L else None)
                assert_close_bf16(got[l].view(np.uint16), r["out_bits"], what="graph replay t=%d l=%d" % (t, l))
            for k in ("table", "owner", "usage", "recency"):
                assert list(snap_b[k]) == getattr(orc.cache, k), ("oracle " + k, t)
        st = graph_eng.stats()
        assert st["host"] > 0 and st["fetched"] > 0 and st["hits"] > 0, st
        assert st == {**st, **{k: eager.stats()[k] for k in ("calls", "hits", "fetched", "host", "spec_fetched")}}
        del g
    finally:
        for e in (eager, graph_eng):
            if e is not None:
                e.close()
        pool.free()
