"""GPU parity of the integer control path against the oracle, bit for bit:
q* (every f for m <= 64), router ids, and whole ensure/split call sequences
(slots, host ids, counts, fetch lists, final tables), including speculative
calls, S = 0, tiny caches, calls with more than 4 victims (the radix select,
up to four 8-bit passes) and calls with more than 64 entries (the expert-table
ensure at most 2048 experts, the sweep ensure above)."""
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from oracle.policy import SlotCache  # noqa: E402
from oracle.qstar import Q16  # noqa: E402
from oracle.router import logits_fixed_order, topk_softmax  # noqa: E402
from tests.helpers import PinnedPool, make_engine  # noqa: E402


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    assert torch.cuda.is_available()
    return e


def brute_all_f(m):
    F = np.arange(m + 1, dtype=np.int64)[:, None]
    f = np.arange(Q16 + 1, dtype=np.int64)[None, :]
    return np.argmin(np.maximum(F * (Q16 - f), (m - F) * f), axis=0)


def test_qstar_batch_every_f(eff):
    ms = np.repeat(np.arange(65, dtype=np.int32), Q16 + 1)
    fs = np.tile(np.arange(Q16 + 1, dtype=np.uint32), 65)
    m_d = torch.from_numpy(ms).cuda()
    f_d = torch.from_numpy(fs.view(np.int32)).cuda()
    q_d = torch.empty_like(m_d)
    eff.qstar_batch(m_d, f_d, q_d)
    got = q_d.cpu().numpy().reshape(65, Q16 + 1)
    for m in range(65):
        assert np.array_equal(got[m], brute_all_f(m)), m
    # large m, random f
    rng = np.random.default_rng(1)
    m2 = rng.integers(0, 4097, 20000).astype(np.int32)
    f2 = rng.integers(0, Q16 + 1, 20000).astype(np.uint32)
    q2 = torch.empty(20000, dtype=torch.int32, device="cuda")
    eff.qstar_batch(torch.from_numpy(m2).cuda(), torch.from_numpy(f2.view(np.int32)).cuda(), q2)
    from oracle.qstar import qstar_bruteforce
    got2 = q2.cpu().numpy()
    for i in range(0, 20000, 97):
        assert got2[i] == qstar_bruteforce(int(m2[i]), int(f2[i]))


@pytest.mark.parametrize("H,E,K,B", [(64, 8, 2, 1), (2048, 256, 8, 1), (2560, 512, 10, 16), (4096, 256, 6, 4),
                                     (4096, 256, 6, 77), (2048, 64, 8, 33)])
def test_route_ids_bit_exact(eff, H, E, K, B):
    pool = PinnedPool(eff, 5, 1, 1, 64, 64, synth.FMT_INT4)   # engine needs a pool; routing does not read it
    cfg = eff.make_config(1, E, K, H, 64, 0, 0, min(B, 32), max(B, 1), 65536, 2)
    eng = eff.Engine(cfg, pool.ptr)
    try:
        x = synth.activations(7, 0, 0, B, H)
        wr = synth.router_weights(7, 0, E, H)
        ids = torch.empty((B, K), dtype=torch.int32, device="cuda")
        w = torch.empty((B, K), dtype=torch.float32, device="cuda")
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        wd = torch.from_numpy(wr.view(np.int16)).cuda()
        eng.route(xd, wd, ids, w)
        torch.cuda.synchronize()
        rid, rw = topk_softmax(logits_fixed_order(x, wr), K)
        assert np.array_equal(ids.cpu().numpy(), rid)
        assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    finally:
        eng.close()
        pool.free()


@pytest.mark.parametrize("H,E,B", [(2048, 256, 4), (2560, 512, 3), (4096, 256, 5), (512, 64, 2)])
def test_route_logits_bit_exact(eff, H, E, B):
    """The fp32 router logits themselves (not only the ids) equal the oracle's fixed-order sums bit for
    bit at the real hidden sizes, where each lane adds blocks of V = 8 consecutive inputs."""
    pool = PinnedPool(eff, 5, 1, 1, 64, 64, synth.FMT_INT4)
    cfg = eff.make_config(1, E, 6, H, 64, 0, 0, B, B, 65536, 2)
    eng = eff.Engine(cfg, pool.ptr)
    try:
        x = synth.activations(17, 0, 0, B, H)
        wr = synth.router_weights(17, 0, E, H)
        ids = torch.empty((B, 6), dtype=torch.int32, device="cuda")
        w = torch.empty((B, 6), dtype=torch.float32, device="cuda")
        eng.route(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(wr.view(np.int16)).cuda(), ids, w)
        got = eng.last_logits(B)
        ref = logits_fixed_order(x, wr)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    finally:
        eng.close()
        pool.free()


def test_route_logits_order_cases(eff):
    """The hand-derived order cases of the oracle's router pins, on the GPU: each case is one router
    row against x = 1, so its logit must equal the case's value exactly."""
    from tests.test_oracle_router import ORDER_CASES, order_case_inputs
    pool = PinnedPool(eff, 5, 1, 1, 64, 64, synth.FMT_INT4)
    try:
        for H in sorted({c[0] for c in ORDER_CASES}):
            cases = [c for c in ORDER_CASES if c[0] == H]
            E = 8
            wr = np.zeros((E, H), np.uint16)
            x = None
            for e, (_, prods, _) in enumerate(cases):
                x, w1 = order_case_inputs(H, prods)
                wr[e] = w1[0]
            cfg = eff.make_config(1, E, 2, H, 64, 0, 0, 1, 1, 65536, 2)
            eng = eff.Engine(cfg, pool.ptr)
            try:
                ids = torch.empty((1, 2), dtype=torch.int32, device="cuda")
                w = torch.empty((1, 2), dtype=torch.float32, device="cuda")
                eng.route(torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(wr.view(np.int16)).cuda(),
                          ids, w)
                got = eng.last_logits(1)[0]
                for e, (_, _, want) in enumerate(cases):
                    assert float(got[e]) == want, (H, e, float(got[e]), want)
                assert np.all(got[len(cases):] == 0)
            finally:
                eng.close()
    finally:
        pool.free()


@pytest.mark.parametrize("E", [256, 512])
def test_route_logits_traces_and_ties(eff, E):
    pool = PinnedPool(eff, 5, 1, 1, 64, 64, synth.FMT_INT4)
    K, B = 10, 16
    cfg = eff.make_config(1, E, K, 64, 64, 0, 0, B, 0, 65536, 2)
    eng = eff.Engine(cfg, pool.ptr)
    try:
        lg = synth.trace_logits(3, 0, E, 1.2, 0, B)
        lg[0, :] = 0.0            # all tied: ids 0..K-1
        lg[1, 7] = lg[1, 9] = lg[1, 200] = 50.0
        lg[2, [131, 67, 3, 2]] = 40.0   # equal logits inside one lane (3, 67, 131) and beside it (2)
        lg[3, [70, 6, 134]] = 30.0      # one lane's equal logits only
        ids = torch.empty((B, K), dtype=torch.int32, device="cuda")
        w = torch.empty((B, K), dtype=torch.float32, device="cuda")
        eng.route_logits(torch.from_numpy(lg).cuda(), ids, w)
        torch.cuda.synchronize()
        rid, rw = topk_softmax(lg, K)
        got = ids.cpu().numpy()
        assert np.array_equal(got, rid)
        assert list(got[0]) == list(range(K)) and list(got[1][:3]) == [7, 9, 200]
        assert list(got[2][:4]) == [2, 3, 67, 131] and list(got[3][:3]) == [6, 70, 134]
        assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    finally:
        eng.close()
        pool.free()


def run_sequence(eff, L, E, K, S, f, calls, maxB):
    """calls: list of (layer, ids list, speculative).  Compares every call and the final tables."""
    pool = PinnedPool(eff, 9, L, E, 64, 64, synth.FMT_INT4)
    eng = make_engine(eff, pool, K, S, maxB, f)
    orc = SlotCache(L, E, S, f)
    try:
        for i, (layer, ids, spec) in enumerate(calls):
            n = len(ids)
            d_ids = torch.tensor(ids, dtype=torch.int32, device="cuda")
            cpu = torch.full((n,), -7, dtype=torch.int32, device="cuda")
            counts = torch.zeros(3, dtype=torch.int32, device="cuda")
            eng.ensure_experts(layer, d_ids, eff.SPECULATIVE if spec else 0)
            ens = d_ids.cpu().numpy().copy()
            eng.split_misses(d_ids, cpu, counts)
            eng.copy_missing()
            torch.cuda.synchronize()
            o_ens = orc.ensure(layer, ids, speculative=spec)
            r = orc.split()
            assert list(ens) == o_ens, ("ensure", i)
            assert list(d_ids.cpu().numpy()) == r.slots, ("slots", i)
            assert list(cpu.cpu().numpy()) == r.cpu_ids, ("cpu_ids", i)
            assert list(counts.cpu().numpy()) == [r.m, r.q, r.host], ("counts", i)
        snap = eng.snapshot_tables()
        assert list(snap["table"]) == orc.table
        assert list(snap["owner"]) == orc.owner
        assert list(snap["usage"]) == orc.usage
        assert list(snap["recency"]) == orc.recency
        assert (snap["step"], snap["last_real"]) == (orc.step, orc.last_real)
        st = eng.stats()
        return st
    finally:
        eng.close()
        pool.free()


@pytest.mark.parametrize("S", [0, 1, 4, 16])
@pytest.mark.parametrize("f", [0, 1, 16384, 32768, 49152, 65535, 65536])
def test_sequences_tiny(eff, S, f):
    rng = random.Random(S * 100003 + f)
    L, E, K = 2, 8, 2
    calls = [(rng.randrange(L), rng.sample(range(E), K), False) for _ in range(60)]
    run_sequence(eff, L, E, K, S, f, calls, 1)


def test_sequences_batched_speculative(eff):
    rng = random.Random(3)
    L, E, K, B = 4, 64, 10, 16
    calls = []
    for step in range(40):
        layer = step % L
        ids = [e for _ in range(B) for e in rng.sample(range(E), K)]
        calls.append((layer, ids, False))
        if layer + 1 < L:
            calls.append((layer + 1, [e for _ in range(B) for e in rng.sample(range(E), K)], True))
    for S, f in [(40, 65535), (100, 45875), (200, 26214), (0, 65536)]:
        run_sequence(eff, L, E, K, S, f, calls, B)


def test_sequences_many_fetches_sorted_path(eff):
    # many fetches per call (256 entries): the radix victim selection and the expert-table ensure
    rng = random.Random(4)
    L, E, K, B = 3, 256, 8, 32
    calls = [(s % L, [e for _ in range(B) for e in rng.sample(range(E), K)], False) for s in range(18)]
    run_sequence(eff, L, E, K, 700, 65536, calls, B)
    run_sequence(eff, L, E, K, 5000, 65536, calls, B)


def test_sequences_many_experts_sweep_path(eff):
    # more than 64 entries and more than 2048 experts: the ensure takes its sweeps over the entries
    # (the expert-table path covers at most 2048); half of the tokens draw from a small hot set so
    # that ids repeat across tokens, the rest from the whole range (ids above 2048 included)
    rng = random.Random(5)
    L, E, K, B = 2, 3000, 8, 16
    hot = rng.sample(range(E), 24)

    def draw():
        return [e for _ in range(B) for e in rng.sample(hot if rng.random() < 0.5 else range(E), K)]

    calls = []
    for step in range(24):
        layer = step % L
        calls.append((layer, draw(), False))
        if layer + 1 < L:
            calls.append((layer + 1, draw(), True))
    for S, f in [(200, 65535), (300, 45875)]:
        run_sequence(eff, L, E, K, S, f, calls, B)


def test_sequences_long_run_radix_passes(eff):
    # the largest cache (16384 slots) filling up over 1400 calls of about 8 misses each (8 layers of
    # 4096 experts): past step 1024 the empty slots' victim keys (below 2^14) sit beside used ones
    # above 2^24, so the radix select runs four 8-bit passes (every other case here needs at most three)
    rng = random.Random(6)
    L, E, K, B = 8, 4096, 8, 1
    calls = [(s % L, rng.sample(range(E), K), False) for s in range(1400)]
    run_sequence(eff, L, E, K, 16384, 65535, calls, B)


def test_bad_id_reported(eff):
    pool = PinnedPool(eff, 9, 1, 8, 64, 64, synth.FMT_INT4)
    eng = make_engine(eff, pool, 2, 4, 1, 65536)
    try:
        d_ids = torch.tensor([3, 9], dtype=torch.int32, device="cuda")
        eng.ensure_experts(0, d_ids)
        eng.split_misses(d_ids, torch.empty(2, dtype=torch.int32, device="cuda"),
                         torch.empty(3, dtype=torch.int32, device="cuda"))
        with pytest.raises(eff.EffError) as ei:
            eng.copy_missing()
        assert ei.value.code == eff.EFF_EDEVICE
    finally:
        eng.close()
        pool.free()
