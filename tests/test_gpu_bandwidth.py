"""The bandwidth profile and the fetch fraction it yields ([FT-deep] §4 design pattern ②: f is
B_P / B_H in Q16, from a profile of both paths run at the same time; [FT-blog] §六: measured on
the target machine with the real record shapes).

* The profile's f equals the oracle's f of the rates it reports (concurrent and alone).
* The rates are positive and finite, and the link rate is below what one PCIe x16 link can carry.
* Profiling changes nothing of the engine's state: tables, usage, recency, clock and statistics
  are bit-identical afterwards, and later decode calls match a twin engine that was not profiled.
* eff_set_fetch_frac steers the split of later calls: f = 0 sends every miss to the host,
  f = 65536 fetches every miss that has a victim; values above 65536 are rejected.
The rates themselves depend on the machine: parity unpinned beyond these properties."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from oracle.qstar import frac_q16  # noqa: E402
from tests.helpers import PinnedPool, make_engine  # noqa: E402


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    assert torch.cuda.is_available()
    return e


def decode_tokens(eng, X, LG, tokens, L, out):
    side = torch.cuda.Stream()
    res = []
    for t in tokens:
        for l in range(L):
            eng.decode_layer(l, X[l][t:t + 1], out, logits=LG[l][t:t + 1], side=side)
            res.append(out.cpu().numpy().copy())
    torch.cuda.synchronize()
    return res


def test_profile_bandwidth(eff):
    fmt, H, I, L, E, K, S, f = synth.FMT_INT4, 2048, 512, 4, 64, 8, 40, 26214
    print("bandwidth profile: fmt=%d H=%d I=%d L=%d E=%d K=%d S=%d" % (fmt, H, I, L, E, K, S), flush=True)
    seed, T = 33, 12
    pool = PinnedPool(eff, seed, L, E, H, I, fmt)
    a = b = None
    try:
        a = make_engine(eff, pool, K, S, 1, f)
        b = make_engine(eff, pool, K, S, 1, f)
        X = [torch.from_numpy(synth.activations(seed, l, 0, T, H).view(np.int16)).cuda() for l in range(L)]
        LG = [torch.from_numpy(synth.trace_logits(seed, l, E, 1.1, 0, T)).cuda() for l in range(L)]
        out = torch.empty((1, H), dtype=torch.int16, device="cuda")
        ra = decode_tokens(a, X, LG, range(4), L, out)
        rb = decode_tokens(b, X, LG, range(4), L, out)
        snap0, st0 = a.snapshot_tables(), a.stats()

        p = a.profile_bandwidth(64)
        print("  profile:", {k: (round(v / 1e9, 2) if isinstance(v, float) else v) for k, v in p.items()}, flush=True)
        for k in ("pcie_alone", "host_alone", "pcie_concurrent", "host_concurrent"):
            assert math.isfinite(p[k]) and p[k] > 0, (k, p[k])
        assert p["pcie_alone"] < 80e9 and p["pcie_concurrent"] < 80e9   # one PCIe Gen5 x16 link
        assert p["frac_q16"] == frac_q16(p["pcie_concurrent"], p["host_concurrent"])
        assert p["frac_q16_alone"] == frac_q16(p["pcie_alone"], p["host_alone"])
        assert p["record_bytes"] == pool.R and p["records"] == 64

        snap1, st1 = a.snapshot_tables(), a.stats()
        for k in ("table", "owner", "usage", "recency"):
            assert np.array_equal(snap0[k], snap1[k]), k
        assert (snap0["step"], snap0["last_real"]) == (snap1["step"], snap1["last_real"])
        for k in ("calls", "hits", "fetched", "host", "spec_fetched", "host_calls"):
            assert st0[k] == st1[k], k
        # later calls: the profiled engine and its twin agree bit for bit
        ra = decode_tokens(a, X, LG, range(4, 8), L, out)
        rb = decode_tokens(b, X, LG, range(4, 8), L, out)
        assert all(np.array_equal(x, y) for x, y in zip(ra, rb))
        sa, sb = a.snapshot_tables(), b.snapshot_tables()
        for k in ("table", "owner", "usage", "recency"):
            assert np.array_equal(sa[k], sb[k]), k

        # the fetch fraction steers later splits
        with pytest.raises(Exception):
            a.set_fetch_frac(65537)
        a.set_fetch_frac(0)
        s0 = a.stats()
        decode_tokens(a, X, LG, range(8, 10), L, out)
        s1 = a.stats()
        assert s1["fetched"] == s0["fetched"] and s1["host"] > s0["host"]   # f = 0: every miss on the host
        a.set_fetch_frac(65536)
        decode_tokens(a, X, LG, range(10, 12), L, out)
        s2 = a.stats()
        assert s2["fetched"] > s1["fetched"] and s2["host"] == s1["host"]   # S >> K: a victim for every miss
    finally:
        for e in (a, b):
            if e is not None:
                e.close()
        pool.free()
