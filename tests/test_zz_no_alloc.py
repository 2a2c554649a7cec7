"""eff_expert_ffn_decode_noalloc (plan and SwiGLU staging in the library's static device scratch)
against eff_expert_ffn_decode (the same kernels on engine buffers), through the C ABI: two calls in a
row on one engine, the second with fewer tokens, outputs compared for every GPU entry (bit for bit,
and within the parity bar rel-L2 <= 5e-3 / max-abs <= 2e-2 against the oracle's fp64 expert FFN);
entries the host owns are not written; a call needing more than the static scratch is refused
before anything is launched."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests.helpers import MAX_ABS, PinnedPool, make_engine, rel_l2  # noqa: E402


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    assert torch.cuda.is_available()
    return e


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def routed_slots(eff, eng, E, K, B, seed):
    """Distinct-per-token expert ids, made resident (f = 65536, S = E), as slots on the device."""
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(B)]).astype(np.int32)
    d = torch.from_numpy(ids.reshape(-1).copy()).cuda()
    eng.ensure_experts(0, d)
    eng.split_misses(d, torch.empty_like(d), torch.zeros(3, dtype=torch.int32, device="cuda"))
    eng.copy_missing()
    torch.cuda.synchronize()
    return ids, d


@pytest.mark.parametrize("fmt,H,I,E,K,maxB,Bs", [(synth.FMT_NVFP4, 2560, 640, 40, 10, 16, (16, 5)),
                                                  (synth.FMT_INT4, 2048, 512, 32, 8, 4, (4, 1))])
def test_noalloc_matches_engine_scratch(eff, fmt, H, I, E, K, maxB, Bs):
    from oracle.cffn import expert_ffn_batch
    print("noalloc decode: fmt=%d H=%d I=%d E=%d K=%d max_tokens=%d B=%s" % (fmt, H, I, E, K, maxB, Bs), flush=True)
    pool = PinnedPool(eff, 37, 1, E, H, I, fmt)
    eng = make_engine(eff, pool, K, E, maxB, 65536)
    L = eff.lib()
    try:
        for i, B in enumerate(Bs):
            ids, slots = routed_slots(eff, eng, E, K, B, 100 + i)
            if i == 1:   # one entry the host owns: neither call writes it
                slots[3] = -1
            x = synth.activations(37, 0, 10 * i, B, H)
            xd = dev_bf16(x)
            y_ref = torch.full((B, K, H), 7.0, dtype=torch.float32, device="cuda")
            y_na = torch.full((B, K, H), 7.0, dtype=torch.float32, device="cuda")
            eng.expert_ffn_decode(0, xd, slots, y_ref)
            rc = L.eff_expert_ffn_decode_noalloc(eng.h, 0, xd.data_ptr(), slots.data_ptr(), B, y_na.data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream)
            assert rc == 0, L.eff_last_error().decode()
            torch.cuda.synchronize()
            a, b = y_ref.cpu().numpy(), y_na.cpu().numpy()
            assert np.array_equal(a, b), ("noalloc differs from the engine-scratch call", B)
            sl = slots.cpu().numpy().reshape(B, K)
            xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            jobs, where = [], []
            for t in range(B):
                for k in range(K):
                    if sl[t, k] < 0:
                        assert np.all(b[t, k] == 7.0)
                        continue
                    jobs.append((pool.record(int(ids[t, k])), pool.tensor_scales(int(ids[t, k])), xf[t:t + 1]))
                    where.append((t, k))
            refs = expert_ffn_batch(jobs, fmt, H, I, nthreads=16)
            for (t, k), r in zip(where, refs):
                assert rel_l2(b[t, k], r[0]) <= 5e-3 and float(np.max(np.abs(b[t, k] - r[0]))) <= MAX_ABS, (B, t, k)
    finally:
        eng.close()
        pool.free()


def test_noalloc_refuses_calls_beyond_the_scratch(eff):
    """max_tokens 32, top-8, 24 experts of inter 4096, B = 4: 73,984 + 3 * min(32, 24) * 32 * 4096 bytes,
    more than 8 MiB."""
    E, K, H, I, maxB = 24, 8, 2048, 4096, 32
    pool = PinnedPool(eff, 38, 1, E, H, I, synth.FMT_INT4)
    eng = make_engine(eff, pool, K, E, maxB, 65536)
    L = eff.lib()
    try:
        B = 4
        ids, slots = routed_slots(eff, eng, E, K, B, 7)
        x = dev_bf16(synth.activations(38, 0, 0, B, H))
        y = torch.full((B, K, H), 7.0, dtype=torch.float32, device="cuda")
        rc = L.eff_expert_ffn_decode_noalloc(eng.h, 0, x.data_ptr(), slots.data_ptr(), B, y.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream)
        assert rc == eff.EFF_EINVAL and b"scratch" in L.eff_last_error()
        torch.cuda.synchronize()
        assert torch.all(y == 7.0)
        # the same engine still serves the engine-scratch entry point
        eng.expert_ffn_decode(0, x, slots, y)
        torch.cuda.synchronize()
        assert not torch.all(y == 7.0)
    finally:
        eng.close()
        pool.free()
