"""GPU parity of whole-layer prefill against the oracle.

Streams each layer into buffer layer % 2 (slot bytes must equal the host
records; the table must match the oracle's after every layer, leaving the last
two layers resident), runs the MFMA grouped GEMM and compares the bf16 output
within rel-L2 <= 5e-3 / max-abs <= 2e-2.  Also the on-demand fallback (S < 2E)
and chunks with more than 64 tokens per expert (several M passes)."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from synth.configs import TINY  # noqa: E402
from tests.helpers import PinnedPool, assert_close_bf16, make_engine, oracle_engine  # noqa: E402


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    assert torch.cuda.is_available()
    return e


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def slot_bytes(eff, eng, slot, R):
    host = np.empty(R, np.uint8)
    eff._memcpy_d2h(host.ctypes.data, eng.slot_ptr(slot), R)
    return host


def run_prefill(eff, pool, K, S, T, layers, seed, tokens_checked=None, check_bytes=True):
    L, E, H = pool.L, pool.E, pool.H
    eng = make_engine(eff, pool, K, S, 1, 65536, max_prefill_tokens=T)
    orc = oracle_engine(pool, K, S, 65536)
    side = torch.cuda.Stream()
    try:
        for l in layers:
            X = synth.activations(seed, l, 0, T, H, tag=synth.TAG_PREFILL_X)
            wr = synth.router_weights(seed, l, E, H)
            xd, wd = dev_bf16(X), dev_bf16(wr)
            ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
            w = torch.empty((T, K), dtype=torch.float32, device="cuda")
            out = torch.empty((T, H), dtype=torch.int16, device="cuda")
            if S >= 2 * E:
                eng.prefill_stream_layer(l, side)
            eng.route(xd, wd, ids, w)
            eng.expert_ffn_prefill_layer(l, xd, ids, w, out)
            torch.cuda.synchronize()
            r = orc.prefill_layer(l, X, wr, tokens=tokens_checked)
            toks = r["tokens"]
            assert np.array_equal(ids.cpu().numpy()[toks], r["ids"]), ("ids", l)
            got = out.cpu().numpy().view(np.uint16)[toks]
            assert_close_bf16(got, r["out_bits"], what="prefill layer %d" % l)
            if S >= 2 * E and check_bytes:
                b = l % 2
                for e in (0, E // 2, E - 1):
                    assert np.array_equal(slot_bytes(eff, eng, b * E + e, pool.R), pool.record(l * E + e))
            snap = eng.snapshot_tables()
            assert list(snap["table"]) == orc.cache.table, ("table", l)
            assert list(snap["owner"]) == orc.cache.owner, ("owner", l)
        return eng.stats()
    finally:
        eng.close()


def test_tiny_prefill_double_buffer(eff):
    pool = PinnedPool(eff, TINY.seed, TINY.L, TINY.E, TINY.H, TINY.I, TINY.fmt)
    try:
        run_prefill(eff, pool, TINY.K, 2 * TINY.E + 3, 40, range(TINY.L), TINY.seed)
    finally:
        pool.free()


def test_tiny_prefill_fallback(eff):
    pool = PinnedPool(eff, TINY.seed, TINY.L, TINY.E, TINY.H, TINY.I, TINY.fmt)
    try:
        run_prefill(eff, pool, TINY.K, TINY.S, 40, range(TINY.L), TINY.seed)
    finally:
        pool.free()


@pytest.mark.parametrize("fmt,H,I,E,K,T", [
    (synth.FMT_NVFP4, 4096, 2048, 16, 6, 256),    # ~96 tokens per expert: two M passes
    (synth.FMT_INT4, 2048, 512, 16, 8, 70),
    (synth.FMT_NVFP4, 2560, 640, 32, 10, 33),     # I/64 = 10 row blocks: a partial 4-block group
])
def test_prefill_shapes(eff, fmt, H, I, E, K, T):
    L = 3
    pool = PinnedPool(eff, 31, L, E, H, I, fmt)
    try:
        run_prefill(eff, pool, K, 2 * E + 5, T, range(L), 31)
    finally:
        pool.free()


def test_prefill_fp16_range_reported(eff):
    """An activation beyond the fp16 range (the GEMMs take fp16 inputs) is reported as EFF_EDEVICE by
    the next host-waiting call instead of flowing on as inf; a normal layer after it reports nothing."""
    pool = PinnedPool(eff, TINY.seed, TINY.L, TINY.E, TINY.H, TINY.I, TINY.fmt)
    T, E, K = 24, TINY.E, TINY.K
    eng = make_engine(eff, pool, K, 2 * E, 1, 65536, max_prefill_tokens=T)
    side = torch.cuda.Stream()
    try:
        X = synth.activations(TINY.seed, 0, 0, T, TINY.H, tag=synth.TAG_PREFILL_X).copy()
        wr = synth.router_weights(TINY.seed, 0, E, TINY.H)
        ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        out = torch.empty((T, TINY.H), dtype=torch.int16, device="cuda")
        big = X.copy()
        big[5, 7] = 0x47C3  # bf16 of 99840, above the fp16 maximum 65504
        eng.prefill_stream_layer(0, side)
        eng.route(dev_bf16(X), dev_bf16(wr), ids, w)   # routing from the in-range rows
        eng.expert_ffn_prefill_layer(0, dev_bf16(big), ids, w, out)
        torch.cuda.synchronize()
        with pytest.raises(eff.EffError) as ei:
            eng.snapshot_tables()
        assert ei.value.code == eff.EFF_EDEVICE and "fp16" in str(ei.value)
        # reported once; an in-range layer afterwards is clean
        eng.prefill_stream_layer(1, side)
        eng.route(dev_bf16(X), dev_bf16(wr), ids, w)
        eng.expert_ffn_prefill_layer(1, dev_bf16(X), ids, w, out)
        torch.cuda.synchronize()
        eng.snapshot_tables()
    finally:
        eng.close()
        pool.free()
