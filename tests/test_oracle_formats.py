"""Pins of the oracle's number formats and record decoder.

* e2m1: the 16 codes against the FP4 value set of the OCP microscaling spec.
* e4m3: the 256 codes against torch's float8_e4m3fn (a library routine).
* bf16: against torch's bfloat16 rounding.
* record sizes against the byte counts printed on the pages (tests/golden/page_byte_counts.txt).
* round trip: the generator's float weights, encoded, come back within half a
  quantization step (a wrong index, nibble order or scale placement breaks it);
  a decoder with the nibbles swapped must fail it (negative control, as the
  NVMe streaming page's "작동 방식 확인 방법" runs swapped nibbles as a must-fail control).
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_byte_counts.txt")


def gold():
    out = {}
    for ln in open(GOLD):
        if ln.startswith("#") or not ln.strip():
            continue
        name, val = [c.strip() for c in ln.split("|")[:2]]
        out[name] = float(val)
    return out


def test_e2m1_all_codes():
    ocp = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = F.e2m1_value(np.arange(16))
    assert np.array_equal(got[:8], ocp)
    assert np.array_equal(got[8:], [-v for v in ocp])
    assert np.signbit(got[8])  # code 8 is -0


def test_e4m3_all_codes_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = F.e4m3_value(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9 and got[0x38] == 1.0


def test_bf16_roundtrip_vs_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-20, 20, 5000), [0.0, -0.0, 1.0]])
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.f64_to_bf16_bits(x.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, ref)
    back = F.bf16_bits_to_f64(ref)
    assert np.array_equal(back, torch.tensor(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_int4_values():
    assert list(F.int4_value(np.arange(16))) == list(range(-8, 8))


def test_record_sizes_match_pages():
    g = gold()
    r_a3b = F.record_bytes(2048, 512)
    assert r_a3b == synth.record_bytes(2048, 512) == 1_769_472
    assert round(r_a3b / 1e6, 2) == g["a3b_expert_record"]
    assert round(256 * r_a3b / 1e6) == g["a3b_layer_experts"]
    assert round(40 * 256 * r_a3b / 1e9) == g["a3b_all_experts"]
    assert round(40 * 256 * r_a3b / 2 ** 30, 1) == g["a3b_all_experts_gib"]
    r_next = F.record_bytes(2560, 640)
    assert r_next == g["next_expert_record"] == 675 * 4096 == g["next_expert_pages"] * 4096
    assert round(48 * 512 * r_next / 2 ** 30) == g["next_all_experts"]
    assert round(10 * 48 * r_next / 1e9, 2) == g["next_token_bytes"]
    payload = 43 * 256 * 3 * 4096 * 2048 // 2
    assert abs(payload / 1e9 - g["dsv4_fp4_pool"]) / g["dsv4_fp4_pool"] < 0.02
    assert F.record_bytes(4096, 2048) == 14_155_776
    assert F.record_bytes(64, 128) == 13_824


def _roundtrip(fmt, H, I, l=1, e=3, seed=99):
    rec, ts = synth.record(seed, 8, l, e, H, I, fmt)
    outs = []
    for m in range(3):
        w = synth.weights_f32(seed, 8, l, e, m, H, I).astype(np.float64)
        wq = F.dequant_matrix(rec, fmt, H, I, m, ts[m])
        outs.append((w, wq))
    return rec, ts, outs


def test_int4_roundtrip_half_step():
    H, I = 128, 192
    rec, ts, outs = _roundtrip(F.INT4, H, I)
    for w, wq in outs:
        N, Kd = w.shape
        g = w.reshape(N, Kd // 32, 32)
        s = np.abs(g).max(axis=2) / 7.0  # scale before bf16 rounding
        err = np.abs(w - wq).reshape(N, Kd // 32, 32).max(axis=2)
        # half a step (plus bf16 rounding of the scale and the clamp at +7 it can cause)
        assert np.all(err <= 0.5 * s * (1 + 2 ** -7) + 7 * s * 2 ** -8 + 1e-12)
        rel = np.linalg.norm(w - wq) / np.linalg.norm(w)
        assert 0.02 < rel < 0.2


def test_nvfp4_roundtrip_half_step():
    H, I = 128, 192
    rec, ts, outs = _roundtrip(F.NVFP4, H, I)
    for (w, wq), t in zip(outs, ts):
        N, Kd = w.shape
        assert t == np.float32(np.abs(w).max() / (6 * 448))
        # per 16-block: the decoded block scale times ts is the grid step unit u; the e2m1 grid
        # has gaps of 0.5 / 1 / 2 units, so an element is within one unit of its decoded value
        blocks = np.abs(w - wq).reshape(N, Kd // 16, 16)
        amax = np.abs(w).reshape(N, Kd // 16, 16).max(axis=2)
        unit = amax / 6.0 * (1 + 2 ** -4)
        assert np.all(blocks.max(axis=2) <= unit + 1e-12)
        rel = np.linalg.norm(w - wq) / np.linalg.norm(w)
        assert 0.03 < rel < 0.2


@pytest.mark.parametrize("fmt", [F.INT4, F.NVFP4])
def test_negative_control_swapped_nibbles_fails(fmt):
    H, I = 64, 128
    rec, ts, outs = _roundtrip(fmt, H, I)
    pay = 3 * H * I // 2
    bad = rec.copy()
    bad[:pay] = ((rec[:pay] & 0x0F) << 4) | (rec[:pay] >> 4)
    w = outs[0][0]
    wq_bad = F.dequant_matrix(bad, fmt, H, I, 0, ts[0])
    assert np.linalg.norm(w - wq_bad) / np.linalg.norm(w) > 0.5


def test_negative_control_transposed_tiles_fail():
    """Reading the tiles inputs-outer (instead of row slices outer) must fail the round trip."""
    H, I = 64, 128
    rec, ts, outs = _roundtrip(F.INT4, H, I)
    w = outs[0][0]
    N, Kd = w.shape
    n, k = np.meshgrid(np.arange(N), np.arange(Kd), indexing="ij")
    _, sh = F.payload_index(Kd, n, k)
    r, q, i = n % 16, (k % 32) // 8, k % 8
    off_bad = ((k // 32) * (N // 16) + n // 16) * 256 + (q * 16 + r) * 4 + i // 2
    codes_bad = (rec[off_bad].astype(np.int64) >> sh) & 15
    sca = rec[3 * H * I // 2:]
    so = F.scale_index(F.INT4, Kd, n, k)
    s = F.bf16_bits_to_f64(sca[so].astype(np.uint16) | (sca[so + 1].astype(np.uint16) << 8))
    bad = F.int4_value(codes_bad) * s
    assert np.linalg.norm(bad - w) / np.linalg.norm(w) > 0.5


def test_layout_is_a_bijection():
    for (N, Kd) in [(128, 64), (64, 128), (640, 2560)]:
        n, k = np.meshgrid(np.arange(N), np.arange(Kd), indexing="ij")
        off, sh = F.payload_index(Kd, n, k)
        lin = off * 2 + sh // 4
        assert np.array_equal(np.sort(lin.reshape(-1)), np.arange(N * Kd))
