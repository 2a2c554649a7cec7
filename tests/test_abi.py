"""The C-ABI library loads, exports every function include/eff.h declares, and the
Python binding passes each one the number of arguments the header declares.
Host-only entry points (no GPU work) are exercised here as well."""
import os
import re

import pytest

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "eff.h")


def prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(eff_\w+)\s*\(([^;{]*?)\)\s*;", text, re.S):
        args = m.group(2).strip()
        out[m.group(1)] = 0 if args in ("", "void") else len(args.split(","))
    return out


@pytest.fixture(scope="module")
def eff():
    import expert_ffn_serving_amd as e
    e.lib()
    return e


def test_every_declared_symbol_exported(eff):
    protos = prototypes()
    assert len(protos) >= 20
    assert set(protos) == set(eff.declared_functions())
    for name in protos:
        assert hasattr(eff.lib(), name), name


def test_binding_argument_counts_match_header(eff):
    L = eff.lib()
    for name, n in prototypes().items():
        assert len(getattr(L, name).argtypes) == n, (name, n, len(getattr(L, name).argtypes))


def test_frac_q16_matches_the_oracle(eff):
    import random
    from oracle.qstar import frac_q16
    rnd = random.Random(3)
    cases = [(0.4, 1.0), (0.7, 1.0), (1.0, 1.0), (2.0, 1.0), (0.0, 3.0), (3.0, 0.0), (1.0, 65536.0),
             (1.0, 65537.0), (65535.0, 65536.0), (55e9, 330e9), (float("inf"), 1.0), (1.0, float("inf"))]
    cases += [(rnd.uniform(0, 2e11), rnd.uniform(1, 4e11)) for _ in range(3000)]
    # quotients just below and at integers, where a rounded division would land on the wrong side
    cases += [(k * 3.0 - 1e-12, 3.0 * 65536) for k in range(1, 200)] + [(k * 7.0, 7.0 * 65536) for k in range(200)]
    for bp, bh in cases:
        assert eff.frac_q16(bp, bh) == frac_q16(bp, bh), (bp, bh)
    for bad in ((-1.0, 1.0), (1.0, -2.0), (float("nan"), 1.0)):
        assert eff.frac_q16(*bad) == 0xFFFFFFFF


def test_host_only_entry_points(eff):
    assert eff.qstar(3, 32768) == 1 and eff.qstar(16, 45875) == 11 and eff.qstar(5, 0) == 0
    assert eff.qstar(-1, 5) == -1 and eff.qstar(4, 65537) == -1
    from oracle.qstar import qstar_bruteforce
    for m in range(0, 40):
        for f in (0, 1, 16384, 26214, 32768, 45875, 49152, 65535, 65536):
            assert eff.qstar(m, f) == qstar_bruteforce(m, f)
    assert eff.record_bytes(eff.make_config(40, 256, 8, 2048, 512, 0, 5120, 1)) == 1_769_472
    assert eff.record_bytes(eff.make_config(48, 512, 10, 2560, 640, 1, 2457, 16)) == 2_764_800
    assert eff.record_bytes(eff.make_config(1, 8, 2, 65, 128, 0, 4, 1)) == 0      # H not a multiple of 64
    assert eff.record_bytes(eff.make_config(1, 8, 9, 64, 128, 0, 4, 1)) == 0      # K > E
    assert eff.record_bytes(eff.make_config(1, 8, 2, 64, 128, 0, 20000, 1)) == 0  # too many slots


def test_create_rejects_bad_config_without_side_effects(eff):
    cfg = eff.make_config(1, 8, 2, 64, 128, 0, 4, 0)   # max_tokens 0
    with pytest.raises(eff.EffError) as ei:
        eff.Engine(cfg, 0)
    assert ei.value.code == eff.EFF_EINVAL
