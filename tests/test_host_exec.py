"""The library's host executor (the host share of a decode step) against the oracle, on the
CPU: entries with a host id get y = W_d(silu(W_g x) * W_u x) from the pool, others untouched.
Built from the library's own host_exec.cpp with a small shim (no GPU needed)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import synth
from oracle import cffn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "expert_ffn_serving_amd", "csrc", "host_exec.cpp"),
       os.path.join(ROOT, "tests", "native", "host_exec_shim.cpp")]


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("shim") / "libhostshim.so")
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    subprocess.check_call([hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950", "--cuda-host-only", "-fPIC", "-shared",
                           "-o", so] + SRC)
    lib = ctypes.CDLL(so)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.shim_host_ffn.argtypes = [i, i, i, i, i, i, vp, vp, i, vp, vp, i, vp, i, i]
    return lib


SCALAR, AVX2, AVX512F, AVX512_BF16 = 0, 1, 2, 3


def isas(shim):
    """The levels this CPU can run: every level up to the best it supports."""
    return list(range(shim.shim_host_isa_best() + 1))


@pytest.mark.parametrize("fmt,H,I,E,K,B", [(synth.FMT_INT4, 64, 128, 8, 2, 3), (synth.FMT_INT4, 256, 128, 8, 4, 5),
                                           (synth.FMT_NVFP4, 128, 192, 8, 3, 4), (synth.FMT_NVFP4, 320, 128, 6, 2, 2),
                                           (synth.FMT_INT4, 2048, 512, 8, 4, 6), (synth.FMT_NVFP4, 2560, 640, 6, 3, 5)])
@pytest.mark.parametrize("isa", [SCALAR, AVX2, AVX512F, AVX512_BF16])
def test_host_executor_matches_oracle(shim, fmt, H, I, E, K, B, isa):
    if isa not in isas(shim):
        pytest.skip("this CPU does not support host level %d" % isa)
    if isa == SCALAR and H * I > 256 * 1024:
        pytest.skip("the scalar level is checked at the small shapes (it is slow by design)")
    L, layer = 2, 1
    pool, ts = synth.pool_numpy(41, L, E, H, I, fmt)
    x = synth.activations(41, layer, 0, B, H)
    rng = np.random.default_rng(fmt * 100 + H)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(B)]).astype(np.int32)
    cpu = ids.reshape(-1).copy()
    cpu[rng.random(cpu.size) < 0.3] = -1            # those entries belong to the GPU
    y = np.full((B, K, H), 7.0, np.float32)
    used = shim.shim_host_ffn(L, E, K, H, I, fmt, pool.ctypes.data, ts.ctypes.data, layer, x.ctypes.data,
                              cpu.ctypes.data, B, y.ctypes.data, 4, isa)
    assert used == isa
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for p, e in enumerate(cpu):
        b, k = divmod(p, K)
        if e < 0:
            assert np.all(y[b, k] == 7.0)      # GPU-owned entries are not written
            continue
        ref = cffn.expert_ffn_batch([(pool[layer * E + e], ts[layer * E + e], xf[b:b + 1])], fmt, H, I, 1)[0][0]
        err = np.linalg.norm(y[b, k] - ref) / np.linalg.norm(ref)
        assert err < 1e-5, (p, e, err)


def test_best_level_follows_cpu_flags(shim):
    """The level picked at run time is the best the CPU flags allow (AVX-512 BF16 needs F, BW, VBMI and
    BF16; AVX2 needs FMA too)."""
    flags = set()
    for ln in open("/proc/cpuinfo"):
        if ln.startswith("flags"):
            flags = set(ln.split(":", 1)[1].split())
            break
    if {"avx512f", "avx512bw", "avx512vbmi", "avx512_bf16"} <= flags:
        want = AVX512_BF16
    elif "avx512f" in flags:
        want = AVX512F
    elif {"avx2", "fma"} <= flags:
        want = AVX2
    else:
        want = SCALAR
    assert shim.shim_host_isa_best() == want


def test_levels_agree_with_each_other(shim):
    """Every level the CPU runs gives the same outputs within fp32 summation-order error, on one case
    with several tokens per expert (the hi + lo rows of the down input included)."""
    fmt, H, I, E, K, B, L, layer = synth.FMT_NVFP4, 256, 128, 4, 2, 6, 1, 0
    pool, ts = synth.pool_numpy(43, L, E, H, I, fmt)
    x = synth.activations(43, layer, 0, B, H)
    cpu = np.tile(np.array([0, 1], np.int32), B)
    outs = []
    for isa in isas(shim):
        y = np.zeros((B, K, H), np.float32)
        shim.shim_host_ffn(L, E, K, H, I, fmt, pool.ctypes.data, ts.ctypes.data, layer, x.ctypes.data,
                           cpu.ctypes.data, B, y.ctypes.data, 3, isa)
        outs.append(y)
    for y in outs[1:]:
        assert np.linalg.norm(y - outs[0]) / np.linalg.norm(outs[0]) < 1e-6


def test_physical_core_topology(shim):
    """One logical CPU per physical core of the affinity mask: no two share a core, and each is allowed."""
    buf = (ctypes.c_int * 1024)()
    n = shim.shim_physical_core_cpus(buf, 1024)
    cpus = list(buf[:n])
    allowed = os.sched_getaffinity(0)
    assert 1 <= n <= len(allowed) and set(cpus) <= allowed and len(set(cpus)) == n
    cores = set()
    for c in cpus:
        base = "/sys/devices/system/cpu/cpu%d/topology/" % c
        if os.path.exists(base + "core_id"):
            key = (open(base + "physical_package_id").read().strip(), open(base + "core_id").read().strip())
            assert key not in cores
            cores.add(key)
