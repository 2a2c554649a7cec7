"""Builds libeff.so (HIP for gfx950) in-tree with hipcc.

    python -m expert_ffn_serving_amd.build        # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libeff.so")
BUILD = os.path.join(HERE, "_build")

HIP_SOURCES = ["k_cache.hip", "k_route.hip", "k_decode.hip", "k_prefill.hip"]
CPP_SOURCES = ["engine.cpp", "host_exec.cpp"]

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function"]
# packed fp32 instructions stay disabled in device code
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]
# host-only translation units (no kernels): no device pass.  Built for baseline x86-64: the host
# executor's AVX2 and AVX-512 kernels carry their own target attributes and are chosen at run time,
# so the library also loads (and runs its scalar kernels) on a CPU without them.
HOST_CPU = ["--offload-arch=" + ARCH, "--cuda-host-only"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(args):
    cmd, src = args
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s" % (src, err))
    return err


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(([hipcc, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE, src))
        objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(([hipcc, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + HOST_CPU, src))
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for msg in ex.map(_compile, jobs):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = OUT + ".tmp%d" % os.getpid()
    link = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs + ["-lpthread"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
