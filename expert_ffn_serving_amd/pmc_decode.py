"""The 35b-a3b decode through the standalone entry points, for hardware-counter runs.

    rocprofv3 --pmc FETCH_SIZE -d DIR -o pmc --output-format csv -- \\
        python3 -m expert_ffn_serving_amd.pmc_decode [--warmup 256] [--tokens 64]

Per layer call: route_logits (trace logits), ensure_experts, split_misses, copy_missing (the
fetched records by SDMA before the kernels run), expert_ffn_decode (plan, gate/up, down).  The
policy, the slot state and the expert kernels are those of the bench's decode step at the same
workload; the host share and the combine are left out (they do not touch the expert kernels), and
a fetched record is already in HBM when k_gateup reads it.  A 1 GiB device-to-device copy comes
first, the calibration that `profile_summary traffic` scales the counters by.  The last
tokens * 40 k_gateup dispatches are the measured window; the script prints the distinct GPU
experts per layer call over that window, which the algorithmic bytes per launch follow from.
"""
import argparse
import sys


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--warmup", type=int, default=256)
    p.add_argument("--tokens", type=int, default=64)
    p.add_argument("--threads", type=int, default=16)
    a = p.parse_args(argv)
    import numpy as np
    import torch
    import expert_ffn_serving_amd as eff
    import synth
    from synth.configs import A3B as W
    eff.lib()
    n = (1 << 30) // 4   # the calibration copy
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    R = synth.record_bytes(W.H, W.I)
    ptr = eff.host_alloc(W.L * W.E * R)
    ts = np.empty(W.L * W.E * 3, np.float32)
    synth.fill_records(W.seed, W.E, W.H, W.I, W.fmt, 0, W.L * W.E, ptr, ts, a.threads)
    eng = None
    try:
        cfg = eff.make_config(W.L, W.E, W.K, W.H, W.I, W.fmt, W.S, 1, 0, W.f_q16, a.threads)
        eng = eff.Engine(cfg, ptr, None)
        T = a.warmup + a.tokens
        X = [torch.from_numpy(synth.activations(W.seed, l, 0, T, W.H).view(np.int16)).cuda() for l in range(W.L)]
        LG = [torch.from_numpy(synth.trace_logits(W.seed, l, W.E, W.zipf_s, 0, T)).cuda() for l in range(W.L)]
        ids = torch.empty((1, W.K), dtype=torch.int32, device="cuda")
        w = torch.empty((1, W.K), dtype=torch.float32, device="cuda")
        cpu = torch.empty(W.K, dtype=torch.int32, device="cuda")
        counts = torch.empty(3, dtype=torch.int32, device="cuda")
        y = torch.empty((1, W.K, W.H), dtype=torch.float32, device="cuda")
        s0 = None
        for t in range(T):
            if t == a.warmup:
                torch.cuda.synchronize()
                s0 = eng.stats()
            for l in range(W.L):
                eng.route_logits(LG[l][t:t + 1], ids, w)
                eng.ensure_experts(l, ids.view(-1))
                eng.split_misses(ids.view(-1), cpu, counts)
                eng.copy_missing()
                eng.expert_ffn_decode(l, X[l][t:t + 1], ids.view(-1), y)
        torch.cuda.synchronize()
        s1 = eng.stats()
        calls = s1["calls"] - s0["calls"]
        gpu = (s1["hits"] - s0["hits"]) + (s1["fetched"] - s0["fetched"])
        print("measured window: %d layer calls, %.3f distinct GPU experts per call, %d fetched" % (
            calls, gpu / max(1, calls), s1["fetched"] - s0["fetched"]), flush=True)
    finally:
        if eng is not None:
            eng.close()
        eff.host_free(ptr)


if __name__ == "__main__":
    sys.exit(main())
