#!/usr/bin/env python3
"""Benchmark of the routed-expert FFN step over an HBM slot cache on one MI355X.

`python bench.py [--steps K] [--warmup W]` prints one JSON line on stdout (progress on stderr).

value: the qwen3.8-flash-next decode end to end over its whole pool, the largest decode workload
  that fits one GPU: 48 layers x 512 NVFP4 experts of 2560 x 640 (2,764,800-byte records, 68 GB
  pinned in host memory), top-10, 2457 HBM slots (10 %), f = 65535, Zipf(1.2) routing, speculative
  next-layer requests keeping 65 % of the true top-10, B = 16.  A step is 16 tokens through all 48
  layers: control (top-K, ensure, split, speculative request, plan), in-kernel record fetches over
  PCIe, GPU expert FFN, host share, combine.  The slot cache is first warmed by the workload's 512
  trace tokens, then W untimed and K timed steps.  Inputs (x, trace logits, predictions) are resident
  in HBM before timing.  Speculative fetches are capped by the link: a request fetches at most G
  records less the layer's own fetches, G the records the link (its rate alone, from the engine's
  bandwidth profile) carries while the layer's expert kernels run with nothing to fetch (their
  all-resident time at the same batch, below), i.e. the link time a layer leaves idle.  B = 1 and 8
  run beside it with the same settings, and each batch also without speculation.

Beside it (context, not `value`):
  roofline       the dominant kernel, the decode gate/up GEMV (k_gateup, NVFP4, 8-token chunks) at
                 the same expert shape and B = 16 with every expert resident (two layers streamed
                 whole into the slots), timed with HIP events that the launch sets at the kernel's own
                 start and end (on its stream); algorithmic bytes per
                 launch over its average duration.  In the end-to-end run a fetched record crosses
                 PCIe inside this kernel, which makes those launches link-bound: `link` reports them.
  decode_kernels the same for B = 1, 8, 16 and for the dsv4-flash expert shape (B = 1, 4).
  prefill        whole-layer prefill on the dsv4-flash shape (2048 tokens, 256 experts, top-6, 4096 x
                 2048 NVFP4): grouped-GEMM TFLOP/s against the MFMA peak, weight-stream HBM rate, and the
                 overlap of the double-buffered layer streaming (copy time / wall).
  decode_e2e_*   the 35b-a3b decode (int4, 40 x 256, f = 0.4, B = 1; eager and graph replay) and the
                 dsv4-flash decode on 16 of its 43 layers (the whole 155.8 GB pool does not pin).
  cpu_baseline   the CPU oracle on a bounded sample of the qwen3.8-flash-next decode.

`--counters-pass` runs only a program for rocprofv3 counter passes: the roofline kernel's workload
through the standalone entry points (no fused control kernel), after a 1 GiB calibration copy.
`--counters-prefill` does the same for the prefill grouped GEMMs (two dsv4-flash layers streamed);
`--counters-shape dsv4` runs the counters pass at the dsv4-flash expert shape (B = 4) instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA
METRIC = "decode expert-FFN tok/s + HBM GB/s (% peak); prefill MoE TFLOP/s (% MFMA)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_gateup_traffic_qwen_next_b16.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fill_pool(eff, synth, seed, L, E, H, I, fmt, nthreads=16):
    import numpy as np
    R = synth.record_bytes(H, I)
    t0 = time.time()
    ptr = eff.host_alloc(L * E * R)
    ts = np.empty(L * E * 3, np.float32)
    synth.fill_records(seed, E, H, I, fmt, 0, L * E, ptr, ts, nthreads)
    log("  pool %.2f GB pinned and filled in %.1f s" % (L * E * R / 1e9, time.time() - t0))
    return ptr, ts, R


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "expert_ffn_serving_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(path, kernel_sources):
    """HBM bytes per launch from a committed counter summary, when it matches the current sources."""
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != src_hash(*kernel_sources):
        return None
    return d.get("hbm_bytes_per_launch")


def mat_bytes(W):
    return W.H * W.I // 2 + W.H * W.I // 16       # one matrix: 4-bit payload + 1-byte-per-16 scales


def gateup_alg_bytes(W, B, units, launches):
    """k_gateup per pass: gate and up of every GPU expert once, x read once per launch, the SwiGLU
    output written (fp16 plus one 8-byte scale/sum pair per 8 values: 3 bytes per activation) for
    every GPU entry."""
    return units * 2 * mat_bytes(W) + launches * B * W.H * 2 + launches * B * W.K * W.I * 3


def down_alg_bytes(W, B, units, launches):
    """k_down per pass: down of every GPU expert once, the SwiGLU output read, y written (fp32)."""
    return units * mat_bytes(W) + launches * B * W.K * (W.I * 3 + W.H * 4)


# ------------------------------------------------------------------------------ decode end to end
def decode_inputs(torch, synth, W, L, B, n_steps):
    """x, trace logits and speculative predictions for n_steps steps of B tokens, resident in HBM."""
    import numpy as np
    n_rows = n_steps * B
    X = [torch.from_numpy(synth.activations(W.seed, l, 0, n_rows, W.H).view(np.int16)).cuda() for l in range(L)]
    lg_host = [synth.trace_logits(W.seed, l, W.E, W.zipf_s, 0, n_rows) for l in range(L)]
    LG = [torch.from_numpy(a).cuda() for a in lg_host]
    SP = []
    if W.spec_keep >= 0:
        for l in range(L - 1):   # predictions of layer l+1's sets, made at layer l
            truth = synth.gumbel_topk_sets(lg_host[l + 1], W.K)
            SP.append(torch.from_numpy(np.stack([synth.spec_ids(W.seed, l + 1, W.E, W.zipf_s, r, truth[r], W.spec_keep)
                                                 for r in range(n_rows)]).astype(np.int32).reshape(-1)).cuda())
    torch.cuda.synchronize()
    return X, LG, SP


def e2e_run(eff, torch, W, pool, inputs, B, f, steps, warmup, warm_tokens, L=None, S=None, spec_budget=-1,
            spec_gap=False, spec=True, threads=0, timing=False, spec_link=-1):
    """One end-to-end decode run on a fresh engine: the cache warmed by `warm_tokens` trace tokens,
    `warmup` untimed steps, then `steps` timed steps (bracketed by device synchronizations)."""
    ptr, ts, R = pool
    L = L or W.L
    S = W.S if S is None else S
    X, LG, SP = inputs
    cfg = eff.make_config(L, W.E, W.K, W.H, W.I, W.fmt, S, B, 0, f, threads)
    eng = eff.Engine(cfg, ptr, ts if W.fmt == 1 else None)
    eng.set_speculation(spec_budget, spec_gap)
    eng.set_speculation_link(spec_link)
    comp, side = torch.cuda.Stream(), torch.cuda.Stream()
    L_, h = eff.lib(), eng.h
    cs, ss = comp.cuda_stream, side.cuda_stream
    out = torch.empty((B, W.H), dtype=torch.int16, device="cuda")
    op = out.data_ptr()
    use_spec = spec and W.spec_keep >= 0
    K = W.K

    def step(t):
        for l in range(L):
            sp = SP[l][t * B * K:(t + 1) * B * K].data_ptr() if use_spec and l + 1 < L else None
            rc = L_.eff_decode_layer(h, l, X[l][t * B:(t + 1) * B].data_ptr(), None,
                                     LG[l][t * B:(t + 1) * B].data_ptr(), B, sp, op, cs, ss)
            if rc:
                raise eff.EffError(rc, L_.eff_last_error().decode())

    n_warm = (warm_tokens + B - 1) // B
    for t in range(n_warm + warmup):
        step(t)
    torch.cuda.synchronize()
    s0 = eng.stats()
    if timing:
        eng.reset_stats()
        eng.set_flags(eff.CFG_TIMING)
        s0 = eng.stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(n_warm + warmup, n_warm + warmup + steps):
        step(t)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    s1 = eng.stats()
    hi = eng.host_info()
    eng.close()
    n = steps * L
    per = {k: round((s1[k] - s0[k]) / n, 3) for k in ("hits", "fetched", "host", "spec_fetched")}
    link = (per["fetched"] + per["spec_fetched"]) * R
    res = {"B": B, "frac_q16": f, "spec": use_spec, "spec_budget": spec_budget, "spec_in_gap": spec_gap,
           "spec_link_records": spec_link if use_spec else None,
           "cache_warmup_tokens": n_warm * B, "warmup_steps": warmup, "steps": steps,
           "tok_s": round(steps * B / dt, 2), "ms_per_step": round(dt * 1e3 / steps, 3),
           "us_per_layer": round(dt * 1e6 / n, 1), "per_layer_call": per,
           "link_MB_per_layer": round(link / 1e6, 2), "link_GBps": round(link / (dt / n) / 1e9, 2),
           "host_executor": {"isa": eff.HOST_ISA_NAMES.get(hi["isa"], "?"), "threads": hi["threads"],
                             "pinned": bool(hi["pinned"]), "physical_cores": hi["physical_cores"],
                             "us_per_layer_call_with_host": round(
                                 (s1["host_ms"] - s0["host_ms"]) * 1e3 / max(1, s1["host_calls"] - s0["host_calls"]),
                                 2)}}
    if timing:
        for slot, name in ((eff.T_DECODE_GATEUP, "gateup"), (eff.T_DECODE_DOWN, "down")):
            nl = s1["launches"][slot]
            res[name + "_us_avg"] = round(s1["kernel_ms"][slot] * 1e3 / max(1, nl), 2)
    return res, dt


def run_headline(eff, torch, synth, W, steps, warmup, threads, compute_us, skip_variants=False):
    """The workload's end-to-end decode at B = 16 (value) and B = 1, 8, plus context variants."""
    log("decode end to end %s: L=%d E=%d K=%d H=%d I=%d S=%d f=%d spec keep %.2f" % (
        W.name, W.L, W.E, W.K, W.H, W.I, W.S, W.f_q16, W.spec_keep))
    pool = fill_pool(eff, synth, W.seed, W.L, W.E, W.H, W.I, W.fmt)
    ptr, ts, R = pool
    res = {"workload": W.name, "record_bytes": R}
    # the bandwidth profile of this machine ([FT-deep] §4 design pattern ②), for the context variants
    cfg = eff.make_config(W.L, W.E, W.K, W.H, W.I, W.fmt, W.S, max(W.batches), 0, W.f_q16, threads)
    eng = eff.Engine(cfg, ptr, ts)
    bw = eng.profile_bandwidth(256)
    eng.close()
    res["bandwidth_profile"] = {"frac_q16": bw["frac_q16"], "frac_q16_alone": bw["frac_q16_alone"],
                                "pcie_GBps_concurrent": round(bw["pcie_concurrent"] / 1e9, 2),
                                "host_GBps_concurrent": round(bw["host_concurrent"] / 1e9, 2),
                                "pcie_GBps_alone": round(bw["pcie_alone"] / 1e9, 2),
                                "host_GBps_alone": round(bw["host_alone"] / 1e9, 2)}
    log("  bandwidth profile: link %.1f GB/s, host %.1f GB/s at once -> f = %d (workload: %d)" % (
        bw["pcie_concurrent"] / 1e9, bw["host_concurrent"] / 1e9, bw["frac_q16"], W.f_q16))
    head = None
    link_Bps = bw["pcie_alone"]

    def link_cap(B):
        """Records the link (its rate alone) carries while the layer's expert kernels run with every
        expert resident (gate/up + down at this batch, measured by decode_kernel_rates): the link
        time a layer leaves when its own reads take none."""
        return int(link_Bps * compute_us[B] * 1e-6 / R)

    def show(tag, r):
        log("  B=%d, %s (f=%d, link cap %s): %.2f tok/s (%.1f us per layer), per layer call %s, %.1f MB/layer over "
            "the link (%.1f GB/s)" % (r["B"], tag, r["frac_q16"], r["spec_link_records"], r["tok_s"], r["us_per_layer"],
                                      r["per_layer_call"], r["link_MB_per_layer"], r["link_GBps"]))

    for B in sorted(W.batches, reverse=True):
        n_steps = (W.warmup_tokens + B - 1) // B + warmup + steps
        inputs = decode_inputs(torch, synth, W, W.L, B, n_steps)

        def run(f, **kw):
            return e2e_run(eff, torch, W, pool, inputs, B, f, steps, warmup, W.warmup_tokens, threads=threads, **kw)

        # speculation reads guesses only in the link time the layer's real reads leave ([NVMe-8GB] "엔진"
        # item 3): the cap is the link's records per layer of the same step without speculation
        nospec, _ = run(W.f_q16, spec=False)
        res["B%d_nospec" % B] = nospec
        show("no speculation", nospec)
        r, dt = run(W.f_q16, spec_link=link_cap(B))
        res["B%d" % B] = r
        show("workload settings", r)
        if B == 16:
            head = (r, dt)
            if not skip_variants:
                rv, _ = run(W.f_q16)
                res["B16_spec_uncapped"] = rv
                show("speculation without the link cap", rv)
                pn, _ = run(bw["frac_q16"], spec=False)
                res["B16_profiled_f_nospec"] = pn
                show("profiled f, no speculation", pn)
                pc, _ = run(bw["frac_q16"], spec_link=link_cap(B))
                res["B16_profiled_f"] = pc
                show("profiled f", pc)
        del inputs
        torch.cuda.empty_cache()
    eff.host_free(ptr)
    return res, head


# ---------------------------------------------------------------------- decode kernels, all resident
def decode_kernel_rates(eff, torch, synth, W, batches, tokens=64, threads=0, label=""):
    """HBM rates of the decode expert kernels at a workload's expert shape: layers 0 and 1 streamed
    whole into the two slot buffers (S = 2E, every expert resident, no call misses), then `tokens`
    decode steps per batch size on the workload's Zipf trace, alternating the two layers, with the
    expert kernels timed by HIP events that each launch sets at its kernel's start and end (EFF_CFG_TIMING)."""
    import numpy as np
    pool = fill_pool(eff, synth, W.seed, 2, W.E, W.H, W.I, W.fmt)
    ptr, ts, R = pool
    E, K, H, I = W.E, W.K, W.H, W.I
    cfg = eff.make_config(2, E, K, H, I, W.fmt, 2 * E, max(batches), 0, 65536, threads)
    eng = eff.Engine(cfg, ptr, ts)
    comp, side = torch.cuda.Stream(), torch.cuda.Stream()
    x = torch.from_numpy(synth.activations(W.seed, 0, 0, max(batches), H).view(np.int16)).cuda()
    out = torch.empty((max(batches), H), dtype=torch.int16, device="cuda")
    eng.prefill_stream_layer(0, side)
    eng.prefill_stream_layer(1, side)
    torch.cuda.synchronize()
    res = {"workload": "%s expert shape (H=%d I=%d E=%d K=%d %s), 2 layers, every expert resident" % (
        W.name, H, I, E, K, "NVFP4" if W.fmt == 1 else "int4"), "tokens": tokens, "zipf": W.zipf_s}
    for B in batches:
        LG = [torch.from_numpy(synth.trace_logits(W.seed, l, E, W.zipf_s, 0, tokens * B)).cuda() for l in range(2)]
        with torch.cuda.stream(comp):   # one untimed step first
            for l in range(2):
                eng.decode_layer(l, x[:B], out[:B], logits=LG[l][:B], compute=comp, side=side)
        torch.cuda.synchronize()
        eng.reset_stats()
        eng.set_flags(eff.CFG_TIMING)
        with torch.cuda.stream(comp):
            for t in range(tokens):
                for l in range(2):
                    eng.decode_layer(l, x[:B], out[:B], logits=LG[l][t * B:(t + 1) * B], compute=comp, side=side)
        torch.cuda.synchronize()
        st = eng.stats()
        eng.set_flags(0)
        n = st["launches"][eff.T_DECODE_GATEUP]
        g_ms, d_ms = st["kernel_ms"][eff.T_DECODE_GATEUP], st["kernel_ms"][eff.T_DECODE_DOWN]
        U = st["hits"] + st["fetched"]
        gu, dn = gateup_alg_bytes(W, B, U, n), down_alg_bytes(W, B, U, n)
        res["B%d" % B] = {
            "launches": n, "gpu_experts_per_launch": round(U / max(1, n), 3), "fetched": st["fetched"],
            "gateup_alg_bytes_per_launch": int(gu / max(1, n)),
            "gateup_us": round(g_ms * 1e3 / max(1, n), 2), "gateup_GBps": round(gu / (g_ms * 1e-3) / 1e9, 1),
            "gateup_frac": round(gu / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "down_alg_bytes_per_launch": int(dn / max(1, n)),
            "down_us": round(d_ms * 1e3 / max(1, n), 2), "down_GBps": round(dn / (d_ms * 1e-3) / 1e9, 1),
            "down_frac": round(dn / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        log("  decode kernels at the %s shape, B=%d: %.1f experts/launch, gate/up %.2f us (%.0f GB/s, %.1f%%), "
            "down %.2f us (%.0f GB/s, %.1f%%)" % (label or W.name, B, U / max(1, n), g_ms * 1e3 / max(1, n),
                                                 gu / (g_ms * 1e-3) / 1e9, 100 * gu / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                                 d_ms * 1e3 / max(1, n), dn / (d_ms * 1e-3) / 1e9,
                                                 100 * dn / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS))
    eng.close()
    eff.host_free(ptr)
    return res


def calibration_copy(torch):
    """A 1 GiB device-to-device copy: what a counter reads for it scales the counter to bytes."""
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def counters_prefill(eff, torch, synth, W, layers=2, threads=0):
    """A program for rocprofv3 counter passes over the prefill grouped GEMMs: the calibration copy,
    then run_prefill on `layers` layers of the prefill workload (route, sort, fp16 rows, gate/up and
    down GEMMs, combine; no decode kernels)."""
    calibration_copy(torch)
    run_prefill(eff, torch, synth, W, layers, threads)


def counters_pass(eff, torch, synth, W, B=16, tokens=64, warm=8, threads=0):
    """A program for rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE): a 1 GiB device-to-device copy
    (the calibration), then the roofline kernel's workload (the same expert shape, B, trace and
    resident slots as decode_kernel_rates) through the standalone entry points: route_logits,
    ensure_experts, split_misses, copy_missing (nothing to copy: every expert is resident),
    expert_ffn_decode.  The fused control kernel is not launched.  The last tokens * 2 k_gateup
    dispatches are the measured window."""
    import numpy as np
    calibration_copy(torch)
    ptr, ts, R = fill_pool(eff, synth, W.seed, 2, W.E, W.H, W.I, W.fmt)
    E, K, H = W.E, W.K, W.H
    cfg = eff.make_config(2, E, K, H, W.I, W.fmt, 2 * E, B, 0, 65536, threads)
    eng = eff.Engine(cfg, ptr, ts)
    try:
        side = torch.cuda.Stream()
        eng.prefill_stream_layer(0, side)
        eng.prefill_stream_layer(1, side)
        torch.cuda.synchronize()
        x = torch.from_numpy(synth.activations(W.seed, 0, 0, B, H).view(np.int16)).cuda()
        LG = [torch.from_numpy(synth.trace_logits(W.seed, l, E, W.zipf_s, 0, (tokens + warm) * B)).cuda()
              for l in range(2)]
        ids = torch.empty((B, K), dtype=torch.int32, device="cuda")
        w = torch.empty((B, K), dtype=torch.float32, device="cuda")
        cpu = torch.empty(B * K, dtype=torch.int32, device="cuda")
        counts = torch.empty(3, dtype=torch.int32, device="cuda")
        y = torch.empty((B, K, H), dtype=torch.float32, device="cuda")
        s0 = None
        for t in range(warm + tokens):
            if t == warm:
                torch.cuda.synchronize()
                s0 = eng.stats()
            for l in range(2):
                eng.route_logits(LG[l][t * B:(t + 1) * B], ids, w)
                eng.ensure_experts(l, ids.view(-1))
                eng.split_misses(ids.view(-1), cpu, counts)
                eng.copy_missing()
                eng.expert_ffn_decode(l, x, ids.view(-1), y)
        torch.cuda.synchronize()
        s1 = eng.stats()
        calls = s1["calls"] - s0["calls"]
        gpu = (s1["hits"] - s0["hits"]) + (s1["fetched"] - s0["fetched"])
        print("counters pass %s B=%d: window of %d k_gateup dispatches, %.3f distinct GPU experts per call, "
              "%d fetched; algorithmic bytes per k_gateup launch %d" % (
                  W.name, B, calls, gpu / max(1, calls), s1["fetched"] - s0["fetched"],
                  int(gateup_alg_bytes(W, B, gpu, calls) / max(1, calls))), flush=True)
    finally:
        eng.close()
        eff.host_free(ptr)


# ------------------------------------------------------------------------------ 35b-a3b end to end
def run_a3b(eff, torch, synth, W, steps, warmup, threads):
    """The 35b-a3b decode end to end at B = 1 (eager calls, then the decode step captured once as a HIP
    graph and replayed per token after one untimed replay)."""
    import numpy as np
    log("decode end to end %s: L=%d E=%d K=%d H=%d I=%d S=%d f=%d" % (W.name, W.L, W.E, W.K, W.H, W.I, W.S,
                                                                       W.f_q16))
    pool = fill_pool(eff, synth, W.seed, W.L, W.E, W.H, W.I, W.fmt)
    B = 1
    n_tok = W.warmup_tokens + warmup + 2 * steps + 1
    inputs = decode_inputs(torch, synth, W, W.L, B, n_tok)
    r, _ = e2e_run(eff, torch, W, pool, inputs, B, W.f_q16, steps, warmup, W.warmup_tokens, threads=threads)
    log("  eager: %.1f tok/s, per layer call %s" % (r["tok_s"], r["per_layer_call"]))
    # graph replay: one engine, the same warm-up, then one decode step captured and replayed per token
    ptr, ts, R = pool
    X, LG, _ = inputs
    cfg = eff.make_config(W.L, W.E, W.K, W.H, W.I, W.fmt, W.S, B, 0, W.f_q16, threads)
    eng = eff.Engine(cfg, ptr, None)
    comp, side = torch.cuda.Stream(), torch.cuda.Stream()
    L_, h = eff.lib(), eng.h
    cs, ss = comp.cuda_stream, side.cuda_stream
    out = torch.empty((B, W.H), dtype=torch.int16, device="cuda")
    for t in range(W.warmup_tokens + warmup):
        for l in range(W.L):
            rc = L_.eff_decode_layer(h, l, X[l][t:t + 1].data_ptr(), None, LG[l][t:t + 1].data_ptr(), B, None,
                                     out.data_ptr(), cs, ss)
            if rc:
                raise eff.EffError(rc, L_.eff_last_error().decode())
    gx = torch.empty((W.L, B, W.H), dtype=torch.int16, device="cuda")
    gl = torch.empty((W.L, B, W.E), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=comp):
        for l in range(W.L):
            rc = L_.eff_decode_layer(h, l, gx[l].data_ptr(), None, gl[l].data_ptr(), B, None, out.data_ptr(), cs, ss)
            if rc:
                raise eff.EffError(rc, L_.eff_last_error().decode())
    Xs, LGs = torch.stack([x[:, :] for x in X]), torch.stack(LG)

    def gstep(t):
        with torch.cuda.stream(comp):
            gx.copy_(Xs[:, t:t + 1])
            gl.copy_(LGs[:, t:t + 1])
            graph.replay()

    t_next = W.warmup_tokens + warmup
    gstep(t_next)            # the first replay after capture, untimed
    torch.cuda.synchronize()
    t_next += 1
    t0 = time.perf_counter()
    for t in range(t_next, t_next + steps):
        gstep(t)
    torch.cuda.synchronize()
    dtg = time.perf_counter() - t0
    del graph
    eng.close()
    r["graph_replay_tok_s"] = round(steps * B / dtg, 2)
    log("  graph replay: %.1f tok/s" % (steps * B / dtg))
    del inputs, Xs, LGs
    eff.host_free(ptr)
    return r


# ------------------------------------------------------------------------------------- prefill
def run_prefill(eff, torch, synth, W, layers, threads, cpu_tokens=0, cpu_threads=1):
    import numpy as np
    T = W.prefill_T
    log("prefill %s: T=%d E=%d K=%d H=%d I=%d (%d layers streamed)" % (W.name, T, W.E, W.K, W.H, W.I, layers))
    ptr, ts, R = fill_pool(eff, synth, W.seed, layers, W.E, W.H, W.I, W.fmt)
    cfg = eff.make_config(layers, W.E, W.K, W.H, W.I, W.fmt, W.S, 1, T, W.f_q16, threads, eff.CFG_TIMING)
    eng = eff.Engine(cfg, ptr, ts)
    X = [torch.from_numpy(synth.activations(W.seed, l, 0, T, W.H, tag=synth.TAG_PREFILL_X).view(np.int16)).cuda()
         for l in range(layers)]
    WR = [torch.from_numpy(synth.router_weights(W.seed, l, W.E, W.H).view(np.int16)).cuda() for l in range(layers)]
    ids = torch.empty((T, W.K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, W.K), dtype=torch.float32, device="cuda")
    out = torch.empty((T, W.H), dtype=torch.int16, device="cuda")
    side = torch.cuda.Stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(layers)]
    torch.cuda.synchronize()
    eng.reset_stats()

    def stream(l):
        ev[l][0].record(side)
        eng.prefill_stream_layer(l, side)
        ev[l][1].record(side)

    t0 = time.perf_counter()
    stream(0)
    for l in range(layers):
        if l + 1 < layers:
            stream(l + 1)
        eng.route(X[l], WR[l], ids, w)
        eng.expert_ffn_prefill_layer(l, X[l], ids, w, out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    copy_ms = sum(a.elapsed_time(b) for a, b in ev)
    st = eng.stats()
    g_ms = st["kernel_ms"][eff.T_PREFILL_GATEUP]
    d_ms = st["kernel_ms"][eff.T_PREFILL_DOWN]
    n = st["launches"][eff.T_PREFILL_GATEUP]
    flops = 2.0 * T * W.K * 3 * W.H * W.I           # per layer
    tflops = flops * n / ((g_ms + d_ms) * 1e-3) / 1e12
    wbytes = W.E * R
    res = {
        "workload": W.name, "tokens": T, "layers_timed": n, "pool_layers": layers,
        "gflop_per_layer": round(flops / 1e9, 1),
        "tflops": round(tflops, 1), "peak_tflops": MFMA_PEAK_TFLOPS, "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
        "gemm_ms_per_layer": round((g_ms + d_ms) / max(1, n), 3),
        "gateup_ms_per_layer": round(g_ms / max(1, n), 3), "down_ms_per_layer": round(d_ms / max(1, n), 3),
        "weight_GBps": round(wbytes * n / ((g_ms + d_ms) * 1e-3) / 1e9, 1),
        "weight_hbm_frac": round(wbytes * n / ((g_ms + d_ms) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "wall_ms_per_layer_with_streaming": round(wall * 1e3 / layers, 2),
        "stream_GBps": round(wbytes * layers / (copy_ms * 1e-3) / 1e9, 1),
        "stream_overlap": {"copy_ms_total": round(copy_ms, 2), "wall_ms": round(wall * 1e3, 2),
                           "efficiency": round(copy_ms / (wall * 1e3), 3),
                           "definition": "sum over the streamed layers of the side-stream copy time (HIP events "
                                         "around each layer's install + record copy) / wall time of the whole "
                                         "prefill; 1.0 = the link never idles"},
        "source_sha": src_hash("k_prefill.hip"),
    }
    log("  prefill: %.1f TFLOP/s (%.1f%% of MFMA peak), weights %.0f GB/s (%.1f%% of HBM peak), GEMM %.3f ms/layer, "
        "wall %.1f ms/layer, stream overlap %.3f" % (
            tflops, 100 * tflops / MFMA_PEAK_TFLOPS, res["weight_GBps"], 100 * res["weight_hbm_frac"],
            res["gemm_ms_per_layer"], wall * 1e3 / layers, res["stream_overlap"]["efficiency"]))
    eng.close()
    if cpu_tokens > 0:
        res["cpu_oracle"] = prefill_oracle(synth, W, (ptr, ts, R), cpu_tokens, cpu_threads)
        log("  prefill cpu oracle: %.2f GFLOP/s (%s)" % (res["cpu_oracle"]["value"], res["cpu_oracle"]["sample"]))
    eff.host_free(ptr)
    return res


# ------------------------------------------------------------------------------------- CPU oracle
def host_cpu():
    """CPU model, sockets, cores per socket, threads per core (lscpu), and the CPUs of this process."""
    info = {"model": "?", "sockets": None, "cores_per_socket": None, "threads_per_core": None}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        keys = {"Model name": "model", "Socket(s)": "sockets", "Core(s) per socket": "cores_per_socket",
                "Thread(s) per core": "threads_per_core"}
        for ln in out.splitlines():
            k, _, v = ln.partition(":")
            if k.strip() in keys:
                v = v.strip()
                info[keys[k.strip()]] = int(v) if v.isdigit() else v
    except (OSError, subprocess.SubprocessError):
        pass
    info["cpus_available"] = len(os.sched_getaffinity(0))
    return info


def host_read_gbps(ptr, nbytes, threads, reps=3):
    """Host memory read bandwidth over `nbytes` of the pinned pool (what the host share streams), with
    `threads` threads each summing its own contiguous part (NumPy releases the GIL in the reduction)."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    words = nbytes // 8 // threads * threads
    a = np.frombuffer((ctypes.c_uint64 * words).from_address(ptr), np.uint64)
    parts = np.array_split(a, threads)
    best = 0.0
    with ThreadPoolExecutor(threads) as ex:
        for _ in range(reps):
            t0 = time.perf_counter()
            list(ex.map(lambda v: int(np.add.reduce(v)), parts))
            best = max(best, words * 8 / (time.perf_counter() - t0) / 1e9)
    return round(best, 1)


def prefill_oracle(synth, W, pool, tokens, threads):
    """The oracle's prefill layer (as it stands) on `tokens` tokens of layer 0, in GFLOP/s of expert math."""
    import ctypes

    import numpy as np

    from oracle.engine import OracleEngine
    ptr, ts, R = pool

    def rec(flat):
        return np.frombuffer((ctypes.c_uint8 * R).from_address(ptr + flat * R), np.uint8)

    eng = OracleEngine(2, W.E, W.K, W.H, W.I, W.fmt, W.S, W.f_q16, rec, lambda f: ts[3 * f:3 * f + 3],
                       use_c=True, nthreads=threads)
    x = synth.activations(W.seed, 0, 0, W.prefill_T, W.H, tag=synth.TAG_PREFILL_X)
    wr = synth.router_weights(W.seed, 0, W.E, W.H)
    sample = list(range(0, W.prefill_T, W.prefill_T // tokens))[:tokens]
    t0 = time.perf_counter()
    eng.prefill_layer(0, x, wr, tokens=sample)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(sample) * W.K * 3 * W.H * W.I
    return {"value": round(flops / dt / 1e9, 2), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of the %d tokens of layer 0 (every %dth), including the oracle's copy of the layer's %d "
                      "records into its buffer; fp64 C evaluator" % (len(sample), W.prefill_T,
                                                                    W.prefill_T // tokens, W.E)}


def cpu_baseline(eff, synth, W, tokens, threads, layers_1core=6):
    """The oracle as it stands on the headline workload's decode: `tokens` tokens (B = 1) through every
    layer of the same trace from a cold cache, on `threads` threads, and the first token's first
    `layers_1core` layers on one thread (scaled to a whole token); tok/s per token of that sample.  Only
    the records the sample routes to are generated (the generator keys a record by its flat id, so they
    are the pool's); their generation is not timed."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle.engine import OracleEngine
    R = synth.record_bytes(W.H, W.I)
    lg = [synth.trace_logits(W.seed, l, W.E, W.zipf_s, 0, tokens) for l in range(W.L)]
    xs = [synth.activations(W.seed, l, 0, tokens, W.H) for l in range(W.L)]
    flats = sorted({l * W.E + int(e) for l in range(W.L) for row in synth.gumbel_topk_sets(lg[l], W.K) for e in row})
    buf = np.empty((len(flats), R), np.uint8)
    tsb = np.empty((len(flats), 3), np.float32)

    def gen(i):
        synth.fill_records(W.seed, W.E, W.H, W.I, W.fmt, flats[i], 1, buf[i].ctypes.data, tsb[i], 1)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(gen, range(len(flats))))
    where = {fl: i for i, fl in enumerate(flats)}

    def timed(n, nthreads, layers):
        eng = OracleEngine(W.L, W.E, W.K, W.H, W.I, W.fmt, W.S, W.f_q16, lambda f: buf[where[f]],
                           lambda f: tsb[where[f]], use_c=True, nthreads=nthreads)
        t0 = time.perf_counter()
        for t in range(n):
            for l in range(layers):
                eng.decode_layer(l, xs[l][t:t + 1], logits=lg[l][t:t + 1])
        return n * layers / W.L / (time.perf_counter() - t0)

    value = timed(tokens, threads, W.L)
    one = timed(1, 1, layers_1core)
    info = host_cpu()
    ptr = eff.host_alloc(2 << 30)
    try:
        ctypes.memset(ptr, 1, 2 << 30)
        rd = host_read_gbps(ptr, 2 << 30, threads)
    finally:
        eff.host_free(ptr)
    return {"value": round(value, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": "%d token(s) (B = 1) x %d layers of the %s trace from a cold cache (all records the sample "
                      "routes to, generated beforehand); fp64 C evaluator on %d threads plus single-threaded "
                      "NumPy routing and policy" % (tokens, W.L, W.name, threads),
            "value_1core": round(one, 4),
            "sample_1core": "the first %d of the first token's %d layers on 1 thread, scaled to a whole token" % (
                layers_1core, W.L),
            "host_cpu": info, "host_read_GBps": rd,
            "host_read_probe": "NumPy sums over 2 GiB of pinned host memory, %d threads, best of 3" % threads}


# ------------------------------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the headline decode")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps after the cache warm-up")
    ap.add_argument("--kernel-tokens", type=int, default=64, help="decode steps per batch in the kernel passes")
    ap.add_argument("--prefill-layers", type=int, default=6)
    ap.add_argument("--cpu-tokens", type=int, default=1)
    ap.add_argument("--threads", type=int, default=0,
                    help="host executor threads (0: one per physical core, one core left for the enqueuing thread)")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-context", action="store_true",
                    help="skip the 35b-a3b and dsv4-flash end-to-end runs and the headline's context variants")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--counters-pass", action="store_true",
                    help="only run the roofline kernel's workload for rocprofv3 counter passes (no JSON line)")
    ap.add_argument("--counters-prefill", action="store_true",
                    help="only run two prefill layers for rocprofv3 counter passes (no JSON line)")
    ap.add_argument("--counters-shape", choices=("qwen", "dsv4"), default="qwen",
                    help="--counters-pass at the qwen3.8-flash-next shape (B = 16) or the dsv4-flash one (B = 4)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path, and this machine runs one "
              "GPU per job (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import expert_ffn_serving_amd as eff
    import synth
    from synth.configs import A3B, DSV4_DECODE, DSV4_PREFILL, QWEN_NEXT

    eff.lib()   # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    if args.counters_pass:
        if args.counters_shape == "dsv4":
            counters_pass(eff, torch, synth, DSV4_DECODE, B=4, tokens=args.kernel_tokens, threads=args.threads)
        else:
            counters_pass(eff, torch, synth, QWEN_NEXT, B=16, tokens=args.kernel_tokens, threads=args.threads)
        return
    if args.counters_prefill:
        counters_prefill(eff, torch, synth, DSV4_PREFILL, layers=2, threads=args.threads)
        return
    W = QWEN_NEXT
    # the dominant kernel at the headline's shape and batches, every expert resident (first: the
    # headline's speculative link cap takes the expert kernels' time from it)
    log("decode kernels %s (2 layers resident)" % W.name)
    kq = decode_kernel_rates(eff, torch, synth, W, W.batches, args.kernel_tokens, args.threads)
    k16 = kq["B16"]
    compute_us = {B: kq["B%d" % B]["gateup_us"] + kq["B%d" % B]["down_us"] for B in W.batches}
    head_res, (head, dt) = run_headline(eff, torch, synth, W, args.steps, args.warmup, args.threads, compute_us,
                                        skip_variants=args.skip_context)
    srcs = ("k_decode.hip",)
    roofline = {
        "bound": "hbm", "achieved": k16["gateup_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": k16["gateup_frac"], "traffic": traffic_from_profile(TRAFFIC_FILE, srcs),
        "kernel": "k_gateup<NVFP4, 8, 1> (decode gate+up GEMV with SwiGLU, B = 16, one launch per layer call)",
        "workload": "%s expert shape, B = 16, every expert resident (2 layers streamed whole into the slots), "
                    "%d steps x 2 layers of the workload's Zipf(%.1f) trace" % (W.name, args.kernel_tokens, W.zipf_s),
        "algorithmic_bytes_per_launch": k16["gateup_alg_bytes_per_launch"],
        "gpu_experts_per_launch": k16["gpu_experts_per_launch"], "avg_launch_us": k16["gateup_us"],
        "launches": k16["launches"],
        "timed_as": "HIP events that each launch sets at its kernel's start and end (hipExtLaunchKernelGGL), "
                    "on the kernel's stream",
        "source_sha": src_hash(*srcs),
        "down": {"kernel": "k_down<NVFP4, 4, 1, true> (weights kept in registers across token chunks)", "achieved": k16["down_GBps"], "frac": k16["down_frac"],
                 "algorithmic_bytes_per_launch": k16["down_alg_bytes_per_launch"], "avg_launch_us": k16["down_us"]},
    }
    link = {"bound": "pcie", "achieved_GBps": head["link_GBps"],
            "peak_GBps_measured": head_res["bandwidth_profile"]["pcie_GBps_alone"],
            "frac_of_measured": round(head["link_GBps"] / max(1e-9, head_res["bandwidth_profile"]["pcie_GBps_alone"]),
                                      3),
            "MB_per_layer": head["link_MB_per_layer"],
            "note": "the headline step at f = 65535: every miss and every speculative guess crosses PCIe inside "
                    "the layer's expert kernels (speculative records in extra workgroups of the same kernels); "
                    "its rate against the link rate the bandwidth profile measured on this machine"}
    dk = None
    if not args.skip_prefill:
        log("decode kernels %s (2 layers resident)" % DSV4_DECODE.name)
        dk = decode_kernel_rates(eff, torch, synth, DSV4_DECODE, DSV4_DECODE.batches, args.kernel_tokens,
                                 args.threads)
    a3b = ds = None
    if not args.skip_context:
        a3b = run_a3b(eff, torch, synth, A3B, max(args.steps * 8, 128), args.warmup, args.threads)
        log("decode end to end %s, 16 of 43 layers" % DSV4_DECODE.name)
        W3 = DSV4_DECODE
        Ls, Ss = 16, int(DSV4_DECODE.S * 16 / DSV4_DECODE.L)
        pool = fill_pool(eff, synth, W3.seed, Ls, W3.E, W3.H, W3.I, W3.fmt)
        ds = {"workload": "%s, the first 16 of 43 layers, %d slots (20 %% of their experts)" % (W3.name, Ss)}
        for B in W3.batches:
            inputs = decode_inputs(torch, synth, W3, Ls, B, (W3.warmup_tokens + B - 1) // B + args.warmup + args.steps)
            r, _ = e2e_run(eff, torch, W3, pool, inputs, B, W3.f_q16, args.steps, args.warmup, W3.warmup_tokens,
                           L=Ls, S=Ss, threads=args.threads)
            ds["B%d" % B] = r
            log("  B=%d: %.2f tok/s over 16 layers (%.1f us per layer), per layer call %s" % (
                B, r["tok_s"], r["us_per_layer"], r["per_layer_call"]))
            del inputs
        eff.host_free(pool[0])
    pre = None
    ncpu = len(os.sched_getaffinity(0))
    if not args.skip_prefill:
        pre = run_prefill(eff, torch, synth, DSV4_PREFILL, args.prefill_layers, args.threads,
                          0 if args.skip_cpu else 16, ncpu)
        pre["decode_kernels_dsv4_shape"] = dk
    cpu = None
    if not args.skip_cpu:
        t0 = time.time()
        cpu = cpu_baseline(eff, synth, W, args.cpu_tokens, ncpu)
        log("  cpu oracle: %.3f tok/s on %d threads, %.3f tok/s on 1; host reads %.1f GB/s (%.1f s)" % (
            cpu["value"], ncpu, cpu["value_1core"], cpu["host_read_GBps"], time.time() - t0))
    B = 16
    line = {
        "metric": METRIC, "value": head["tok_s"], "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "nvfp4 weights, bf16 activations, fp32 accumulation",
        "data": "synthetic (seeded generator; random-init NVFP4 experts, Zipf(1.2) routing trace)",
        "config": {"workload": W.name, "layers": W.L, "experts": W.E, "top_k": W.K, "hidden": W.H, "inter": W.I,
                   "weights": "nvfp4 (e2m1, e4m3 per 16, fp32 per matrix)", "record_bytes": head_res["record_bytes"],
                   "slots": W.S, "fetch_frac_q16": W.f_q16, "batch": B, "routing": "zipf(%.1f) trace" % W.zipf_s,
                   "speculative_keep": W.spec_keep, "speculative_link_cap_records": head["spec_link_records"],
                   "cache_warmup_tokens": head["cache_warmup_tokens"],
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "link": link,
        "cpu_baseline": cpu,
        "decode_e2e": head_res,
        "decode_kernels": kq,
        "prefill": pre,
        "decode_e2e_35b_a3b": a3b,
        "decode_e2e_dsv4_16_layers": ds,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
