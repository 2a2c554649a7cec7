#!/usr/bin/env python3
"""Benchmark of the routed-expert FFN step over an HBM slot cache on one MI355X.

Default workload (one JSON line on stdout, progress on stderr):
  decode, 35B-A3B shape: 40 layers x 256 experts, top-8, hidden 2048, expert
  intermediate 512, int4-g32 weights, 5120 HBM slots (50 %), f = 26214, batch 1,
  Zipf(1.1) routing trace.  A step is one token through all 40 layers: route,
  ensure, split (q*), fetch copies, GPU expert FFN, host share, combine.
  value = tokens/s over `--steps` steps after `--warmup` untimed steps.

Extra fields:
  roofline      the decode expert-FFN kernels (gate/up + down), algorithmic bytes per
                launch over their average duration (HIP events on their stream,
                measured in a separate pass of --profile-steps steps)
  prefill       whole-layer prefill on the DeepSeek-V4-Flash shape (2048 tokens, 256
                experts, top-6, 4096 x 2048 NVFP4); MoE TFLOP/s of the grouped GEMM
  cpu_baseline  the CPU oracle on a bounded sample of the same decode trace
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA
METRIC = "decode expert-FFN tok/s + HBM GB/s (% peak); prefill MoE TFLOP/s (% MFMA)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fill_pool(eff, synth, seed, L, E, H, I, fmt, nthreads):
    import numpy as np
    R = synth.record_bytes(H, I)
    ptr = eff.host_alloc(L * E * R)
    ts = np.empty(L * E * 3, np.float32)
    t0 = time.time()
    synth.fill_records(seed, E, H, I, fmt, 0, L * E, ptr, ts, nthreads)
    log("  pool %.2f GB filled in %.1f s" % (L * E * R / 1e9, time.time() - t0))
    return ptr, ts, R


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "expert_ffn_serving_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_sources, n_launch_units):
    """HBM bytes per launch from committed PMC summaries, when they match the current sources."""
    path = os.path.join(ROOT, "profiles", "decode_ffn_traffic_35b_a3b.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != src_hash(*kernel_sources):
        return None
    return d.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------------------------- decode
def run_decode(eff, torch, synth, W, steps, warmup, profile_steps, threads, use_graph=True):
    import numpy as np
    log("decode %s: L=%d E=%d K=%d H=%d I=%d S=%d f=%d" % (W.name, W.L, W.E, W.K, W.H, W.I, W.S, W.f_q16))
    ptr, ts, R = fill_pool(eff, synth, W.seed, W.L, W.E, W.H, W.I, W.fmt, threads)
    B = W.batches[0]
    cfg = eff.make_config(W.L, W.E, W.K, W.H, W.I, W.fmt, W.S, B, 0, W.f_q16, threads)
    eng = eff.Engine(cfg, ptr, ts if W.fmt == synth.FMT_NVFP4 else None)
    n_tok = warmup + steps * (2 if use_graph else 1) + profile_steps
    t0 = time.time()
    # inputs resident in HBM before timing: x [L, n_tok*B, H] bf16 and trace logits [L, n_tok*B, E]
    X = torch.empty((W.L, n_tok * B, W.H), dtype=torch.int16, device="cuda")
    LG = torch.empty((W.L, n_tok * B, W.E), dtype=torch.float32, device="cuda")
    for l in range(W.L):
        X[l].copy_(torch.from_numpy(synth.activations(W.seed, l, 0, n_tok * B, W.H).view(np.int16)))
        LG[l].copy_(torch.from_numpy(synth.trace_logits(W.seed, l, W.E, W.zipf_s, 0, n_tok * B)))
    out = torch.empty((B, W.H), dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    log("  inputs generated in %.1f s" % (time.time() - t0))
    L_ = eff.lib()
    h = eng.h
    comp, side = torch.cuda.Stream(), torch.cuda.Stream()   # every decode call runs on `comp`
    cs, ss = comp.cuda_stream, side.cuda_stream
    xs, ls = X.stride(1) * 2, LG.stride(1) * 4
    xb, lb = X.data_ptr(), LG.data_ptr()
    xl, ll = X.stride(0) * 2, LG.stride(0) * 4
    op = out.data_ptr()

    def step(t):
        for l in range(W.L):
            rc = L_.eff_decode_layer(h, l, xb + l * xl + t * B * xs, None, lb + l * ll + t * B * ls, B, None, op,
                                     cs, ss)
            if rc:
                raise eff.EffError(rc, L_.eff_last_error().decode())

    t0 = time.time()
    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    log("  warmup %d steps in %.1f s" % (warmup, time.time() - t0))
    eng.reset_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        step(t)
    torch.cuda.synchronize()
    dt_eager = time.perf_counter() - t0
    st = eng.stats()
    calls = W.L * steps
    log("  timed %d steps (eager calls): %.3f s -> %.1f tok/s; per layer-call hit %.2f fetch %.2f host %.2f" % (
        steps, dt_eager, steps * B / dt_eager, st["hits"] / calls, st["fetched"] / calls, st["host"] / calls))
    dt_graph, t_next = None, warmup + steps
    if use_graph:
        # the decode step (all layers) captured once as a HIP graph on fixed input rows; each token's x
        # and logits rows are copied in (two device copies) and the graph replayed
        gx = torch.empty((W.L, B, W.H), dtype=torch.int16, device="cuda")
        gl = torch.empty((W.L, B, W.E), dtype=torch.float32, device="cuda")
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=comp):
            for l in range(W.L):
                rc = L_.eff_decode_layer(h, l, gx[l].data_ptr(), None, gl[l].data_ptr(), B, None, op, cs, ss)
                if rc:
                    raise eff.EffError(rc, L_.eff_last_error().decode())

        def gstep(t):
            with torch.cuda.stream(comp):
                gx.copy_(X[:, t * B:(t + 1) * B])
                gl.copy_(LG[:, t * B:(t + 1) * B])
                graph.replay()

        eng.reset_stats()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(t_next, t_next + steps):
            gstep(t)
        torch.cuda.synchronize()
        dt_graph = time.perf_counter() - t0
        t_next += steps
        sg = eng.stats()
        log("  timed %d steps (graph replay): %.3f s -> %.1f tok/s; per layer-call hit %.2f fetch %.2f host %.2f" % (
            steps, dt_graph, steps * B / dt_graph, sg["hits"] / calls, sg["fetched"] / calls, sg["host"] / calls))
    # `value` is the eager window: replaying the 160-kernel step as a graph measured a few percent slower
    # on this runtime (per-node dispatch), so the graph rate is reported beside it
    dt = dt_eager
    # profiled pass: the same path with the expert kernels bracketed by HIP events
    eng.reset_stats()
    eng.set_flags(eff.CFG_TIMING)
    for t in range(t_next, t_next + profile_steps):
        step(t)
    torch.cuda.synchronize()
    sp = eng.stats()
    eng.set_flags(0)
    n_launch = sp["launches"][eff.T_DECODE_GATEUP]
    g_ms, d_ms = sp["kernel_ms"][eff.T_DECODE_GATEUP], sp["kernel_ms"][eff.T_DECODE_DOWN]
    gpu_unique = sp["hits"] + sp["fetched"]               # distinct GPU experts over the pass (= entries, B = 1)
    mat_bytes = W.H * W.I // 2 + W.H * W.I // 16           # one matrix: payload + scales
    # algorithmic bytes of k_gateup: gate and up of every GPU expert once, x read, SwiGLU output written
    # (fp16 values plus one 8-byte scale/sum pair per 8 of them: 3 bytes per activation)
    def gu_alg(units, launches):
        return units * 2 * mat_bytes + launches * B * W.H * 2 + units * W.I * 3

    # k_down: down of every GPU expert once, SwiGLU output read, y written (fp32)
    def dn_alg(units):
        return units * mat_bytes + units * W.I * 3 + units * W.H * 4

    gu_bytes, dn_bytes = gu_alg(gpu_unique, n_launch), dn_alg(gpu_unique)
    gu_gbps = gu_bytes / (g_ms * 1e-3) / 1e9 if g_ms > 0 else 0.0
    dn_gbps = dn_bytes / (d_ms * 1e-3) / 1e9 if d_ms > 0 else 0.0
    src = ("k_decode.hip",)
    traffic = traffic_from_profile(src, n_launch)
    roofline = {
        "bound": "hbm", "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(gu_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
        "kernel": "k_gateup (decode gate+up GEMV with SwiGLU, one launch per layer)",
        "algorithmic_bytes_per_launch": int(gu_bytes / max(1, n_launch)),
        "avg_launch_us": round(g_ms * 1e3 / max(1, n_launch), 2),
        "gpu_experts_per_launch": round(gpu_unique / max(1, n_launch), 3),
        "launches": n_launch, "source_sha": src_hash(*src),
        "down": {"kernel": "k_down", "achieved": round(dn_gbps, 1), "frac": round(dn_gbps / HBM_PEAK_GBPS, 4),
                 "algorithmic_bytes_per_launch": int(dn_bytes / max(1, n_launch)),
                 "avg_launch_us": round(d_ms * 1e3 / max(1, n_launch), 2)},
    }
    # the same kernels on the calls that fetched nothing: HBM reads only, no wait on the host link
    nf = sp["launches_nofetch"][eff.T_DECODE_GATEUP]
    if nf > 0:
        g_nf, d_nf = sp["kernel_ms_nofetch"][eff.T_DECODE_GATEUP], sp["kernel_ms_nofetch"][eff.T_DECODE_DOWN]
        u_nf = sp["gpu_experts_nofetch"]
        gnf_gbps = gu_alg(u_nf, nf) / (g_nf * 1e-3) / 1e9
        dnf_gbps = dn_alg(u_nf) / (d_nf * 1e-3) / 1e9
        roofline["nofetch_launches"] = {
            "share_of_launches": round(nf / max(1, n_launch), 3), "gpu_experts_per_launch": round(u_nf / nf, 3),
            "gateup": {"avg_launch_us": round(g_nf * 1e3 / nf, 2), "achieved": round(gnf_gbps, 1),
                       "frac": round(gnf_gbps / HBM_PEAK_GBPS, 4)},
            "down": {"avg_launch_us": round(d_nf * 1e3 / nf, 2), "achieved": round(dnf_gbps, 1),
                     "frac": round(dnf_gbps / HBM_PEAK_GBPS, 4)}}
    kernel_tok_s = profile_steps * B / ((g_ms + d_ms) * 1e-3) if g_ms + d_ms > 0 else 0.0
    detail = {
        "per_layer_call": {k: round(st[k] / calls, 3) for k in ("hits", "fetched", "host")},
        "host_executor_us_per_layer": round(st["host_ms"] * 1e3 / calls, 2),
        "control_wait_us_per_layer": round(st["wait_ms"] * 1e3 / calls, 2),
        "layers_with_host_share": round(st["host_calls"] / calls, 3),
        "bytes_fetched_per_token": int(st["bytes_fetched"] / steps),
        "kernel_only_tok_s": round(kernel_tok_s, 1),
        "profile_steps": profile_steps,
        "timed_as": "eager calls on one stream (no host synchronization)",
        "graph_replay_tok_s": round(steps * B / dt_graph, 2) if dt_graph else None,
    }
    # the fetch fraction this machine would give ([FT-deep] §4 ②): link and host expert rates, run
    # at the same time; the timed run keeps the workload's f
    bw = eng.profile_bandwidth(512)
    detail["bandwidth_profile"] = {
        "records": bw["records"], "record_bytes": bw["record_bytes"],
        "pcie_GBps_concurrent": round(bw["pcie_concurrent"] / 1e9, 2),
        "host_GBps_concurrent": round(bw["host_concurrent"] / 1e9, 2),
        "pcie_GBps_alone": round(bw["pcie_alone"] / 1e9, 2), "host_GBps_alone": round(bw["host_alone"] / 1e9, 2),
        "frac_q16": bw["frac_q16"], "frac_q16_alone": bw["frac_q16_alone"], "frac_q16_workload": W.f_q16}
    log("  bandwidth profile: link %.1f GB/s, host %.1f GB/s at once (alone %.1f / %.1f) -> f = %d (workload: %d)" % (
        bw["pcie_concurrent"] / 1e9, bw["host_concurrent"] / 1e9, bw["pcie_alone"] / 1e9, bw["host_alone"] / 1e9,
        bw["frac_q16"], W.f_q16))
    eng.close()
    # context only: the same timed steps at the profiled f, from an empty cache after the same warm-up
    cfg2 = eff.make_config(W.L, W.E, W.K, W.H, W.I, W.fmt, W.S, B, 0, bw["frac_q16"], threads)
    eng2 = eff.Engine(cfg2, ptr, ts if W.fmt == synth.FMT_NVFP4 else None)
    h = eng2.h   # step() calls through h
    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        step(t)
    torch.cuda.synchronize()
    dt2 = time.perf_counter() - t0
    st2 = eng2.stats()
    eng2.close()
    detail["bandwidth_profile"]["tok_s_at_profiled_f"] = round(steps * B / dt2, 2)
    detail["bandwidth_profile"]["host_share_of_misses_at_profiled_f"] = round(
        st2["host"] / max(1, st2["host"] + st2["fetched"]), 3)
    log("  at the profiled f: %.1f tok/s (workload f: %.1f)" % (steps * B / dt2, steps * B / dt))
    del X, LG
    return dict(value=steps * B / dt, ms=dt * 1e3 / steps, roofline=roofline, detail=detail,
                pool=(ptr, ts, R), B=B)


# ------------------------------------------------------------------------------------- prefill
def run_prefill(eff, torch, synth, W, layers, threads, cpu_tokens=0, cpu_threads=1, decode_kernels=True):
    import numpy as np
    T = W.prefill_T
    log("prefill %s: T=%d E=%d K=%d H=%d I=%d (%d layers streamed)" % (W.name, T, W.E, W.K, W.H, W.I, layers))
    ptr, ts, R = fill_pool(eff, synth, W.seed, layers, W.E, W.H, W.I, W.fmt, threads)
    # the decode kernels at this expert shape first, on a fresh engine
    dk = decode_kernel_rates(eff, torch, synth, W, (ptr, ts, R), layers, threads) if decode_kernels else None
    cfg = eff.make_config(layers, W.E, W.K, W.H, W.I, W.fmt, W.S, 1, T, W.f_q16, threads, eff.CFG_TIMING)
    eng = eff.Engine(cfg, ptr, ts)
    X = [torch.from_numpy(synth.activations(W.seed, l, 0, T, W.H, tag=synth.TAG_PREFILL_X).view(np.int16)).cuda()
         for l in range(layers)]
    WR = [torch.from_numpy(synth.router_weights(W.seed, l, W.E, W.H).view(np.int16)).cuda() for l in range(layers)]
    ids = torch.empty((T, W.K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, W.K), dtype=torch.float32, device="cuda")
    out = torch.empty((T, W.H), dtype=torch.int16, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    eng.reset_stats()
    t0 = time.perf_counter()
    eng.prefill_stream_layer(0, side)
    for l in range(layers):
        if l + 1 < layers:
            eng.prefill_stream_layer(l + 1, side)
        eng.route(X[l], WR[l], ids, w)
        eng.expert_ffn_prefill_layer(l, X[l], ids, w, out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
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
        "stream_GBps": round(wbytes * layers / wall / 1e9, 1),
        "source_sha": src_hash("k_prefill.hip"),
    }
    log("  prefill: %.1f TFLOP/s (%.1f%% of MFMA peak), weights %.0f GB/s (%.1f%% of HBM peak), GEMM %.3f ms/layer, "
        "wall %.1f ms/layer" % (tflops, 100 * tflops / MFMA_PEAK_TFLOPS, wbytes * n / ((g_ms + d_ms) * 1e-3) / 1e9,
                                100 * wbytes * n / ((g_ms + d_ms) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                (g_ms + d_ms) / max(1, n), wall * 1e3 / layers))
    eng.close()
    if decode_kernels:
        res["decode_kernels"] = dk
    if cpu_tokens > 0:
        res["cpu_oracle"] = prefill_oracle(synth, W, (ptr, ts, R), cpu_tokens, cpu_threads)
        log("  prefill cpu oracle: %.1f GFLOP/s (%s)" % (res["cpu_oracle"]["value"], res["cpu_oracle"]["sample"]))
    eff.host_free(ptr)
    return res


# ---------------------------------------------------------------------- decode kernels at a large shape
def decode_kernel_rates(eff, torch, synth, W, pool, layers, threads, batches=(1, 4), tokens=64, zipf=1.0,
                        label="dsv4"):
    """HBM rates of the decode expert kernels at a workload's expert shape (e.g. the DeepSeek-V4-Flash
    4096 x 2048 NVFP4 experts, tens of MB per layer): layers 0 and 1 of the pool streamed whole into the
    two slot buffers (S = 2E, every expert resident, no call misses), then `tokens` profiled decode steps
    per batch size on Zipf trace logits, alternating the two layers."""
    import numpy as np
    ptr, ts, R = pool
    E, K, H, I = W.E, W.K, W.H, W.I
    cfg = eff.make_config(layers, E, K, H, I, W.fmt, 2 * E, max(batches), 0, 65536, threads)
    eng = eff.Engine(cfg, ptr, ts)
    comp, side = torch.cuda.Stream(), torch.cuda.Stream()
    x = torch.from_numpy(synth.activations(W.seed, 0, 0, max(batches), H).view(np.int16)).cuda()
    out = torch.empty((max(batches), H), dtype=torch.int16, device="cuda")
    eng.prefill_stream_layer(0, side)
    eng.prefill_stream_layer(1, side)
    torch.cuda.synchronize()
    layers = 2
    mat_bytes = H * I // 2 + H * I // 16
    res = {"workload": "%s expert shape (H=%d I=%d E=%d K=%d NVFP4), 2 layers, every expert resident" % (
        W.name, H, I, E, K), "tokens": tokens, "zipf": zipf}
    for B in batches:
        LG = [torch.from_numpy(synth.trace_logits(W.seed, l, E, zipf, 0, tokens * B)).cuda() for l in range(layers)]
        eng.reset_stats()
        eng.set_flags(eff.CFG_TIMING)
        with torch.cuda.stream(comp):
            for t in range(tokens):
                for l in range(layers):
                    eng.decode_layer(l, x[:B], out[:B], logits=LG[l][t * B:(t + 1) * B], compute=comp, side=side)
        torch.cuda.synchronize()
        st = eng.stats()
        eng.set_flags(0)
        n = st["launches"][eff.T_DECODE_GATEUP]
        g_ms, d_ms = st["kernel_ms"][eff.T_DECODE_GATEUP], st["kernel_ms"][eff.T_DECODE_DOWN]
        U = st["hits"] + st["fetched"]
        gu = U * 2 * mat_bytes + n * B * H * 2 + U * B * I * 3   # upper bound on the small terms
        dn = U * mat_bytes + U * B * (I * 3 + H * 4)
        res["B%d" % B] = {
            "gpu_experts_per_launch": round(U / max(1, n), 2), "fetched": st["fetched"],
            "gateup_us": round(g_ms * 1e3 / max(1, n), 2), "gateup_GBps": round(gu / (g_ms * 1e-3) / 1e9, 1),
            "gateup_frac": round(gu / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "down_us": round(d_ms * 1e3 / max(1, n), 2), "down_GBps": round(dn / (d_ms * 1e-3) / 1e9, 1),
            "down_frac": round(dn / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        log("  decode kernels at the %s shape, B=%d: %.1f experts/launch, gate/up %.1f us (%.0f GB/s), "
            "down %.1f us (%.0f GB/s), fetched %d" % (label, B, U / max(1, n), g_ms * 1e3 / max(1, n),
                                                       gu / (g_ms * 1e-3) / 1e9, d_ms * 1e3 / max(1, n),
                                                       dn / (d_ms * 1e-3) / 1e9, st["fetched"]))
    eng.close()
    return res


def decode_e2e(eff, torch, synth, W, threads, warm=48, timed=16, layers=None, slots=None):
    """End-to-end decode over a workload's whole pool (every layer, its slot count) with speculative
    next-layer requests, for each batch size in W.batches: `warm` untimed then `timed` timed steps of all
    W.L layers, each from an empty cache.  Run at the workload's fetch fraction and at the one the
    bandwidth profile gives on this machine ([FT-deep] §4 ②), which sends part of the misses to the host
    executor and fetches fewer of the speculative ones; each with speculative copies as requested, with at
    most two per request copied after the gate/up kernel ([NVMe-8GB] "엔진" item 3), and with none.  Reports tok/s and the per-layer-call policy counts;
    the link bytes are the demand and speculative fetches times the record size.  `layers` and `slots`
    run the first `layers` layers of the pool with `slots` slots instead (a pool too large to pin)."""
    import numpy as np
    L = layers or W.L
    S = slots or W.S
    spec_on = W.spec_keep >= 0
    ptr, ts, R = fill_pool(eff, synth, W.seed, L, W.E, W.H, W.I, W.fmt, 16)
    res = {"workload": "%s (L=%d E=%d K=%d H=%d I=%d NVFP4, S=%d%s)" % (
        W.name, L, W.E, W.K, W.H, W.I, S, ", speculative keep %.2f" % W.spec_keep if spec_on else ""),
        "warmup": warm, "steps": timed, "record_bytes": R}
    side = torch.cuda.Stream()
    cfg = eff.make_config(L, W.E, W.K, W.H, W.I, W.fmt, S, max(W.batches), 0, W.f_q16, threads)
    eng = eff.Engine(cfg, ptr, ts)
    bw = eng.profile_bandwidth(256)
    eng.close()
    res["profiled_f"] = {"frac_q16": bw["frac_q16"], "pcie_GBps_concurrent": round(bw["pcie_concurrent"] / 1e9, 2),
                         "host_GBps_concurrent": round(bw["host_concurrent"] / 1e9, 2)}
    log("  bandwidth profile at this record size: link %.1f GB/s, host %.1f GB/s -> f = %d" % (
        bw["pcie_concurrent"] / 1e9, bw["host_concurrent"] / 1e9, bw["frac_q16"]))
    for B in W.batches:
        n_rows = (warm + timed) * B
        X = [torch.from_numpy(synth.activations(W.seed, l, 0, n_rows, W.H).view(np.int16)).cuda() for l in range(L)]
        lg_host = [synth.trace_logits(W.seed, l, W.E, W.zipf_s, 0, n_rows) for l in range(L)]
        LG = [torch.from_numpy(a).cuda() for a in lg_host]
        SP = []
        for l in range(L - 1 if spec_on else 0):   # predictions of layer l+1's sets, made at layer l
            truth = synth.gumbel_topk_sets(lg_host[l + 1], W.K)
            SP.append(torch.from_numpy(np.stack([synth.spec_ids(W.seed, l + 1, W.E, W.zipf_s, r, truth[r], W.spec_keep)
                                                 for r in range(n_rows)]).astype(np.int32).reshape(-1)).cuda())
        out = torch.empty((B, W.H), dtype=torch.int16, device="cuda")
        fp = bw["frac_q16"]
        variants = ((("workload_f", W.f_q16, -1, False), ("workload_f_gap2", W.f_q16, 2, True),
                     ("workload_f_nospec", W.f_q16, 0, False), ("profiled_f", fp, -1, False),
                     ("profiled_f_gap2", fp, 2, True), ("profiled_f_nospec", fp, 0, False)) if spec_on else
                    (("workload_f", W.f_q16, -1, False), ("profiled_f", fp, -1, False)))
        for tag, f, budget, gap in variants:
            cfg = eff.make_config(L, W.E, W.K, W.H, W.I, W.fmt, S, B, 0, f, threads)
            eng = eff.Engine(cfg, ptr, ts)
            eng.set_speculation(budget, gap)

            def run(t0, t1):
                for t in range(t0, t1):
                    r = slice(t * B, (t + 1) * B)
                    for l in range(L):
                        eng.decode_layer(l, X[l][r], out, logits=LG[l][r], side=side,
                                         spec_ids=SP[l][t * B * W.K:(t + 1) * B * W.K] if spec_on and l + 1 < L
                                         else None)
            run(0, warm)
            torch.cuda.synchronize()
            s0 = eng.stats()
            t0 = time.perf_counter()
            run(warm, warm + timed)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            s1 = eng.stats()
            eng.close()
            n = timed * L
            per = {k: round((s1[k] - s0[k]) / n, 2) for k in ("hits", "fetched", "host", "spec_fetched")}
            link = (per["fetched"] + per["spec_fetched"]) * R
            res.setdefault("B%d" % B, {})[tag] = {
                "frac_q16": f, "spec_budget": budget, "spec_in_gap": gap, "tok_s": round(timed * B / dt, 2), "ms_per_step": round(dt * 1e3 / timed, 3),
                "us_per_layer": round(dt * 1e6 / n, 1), "per_layer_call": per,
                "link_MB_per_layer": round(link / 1e6, 1), "link_GBps": round(link / (dt / n) / 1e9, 1)}
            log("  %s end to end, B=%d, %s (f=%d): %.1f tok/s (%.1f us per layer), per layer call %s, %.0f MB "
                "over the link per layer (%.1f GB/s)" % (W.name, B, tag, f, timed * B / dt, dt * 1e6 / n, per,
                                                        link / 1e6, link / (dt / n) / 1e9))
        del X, LG, SP
    eff.host_free(ptr)
    return res


# ------------------------------------------------------------------------------------- CPU oracle
def host_cpu():
    """CPU model and the cores this process may run on."""
    model = "?"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


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

def cpu_baseline(synth, W, pool, tokens, threads, tokens_1core=1):
    """The oracle as it stands, on `tokens` decode steps of the same trace (cold cache), on `threads`
    threads, and on one thread over the first `tokens_1core` steps."""
    import ctypes

    import numpy as np

    from oracle.engine import OracleEngine
    ptr, ts, R = pool

    def rec(flat):
        return np.frombuffer((ctypes.c_uint8 * R).from_address(ptr + flat * R), np.uint8)

    lg = [synth.trace_logits(W.seed, l, W.E, W.zipf_s, 0, tokens) for l in range(W.L)]
    xs = [synth.activations(W.seed, l, 0, tokens, W.H) for l in range(W.L)]

    def timed(n, nthreads):
        eng = OracleEngine(W.L, W.E, W.K, W.H, W.I, W.fmt, W.S, W.f_q16, rec, lambda f: ts[3 * f:3 * f + 3],
                           use_c=True, nthreads=nthreads)
        t0 = time.perf_counter()
        for t in range(n):
            for l in range(W.L):
                eng.decode_layer(l, xs[l][t:t + 1], logits=lg[l][t:t + 1])
        return n / (time.perf_counter() - t0)

    value = timed(tokens, threads)
    one = timed(tokens_1core, 1)
    model, avail = host_cpu()
    return {"value": round(value, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": "%d tokens x %d layers of the %s trace from a cold cache; fp64 C evaluator on %d threads "
                      "plus single-threaded NumPy routing/policy" % (tokens, W.L, W.name, threads),
            "value_1core": round(one, 3),
            "sample_1core": "the first %d token(s) of the same sample on 1 thread" % tokens_1core,
            "host_cpu": model, "host_cores_available": avail,
            "host_read_GBps": host_read_gbps(ptr, 2 << 30, threads),
            "host_read_probe": "NumPy sums over 2 GiB of the pinned expert pool, %d threads, best of 3" % threads}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=1024)
    ap.add_argument("--profile-steps", type=int, default=64)
    ap.add_argument("--prefill-layers", type=int, default=4)
    ap.add_argument("--cpu-tokens", type=int, default=4)
    # host-share pool: 11 workers + the engine's worker thread, which leaves cores of a 16-core host for
    # the enqueuing thread and the runtime (on 16 cores: 15 threads gave 430-446 tok/s, 12 gave 476-478)
    ap.add_argument("--threads", type=int, default=12)
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-qwen-next-kernels", action="store_true",
                    help="skip the decode kernels at the qwen3.8-flash-next expert shape (B = 1, 8, 16)")
    ap.add_argument("--qwen-next-e2e", action="store_true",
                    help="also run the qwen3.8-flash-next decode end to end over its whole pool (about 70 GB of "
                         "pinned host memory, B = 1, 8, 16)")
    ap.add_argument("--dsv4-e2e", action="store_true",
                    help="also run the dsv4-flash decode end to end on 16 of its 43 layers (58 GB pinned; the whole "
                         "pool does not pin) with the slots scaled to its 20 %%, B = 1 and 4")
    ap.add_argument("--no-graph", action="store_true", help="time eager decode calls only (no HIP graph)")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="first copy this many GiB device to device with torch (a plain copy kernel of known size, "
                         "the reference for HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch

    import expert_ffn_serving_amd as eff
    import synth
    from synth.configs import A3B, DSV4_DECODE, DSV4_PREFILL, QWEN_NEXT

    eff.lib()   # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    if args.calibrate_copy_gib > 0:
        n = int(args.calibrate_copy_gib * (1 << 30)) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("  copy calibration: %d bytes device to device" % (n * 4))
        del a, b
    dec = run_decode(eff, torch, synth, A3B, args.steps, args.warmup, args.profile_steps, args.threads,
                     not args.no_graph)
    cpu = None
    ncpu = len(os.sched_getaffinity(0))
    if not args.skip_cpu:
        t0 = time.time()
        cpu = cpu_baseline(synth, A3B, dec["pool"], args.cpu_tokens, ncpu)
        log("  cpu oracle: %.3f tok/s on %d threads, %.3f tok/s on 1; host reads %.1f GB/s (%.1f s)" % (
            cpu["value"], ncpu, cpu["value_1core"], cpu["host_read_GBps"], time.time() - t0))
    eff.host_free(dec["pool"][0])
    pre = None
    if not args.skip_prefill:
        pre = run_prefill(eff, torch, synth, DSV4_PREFILL, args.prefill_layers, args.threads,
                          0 if args.skip_cpu else 16, ncpu)
    qn = None
    if not args.skip_qwen_next_kernels:   # the decode kernels at the third decode workload's expert shape
        W = QWEN_NEXT
        log("decode kernels %s: E=%d K=%d H=%d I=%d (2 layers resident)" % (W.name, W.E, W.K, W.H, W.I))
        pool = fill_pool(eff, synth, W.seed, 2, W.E, W.H, W.I, W.fmt, args.threads)
        qn = decode_kernel_rates(eff, torch, synth, W, pool, 2, args.threads, batches=W.batches, zipf=W.zipf_s,
                                 label="qwen3.8-flash-next")
        eff.host_free(pool[0])
    qe = None
    if args.qwen_next_e2e:
        log("decode end to end %s" % QWEN_NEXT.name)
        qe = decode_e2e(eff, torch, synth, QWEN_NEXT, args.threads)
    de = None
    if args.dsv4_e2e:
        log("decode end to end %s (16 layers)" % DSV4_DECODE.name)
        de = decode_e2e(eff, torch, synth, DSV4_DECODE, args.threads, layers=16,
                        slots=int(DSV4_DECODE.S * 16 / DSV4_DECODE.L))
    line = {
        "metric": METRIC, "value": round(dec["value"], 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dec["ms"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded generator; random-init int4 experts)",
        "config": {"workload": A3B.name, "layers": A3B.L, "experts": A3B.E, "top_k": A3B.K, "hidden": A3B.H,
                   "inter": A3B.I, "weights": "int4-g32-bf16", "slots": A3B.S, "fetch_frac_q16": A3B.f_q16,
                   "batch": dec["B"], "routing": "zipf(%.1f) trace" % A3B.zipf_s, "parallelism": "single-gpu"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_detail": dec["detail"],
        "prefill": pre,
        "decode_kernels_qwen_next": qn,
        "decode_e2e_qwen_next": qe,
        "decode_e2e_dsv4_16_layers": de,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
