"""Python binding of libeff (routed-expert FFN over an HBM slot cache, MI355X).

Argument marshalling only: every step runs in the HIP library (libeff.so, built
in-tree by ``expert_ffn_serving_amd.build``).  torch is imported first so that
the process has exactly one HIP runtime (torch's), which libeff then binds to.
Device arguments are torch tensors on the GPU; streams are torch.cuda.Stream
objects (or None for the current stream).  Errors raise EffError.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (loads the HIP runtime libeff binds to)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libeff.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "eff.h")

INT4_G32_BF16 = 0
NVFP4_G16_E4M3 = 1
SPECULATIVE = 1
CFG_TIMING = 1
CFG_SYNC_HOST = 2
T_DECODE_GATEUP, T_DECODE_DOWN, T_PREFILL_GATEUP, T_PREFILL_DOWN = 0, 1, 2, 3
HOST_ISA_SCALAR, HOST_ISA_AVX2, HOST_ISA_AVX512F, HOST_ISA_AVX512_BF16 = 0, 1, 2, 3
HOST_ISA_NAMES = {0: "scalar", 1: "avx2+fma", 2: "avx512f", 3: "avx512-bf16"}

EFF_OK, EFF_EINVAL, EFF_ENOMEM, EFF_EHIP, EFF_ECAPTURE, EFF_ESTATE, EFF_EDEVICE = 0, -1, -2, -3, -4, -5, -6
EFF_EREJECTED = -7


class EffError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("libeff error %d: %s" % (code, msg))
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("wformat", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("max_prefill_tokens", ctypes.c_int32), ("fetch_frac_q16", ctypes.c_uint32),
                ("host_threads", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class Stats(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64), ("hits", ctypes.c_int64), ("fetched", ctypes.c_int64),
                ("host", ctypes.c_int64), ("spec_fetched", ctypes.c_int64), ("bytes_fetched", ctypes.c_int64),
                ("qstar_hist", ctypes.c_int64 * 17), ("launches", ctypes.c_int64 * 4),
                ("kernel_ms", ctypes.c_double * 4), ("host_ms", ctypes.c_double), ("wait_ms", ctypes.c_double),
                ("host_calls", ctypes.c_int64), ("launches_nofetch", ctypes.c_int64 * 4),
                ("kernel_ms_nofetch", ctypes.c_double * 4), ("gpu_experts_nofetch", ctypes.c_int64)]


_lib = None
VP, I32, U32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_int64


def lib():
    """Load libeff.so; fails loudly when the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libeff.so is not built (run: python -m expert_ffn_serving_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "eff_last_error": (ctypes.c_char_p, []),
            "eff_record_bytes": (I64, [VP]),
            "eff_create": (I32, [VP, VP, VP, VP]),
            "eff_destroy": (I32, [VP]),
            "eff_host_alloc": (I32, [ctypes.c_size_t, VP]),
            "eff_host_free": (I32, [VP]),
            "eff_route": (I32, [VP, VP, VP, I32, VP, VP, VP]),
            "eff_route_logits": (I32, [VP, VP, I32, VP, VP, VP]),
            "eff_last_logits": (I32, [VP, VP]),
            "eff_ensure_experts": (I32, [VP, I32, VP, I32, U32, VP]),
            "eff_split_misses": (I32, [VP, VP, VP, VP, VP]),
            "eff_qstar": (I64, [I64, U32]),
            "eff_qstar_batch": (I32, [VP, VP, VP, I32, VP]),
            "eff_frac_q16": (U32, [ctypes.c_double, ctypes.c_double]),
            "eff_profile_bandwidth": (I32, [VP, I32, VP]),
            "eff_set_fetch_frac": (I32, [VP, U32]),
            "eff_set_speculation": (I32, [VP, I32, I32]),
            "eff_set_speculation_link": (I32, [VP, I32]),
            "eff_rebuild_cache": (I32, [VP, I32, ctypes.c_uint64]),
            "eff_copy_missing": (I32, [VP, VP, VP]),
            "eff_expert_ffn_decode": (I32, [VP, I32, VP, VP, I32, VP, VP]),
            "eff_expert_ffn_decode_noalloc": (I32, [VP, I32, VP, VP, I32, VP, VP]),
            "eff_host_ffn_decode": (I32, [VP, I32, VP, VP, I32, VP]),
            "eff_combine": (I32, [VP, VP, VP, VP, VP, I32, VP, VP]),
            "eff_decode_layer": (I32, [VP, I32, VP, VP, VP, I32, VP, VP, VP, VP]),
            "eff_last_layer_info": (I32, [VP, VP, VP, VP, VP, VP]),
            "eff_prefill_stream_layer": (I32, [VP, I32, VP]),
            "eff_expert_ffn_prefill_layer": (I32, [VP, I32, VP, VP, VP, I32, VP, VP]),
            "eff_snapshot_tables": (I32, [VP, VP, VP, VP, VP, VP]),
            "eff_get_stats": (I32, [VP, VP]),
            "eff_reset_stats": (I32, [VP]),
            "eff_set_flags": (I32, [VP, U32]),
            "eff_get_host_info": (I32, [VP, VP]),
            "eff_set_host_isa": (I32, [VP, I32]),
            "eff_slot_ptr": (I32, [VP, I32, VP]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def declared_functions():
    """Names of the functions include/eff.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(eff_\w+)\s*\([^;{]*?\)\s*;", text, re.S)))


def _check(rc: int):
    if rc != 0:
        raise EffError(rc, lib().eff_last_error().decode())


def _p(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_hip = None


def _memcpy_d2h(dst: int, src: int, nbytes: int):
    """hipMemcpy device -> host through the HIP runtime torch loaded (the one libeff uses)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemcpy.argtypes = [VP, VP, ctypes.c_size_t, ctypes.c_int]
    rc = _hip.hipMemcpy(dst, src, nbytes, 2)  # hipMemcpyDeviceToHost
    if rc != 0:
        raise EffError(EFF_EHIP, "hipMemcpy failed: %d" % rc)


def qstar(m: int, f: int) -> int:
    return int(lib().eff_qstar(m, f))


def frac_q16(pcie_bytes_per_s: float, host_bytes_per_s: float) -> int:
    """eff_frac_q16: 65536 * B_P / B_H as an integer, capped at 65536 (0xFFFFFFFF: bad input)."""
    return int(lib().eff_frac_q16(pcie_bytes_per_s, host_bytes_per_s))


class HostInfo(ctypes.Structure):
    _fields_ = [("isa", ctypes.c_int32), ("isa_best", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("pinned", ctypes.c_int32), ("physical_cores", ctypes.c_int32), ("pad", ctypes.c_int32)]


class BwProfile(ctypes.Structure):
    _fields_ = [("pcie_alone", ctypes.c_double), ("host_alone", ctypes.c_double),
                ("pcie_concurrent", ctypes.c_double), ("host_concurrent", ctypes.c_double),
                ("frac_q16", ctypes.c_uint32), ("frac_q16_alone", ctypes.c_uint32),
                ("record_bytes", ctypes.c_int64), ("records", ctypes.c_int32), ("pad", ctypes.c_int32)]


def qstar_batch(m, f, q, stream=None):
    _check(lib().eff_qstar_batch(_p(m), _p(f), _p(q), m.numel(), _s(stream)))


def host_alloc(nbytes: int) -> int:
    out = ctypes.c_void_p()
    _check(lib().eff_host_alloc(nbytes, ctypes.byref(out)))
    return out.value


def host_free(ptr: int):
    _check(lib().eff_host_free(ptr))


def make_config(L, E, K, H, I, wformat, S, max_tokens, max_prefill_tokens=0, f_q16=65536, host_threads=0,
                flags=0):
    return Config(L, E, K, H, I, wformat, S, max_tokens, max_prefill_tokens, f_q16, host_threads, flags)


def record_bytes(cfg: Config) -> int:
    return int(lib().eff_record_bytes(ctypes.byref(cfg)))


class Engine:
    """One libeff engine.  host_pool: address of L*E*R bytes of pinned host memory (kept
    alive by the caller); tensor_scales: numpy float32 [L*E*3] or None (int4)."""

    def __init__(self, cfg: Config, host_pool: int, tensor_scales=None):
        self.cfg = cfg
        self._ts = None if tensor_scales is None else tensor_scales.astype("float32").copy()
        h = ctypes.c_void_p()
        _check(lib().eff_create(ctypes.byref(cfg), host_pool,
                                None if self._ts is None else self._ts.ctypes.data, ctypes.byref(h)))
        self.h = h.value

    def close(self):
        if self.h:
            _check(lib().eff_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- decode primitives
    def route(self, x, w_router, ids, w, stream=None):
        _check(lib().eff_route(self.h, _p(x), _p(w_router), x.shape[0], _p(ids), _p(w), _s(stream)))

    def last_logits(self, B: int):
        """Host copy (float32 [B, E]) of the logits the last eff_route computed."""
        import numpy as np
        ptr = ctypes.c_void_p()
        _check(lib().eff_last_logits(self.h, ctypes.byref(ptr)))
        torch.cuda.synchronize()
        out = np.empty((B, self.cfg.num_experts), np.float32)
        _memcpy_d2h(out.ctypes.data, ptr.value, out.nbytes)
        return out

    def route_logits(self, logits, ids, w, stream=None):
        _check(lib().eff_route_logits(self.h, _p(logits), logits.shape[0], _p(ids), _p(w), _s(stream)))

    def ensure_experts(self, layer, ids, flags=0, stream=None):
        _check(lib().eff_ensure_experts(self.h, layer, _p(ids), ids.numel(), flags, _s(stream)))

    def split_misses(self, ids, cpu_ids, counts, stream=None):
        _check(lib().eff_split_misses(self.h, _p(ids), _p(cpu_ids), _p(counts), _s(stream)))

    def copy_missing(self, compute=None, side=None):
        _check(lib().eff_copy_missing(self.h, _s(compute), _s(side) if side is not None else _s(compute)))

    def expert_ffn_decode(self, layer, x, slots, y, stream=None):
        _check(lib().eff_expert_ffn_decode(self.h, layer, _p(x), _p(slots), x.shape[0], _p(y), _s(stream)))

    def expert_ffn_decode_noalloc(self, layer, x, slots, y, stream=None):
        _check(lib().eff_expert_ffn_decode_noalloc(self.h, layer, _p(x), _p(slots), x.shape[0], _p(y), _s(stream)))

    def host_ffn_decode(self, layer, x_host, cpu_ids_host, y_host):
        """numpy arrays: x uint16 [B,H], cpu_ids int32 [B*K], y float32 [B,K,H]."""
        _check(lib().eff_host_ffn_decode(self.h, layer, x_host.ctypes.data, cpu_ids_host.ctypes.data,
                                         x_host.shape[0], y_host.ctypes.data))

    def combine(self, y_gpu, y_host, slots, w, out, stream=None):
        _check(lib().eff_combine(self.h, _p(y_gpu), _p(y_host), _p(slots), _p(w), out.shape[0], _p(out),
                                 _s(stream)))

    def decode_layer(self, layer, x, out, w_router=None, logits=None, spec_ids=None, compute=None, side=None):
        _check(lib().eff_decode_layer(self.h, layer, _p(x), _p(w_router), _p(logits), x.shape[0], _p(spec_ids),
                                      _p(out), _s(compute), _s(side) if side is not None else _s(compute)))

    def last_layer_arrays(self, B: int) -> dict:
        """Host copies of the last eff_decode_layer's ids, slots, host ids (int32 [B*K]) and counts [6]."""
        import numpy as np
        ids, _, slots, cpu, counts = self.last_layer_info()
        n = B * self.cfg.top_k
        torch.cuda.synchronize()
        out = {}
        for name, ptr, cnt in (("ids", ids, n), ("slots", slots, n), ("cpu", cpu, n), ("counts", counts, 6)):
            host = np.empty(cnt, np.int32)
            _memcpy_d2h(host.ctypes.data, ptr, cnt * 4)
            out[name] = host
        return out

    def last_layer_info(self):
        """Device addresses (ids, w, slots, cpu_ids, counts) of the last eff_decode_layer."""
        vals = [ctypes.c_void_p() for _ in range(5)]
        _check(lib().eff_last_layer_info(self.h, *[ctypes.byref(v) for v in vals]))
        return [v.value for v in vals]

    # -- prefill
    def prefill_stream_layer(self, layer, side=None):
        _check(lib().eff_prefill_stream_layer(self.h, layer, _s(side)))

    def expert_ffn_prefill_layer(self, layer, x, ids, w, out, stream=None):
        _check(lib().eff_expert_ffn_prefill_layer(self.h, layer, _p(x), _p(ids), _p(w), x.shape[0], _p(out),
                                                  _s(stream)))

    # -- diagnostics
    def snapshot_tables(self):
        import numpy as np
        c = self.cfg
        table = np.empty(c.num_layers * c.num_experts, np.int32)
        owner = np.empty(max(1, c.num_slots), np.int32)
        usage = np.empty(max(1, c.num_slots), np.int64)
        recency = np.empty(c.num_layers * c.num_experts, np.int64)
        clock = np.empty(2, np.int64)
        _check(lib().eff_snapshot_tables(self.h, table.ctypes.data, owner.ctypes.data, usage.ctypes.data,
                                         recency.ctypes.data, clock.ctypes.data))
        return dict(table=table, owner=owner[:c.num_slots], usage=usage[:c.num_slots], recency=recency,
                    step=int(clock[0]), last_real=int(clock[1]))

    def stats(self) -> dict:
        st = Stats()
        _check(lib().eff_get_stats(self.h, ctypes.byref(st)))
        return dict(calls=st.calls, hits=st.hits, fetched=st.fetched, host=st.host,
                    spec_fetched=st.spec_fetched, bytes_fetched=st.bytes_fetched,
                    qstar_hist=list(st.qstar_hist), launches=list(st.launches), kernel_ms=list(st.kernel_ms),
                    host_ms=st.host_ms, wait_ms=st.wait_ms, host_calls=st.host_calls,
                    launches_nofetch=list(st.launches_nofetch), kernel_ms_nofetch=list(st.kernel_ms_nofetch),
                    gpu_experts_nofetch=st.gpu_experts_nofetch)

    def reset_stats(self):
        _check(lib().eff_reset_stats(self.h))

    def set_flags(self, flags: int):
        _check(lib().eff_set_flags(self.h, flags))
        self.cfg.flags = flags

    def profile_bandwidth(self, records: int) -> dict:
        """eff_profile_bandwidth: link and host expert rates (bytes/s), alone and concurrent, and f."""
        out = BwProfile()
        _check(lib().eff_profile_bandwidth(self.h, records, ctypes.byref(out)))
        return {k: getattr(out, k) for k, _ in BwProfile._fields_ if k != "pad"}

    def set_speculation(self, max_fetch: int = -1, in_gap: bool = False):
        """eff_set_speculation: at most max_fetch records per speculative request (-1: no budget), copied
        right after the control kernel or, with in_gap, after the layer's gate/up kernel."""
        _check(lib().eff_set_speculation(self.h, max_fetch, 1 if in_gap else 0))

    def host_info(self) -> dict:
        """eff_get_host_info: the host executor's instruction set, threads and pinning."""
        out = HostInfo()
        _check(lib().eff_get_host_info(self.h, ctypes.byref(out)))
        return {k: getattr(out, k) for k, _ in HostInfo._fields_ if k != "pad"}

    def set_host_isa(self, isa: int):
        _check(lib().eff_set_host_isa(self.h, isa))

    def set_speculation_link(self, link_records: int):
        """eff_set_speculation_link: speculative fetches limited to the link records a layer leaves (-1: off)."""
        _check(lib().eff_set_speculation_link(self.h, link_records))

    def set_fetch_frac(self, frac_q16: int):
        _check(lib().eff_set_fetch_frac(self.h, frac_q16))
        self.cfg.fetch_frac_q16 = frac_q16

    def rebuild_cache(self, num_slots: int, max_arena_bytes: int = 0):
        """eff_rebuild_cache: the slot cache rebuilt with num_slots slots (EffError with code
        EFF_EREJECTED, and the engine unchanged, when the request does not fit)."""
        _check(lib().eff_rebuild_cache(self.h, num_slots, max_arena_bytes))
        self.cfg.num_slots = num_slots

    def slot_ptr(self, slot: int) -> int:
        out = ctypes.c_void_p()
        _check(lib().eff_slot_ptr(self.h, slot, ctypes.byref(out)))
        return out.value
