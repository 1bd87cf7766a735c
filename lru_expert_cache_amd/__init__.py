"""Python binding of libftmoe.so, the offloaded MoE layer for MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch is used by callers for device memory and streams; this module accepts
raw device pointers or tensors (their .data_ptr()).  The functions keep the
names of the C ABI in include/ftmoe.h.  If the library has not been built the
import of `lib()` fails loudly -- there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libftmoe.so")

FT_OK = 0
FT_WARN_STAGING_SMALL = 1
FT_E_INVALID = -1
FT_E_OOM_DEVICE = -2
FT_E_OOM_PINNED = -3
FT_E_HIP = -4
FT_E_STATE = -5

FT_FMT_MXFP4, FT_FMT_NVFP4, FT_FMT_FP8_B128 = 1, 2, 3
FT_FWD_DECODE, FT_FWD_PREFILL_STAGED = 0, 1
FT_FWD_PREFILL_HIT_D2D = 1 << 8
FT_ACT_BF16, FT_ACT_MXFP8, FT_ACT_MXFP4 = 0 << 4, 1 << 4, 2 << 4
FT_PAIR_HIT, FT_PAIR_MISS_STREAM, FT_PAIR_MISS_CPU = 0, 1, 2

FT_STAGES = ["router", "topk", "resolve", "ffn_gateup", "ffn_down", "combine", "copy", "act_quant", "host_ffn"]

EXPORTED = ["ft_moe_init_pool", "ft_moe_layer_forward", "ft_moe_pool_stats", "ft_moe_last_misses",
            "ft_moe_pool_table", "ft_moe_set_hybrid_share", "ft_moe_host_expert_rate",
            "ft_moe_set_profiling", "ft_moe_profile_read", "ft_moe_destroy_pool", "ft_moe_last_error",
            "ft_moe_reserve", "ft_moe_resize_pool", "ft_moe_decide_mode", "ft_moe_measure_mode",
            "ft_moe_ffn_kernel_name", "ft_moe_mfma_rate", "ft_moe_layer_forward_noalloc",
            "ft_moe_set_hybrid_share_format", "ft_moe_get_hybrid_share", "ft_moe_rebalance",
            "ft_moe_debug_read"]
FT_DBG_H_CODES, FT_DBG_H_SCALES, FT_DBG_ROW_SLOT = 0, 1, 2

FT_MODE_OFFLOAD, FT_MODE_HYBRID, FT_MODE_FUSED = 0, 1, 2


class ft_moe_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("has_shared_expert", ctypes.c_int32), ("layer_fmt", ctypes.POINTER(ctypes.c_int32)),
                ("pool_slots", ctypes.c_int64), ("pool_bytes", ctypes.c_int64),
                ("hybrid_cpu_share", ctypes.c_double), ("cpu_threads", ctypes.c_int32),
                ("device", ctypes.c_int32)]


class ft_moe_weights(ctypes.Structure):
    _fields_ = [("expert", ctypes.POINTER(ctypes.c_void_p)), ("shared", ctypes.POINTER(ctypes.c_void_p)),
                ("router_w", ctypes.c_void_p)]


class ft_moe_trace(ctypes.Structure):
    _fields_ = [("sel", ctypes.c_void_p), ("w", ctypes.c_void_p), ("slot", ctypes.c_void_p),
                ("flag", ctypes.c_void_p), ("row", ctypes.c_void_p)]


class ft_moe_stats(ctypes.Structure):
    _fields_ = [("pair_hits", ctypes.c_uint64), ("pair_misses", ctypes.c_uint64),
                ("expert_hits", ctypes.c_uint64), ("expert_misses", ctypes.c_uint64),
                ("cpu_misses", ctypes.c_uint64), ("evictions", ctypes.c_uint64),
                ("bytes_h2d", ctypes.c_uint64), ("calls", ctypes.c_uint64),
                ("slots_used", ctypes.c_int64), ("slots_total", ctypes.c_int64),
                ("min_topk_gap", ctypes.c_double), ("copy_ms", ctypes.c_double)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class ft_moe_mode_report(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("layers", ctypes.c_int32 * 4), ("expert_bytes", ctypes.c_double * 4),
                ("h2d_bytes_per_s", ctypes.c_double * 4), ("gpu_bytes_per_s", ctypes.c_double * 4),
                ("cpu_bytes_per_s", ctypes.c_double * 4), ("pool_slots", ctypes.c_int64),
                ("all_experts", ctypes.c_int64), ("t_stream", ctypes.c_double), ("t_cpu", ctypes.c_double),
                ("mode", ctypes.c_int32), ("share", ctypes.c_double), ("balanced_share", ctypes.c_double)]

    def as_dict(self):
        d = {}
        for n, _ in self._fields_:
            v = getattr(self, n)
            d[n] = list(v) if isinstance(v, ctypes.Array) else v
        return d


class ft_moe_rebalance_report(ctypes.Structure):
    _fields_ = [("host_bytes", ctypes.c_double * 4), ("host_seconds", ctypes.c_double * 4),
                ("copy_bytes", ctypes.c_double * 4), ("copy_seconds", ctypes.c_double * 4),
                ("gpu_bytes_per_s", ctypes.c_double * 4), ("share", ctypes.c_double * 4),
                ("changed", ctypes.c_int32 * 4)]

    as_dict = ft_moe_mode_report.as_dict


class ft_moe_profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * len(FT_STAGES)), ("bytes", ctypes.c_double * len(FT_STAGES)),
                ("flops", ctypes.c_double * len(FT_STAGES)), ("launches", ctypes.c_uint64 * len(FT_STAGES))]

    def as_dict(self):
        return {st: dict(ms=self.ms[i], bytes=self.bytes[i], flops=self.flops[i], launches=self.launches[i])
                for i, st in enumerate(FT_STAGES)}


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libftmoe.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m lru_expert_cache_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    L.ft_moe_init_pool.argtypes = [ctypes.POINTER(ft_moe_config), ctypes.POINTER(ft_moe_weights), ctypes.POINTER(P)]
    L.ft_moe_init_pool.restype = ctypes.c_int
    L.ft_moe_layer_forward.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_int32, P,
                                       ctypes.POINTER(ft_moe_trace)]
    L.ft_moe_layer_forward.restype = ctypes.c_int
    L.ft_moe_layer_forward_noalloc.argtypes = L.ft_moe_layer_forward.argtypes
    L.ft_moe_layer_forward_noalloc.restype = ctypes.c_int
    L.ft_moe_pool_stats.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ft_moe_stats), ctypes.c_int32]
    L.ft_moe_pool_stats.restype = ctypes.c_int
    I32P = ctypes.POINTER(ctypes.c_int32)
    L.ft_moe_last_misses.argtypes = [P, I32P, I32P, I32P, I32P, I32P, ctypes.c_int32]
    L.ft_moe_last_misses.restype = ctypes.c_int
    L.ft_moe_pool_table.argtypes = [P, I32P, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64),
                                    ctypes.POINTER(ctypes.c_int64)]
    L.ft_moe_pool_table.restype = ctypes.c_int
    L.ft_moe_ffn_kernel_name.argtypes = [ctypes.c_int32]
    L.ft_moe_ffn_kernel_name.restype = ctypes.c_char_p
    L.ft_moe_decide_mode.argtypes = [ctypes.POINTER(ft_moe_mode_report)]
    L.ft_moe_decide_mode.restype = ctypes.c_int
    L.ft_moe_measure_mode.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ft_moe_mode_report)]
    L.ft_moe_measure_mode.restype = ctypes.c_int
    L.ft_moe_resize_pool.argtypes = [P, ctypes.c_int64]
    L.ft_moe_resize_pool.restype = ctypes.c_int
    L.ft_moe_reserve.argtypes = [P, ctypes.c_int32]
    L.ft_moe_reserve.restype = ctypes.c_int
    L.ft_moe_set_hybrid_share.argtypes = [P, ctypes.c_double]
    L.ft_moe_set_hybrid_share.restype = ctypes.c_int
    L.ft_moe_set_hybrid_share_format.argtypes = [P, ctypes.c_int32, ctypes.c_double]
    L.ft_moe_set_hybrid_share_format.restype = ctypes.c_int
    L.ft_moe_get_hybrid_share.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    L.ft_moe_get_hybrid_share.restype = ctypes.c_int
    L.ft_moe_rebalance.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ft_moe_rebalance_report)]
    L.ft_moe_rebalance.restype = ctypes.c_int
    L.ft_moe_debug_read.argtypes = [P, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64]
    L.ft_moe_debug_read.restype = ctypes.c_int
    L.ft_moe_host_expert_rate.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_double)]
    L.ft_moe_host_expert_rate.restype = ctypes.c_int
    L.ft_moe_mfma_rate.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    L.ft_moe_mfma_rate.restype = ctypes.c_int
    L.ft_moe_set_profiling.argtypes = [P, ctypes.c_int32]
    L.ft_moe_set_profiling.restype = ctypes.c_int
    L.ft_moe_profile_read.argtypes = [P, ctypes.POINTER(ft_moe_profile), ctypes.c_int32]
    L.ft_moe_profile_read.restype = ctypes.c_int
    L.ft_moe_destroy_pool.argtypes = [P]
    L.ft_moe_destroy_pool.restype = None
    L.ft_moe_last_error.argtypes = []
    L.ft_moe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


class FtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ftmoe error {code}: {msg}")
        self.code = code


def ft_moe_last_error() -> str:
    r = lib().ft_moe_last_error()
    return r.decode() if r else ""


def _check(rc: int, allow_warn: bool = False) -> int:
    if rc < 0 or (rc > 0 and not allow_warn):
        raise FtError(rc, ft_moe_last_error())
    return rc


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def make_config(num_layers, hidden, inter, num_experts, top_k, layer_fmt: Sequence[int], pool_slots=0,
                pool_bytes=0, shared=False, hybrid_cpu_share=0.0, cpu_threads=0, device=0):
    fmt_arr = (ctypes.c_int32 * num_layers)(*layer_fmt)
    cfg = ft_moe_config(num_layers, hidden, inter, num_experts, top_k, int(bool(shared)),
                        ctypes.cast(fmt_arr, ctypes.POINTER(ctypes.c_int32)), int(pool_slots), int(pool_bytes),
                        float(hybrid_cpu_share), int(cpu_threads), int(device))
    cfg._keep = fmt_arr
    return cfg


def ft_moe_init_pool(cfg: ft_moe_config, expert_blobs: Sequence, router_w, shared_blobs: Optional[Sequence] = None):
    """expert_blobs: [L*E] host buffers (numpy uint8 arrays; repeated objects are stored once);
    router_w: host fp32 array [L,E,H].  Returns (pool handle, status)."""
    import numpy as np

    n = len(expert_blobs)
    arr = (ctypes.c_void_p * n)(*[b.ctypes.data for b in expert_blobs])
    sh = None
    if shared_blobs is not None:
        sh = (ctypes.c_void_p * len(shared_blobs))(*[b.ctypes.data for b in shared_blobs])
    rw = np.ascontiguousarray(router_w, dtype=np.float32)
    w = ft_moe_weights(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
                       ctypes.cast(sh, ctypes.POINTER(ctypes.c_void_p)) if sh is not None else None,
                       rw.ctypes.data)
    out = ctypes.c_void_p()
    rc = lib().ft_moe_init_pool(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(out))
    _check(rc, allow_warn=True)
    return out.value, rc


def ft_moe_layer_forward(pool, layer: int, num_tokens: int, x, router_bias, out, flags: int = 0, stream=None,
                         trace: Optional[dict] = None) -> int:
    tr = None
    if trace is not None:
        tr = ft_moe_trace(_ptr(trace.get("sel")), _ptr(trace.get("w")), _ptr(trace.get("slot")),
                          _ptr(trace.get("flag")), _ptr(trace.get("row")))
    s = 0
    if stream is not None:
        s = stream if isinstance(stream, int) else int(stream.cuda_stream)
    rc = lib().ft_moe_layer_forward(pool, int(layer), int(num_tokens), _ptr(x), _ptr(router_bias), _ptr(out),
                                    int(flags), s, ctypes.byref(tr) if tr is not None else None)
    return _check(rc)


def ft_moe_layer_forward_noalloc(pool, layer: int, num_tokens: int, x, router_bias, out, flags: int = 0,
                                 stream=None, trace: Optional[dict] = None) -> int:
    """ft_moe_layer_forward for a device-driven decode call, with its work
    buffers in the library's static per-GPU scratch (no allocation)."""
    tr = None
    if trace is not None:
        tr = ft_moe_trace(_ptr(trace.get("sel")), _ptr(trace.get("w")), _ptr(trace.get("slot")),
                          _ptr(trace.get("flag")), _ptr(trace.get("row")))
    s = 0
    if stream is not None:
        s = stream if isinstance(stream, int) else int(stream.cuda_stream)
    rc = lib().ft_moe_layer_forward_noalloc(pool, int(layer), int(num_tokens), _ptr(x), _ptr(router_bias), _ptr(out),
                                            int(flags), s, ctypes.byref(tr) if tr is not None else None)
    return _check(rc)


def ft_moe_pool_stats(pool, layer: int = -1, reset: bool = False) -> dict:
    st = ft_moe_stats()
    _check(lib().ft_moe_pool_stats(pool, int(layer), ctypes.byref(st), int(bool(reset))))
    return st.as_dict()


def ft_moe_last_misses(pool, cap: int = 1 << 16):
    se = (ctypes.c_int32 * cap)()
    ss = (ctypes.c_int32 * cap)()
    ce = (ctypes.c_int32 * cap)()
    ns, nc = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ft_moe_last_misses(pool, se, ss, ctypes.byref(ns), ce, ctypes.byref(nc), cap))
    stream = [(se[i], ss[i]) for i in range(min(ns.value, cap))]
    cpu = [ce[i] for i in range(min(nc.value, cap))]
    return stream, cpu


def ft_moe_pool_table(pool, slots: int):
    import numpy as np

    key = np.empty(slots, np.int32)
    last = np.empty(slots, np.uint64)
    clock = ctypes.c_uint64()
    n = ctypes.c_int64()
    _check(lib().ft_moe_pool_table(pool, key.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   last.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ctypes.byref(clock),
                                   ctypes.byref(n)))
    return key, last, clock.value


def ft_moe_resize_pool(pool, new_slots: int) -> int:
    """Returns FT_OK or FT_WARN_STAGING_SMALL."""
    return _check(lib().ft_moe_resize_pool(pool, int(new_slots)), allow_warn=True)


def ft_moe_decide_mode(report: dict) -> dict:
    """The decision alone (host code): report holds the rates as returned by
    ft_moe_measure_mode; returns it with t_stream, t_cpu, mode and share."""
    r = ft_moe_mode_report()
    for n, _ in r._fields_:
        if n in report:
            v = report[n]
            if isinstance(getattr(r, n), ctypes.Array):
                arr = getattr(r, n)
                for i, x in enumerate(v):
                    arr[i] = x
            else:
                setattr(r, n, v)
    _check(lib().ft_moe_decide_mode(ctypes.byref(r)))
    return r.as_dict()


def ft_moe_measure_mode(pool, tokens: int, apply: bool = False) -> dict:
    r = ft_moe_mode_report()
    _check(lib().ft_moe_measure_mode(pool, int(tokens), int(bool(apply)), ctypes.byref(r)))
    return r.as_dict()


def ft_moe_reserve(pool, max_tokens: int):
    _check(lib().ft_moe_reserve(pool, int(max_tokens)))


def ft_moe_set_hybrid_share(pool, share: float):
    _check(lib().ft_moe_set_hybrid_share(pool, float(share)))


def ft_moe_set_hybrid_share_format(pool, fmt: int, share: float):
    _check(lib().ft_moe_set_hybrid_share_format(pool, int(fmt), float(share)))


def ft_moe_get_hybrid_share(pool, fmt: int) -> float:
    v = ctypes.c_double()
    _check(lib().ft_moe_get_hybrid_share(pool, int(fmt), ctypes.byref(v)))
    return v.value


def ft_moe_debug_read(pool, what: int, nbytes: int) -> bytes:
    """A copy of the first nbytes of an internal buffer (FT_DBG_*), for tests."""
    buf = ctypes.create_string_buffer(int(nbytes))
    _check(lib().ft_moe_debug_read(pool, int(what), buf, int(nbytes)))
    return buf.raw


def ft_moe_rebalance(pool, apply: bool = True) -> dict:
    r = ft_moe_rebalance_report()
    _check(lib().ft_moe_rebalance(pool, int(bool(apply)), ctypes.byref(r)))
    return r.as_dict()


def ft_moe_host_expert_rate(pool, layer: int, tokens: int, iters: int = 1) -> float:
    r = ctypes.c_double()
    _check(lib().ft_moe_host_expert_rate(pool, int(layer), int(tokens), int(iters), ctypes.byref(r)))
    return r.value


FT_MFMA_FP4_32X32X64, FT_MFMA_FP8_16X16X128, FT_MFMA_BF16_16X16X32, FT_MFMA_BF16_32X32X16, FT_MFMA_F64_16X16X4 = \
    0, 1, 2, 3, 4


def ft_moe_mfma_rate(kind: int, iters: int = 2000, stream: int = 0) -> float:
    """Measured dense flops per second of one matrix-core instruction kind."""
    r = ctypes.c_double(0.0)
    _check(lib().ft_moe_mfma_rate(int(kind), int(iters), ctypes.c_void_p(stream or None), ctypes.byref(r)))
    return r.value


def ft_moe_ffn_kernel_name(stage: str) -> str:
    """Kernel behind the latest launch of stage "ffn_gateup" or "ffn_down"."""
    return lib().ft_moe_ffn_kernel_name(FT_STAGES.index(stage)).decode()


def ft_moe_set_profiling(pool, stages=None):
    """stages: None = all stages, [] = off, else a list of names from FT_STAGES."""
    if stages is None:
        mask = (1 << len(FT_STAGES)) - 1
    else:
        mask = 0
        for st in stages:
            mask |= 1 << FT_STAGES.index(st)
    _check(lib().ft_moe_set_profiling(pool, int(mask)))


def ft_moe_profile_read(pool, reset: bool = False) -> dict:
    pr = ft_moe_profile()
    _check(lib().ft_moe_profile_read(pool, ctypes.byref(pr), int(bool(reset))))
    return pr.as_dict()


def ft_moe_destroy_pool(pool):
    if pool:
        lib().ft_moe_destroy_pool(pool)
