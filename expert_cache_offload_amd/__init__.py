"""Python binding of the expert-offload MoE layer step (C ABI in include/moe_offload.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libmoe_offload.so``.  Pointers are passed as integers (``tensor.data_ptr()``), streams
as ``torch.cuda.Stream.cuda_stream`` integers (0 = null stream).  Importing this
package fails loudly when the library has not been built (``python -m
expert_cache_offload_amd.build`` or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_OFFLOAD_LIB selects another build of the same ABI (e.g. an instrumented one).
LIB_PATH = os.environ.get("MOE_OFFLOAD_LIB") or os.path.join(_HERE, "libmoe_offload.so")

MOE_OK, MOE_E_INVALID, MOE_E_CAPACITY, MOE_E_BUSY, MOE_E_HIP, MOE_E_NOMEM = 0, -1, -2, -3, -4, -5
MOE_E_HYBRID, MOE_E_SCRATCH = -6, -7
MOE_FMT_BF16, MOE_FMT_FP8_E4M3_K128, MOE_FMT_MXFP4_K32 = 0, 1, 2

# PyTorch ships its own HIP runtime with the same soname (libamdhip64.so.7).  Loading torch
# first makes the library's HIP dependency resolve to that already-loaded runtime, so device
# memory and streams created by PyTorch and the library's launches share one runtime; loading
# the library first would bring up a second runtime and PyTorch would then find no GPU.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m expert_cache_offload_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)


class MoeShape(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("blob_bytes", ctypes.c_int64)]


class MoePlanHost(ctypes.Structure):
    _fields_ = [("n_unique", ctypes.c_int32), ("n_hit", ctypes.c_int32),
                ("n_miss", ctypes.c_int32), ("layer", ctypes.c_int32),
                ("step", ctypes.c_int64), ("n_cpu", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("unique", ctypes.c_void_p), ("slot", ctypes.c_void_p),
                ("hit", ctypes.c_void_p), ("miss_key", ctypes.c_void_p),
                ("miss_slot", ctypes.c_void_p), ("miss_victim", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("cpu_key", ctypes.c_void_p)]


class MoeCounters(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("hits", ctypes.c_int64),
                ("misses", ctypes.c_int64), ("bytes_filled", ctypes.c_int64),
                ("cpu_misses", ctypes.c_int64)]


class MoeProfile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 4), ("ms", ctypes.c_double * 4),
                ("fill_bytes", ctypes.c_int64), ("ffn_weight_bytes", ctypes.c_int64),
                ("gate_up_timed_bytes", ctypes.c_int64), ("fused_timed_bytes", ctypes.c_int64)]


PROF_ROUTE, PROF_FILL, PROF_GATE_UP, PROF_DOWN = 1, 2, 4, 8
PROF_ALL = 15
_PROF_KINDS = ("route", "fill", "gate_up", "down")


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "moe_blob_bytes": (_i64, [_i32, _i32, _i32]),
    "moe_workspace_bytes": (_sz, [ctypes.POINTER(MoeShape), _i32]),
    "moe_host_pool_alloc": (_i32, [_sz, ctypes.POINTER(_vp)]),
    "moe_host_pool_free": (_i32, [_vp]),
    "moe_cache_create": (_i32, [ctypes.POINTER(MoeShape), _i32, _i32, _vp, _vp, _vp, _vp,
                                ctypes.POINTER(_vp)]),
    "moe_cache_create_static": (_i32, [ctypes.POINTER(MoeShape), _i32, _i32, _vp, _vp, _vp,
                                       ctypes.POINTER(_vp)]),
    "moe_cache_destroy": (_i32, [_vp]),
    "moe_cache_resize": (_i32, [_vp, _i32, _vp, _vp]),
    "moe_route_classify": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp]),
    "moe_fill_misses": (_i32, [_vp, _i32, _vp]),
    "moe_expert_ffn": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _vp]),
    "moe_layer_step": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp]),
    "moe_cache_snapshot": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_cache_set_step": (_i32, [_vp, _i64]),
    "moe_plan_read": (_i32, [_vp, ctypes.POINTER(MoePlanHost)]),
    "moe_stats": (_i32, [_vp, ctypes.POINTER(MoeCounters)]),
    "moe_profile_enable": (_i32, [_vp, _i32, _i32]),
    "moe_set_prefetch": (_i32, [_vp, _i32]),
    "moe_set_hybrid": (_i32, [_vp, _i32, _i32, _i32]),
    "moe_auto_capacity": (_i32, [ctypes.POINTER(MoeShape), ctypes.c_uint64, ctypes.c_uint64,
                                 ctypes.c_double, ctypes.POINTER(_i32)]),
    "moe_auto_capacity_device": (_i32, [ctypes.POINTER(MoeShape), ctypes.c_uint64,
                                        ctypes.c_double, ctypes.POINTER(_i32),
                                        ctypes.POINTER(ctypes.c_uint64)]),
    "moe_pool_write": (_i32, [ctypes.c_char_p, ctypes.POINTER(MoeShape), _vp, _i32]),
    "moe_pool_read": (_i32, [ctypes.c_char_p, ctypes.POINTER(MoeShape), _vp, _i32]),
    "moe_miss_split": (_i32, [_i32, _i32, _i32]),
    "moe_choose_mode": (_i32, [_i32, ctypes.c_double, ctypes.c_double]),
    "moe_probe_stream_read": (_i32, [_vp, ctypes.c_uint64, ctypes.c_uint64, _i32, _i32, _vp,
                                     _vp, ctypes.POINTER(ctypes.c_double)]),
    "moe_probe_empty_launch": (_i32, [_i32, _i32, _vp, ctypes.POINTER(ctypes.c_double)]),
    "moe_probe_copy": (_i32, [_vp, _vp, ctypes.c_uint64, _i32, _vp,
                              ctypes.POINTER(ctypes.c_double)]),
    "moe_set_hybrid_timeout": (_i32, [_vp, _i64]),
    "moe_hybrid_hold": (_i32, [_vp, _i32]),
    "moe_hybrid_read": (_i32, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                               ctypes.POINTER(ctypes.c_double)]),
    "moe_cpu_expert_ffn": (_i32, [ctypes.POINTER(MoeShape), _vp, _vp, _i32, _vp, _vp, _i32]),
    "moe_cpu_expert_rate": (_i32, [ctypes.POINTER(MoeShape), _vp, _i32, _i32, _i32,
                                   ctypes.POINTER(ctypes.c_double)]),
    "moe_profile_read": (_i32, [_vp, ctypes.POINTER(MoeProfile)]),
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_last_hip_error": (_i32, [_vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, hip: int = 0):
        msg = _lib.moe_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status}" + (f", hipError {hip})" if hip else ")"))
        self.status = status


def _check(st: int, where: str, handle=None) -> None:
    if st != MOE_OK:
        hip = _lib.moe_last_hip_error(handle) if handle else 0
        raise MoeError(st, where, hip)


def _p(x) -> int | None:
    """Integer address of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def make_shape(layers, experts, top_k, hidden, inter, wfmt, has_shared, max_tokens) -> MoeShape:
    return MoeShape(layers, experts, top_k, hidden, inter, wfmt, int(has_shared), max_tokens,
                    moe_blob_bytes(wfmt, hidden, inter))


def moe_blob_bytes(wfmt: int, hidden: int, inter: int) -> int:
    return int(_lib.moe_blob_bytes(wfmt, hidden, inter))


def moe_workspace_bytes(shape: MoeShape, max_capacity: int) -> int:
    return int(_lib.moe_workspace_bytes(ctypes.byref(shape), max_capacity))


def moe_host_pool_alloc(nbytes: int) -> int:
    out = _vp()
    _check(_lib.moe_host_pool_alloc(nbytes, ctypes.byref(out)), "moe_host_pool_alloc")
    return int(out.value)


def moe_host_pool_free(addr: int) -> None:
    _check(_lib.moe_host_pool_free(addr), "moe_host_pool_free")


def moe_cache_create(shape: MoeShape, capacity: int, max_capacity: int, slot_arena, workspace,
                     host_pool, stream: int = 0) -> int:
    out = _vp()
    st = _lib.moe_cache_create(ctypes.byref(shape), capacity, max_capacity, _p(slot_arena),
                               _p(workspace), _p(host_pool), stream, ctypes.byref(out))
    _check(st, "moe_cache_create")
    return int(out.value)


def moe_cache_create_static(shape: MoeShape, capacity: int, max_capacity: int, slot_arena,
                            host_pool, stream: int = 0) -> int:
    """moe_cache_create with the library's static per-device workspace (no allocation)."""
    out = _vp()
    st = _lib.moe_cache_create_static(ctypes.byref(shape), capacity, max_capacity,
                                      _p(slot_arena), _p(host_pool), stream, ctypes.byref(out))
    _check(st, "moe_cache_create_static")
    return int(out.value)


def moe_cache_destroy(handle: int) -> None:
    _check(_lib.moe_cache_destroy(handle), "moe_cache_destroy")


def moe_cache_resize(handle: int, new_capacity: int, new_arena=None, stream: int = 0) -> None:
    _check(_lib.moe_cache_resize(handle, new_capacity, _p(new_arena), stream),
           "moe_cache_resize", handle)


def moe_route_classify(handle: int, layer: int, x, T: int, w_router, topk_idx=None, topk_w=None,
                       stream: int = 0) -> None:
    _check(_lib.moe_route_classify(handle, layer, _p(x), T, _p(w_router), _p(topk_idx),
                                   _p(topk_w), stream), "moe_route_classify", handle)


def moe_fill_misses(handle: int, groups: int = 2, fill_stream: int = 0) -> None:
    _check(_lib.moe_fill_misses(handle, groups, fill_stream), "moe_fill_misses", handle)


def moe_expert_ffn(handle: int, layer: int, x, T: int, shared_blob, y, stream: int = 0) -> None:
    _check(_lib.moe_expert_ffn(handle, layer, _p(x), T, _p(shared_blob), _p(y), stream),
           "moe_expert_ffn", handle)


def moe_layer_step(handle: int, layer: int, x, T: int, w_router, shared_blob, y, topk_idx=None,
                   topk_w=None, groups: int = 2, compute_stream: int = 0,
                   fill_stream: int = 0) -> None:
    _check(_lib.moe_layer_step(handle, layer, _p(x), T, _p(w_router), _p(shared_blob),
                               _p(topk_idx), _p(topk_w), _p(y), groups, compute_stream,
                               fill_stream), "moe_layer_step", handle)


def moe_cache_snapshot(handle: int, capacity: int, n_keys: int):
    """Returns (key_of, stamp, slot_of, n, step, capacity) as numpy arrays / ints."""
    import numpy as np
    key_of = np.empty(capacity, np.int32)
    stamp = np.empty(capacity, np.int64)
    slot_of = np.empty(n_keys, np.int32)
    n = ctypes.c_int32()
    step = ctypes.c_int64()
    cap = ctypes.c_int32()
    st = _lib.moe_cache_snapshot(handle, key_of.ctypes.data, stamp.ctypes.data,
                                 slot_of.ctypes.data, ctypes.addressof(n),
                                 ctypes.addressof(step), ctypes.addressof(cap))
    _check(st, "moe_cache_snapshot", handle)
    return key_of[:cap.value], stamp[:cap.value], slot_of, n.value, step.value, cap.value


def moe_cache_set_step(handle: int, step: int) -> None:
    """Set the step counter of an empty cache (see the header)."""
    _check(_lib.moe_cache_set_step(handle, int(step)), "moe_cache_set_step", handle)


def moe_plan_read(handle: int, max_unique: int, max_assign: int) -> dict:
    import numpy as np
    bufs = {k: np.zeros(max_unique, np.int32) for k in
            ("unique", "slot", "miss_key", "miss_slot", "miss_victim", "count")}
    bufs["hit"] = np.zeros(max_unique, np.uint8)
    bufs["perm"] = np.zeros(max(1, max_assign), np.int32)
    bufs["cpu_key"] = np.zeros(max_unique, np.int32)
    ph = MoePlanHost(0, 0, 0, 0, 0, 0, 0, *[bufs[k].ctypes.data for k in
                                            ("unique", "slot", "hit", "miss_key", "miss_slot",
                                             "miss_victim", "count", "perm", "cpu_key")])
    _check(_lib.moe_plan_read(handle, ctypes.byref(ph)), "moe_plan_read", handle)
    nu, nm = ph.n_unique, ph.n_miss
    return {"n_unique": nu, "n_hit": ph.n_hit, "n_miss": nm, "layer": ph.layer, "step": ph.step,
            "unique": bufs["unique"][:nu].copy(), "slot": bufs["slot"][:nu].copy(),
            "hit": bufs["hit"][:nu].astype(bool), "miss_key": bufs["miss_key"][:nm].copy(),
            "miss_slot": bufs["miss_slot"][:nm].copy(),
            "miss_victim": bufs["miss_victim"][:nm].copy(), "count": bufs["count"][:nu].copy(),
            "perm": bufs["perm"].copy(), "n_cpu": ph.n_cpu,
            "cpu_key": bufs["cpu_key"][:ph.n_cpu].copy()}


def moe_stats(handle: int) -> dict:
    c = MoeCounters()
    _check(_lib.moe_stats(handle, ctypes.byref(c)), "moe_stats", handle)
    return {"steps": c.steps, "hits": c.hits, "misses": c.misses, "bytes_filled": c.bytes_filled,
            "cpu_misses": c.cpu_misses}


def moe_set_prefetch(handle: int, enable: bool) -> None:
    """Prefetch the next layer's experts during steps of many tokens (see the header)."""
    _check(_lib.moe_set_prefetch(handle, int(bool(enable))), "moe_set_prefetch", handle)


def moe_set_hybrid(handle: int, b_cpu_mbps: int, b_pcie_mbps: int, threads: int) -> None:
    """Split decode misses between fills and in-place CPU compute (b_cpu_mbps 0: off)."""
    _check(_lib.moe_set_hybrid(handle, int(b_cpu_mbps), int(b_pcie_mbps), int(threads)),
           "moe_set_hybrid", handle)


def moe_auto_capacity(shape: MoeShape, free_bytes: int, reserve_bytes: int,
                      offload_ratio: float = -1.0) -> int:
    """Largest cache capacity that fits the budget (see the header)."""
    c = _i32(0)
    _check(_lib.moe_auto_capacity(ctypes.byref(shape), int(free_bytes), int(reserve_bytes),
                                  float(offload_ratio), ctypes.byref(c)), "moe_auto_capacity")
    return int(c.value)


def moe_auto_capacity_device(shape: MoeShape, reserve_bytes: int,
                             offload_ratio: float = -1.0) -> tuple[int, int]:
    """(capacity, free bytes it was sized from): moe_auto_capacity over the device's free
    memory."""
    c, fr = _i32(0), ctypes.c_uint64(0)
    _check(_lib.moe_auto_capacity_device(ctypes.byref(shape), int(reserve_bytes),
                                         float(offload_ratio), ctypes.byref(c),
                                         ctypes.byref(fr)), "moe_auto_capacity_device")
    return int(c.value), int(fr.value)


def moe_pool_write(path: str, shape: MoeShape, pool: int, threads: int = 8) -> None:
    _check(_lib.moe_pool_write(path.encode(), ctypes.byref(shape), pool, int(threads)),
           "moe_pool_write")


def moe_pool_read(path: str, shape: MoeShape, pool: int, threads: int = 8) -> None:
    _check(_lib.moe_pool_read(path.encode(), ctypes.byref(shape), pool, int(threads)),
           "moe_pool_read")


def moe_miss_split(misses: int, b_cpu_mbps: int, b_pcie_mbps: int) -> int:
    return int(_lib.moe_miss_split(int(misses), int(b_cpu_mbps), int(b_pcie_mbps)))


def moe_set_hybrid_timeout(handle: int, microseconds: int) -> None:
    _check(_lib.moe_set_hybrid_timeout(handle, int(microseconds)), "moe_set_hybrid_timeout",
           handle)


def moe_hybrid_hold(handle: int, hold: bool) -> None:
    _check(_lib.moe_hybrid_hold(handle, int(bool(hold))), "moe_hybrid_hold", handle)


def moe_hybrid_read(handle: int) -> dict:
    """Host-side counters of the hybrid server: requests, experts, busy seconds."""
    r, e, b = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(_lib.moe_hybrid_read(handle, ctypes.byref(r), ctypes.byref(e), ctypes.byref(b)),
           "moe_hybrid_read", handle)
    return {"requests": int(r.value), "experts": int(e.value), "busy_s": float(b.value)}


def moe_cpu_expert_ffn(shape: MoeShape, blob: int, x: int, T: int, w: int, y: int,
                       threads: int) -> None:
    """y[t] += w[t] * FFN(x[t]) on the host (host addresses)."""
    _check(_lib.moe_cpu_expert_ffn(ctypes.byref(shape), blob, x, int(T), w, y, int(threads)),
           "moe_cpu_expert_ffn")


def moe_cpu_expert_rate(shape: MoeShape, pool: int, n_blobs: int, threads: int,
                        reps: int = 1) -> float:
    """Expert-weight GB/s of the CPU path over the first n_blobs blobs of a host pool."""
    g = ctypes.c_double(0.0)
    _check(_lib.moe_cpu_expert_rate(ctypes.byref(shape), pool, int(n_blobs), int(threads),
                                    int(reps), ctypes.byref(g)), "moe_cpu_expert_rate")
    return float(g.value)


def moe_choose_mode(wfmt: int, cpu_gbps: float, fill_gbps: float) -> int:
    """1: hybrid decode, 0: fill every miss, -1: invalid (the library's 2.0x rule)."""
    return int(_lib.moe_choose_mode(int(wfmt), float(cpu_gbps), float(fill_gbps)))


def choose_hybrid(cpu_gbps: float, offload_gbps: float, wfmt: int = MOE_FMT_BF16) -> bool:
    """True when the library's mode rule picks hybrid decode for this format and these rates."""
    r = moe_choose_mode(wfmt, cpu_gbps, offload_gbps)
    if r < 0:
        raise ValueError(f"moe_choose_mode: invalid rates or format ({wfmt}, {cpu_gbps}, "
                         f"{offload_gbps})")
    return r == 1


def moe_probe_stream_read(buf, span_bytes: int, bytes_per_launch: int, nontemporal: bool,
                          reps: int, sink, stream: int = 0) -> float:
    """Average duration (us) of a streaming-read launch of bytes_per_launch (see the header)."""
    us = ctypes.c_double(0.0)
    _check(_lib.moe_probe_stream_read(_p(buf), int(span_bytes), int(bytes_per_launch),
                                      int(bool(nontemporal)), int(reps), _p(sink), stream,
                                      ctypes.byref(us)), "moe_probe_stream_read")
    return float(us.value)


def moe_probe_copy(src, dst, nbytes: int, reps: int, stream: int = 0) -> float:
    """Average duration (us) of a plain device copy of nbytes (see the header)."""
    us = ctypes.c_double(0.0)
    _check(_lib.moe_probe_copy(_p(src), _p(dst), int(nbytes), int(reps), stream,
                               ctypes.byref(us)), "moe_probe_copy")
    return float(us.value)


def moe_probe_empty_launch(grid: int, reps: int, stream: int = 0) -> float:
    """Average duration (us) of an empty launch of `grid` workgroups."""
    us = ctypes.c_double(0.0)
    _check(_lib.moe_probe_empty_launch(int(grid), int(reps), stream, ctypes.byref(us)),
           "moe_probe_empty_launch")
    return float(us.value)


def moe_profile_enable(handle: int, mask: int = PROF_ALL, every: int = 1) -> None:
    """Time one launch in `every` of each kind in `mask` (PROF_* bits; 0 switches timing
    off)."""
    _check(_lib.moe_profile_enable(handle, int(mask), int(every)), "moe_profile_enable", handle)


def moe_profile_read(handle: int) -> dict:
    """{kind: {"launches", "ms"}} for route/fill/gate_up/down, plus fill_bytes and
    ffn_weight_bytes (algorithmic bytes of the FFN since moe_profile_enable)."""
    p = MoeProfile()
    _check(_lib.moe_profile_read(handle, ctypes.byref(p)), "moe_profile_read", handle)
    out = {k: {"launches": int(p.launches[i]), "ms": float(p.ms[i])}
           for i, k in enumerate(_PROF_KINDS)}
    out["fill_bytes"] = int(p.fill_bytes)
    out["ffn_weight_bytes"] = int(p.ffn_weight_bytes)
    out["gate_up_timed_bytes"] = int(p.gate_up_timed_bytes)
    out["fused_timed_bytes"] = int(p.fused_timed_bytes)
    return out


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_last_hip_error(handle: int) -> int:
    return int(_lib.moe_last_hip_error(handle))


__all__ = [n for n in _SIGS] + ["MoeShape", "MoePlanHost", "MoeCounters", "MoeProfile", "MoeError",
                                "make_shape", "choose_hybrid", "LIB_PATH"]
