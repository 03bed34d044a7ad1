#!/usr/bin/env python3
"""MoE-layer decode throughput of the expert-offload stack on one MI355X.

Workload (default): the 48-layer 35B-A3B-shaped MoE stack - hidden 2048, 128 experts top-8
with renormalised softmax, SwiGLU intermediate 768, bf16 expert weights N(0, 0.02) in a
pinned host pool (58 GB), one LRU slot cache shared by all layers holding 30% of the pool
(1,843 slots), AR(1) activations per layer, batch 1, seed 0, cold cache.  One step = one
decode token through all 48 layer steps (route, top-k, dedup, classify, LRU, fills, FFN).
The first --warmup tokens are untimed; exactly --steps tokens are timed.

The headline is the hot path as the pages define it: every miss filled from the pinned pool
("offload").  Reported in one JSON line: decode tokens/s of the stack; the dominant FFN kernel
(at one token with bf16 weights the fused gate/up + down kernel, which streams whole blobs;
otherwise the gate/up kernel, two thirds of the expert bytes) against the MI355X HBM roofline
and against the streaming-read ceilings measured by the library's own probe kernel - achieved
= the expert-weight bytes the timed launches were given / their durations, from event pairs
taken by the kernel dispatches on the compute stream over the timed tokens; fill bandwidth
against pinned hipMemcpyAsync H2D measured on the same box; the float64 CPU oracle over a
bounded sample of the same workload on every host core.  For bf16 weights a second block
runs the pages' hybrid decode (misses split between fills and CPU compute by the closed-form
q; the mode rule's choice is reported) with its own rate, roofline and busy fractions.

`--rocprof-summary DIR` (and `--pmc FETCH_DIR WRITE_DIR`) turn rocprofv3 output of a bench
run into the text summaries kept under profiles/; `--phase-log PATH` makes a bench run record
how many launches of its dominant kernel each phase issued, so the summary can average that
kernel over the timed region alone.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0           # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PROBE_SPAN = 4 << 30             # bytes of device memory the read probes stream over
HOST_CORES_MAX = 16              # the host CPU share of one GPU on the measurement boxes


def _die_multi_gpu(n: int) -> None:
    print(f"bench.py: this build runs on one GPU only (--gpus {n} requested); "
          "the expert-offload path is measured on a single MI355X.", file=sys.stderr)
    sys.exit(2)


def _log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(HOST_CORES_MAX, n))


# ------------------------------------------------------------------ CPU baseline (oracle)
# The float64 oracle as it stands, over (token, layer) work items spread across the host's
# cores: each worker routes its item (router GEMM, top-k) and computes its layer output (the
# SwiGLU FFN of the selected experts) with one BLAS thread; the main process then replays
# dedup and the LRU cache over the items in step order.  It runs before the GPU is touched
# (the workers are forked from a process that has not initialised it).

_CPU = {}  # state the forked workers read (copy-on-write)


def _cpu_item(i: int):
    from oracle.ffn import moe_output
    from oracle.formats import bf16_to_f64, decode_blob
    from oracle.router import router_logits, topk_softmax
    c = _CPU
    wl = c["wl"]
    t, l = divmod(i, wl.layers)
    x = bf16_to_f64(c["acts"][t, l]).reshape(-1, wl.hidden)
    idx, w = topk_softmax(router_logits(x, bf16_to_f64(c["router"][l])), wl.top_k)
    shared = None
    if wl.has_shared:
        shared = decode_blob(c["shared"][l], wl.fmt, wl.hidden, wl.inter)
    y = moe_output(x, idx, w, lambda e: decode_blob(c["blobs"][l * wl.experts + int(e)], wl.fmt,
                                                    wl.hidden, wl.inter), shared)
    return i, idx, float(abs(y).sum())


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU["limit"] = threadpool_limits(1)


def cpu_baseline_decode(wl, tokens: int, reps: int) -> dict:
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    import moe_inputs as mi
    from oracle.dedup import dedup
    from oracle.formats import bf16_to_f64
    from oracle.lru import LRUCache
    from oracle.router import router_logits, topk_softmax
    cores = _host_cores()
    t_setup = time.perf_counter()
    L, E, H, I = wl.layers, wl.experts, wl.hidden, wl.inter
    acts = mi.decode_acts(wl.seed, 0, L, wl.tokens_per_step, tokens, H)
    router = mi.router_weights(wl.seed, 0, L, E, H)
    keys = set()
    with threadpool_limits(1):
        for t in range(tokens):  # which blobs the sample reads (untimed): generate only those
            for l in range(L):
                x = bf16_to_f64(acts[t, l]).reshape(-1, H)
                idx, _ = topk_softmax(router_logits(x, bf16_to_f64(router[l])), wl.top_k)
                keys.update(l * E + int(e) for e in np.unique(idx))
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(cores) as ex:  # the generator releases the GIL
        blobs = dict(zip(sorted(keys), ex.map(
            lambda k: mi.expert_blob(wl.seed, wl.fmt, mi.PURPOSE_EXPERT, k // E, k % E, H, I),
            sorted(keys))))
    shared = [mi.shared_blob(wl.seed, wl.fmt, l, H, I) for l in range(L)] if wl.has_shared else None
    _CPU.update(wl=wl, acts=acts, router=router, blobs=blobs, shared=shared)
    setup_s = time.perf_counter() - t_setup
    ctx = mp.get_context("fork")
    n_items = tokens * L
    runs = []
    with threadpool_limits(1):
        with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
            for _ in range(reps):
                t0 = time.perf_counter()
                res = sorted(pool.map(_cpu_item, range(n_items), chunksize=1))
                cache = LRUCache(wl.capacity, wl.n_keys)
                for s, (i, idx, _) in enumerate(res):
                    U = dedup(idx, E)[0]
                    cache.step(i % L, U, E, s)
                runs.append(time.perf_counter() - t0)
    _CPU.clear()
    runs.sort()
    med = runs[len(runs) // 2]
    T = wl.tokens_per_step
    return {"value": round(tokens * T / med, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{tokens} token steps x {L} layers of the same workload ({n_items} "
                      f"(token, layer) items over {cores} worker processes, one BLAS thread "
                      f"each; float64 router, top-k and SwiGLU FFN per item, then dedup and the "
                      f"LRU replayed in step order); median of {reps} repetitions",
            "seconds": [round(r, 3) for r in runs], "setup_s": round(setup_s, 2),
            "blobs_generated": len(blobs), "host_cpus": os.cpu_count(),
            "host_cpu_model": _host_cpu_model()}


def cpu_baseline_prefill(wb, tokens: int) -> dict:
    """The float64 oracle on the first `tokens` tokens of the chunk through the first layer
    (route, top-k, dedup, LRU and the SwiGLU FFN), scaled to the whole layer stack."""
    from threadpoolctl import threadpool_info

    import dataclasses
    from oracle.step import Oracle
    wl = dataclasses.replace(wb.wl, tokens_per_step=tokens)
    orc = Oracle(wl, wb.pool, wb.router_np)
    t0 = time.perf_counter()
    orc.layer_step(0, 0, wb.acts_np[0][:tokens], True)
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {"value": tokens / (dt * wb.wl.layers), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {tokens} tokens of the chunk through layer 0 (full float64 route, "
                      f"top-k, dedup, LRU, SwiGLU FFN), {dt:.1f} s, scaled to "
                      f"{wb.wl.layers} layers",
            "seconds": dt, "host_cpus": os.cpu_count(), "host_cpu_model": _host_cpu_model()}


# ------------------------------------------------------------------ probes
def h2d_memcpy_probe(pool_addr: int, pool_bytes: int, blob: int, dev_buf_ptr: int,
                     dev_buf_bytes: int) -> dict:
    """Pinned host -> device hipMemcpyAsync bandwidth, back-to-back blob-sized copies and one
    large copy, from the same pinned pool the fills read."""
    hip = ctypes.CDLL("libamdhip64.so.7")  # by soname: the runtime already loaded by PyTorch
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    s = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(s)) == 0
    H2D = 1
    out = {}
    n = min(64, dev_buf_bytes // blob, pool_bytes // blob)

    def run(size, count):
        assert hip.hipMemcpyAsync(dev_buf_ptr, pool_addr, size, H2D, s) == 0  # warm
        hip.hipStreamSynchronize(s)
        t0 = time.perf_counter()
        for i in range(count):
            src = pool_addr + ((i * 7919) % (pool_bytes // size)) * size
            dst = dev_buf_ptr + (i % (dev_buf_bytes // size)) * size
            assert hip.hipMemcpyAsync(dst, src, size, H2D, s) == 0
        hip.hipStreamSynchronize(s)
        return size * count / (time.perf_counter() - t0) / 1e9

    out["blob_GBps"] = run(blob, n)
    big = min(1 << 30, dev_buf_bytes, pool_bytes)
    out["large_GBps"] = run(big, 4)
    out["large_bytes"] = big
    hip.hipStreamDestroy(s)
    return out


def read_probes(dev, launch_bytes: int, grid: int) -> dict:
    """The library's streaming-read kernel: the chip's sustained read rate over 4 GiB, and one
    launch of the dominant FFN kernel's size (windows of a 4 GiB buffer read in turn, so none
    is cache-resident), both with plain and with streaming loads; and an empty launch of the
    FFN kernel's grid."""
    import torch

    from expert_cache_offload_amd import (moe_probe_copy, moe_probe_empty_launch,
                                          moe_probe_stream_read)
    buf = torch.empty(PROBE_SPAN, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    out = {"span_bytes": PROBE_SPAN}
    for nt in (0, 1):
        tag = "nt" if nt else "plain"
        us = moe_probe_stream_read(buf, PROBE_SPAN, PROBE_SPAN, nt, 4, sink)
        out[f"read_4GiB_{tag}_GBps"] = round(PROBE_SPAN / us / 1e3, 1)
        lb = launch_bytes // 16 * 16
        if lb >= 16:
            reps = max(8, min(48, PROBE_SPAN // lb))
            us = moe_probe_stream_read(buf, PROBE_SPAN, lb, nt, reps, sink)
            out[f"read_launch_{tag}_GBps"] = round(lb / us / 1e3, 1)
            out[f"read_launch_{tag}_us"] = round(us, 3)
    out["launch_bytes"] = launch_bytes
    out["read_GBps"] = max(out["read_4GiB_plain_GBps"], out["read_4GiB_nt_GBps"])
    if launch_bytes >= 16:
        out["read_launch_GBps"] = max(out["read_launch_plain_GBps"], out["read_launch_nt_GBps"])
    half = PROBE_SPAN // 2  # 2 GiB copied from the buffer's first half to its second
    us = moe_probe_copy(buf, buf.data_ptr() + half, half, 4)
    out["copy_2GiB_GBps"] = round(2 * half / us / 1e3, 1)  # bytes read + written
    out["empty_launch_us"] = round(moe_probe_empty_launch(max(1, grid), 200), 3)
    out["empty_launch_grid"] = grid
    del buf, sink
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ traffic from counters
def _ffn_source_hash() -> str:
    here = os.path.dirname(os.path.abspath(__file__))
    p = os.path.join(here, "expert_cache_offload_amd", "csrc", "ffn_decode.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _traffic_ratio_from_profile(name: str) -> float | None:
    """HBM bytes per algorithmic byte of the dominant decode FFN kernel from a committed
    counter summary, if it was taken on the current kernel source (its hash line)."""
    here = os.path.dirname(os.path.abspath(__file__))
    p = os.path.join(here, "profiles", name)
    if not os.path.exists(p):
        return None
    h = _ffn_source_hash()
    val, src_ok = None, False
    for line in open(p):
        if line.startswith("ffn_source_sha256_16:") and line.split(":", 1)[1].strip() == h:
            src_ok = True
        if line.startswith("hbm_bytes_per_algorithmic_byte:"):
            val = float(line.split(":", 1)[1])
    return val if src_ok else None


# ------------------------------------------------------------------ decode
def _with_cache_frac(wl, frac: float):
    import dataclasses
    return dataclasses.replace(wl, name=f"{wl.name}_cache{frac:g}", cache_frac=frac,
                               fixed_capacity=0)


def decode_block(wb, args, mode: str, phases: list, rates=None) -> dict:
    """One measured decode run from a cold cache: warmup, the timed tokens in five windows (one
    launch in `--profile-every` of the dominant FFN kernel event-timed), then a few untimed
    tokens with every kernel timed (the breakdown).  mode "hybrid": misses split with the CPU
    at `rates` (CPU, fill) MB/s; the CPU rate is re-measured on the warmup's own requests."""
    import torch

    from expert_cache_offload_amd import (PROF_ALL, PROF_GATE_UP, moe_hybrid_read,
                                          moe_profile_enable, moe_profile_read)
    wl = wb.wl
    L, T = wl.layers, wl.tokens_per_step
    n_tok = args.warmup + args.steps
    resize_at = wl.resize_at if 0 <= wl.resize_at < n_tok else -1
    out = {"mode": mode}
    wb.set_hybrid(0)
    if wb.capacity != wl.capacity and wl.resize_at >= 0:
        wb.capacity = wl.capacity
    if mode == "hybrid":
        wb.set_hybrid(rates[0], rates[1], args.cpu_threads)
    wb.reset()

    def token(t):
        for l in range(L):
            wb.step(t, l)

    h0 = moe_hybrid_read(wb.handle)
    for t in range(args.warmup):
        if t == resize_at:
            wb.sync()
            wb.resize(wl.resize_capacity)
        token(t)
        if t % 16 == 15:
            wb.sync()
            _log(f"{mode} warmup token {t}")
    wb.sync()
    phases.append([f"{mode}_warmup", args.warmup * L])
    if mode == "hybrid":
        h1 = moe_hybrid_read(wb.handle)
        busy = h1["busy_s"] - h0["busy_s"]
        if busy > 0 and h1["experts"] > h0["experts"]:
            eff = (h1["experts"] - h0["experts"]) * wl.blob_bytes / busy / 1e9
            out["cpu_rate_warmup_GBps"] = round(eff, 2)
            wb.set_hybrid(int(eff * 1000), rates[1], args.cpu_threads)
            _log(f"CPU path sustained {eff:.1f} GB/s over the warmup: split recomputed with it")
    st0 = wb.stats()
    hy0 = moe_hybrid_read(wb.handle)
    if not args.no_profile:
        moe_profile_enable(wb.handle, PROF_GATE_UP, args.profile_every)
    n_win = 5
    bounds = [args.warmup + (args.steps * i) // n_win for i in range(n_win + 1)]
    segments, resize_s = [], None
    torch.cuda.synchronize()
    for w in range(n_win):
        t, t_end = bounds[w], bounds[w + 1]
        while t < t_end:
            if t == resize_at:
                r0 = time.perf_counter()
                wb.resize(wl.resize_capacity)
                torch.cuda.synchronize()
                resize_s = time.perf_counter() - r0
            stop = resize_at if t < resize_at < t_end else t_end
            t0 = time.perf_counter()
            for tt in range(t, stop):
                token(tt)
            torch.cuda.synchronize()
            segments.append((stop - t, time.perf_counter() - t0,
                             "after" if 0 <= resize_at <= t else "before"))
            _log(f"{mode} tokens {t}..{stop - 1}: "
                 f"{(stop - t) * T / segments[-1][1]:.2f} tok/s")
            t = stop
    phases.append([f"{mode}_timed", args.steps * L])
    wall = sum(dt for _, dt, _ in segments) + (resize_s or 0.0)
    prof = moe_profile_read(wb.handle) if not args.no_profile else None
    st1 = wb.stats()
    hy1 = moe_hybrid_read(wb.handle)
    brk = None
    if not args.no_profile and args.breakdown_steps > 0:
        moe_profile_enable(wb.handle, PROF_ALL)
        for t in range(n_tok, n_tok + args.breakdown_steps):
            token(t)
        brk = moe_profile_read(wb.handle)
        moe_profile_enable(wb.handle, 0)
        phases.append([f"{mode}_breakdown", args.breakdown_steps * L])
    hits = st1["hits"] - st0["hits"]
    misses = st1["misses"] - st0["misses"]
    cpu_misses = st1["cpu_misses"] - st0["cpu_misses"]
    tokens = args.steps * T
    out.update({"tok_s": tokens / wall, "wall_s": wall, "ms_per_step": wall / args.steps * 1e3,
                "miss_rate": round(misses / max(1, hits + misses), 4),
                "misses_per_token": round(misses / max(1, tokens), 2),
                "cpu_misses_per_token": round(cpu_misses / max(1, tokens), 2),
                "fill_bytes": st1["bytes_filled"] - st0["bytes_filled"]})
    rates_w = sorted(n * T / dt for n, dt, _ in segments if n > 0)
    out["repeats"] = {"windows": len(rates_w), "tok_s": [round(r, 3) for r in rates_w],
                      "median": round(rates_w[len(rates_w) // 2], 3),
                      "min": round(rates_w[0], 3), "max": round(rates_w[-1], 3)}
    if prof is not None and prof["gate_up"]["launches"] > 0:
        gu = prof["gate_up"]
        gu_bytes = prof["gate_up_timed_bytes"]
        fused = gu_bytes > 0 and prof["fused_timed_bytes"] == gu_bytes
        # both kernels run I / 8 workgroups per expert entry; an entry streams the whole blob
        # in the fused kernel, its gate and up rows (two thirds) in the gate/up kernel
        out["ffn"] = {"kernel": "ffn_fused_kernel" if fused else "ffn_gate_up_kernel",
                      "launches": gu["launches"], "seconds": gu["ms"] / 1e3, "bytes": gu_bytes,
                      "entry_bytes": wl.blob_bytes if fused else wl.blob_bytes * 2 // 3,
                      "grid_per_entry": wl.inter // 8}
    if brk is not None:
        nb = args.breakdown_steps
        per = lambda k: round(brk[k]["ms"] * 1e3 / max(1, brk[k]["launches"]), 2)  # noqa: E731
        fk = brk["fill"]
        out["fill_kernel_GBps"] = brk["fill_bytes"] / (fk["ms"] / 1e3) / 1e9 if fk["ms"] else 0.0
        out["breakdown"] = {
            "tokens": nb, "note": "untimed tokens after the timed region, every launch timed",
            "route_us_per_launch": per("route"), "fill_us_per_launch": per("fill"),
            "ffn_us_per_launch": per("gate_up"), "second_stage_us_per_launch": per("down"),
            "route_ms_per_token": round(brk["route"]["ms"] / nb, 3),
            "fill_ms_per_token": round(fk["ms"] / nb, 3),
            "ffn_ms_per_token": round(brk["gate_up"]["ms"] / nb, 3),
            "second_stage_ms_per_token": round(brk["down"]["ms"] / nb, 3)}
    if mode == "hybrid":
        busy = hy1["busy_s"] - hy0["busy_s"]
        ex = hy1["experts"] - hy0["experts"]
        out["cpu_busy_frac"] = round(busy / wall, 4) if wall > 0 else None
        out["cpu_effective_GBps"] = round(ex * wl.blob_bytes / busy / 1e9, 2) if busy else None
        out["requests"] = hy1["requests"] - hy0["requests"]
    if resize_s is not None:
        side = {k: (sum(n for n, _, sd in segments if sd == k),
                    sum(dt for _, dt, sd in segments if sd == k)) for k in ("before", "after")}
        out["resize"] = {
            "at_token_step": resize_at, "from_slots": wl.capacity,
            "to_slots": wl.resize_capacity, "latency_ms": round(resize_s * 1e3, 3),
            "tok_s_before": round(side["before"][0] * T / side["before"][1], 3)
            if side["before"][1] > 0 else None,
            "tok_s_after": round(side["after"][0] * T / side["after"][1], 3)
            if side["after"][1] > 0 else None}
    return out


def _roofline(block: dict, wl, probes: dict | None) -> dict | None:
    f = block.get("ffn")
    if not f or f["seconds"] <= 0:
        return None
    achieved = f["bytes"] / f["seconds"] / 1e9
    per_launch = f["bytes"] / max(1, f["launches"])
    r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": f["kernel"],
         "launches": f["launches"],
         "avg_launch_us": round(f["seconds"] * 1e6 / max(1, f["launches"]), 3),
         "algorithmic_bytes_per_launch": round(per_launch)}
    if f["kernel"] == "ffn_fused_kernel":
        ratio = _traffic_ratio_from_profile(f"ffn_fused_{wl.name}_pmc.txt")
        if ratio:
            r["traffic"] = round(ratio * per_launch)
    if probes:
        r["frac_of_measured_read"] = round(achieved / probes["read_GBps"], 4)
        if "read_launch_GBps" in probes:
            r["frac_of_launch_sized_read"] = round(achieved / probes["read_launch_GBps"], 4)
    return r


def run_decode(args, wl, cpu) -> None:
    import torch

    from expert_cache_offload_amd import (make_shape, moe_auto_capacity_device, moe_choose_mode,
                                          moe_cpu_expert_rate)
    from expert_cache_offload_amd.runner import Workbench
    n_all = args.warmup + args.steps + args.breakdown_steps
    wl = wl.with_steps(n_all)
    auto = None
    if args.auto_capacity:
        import dataclasses
        shape = make_shape(wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.fmt,
                           wl.has_shared, wl.tokens_per_step)
        reserve = int(args.reserve_gb * 2**30)
        cap, free = moe_auto_capacity_device(shape, reserve, args.offload_ratio)
        auto = {"slots": cap, "free_bytes": free, "reserve_bytes": reserve,
                "offload_ratio": args.offload_ratio}
        wl = dataclasses.replace(wl, name=f"{wl.name}_auto", fixed_capacity=cap)
        _log(f"auto-sized cache: {cap} slots from {free / 2**30:.1f} GiB free")
    _log(f"workload {wl.name}: L={wl.layers} H={wl.hidden} E={wl.experts} k={wl.top_k} "
         f"I={wl.inter} fmt={wl.fmt} C={wl.capacity} pool={wl.pool_bytes / 1e9:.2f} GB")
    t_setup = time.perf_counter()
    wb = Workbench(wl, groups=args.groups, pool_file=args.pool_file or None)
    _log(f"setup {time.perf_counter() - t_setup:.1f} s")
    phases = []
    off = decode_block(wb, args, "offload", phases)
    _log(f"offload: {off['tok_s']:.2f} tok/s, miss rate {off['miss_rate']:.3f}")
    hybrid = None
    rule = None
    if wl.fmt == 0 and not args.no_hybrid:
        fill_rate = off.get("fill_kernel_GBps") or 0.0
        cpu_rate = moe_cpu_expert_rate(wb.shape, wb.pool_addr, 48, args.cpu_threads, 2)
        rule = moe_choose_mode(wl.fmt, cpu_rate, fill_rate)
        _log(f"CPU expert path {cpu_rate:.1f} GB/s, fills {fill_rate:.1f} GB/s -> mode rule "
             f"{'hybrid' if rule == 1 else 'offload'}")
        if fill_rate > 0 and cpu_rate > 0:
            hybrid = decode_block(wb, args, "hybrid", phases,
                                  (int(cpu_rate * 1000), int(fill_rate * 1000)))
            hybrid.update({"cpu_expert_GBps": round(cpu_rate, 2),
                           "offload_GBps": round(fill_rate, 2),
                           "ratio": round(cpu_rate / fill_rate, 3), "threshold": 2.0,
                           "cpu_threads": args.cpu_threads})
            _log(f"hybrid: {hybrid['tok_s']:.2f} tok/s")
    elif wl.fmt != 0:
        rule = moe_choose_mode(wl.fmt, 0.0, off.get("fill_kernel_GBps") or 0.0)
    head = off
    if args.mode == "hybrid" and hybrid is not None:
        head = hybrid
    elif args.mode == "auto" and rule == 1 and hybrid is not None:
        head = hybrid
    if args.phase_log:
        with open(args.phase_log, "w") as f:
            kname = (off.get("ffn") or {}).get("kernel", "")
            json.dump({"kernel": kname, "phases": phases, "layers": wl.layers}, f)
    scratch = torch.empty(min(1 << 30, wl.capacity * wl.blob_bytes), dtype=torch.uint8,
                          device=wb.dev)
    h2d = h2d_memcpy_probe(wb.pool_addr, wb.pool_bytes, wl.blob_bytes, scratch.data_ptr(),
                           scratch.numel())
    del scratch
    probes = None
    f = head.get("ffn")
    if not args.no_probes:
        lb = f["bytes"] // max(1, f["launches"]) if f else 0
        grid = round(lb / f["entry_bytes"]) * f["grid_per_entry"] if f else 1
        probes = read_probes(wb.dev, lb, grid)
    wb.close()

    def fill_of(b):
        wall = b["wall_s"]
        fl = {"bytes": b["fill_bytes"], "link_GBps": round(b["fill_bytes"] / wall / 1e9, 2),
              "h2d_memcpy_blob_GBps": round(h2d["blob_GBps"], 2),
              "h2d_memcpy_1GiB_GBps": round(h2d["large_GBps"], 2)}
        fl["link_frac_of_memcpy"] = round(fl["link_GBps"] / h2d["blob_GBps"], 3)
        if b.get("fill_kernel_GBps"):
            k = b["fill_kernel_GBps"]
            fl["kernel_GBps"] = round(k, 2)
            fl["kernel_frac_of_memcpy"] = round(k / h2d["blob_GBps"], 3)
            fl["link_busy_frac"] = round(b["fill_bytes"] / (k * 1e9) / wall, 4)
        return fl

    roof = _roofline(head, wl, probes)
    hyb_out = None
    if hybrid is not None:
        hyb_out = {k: v for k, v in hybrid.items() if k not in ("ffn", "fill_bytes", "wall_s")}
        hyb_out["tok_s"] = round(hybrid["tok_s"], 3)
        hyb_out["ms_per_step"] = round(hybrid["ms_per_step"], 3)
        hyb_out["roofline"] = _roofline(hybrid, wl, probes)
        hyb_out["fill"] = fill_of(hybrid)
        hyb_out["mode_rule"] = "hybrid" if rule == 1 else "offload"
        hyb_out["note"] = ("the pages' hybrid decode (f1): the last q misses of a step computed "
                           "by the host CPU from the pinned pool, q the closed-form split of "
                           "the measured CPU and fill rates; CPU misses are not cached")
    elif rule is not None:
        hyb_out = {"mode_rule": "hybrid" if rule == 1 else "offload",
                   "note": "no CPU expert path for this weight format: every miss is filled"}
    if head is hybrid:
        off_out = {"tok_s": round(off["tok_s"], 3), "roofline": _roofline(off, wl, probes),
                   "fill": fill_of(off), "miss_rate": off["miss_rate"]}
    else:
        off_out = None
    dtype = {0: "bf16", 1: "fp8", 2: "mxfp4"}[wl.fmt]
    line = {
        "metric": "MoE decode tokens/s per layer stack + HBM GB/s fraction; miss-fill PCIe GB/s",
        "value": round(head["tok_s"], 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "mode": head["mode"], "layers": wl.layers,
                   "hidden": wl.hidden, "experts": wl.experts, "top_k": wl.top_k,
                   "inter": wl.inter, "cache_slots": wl.capacity, "pool_bytes": wl.pool_bytes,
                   "tokens_per_step": wl.tokens_per_step, "fill_groups": args.groups,
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "fill": fill_of(head),
        "miss_rate": head["miss_rate"],
        "misses_per_token": head["misses_per_token"],
        "cpu_misses_per_token": head["cpu_misses_per_token"],
        "repeats": head["repeats"],
        "breakdown": head.get("breakdown"),
        "hybrid": hyb_out,
        "probes": probes,
    }
    if off_out is not None:
        line["offload"] = off_out
    if head.get("resize"):
        line["resize"] = head["resize"]
    if auto is not None:
        line["config"]["auto_capacity"] = auto
    if args.pool_file:
        line["config"]["pool_file"] = os.path.basename(args.pool_file)
    print(json.dumps(line), flush=True)


# ------------------------------------------------------------------ prefill
def run_prefill(args, wl) -> None:
    """Prefill chunks through the layer stack from a cold cache, each layer step prefetching
    the next layer's experts on the fill stream: tokens/s, the matrix-core FFN against the
    bf16 MFMA roofline, fills against pinned hipMemcpyAsync, and the ablation: the same chunk
    in stream order (each layer's fills, then its FFN: no overlap, no prefetch), with the
    layer's own fills double-buffered in groups, and with both."""
    import torch

    from expert_cache_offload_amd import (PROF_DOWN, PROF_FILL, PROF_GATE_UP, moe_profile_enable,
                                          moe_profile_read)
    from expert_cache_offload_amd.runner import Workbench

    groups = args.groups  # 0: the layer's own fills in stream order, prefetch on the side
    ab_groups = 16  # double-buffered fill groups of the ablation chunks
    steps = args.steps if args.steps_given else 5
    warmup = args.warmup if args.warmup_given else 1
    T, L, H, I, K = wl.tokens_per_step, wl.layers, wl.hidden, wl.inter, wl.top_k
    _log(f"prefill {wl.name}: L={L} T={T} H={H} E={wl.experts} k={K} I={I} C={wl.capacity} "
         f"pool={wl.pool_bytes / 1e9:.2f} GB, {groups} fill groups")
    wb = Workbench(wl, groups=groups, max_capacity=wl.capacity)

    def chunk(g: int, prefetch: bool = True) -> float:
        wb.groups = g
        wb.prefetch = prefetch
        wb.reset()
        t0 = time.perf_counter()
        for l in range(L):
            wb.step(0, l)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    for _ in range(warmup):
        chunk(groups)
    times = []
    for i in range(steps):
        times.append(chunk(groups))
        _log(f"chunk {i}: {times[-1]:.3f} s")
    wall = sum(times)
    tok_s = steps * T / wall
    wb.groups = groups
    wb.prefetch = True
    wb.reset()
    moe_profile_enable(wb.handle, PROF_GATE_UP | PROF_DOWN | PROF_FILL, 1)
    for l in range(L):
        wb.step(0, l)
    torch.cuda.synchronize()
    prof = moe_profile_read(wb.handle)
    st = wb.stats()
    stream_order = chunk(0, prefetch=False)
    db_prefetch = chunk(ab_groups)
    no_prefetch = chunk(ab_groups, prefetch=False)
    _log(f"ablation: stream order {stream_order:.3f} s, {ab_groups} groups + prefetch "
         f"{db_prefetch:.3f} s, {ab_groups} groups {no_prefetch:.3f} s")
    # the matrix-core kernels without concurrent fills: a chunk in stream order, GEMMs timed
    wb.groups = 0
    wb.prefetch = False
    wb.reset()
    moe_profile_enable(wb.handle, PROF_GATE_UP | PROF_DOWN)
    for l in range(L):
        wb.step(0, l)
    torch.cuda.synchronize()
    iso = moe_profile_read(wb.handle)
    moe_profile_enable(wb.handle, 0)
    fl_gu = 2.0 * T * K * (2 * I) * H * L  # gate/up FLOPs of the chunk (every routed row)
    fl_dn = 2.0 * T * K * I * H * L
    gu_s = prof["gate_up"]["ms"] / 1e3
    dn_s = prof["down"]["ms"] / 1e3
    achieved = fl_gu / gu_s / 1e12 if gu_s > 0 else 0.0
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=wb.dev)
    h2d = h2d_memcpy_probe(wb.pool_addr, wb.pool_bytes, wl.blob_bytes, scratch.data_ptr(),
                           scratch.numel())
    del scratch
    fill_bytes = prof["fill_bytes"]
    fk_s = prof["fill"]["ms"] / 1e3
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(wb, 512)
        _log(f"oracle {cpu['value']:.2f} tok/s ({cpu['seconds']:.1f} s)")
    misses = st["misses"]
    wb.close()
    med = sorted(times)[len(times) // 2]
    iso_gu = iso["gate_up"]["ms"] / 1e3
    iso_dn = iso["down"]["ms"] / 1e3
    line = {
        "metric": "MoE prefill tokens/s per layer stack (cold cache) + MFMA TFLOP/s fraction; "
                  "miss-fill PCIe GB/s",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "hidden": H, "experts": wl.experts,
                   "top_k": K, "inter": I, "cache_slots": wl.capacity,
                   "pool_bytes": wl.pool_bytes, "tokens_per_step": T, "fill_groups": groups,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "ffn_prefill_gate_up_kernel",
                     "launches": prof["gate_up"]["launches"],
                     "avg_launch_us": round(prof["gate_up"]["ms"] * 1e3 /
                                            max(1, prof["gate_up"]["launches"]), 1),
                     "algorithmic_flops_per_chunk": fl_gu},
        "down_kernel_TFLOPs": round(fl_dn / dn_s / 1e12, 1) if dn_s > 0 else None,
        "isolated": {"note": "one chunk with each layer's fills before its FFN (no concurrent "
                             "fill traffic): the GEMMs' own rate",
                     "gate_up_TFLOPs": round(fl_gu / iso_gu / 1e12, 1) if iso_gu else None,
                     "gate_up_frac": round(fl_gu / iso_gu / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
                     if iso_gu else None,
                     "down_TFLOPs": round(fl_dn / iso_dn / 1e12, 1) if iso_dn else None,
                     "down_frac": round(fl_dn / iso_dn / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
                     if iso_dn else None},
        "cpu_baseline": cpu,
        "fill": {"bytes_per_chunk": fill_bytes, "misses_per_chunk": misses,
                 "kernel_GBps": round(fill_bytes / fk_s / 1e9, 2) if fk_s > 0 else None,
                 "h2d_memcpy_blob_GBps": round(h2d["blob_GBps"], 2),
                 "h2d_memcpy_1GiB_GBps": round(h2d["large_GBps"], 2),
                 "link_GBps_timed": round(fill_bytes / med / 1e9, 2)},
        "ablation": {"note": f"one chunk each against the timed configuration ({groups} fill "
                             f"groups, prefetch of the next layer): stream order (each layer's "
                             f"fills, then its FFN: no overlap, no prefetch), the layer's own "
                             f"fills double-buffered in {ab_groups} groups with and without "
                             f"prefetch",
                     "timed_median_s": round(med, 4),
                     "stream_order_s": round(stream_order, 4),
                     "stream_order_over_timed": round(stream_order / med, 4),
                     "timed_gain_over_stream_order": round(1.0 - med / stream_order, 4),
                     "prefetch_groups_s": round(db_prefetch, 4),
                     "no_prefetch_groups_s": round(no_prefetch, 4),
                     "no_prefetch_groups_over_timed": round(no_prefetch / med, 4)},
        "repeats": {"chunks": len(times),
                    "tok_s": [round(T / t, 1) for t in sorted(times, reverse=True)],
                    "median": round(T / med, 1),
                    "min": round(T / max(times), 1), "max": round(T / min(times), 1)},
    }
    print(json.dumps(line), flush=True)


# ------------------------------------------------------------------ rocprofv3 summaries
def _csv_rows(d: str, suffix: str) -> list:
    import csv
    import glob
    rows = []
    for p in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _kname(r: dict) -> str:
    return r.get("Kernel_Name", r.get("Name", "")).replace("void ", "")


def rocprof_summary(args) -> None:
    """Print the kernel statistics of a rocprofv3 --kernel-trace --stats run of this bench, and
    the dominant kernel's average over each phase the bench logged (--phase-log)."""
    stats = _csv_rows(args.rocprof_summary, "kernel_stats.csv")
    print(f"{'kernel':<64} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>10} "
          f"{'total_ms':>10} {'pct':>6}")
    for r in stats:
        n = _kname(r)
        if "moe::" not in n:
            continue
        print(f"{n[:64]:<64} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
              f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
              f"{float(r['TotalDurationNs']) / 1e6:>10.2f} {float(r['Percentage']):>6.2f}")
    if not args.phase_log:
        return
    ph = json.load(open(args.phase_log))
    trace = _csv_rows(args.rocprof_summary, "kernel_trace.csv")
    key = ph["kernel"]
    disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace
                  if key and f"moe::{key}" in _kname(r))
    print(f"\n{key}: {len(disp)} dispatches; by phase of the bench run (in order):")
    i = 0
    for name, n in ph["phases"]:
        seg = disp[i:i + n]
        i += n
        if seg:
            avg = sum(e - s for s, e in seg) / len(seg) / 1e3
            print(f"  {name:<20} {len(seg):>6} dispatches  avg {avg:9.3f} us")


def pmc_summary(args) -> None:
    """Per-kernel HBM bytes from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of this
    bench, calibrated by the streaming-read probe's 4 GiB launches (known bytes read) in the
    same runs; for the kernel named by --pmc-kernel the HBM bytes per algorithmic byte
    (--pmc-alg-bytes per launch) and the hash of the decode FFN source."""
    fetch_dir, write_dir = args.pmc
    F = [r for r in _csv_rows(fetch_dir, "counter_collection.csv")
         if r.get("Counter_Name") == "FETCH_SIZE"]
    W = [r for r in _csv_rows(write_dir, "counter_collection.csv")
         if r.get("Counter_Name") == "WRITE_SIZE"]
    # the library's plain copy probe in the same runs: 2 GiB read and 2 GiB written
    cb = PROBE_SPAN // 2
    calib = sorted(float(r["Counter_Value"]) * 1024 / cb for r in F
                   if "stream_copy_kernel" in _kname(r))
    ff = calib[len(calib) // 2] if calib else 1.0
    wcal = sorted(float(r["Counter_Value"]) * 1024 / cb for r in W
                  if "stream_copy_kernel" in _kname(r))
    fw = wcal[len(wcal) // 2] if wcal else 1.0
    print(f"calibration (plain copy probe, 2 GiB read + 2 GiB written per launch): FETCH_SIZE / "
          f"bytes read {[round(c, 4) for c in calib]} -> factor {ff:.4f}; WRITE_SIZE / bytes "
          f"written {[round(c, 4) for c in wcal]} -> factor {fw:.4f}")
    agg = {}
    for r in F:
        a = agg.setdefault(_kname(r), [0, 0.0, 0, 0.0])
        a[0] += 1
        a[1] += float(r["Counter_Value"])
    for r in W:
        a = agg.setdefault(_kname(r), [0, 0.0, 0, 0.0])
        a[2] += 1
        a[3] += float(r["Counter_Value"])
    print(f"{'kernel':<52} {'calls':>6} {'FETCH_KiB':>11} {'WRITE_KiB':>11} {'read_MiB':>9} "
          f"{'write_MiB':>9}")
    ratio = None
    for n, (cf, fs, cw, ws) in sorted(agg.items()):
        if "moe::" not in n or cf == 0:
            continue
        fk, wk = fs / cf, (ws / cw if cw else 0.0)
        print(f"{n[:52]:<52} {cf:>6} {fk:>11.1f} {wk:>11.1f} {fk / ff / 1024:>9.2f} "
              f"{wk / fw / 1024:>9.2f}")
        if args.pmc_kernel and f"moe::{args.pmc_kernel}" in n and args.pmc_alg_bytes:
            hbm = (fk / ff + wk / fw) * 1024
            ratio = hbm / args.pmc_alg_bytes
            print(f"  hbm_bytes_per_launch: {hbm:.0f}  per algorithmic byte "
                  f"({args.pmc_alg_bytes / 2**20:.2f} MiB): {ratio:.4f}")
    print(f"\nffn_source_sha256_16: {_ffn_source_hash()}")
    if ratio is not None:
        print(f"hbm_bytes_per_algorithmic_byte: {ratio:.4f}")


# ------------------------------------------------------------------ main
def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480, help="timed decode tokens")
    ap.add_argument("--warmup", type=int, default=32, help="untimed decode tokens before")
    ap.add_argument("--workload", default="qwen35b_decode")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (0 = workload's)")
    ap.add_argument("--groups", type=int, default=0,
                    help="fill groups per step on a side stream (0: whole step on one stream)")
    ap.add_argument("--profile-every", type=int, default=7,
                    help="time one launch of the dominant FFN kernel in this many")
    ap.add_argument("--cache-frac", type=float, default=0.0,
                    help="override the cache fraction (1.0: every expert fits, FFN alone)")
    ap.add_argument("--breakdown-steps", type=int, default=16,
                    help="untimed tokens after the timed region with every kernel timed")
    ap.add_argument("--cpu-tokens", type=int, default=4, help="oracle sample (token steps)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="oracle sample repetitions")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="no per-kernel events")
    ap.add_argument("--no-probes", action="store_true", help="no streaming-read probes")
    ap.add_argument("--mode", choices=("offload", "auto", "hybrid"), default="offload",
                    help="which decode mode the headline reports: every miss filled (offload, "
                         "the hot path), the pages' mode rule (auto), or hybrid")
    ap.add_argument("--no-hybrid", action="store_true", help="skip the hybrid decode block")
    ap.add_argument("--cpu-threads", type=int, default=12,
                    help="host threads of the hybrid CPU expert path")
    ap.add_argument("--auto-capacity", action="store_true",
                    help="size the cache from the device's free memory (moe_auto_capacity_device)")
    ap.add_argument("--reserve-gb", type=float, default=0.0,
                    help="bytes kept out of the auto-sized cache (KV floor), GiB")
    ap.add_argument("--offload-ratio", type=float, default=-1.0,
                    help="auto-sized cache: at most (1 - r) of the experts (negative: no limit)")
    ap.add_argument("--pool-file", default="",
                    help="read the expert pool from this pool file instead of generating it")
    ap.add_argument("--phase-log", default="",
                    help="write the dominant FFN kernel's launches per phase to this JSON file "
                         "(with --rocprof-summary: read it)")
    ap.add_argument("--rocprof-summary", default="",
                    help="summarise a rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE)")
    ap.add_argument("--pmc-kernel", default="ffn_fused_kernel")
    ap.add_argument("--pmc-alg-bytes", type=float, default=0.0)
    args = ap.parse_args()
    args.steps_given = "--steps" in sys.argv
    args.warmup_given = "--warmup" in sys.argv
    if args.rocprof_summary:
        rocprof_summary(args)
        return
    if args.pmc:
        pmc_summary(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _die_multi_gpu(max(args.gpus, world))

    import moe_inputs as mi
    wl = mi.WORKLOADS[args.workload]
    if args.layers:
        wl = wl.with_layers(args.layers)
    if args.cache_frac > 0:
        wl = _with_cache_frac(wl, args.cache_frac)
    if wl.resize_at >= 0 and not args.steps_given:
        args.steps = wl.token_steps - args.warmup  # run through the resize to the end
    if wl.kind != "decode":
        run_prefill(args, wl)
        return
    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is touched: its workers are forked from this process
        cpu = cpu_baseline_decode(wl, args.cpu_tokens, args.cpu_reps)
        _log(f"oracle {cpu['value']:.4f} tok/s on {cpu['cores']} cores "
             f"(runs {cpu['seconds']} s, setup {cpu['setup_s']} s)")
    run_decode(args, wl, cpu)


if __name__ == "__main__":
    main()
