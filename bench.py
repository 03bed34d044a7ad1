#!/usr/bin/env python3
"""MoE-layer decode throughput of the expert-offload stack on one MI355X.

Workload (default): the 48-layer 35B-A3B-shaped MoE stack - hidden 2048, 128 experts top-8
with renormalised softmax, SwiGLU intermediate 768, bf16 expert weights N(0, 0.02) in a
pinned host pool (58 GB), one LRU slot cache shared by all layers holding 30% of the pool
(1,843 slots), AR(1) activations per layer, batch 1, seed 0, cold cache.  One step = one
decode token through all 48 layer steps (route, dedup, classify, LRU, fills, FFN).  The
first --warmup tokens are untimed; exactly --steps tokens are timed.

Reported (one JSON line): decode tokens/s of the stack; the dominant FFN kernel against the
MI355X HBM roofline (at one token with bf16 weights the fused gate/up + down kernel, which
streams whole blobs; otherwise the gate/up kernel, two thirds of the expert bytes) -
achieved = the expert-weight bytes it was given / its launch durations, timed
with event pairs on the compute stream over the timed tokens; fill bandwidth against pinned
hipMemcpyAsync H2D measured on the same box; the float64 CPU oracle on a bounded sample of
the same workload.  A short untimed pass after the timed tokens times the other kernels
(route/plan, fill, down) for the breakdown.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth


def _die_multi_gpu(n: int) -> None:
    print(f"bench.py: this build runs on one GPU only (--gpus {n} requested); "
          "the expert-offload path is measured on a single MI355X.", file=sys.stderr)
    sys.exit(2)


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
        # warm once, then time
        assert hip.hipMemcpyAsync(dev_buf_ptr, pool_addr, size, H2D, s) == 0
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


def _host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wb, tokens: int) -> dict:
    """The float64 oracle as it stands, on the first `tokens` token steps of the workload."""
    from threadpoolctl import threadpool_info

    from oracle.step import Oracle
    wl = wb.wl
    shared = (lambda l: wb.shared_np[l]) if wl.has_shared else None
    orc = Oracle(wl, wb.pool, wb.router_np, shared)
    t0 = time.perf_counter()
    for t in range(tokens):
        for l in range(wl.layers):
            x = wb.acts_np[t, l] if wl.kind == "decode" else wb.acts_np[l]
            orc.layer_step(t, l, x, True)
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {"value": tokens * wl.tokens_per_step / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {tokens} token step(s) x {wl.layers} layers of the same workload, "
                      f"full float64 route+top-k+dedup+LRU+SwiGLU FFN, {dt:.1f} s",
            "seconds": dt, "host_cpus": os.cpu_count(), "host_cpu_model": _host_cpu_model(),
            "lru_only_steps_per_s": _lru_only_rate(wb)}


def _lru_only_rate(wb, tokens: int = 64) -> float:
    """The oracle's LRU rule alone, single-threaded, in layer steps per second: the distinct
    expert sets of the first `tokens` token steps are routed by the oracle first (untimed),
    then replayed through a cold cache of the workload's size."""
    from oracle.dedup import dedup
    from oracle.formats import bf16_to_f64
    from oracle.lru import LRUCache
    from oracle.router import router_logits, topk_softmax
    wl = wb.wl
    tokens = min(tokens, wb.acts_np.shape[0])
    sets = []
    for t in range(tokens):
        for l in range(wl.layers):
            x = bf16_to_f64(wb.acts_np[t, l]).reshape(-1, wl.hidden)
            idx, _ = topk_softmax(router_logits(x, bf16_to_f64(wb.router_np[l])), wl.top_k)
            sets.append((l, dedup(idx, wl.experts)[0]))
    cache = LRUCache(wl.capacity, wl.n_keys)
    t0 = time.perf_counter()
    for s, (l, U) in enumerate(sets):
        cache.step(l, U, wl.experts, s)
    return round(len(sets) / (time.perf_counter() - t0), 1)


def hbm_stream_probe(dev) -> dict:
    """Measured device-memory streaming rates on this GPU (reference for the HBM roofline):
    a 4 GiB device-to-device copy (read + write bytes) and a 4 GiB sum (read bytes)."""
    import torch
    n = 1 << 32
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    copy = 2 * n * 5 / (time.perf_counter() - t0) / 1e9
    f = a.view(torch.float32)
    f.sum()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        f.sum()
    torch.cuda.synchronize()
    read = n * 5 / (time.perf_counter() - t0) / 1e9
    del a, b, f
    return {"copy_GBps": round(copy, 1), "read_GBps": round(read, 1), "bytes": n}


def _with_cache_frac(wl, frac: float):
    import dataclasses
    return dataclasses.replace(wl, name=f"{wl.name}_cache{frac:g}", cache_frac=frac,
                               fixed_capacity=0)


GATE_UP_END = "// ---------------------------------------------------------------- down role"


def _ffn_source_hash(kernel: str = "ffn_gate_up_kernel") -> str:
    """Hash of the decode FFN source a kernel's traffic depends on: for the gate/up kernel the
    source up to the down role (formats, entry resolution, the gate/up role; the down and
    combine kernels that follow do not change its traffic), for the fused kernel the file."""
    here = os.path.dirname(os.path.abspath(__file__))
    p = os.path.join(here, "expert_cache_offload_amd", "csrc", "ffn_decode.hip")
    text = open(p, "rb").read()
    cut = text.find(GATE_UP_END.encode()) if kernel == "ffn_gate_up_kernel" else -1
    return hashlib.sha256(text[:cut] if cut > 0 else text).hexdigest()[:16]


def _traffic_ratio_from_profile(name: str, kernel: str = "ffn_gate_up_kernel") -> float | None:
    """HBM bytes per algorithmic byte of the gate/up kernel from a committed counter summary,
    if it was taken on the current kernel source (its header line records the source hash).
    The counters are taken with every launch streaming the same number of experts; the bench
    scales the ratio by its own algorithmic bytes per launch."""
    here = os.path.dirname(os.path.abspath(__file__))
    p = os.path.join(here, "profiles", name)
    if not os.path.exists(p):
        return None
    h = _ffn_source_hash(kernel)
    val = None
    src_ok = False
    for line in open(p):
        if line.startswith("ffn_source_sha256_16:") and line.split(":", 1)[1].strip() == h:
            src_ok = True
        if line.startswith("hbm_bytes_per_algorithmic_byte:"):
            val = float(line.split(":", 1)[1])
    return val if src_ok else None


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


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


def run_prefill(args, wl) -> None:
    """Prefill chunks through the layer stack from a cold cache, each layer step prefetching
    the next layer's experts on the fill stream: tokens/s, the matrix-core FFN against the
    bf16 MFMA roofline, fills against pinned hipMemcpyAsync, and the same chunk with the
    layer's own fills double-buffered in groups, with and without prefetch."""
    import torch

    from expert_cache_offload_amd import (PROF_DOWN, PROF_FILL, PROF_GATE_UP, moe_profile_enable,
                                          moe_profile_read)
    from expert_cache_offload_amd.runner import Workbench

    groups = args.groups  # 0: the layer's own fills in stream order, prefetch on the side
    ab_groups = 16  # double-buffered fill groups of the ablation chunks
    steps = args.steps if args.steps_given else 5
    warmup = args.warmup if args.warmup_given else 1
    T, L, H, I, K = wl.tokens_per_step, wl.layers, wl.hidden, wl.inter, wl.top_k
    print(f"[bench] prefill {wl.name}: L={L} T={T} H={H} E={wl.experts} k={K} I={I} "
          f"C={wl.capacity} pool={wl.pool_bytes / 1e9:.2f} GB, {groups} fill groups",
          file=sys.stderr, flush=True)
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
        print(f"[bench] chunk {i}: {times[-1]:.3f} s", file=sys.stderr, flush=True)
    wall = sum(times)
    tok_s = steps * T / wall
    # one more chunk with the FFN kernels and fills timed (event pairs on the dispatches)
    wb.groups = groups
    wb.prefetch = True
    wb.reset()
    moe_profile_enable(wb.handle, PROF_GATE_UP | PROF_DOWN | PROF_FILL, 1)
    for l in range(L):
        wb.step(0, l)
    torch.cuda.synchronize()
    prof = moe_profile_read(wb.handle)
    st = wb.stats()
    db_prefetch = chunk(ab_groups)
    no_prefetch = chunk(ab_groups, prefetch=False)
    # the matrix-core kernels without concurrent fills: a chunk in stream order (each layer's
    # fills, then its FFN), gate/up and down timed
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
        print(f"[bench] oracle {cpu['value']:.2f} tok/s ({cpu['seconds']:.1f} s)",
              file=sys.stderr, flush=True)
    misses = st["misses"]
    wb.close()
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
                     "gate_up_TFLOPs": round(fl_gu / (iso["gate_up"]["ms"] / 1e3) / 1e12, 1)
                     if iso["gate_up"]["ms"] else None,
                     "gate_up_frac": round(fl_gu / (iso["gate_up"]["ms"] / 1e3) / 1e12 /
                                           MFMA_BF16_PEAK_TFLOPS, 4)
                     if iso["gate_up"]["ms"] else None,
                     "down_TFLOPs": round(fl_dn / (iso["down"]["ms"] / 1e3) / 1e12, 1)
                     if iso["down"]["ms"] else None},
        "cpu_baseline": cpu,
        "fill": {"bytes_per_chunk": fill_bytes, "misses_per_chunk": misses,
                 "kernel_GBps": round(fill_bytes / fk_s / 1e9, 2) if fk_s > 0 else None,
                 "h2d_memcpy_blob_GBps": round(h2d["blob_GBps"], 2),
                 "h2d_memcpy_1GiB_GBps": round(h2d["large_GBps"], 2)},
        "ablation": {"note": f"one chunk each, against the timed configuration ({groups} fill "
                             f"groups, prefetch of the next layer): the layer's own fills "
                             f"double-buffered in {ab_groups} groups with prefetch, and the "
                             f"same without prefetch",
                     "timed_median_s": round(sorted(times)[len(times) // 2], 4),
                     "prefetch_groups_s": round(db_prefetch, 4),
                     "no_prefetch_groups_s": round(no_prefetch, 4),
                     "no_prefetch_groups_over_timed":
                         round(no_prefetch / sorted(times)[len(times) // 2], 4)},
        "repeats": {"chunks": len(times),
                    "tok_s": [round(T / t, 1) for t in sorted(times, reverse=True)],
                    "median": round(T / sorted(times)[len(times) // 2], 1),
                    "min": round(T / max(times), 1), "max": round(T / min(times), 1)},
    }
    print(json.dumps(line), flush=True)


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
                    help="time one gate/up launch in this many during the timed region")
    ap.add_argument("--cache-frac", type=float, default=0.0,
                    help="override the cache fraction (1.0: every expert fits, FFN alone)")
    ap.add_argument("--breakdown-steps", type=int, default=16,
                    help="untimed tokens after the timed region with every kernel timed")
    ap.add_argument("--cpu-tokens", type=int, default=1, help="oracle sample (token steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="no per-kernel events")
    ap.add_argument("--mode", choices=("auto", "offload", "hybrid"), default="auto",
                    help="decode misses: fill all (offload), split with the CPU (hybrid), or "
                         "choose by the measured CPU/offload rate ratio against 2.0 (auto)")
    ap.add_argument("--cpu-threads", type=int, default=12,
                    help="host threads of the hybrid CPU expert path")
    ap.add_argument("--hybrid-rates", default="",
                    help="CPU,PCIe rates in MB/s: hybrid mode with these rates, no probe")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the offload run that follows a hybrid run")
    args = ap.parse_args()
    args.steps_given = "--steps" in sys.argv
    args.warmup_given = "--warmup" in sys.argv
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        _die_multi_gpu(max(args.gpus, world))

    import torch

    import moe_inputs as mi
    from expert_cache_offload_amd import (PROF_ALL, PROF_FILL, PROF_GATE_UP, choose_hybrid,
                                          moe_cpu_expert_rate, moe_hybrid_read,
                                          moe_profile_enable, moe_profile_read)
    from expert_cache_offload_amd.runner import Workbench

    wl = mi.WORKLOADS[args.workload]
    if args.layers:
        wl = wl.with_layers(args.layers)
    if args.cache_frac > 0:
        wl = _with_cache_frac(wl, args.cache_frac)
    if wl.resize_at >= 0 and not args.steps_given:
        args.steps = wl.token_steps - args.warmup  # run through the resize to the end
    n_tok = args.warmup + args.steps
    n_all = n_tok + args.breakdown_steps
    if wl.kind != "decode":
        run_prefill(args, wl)
        return
    wl = wl.with_steps(max(n_all, args.cpu_tokens))
    print(f"[bench] workload {wl.name}: L={wl.layers} H={wl.hidden} E={wl.experts} k={wl.top_k} "
          f"I={wl.inter} fmt={wl.fmt} C={wl.capacity} pool={wl.pool_bytes / 1e9:.2f} GB",
          file=sys.stderr, flush=True)
    t_setup = time.perf_counter()
    wb = Workbench(wl, groups=args.groups)
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    L = wl.layers
    resize_at = wl.resize_at if 0 <= wl.resize_at < n_tok else -1

    def token(t):
        for l in range(L):
            wb.step(t, l)

    def warm():
        for t in range(args.warmup):
            if t == resize_at:
                wb.sync()
                wb.resize(wl.resize_capacity)
            token(t)
            if t % 16 == 15:
                wb.sync()
                print(f"[bench] warmup token {t}", file=sys.stderr, flush=True)
        wb.sync()

    warm()
    # mode choice (bf16 only has a CPU path): the fill kernel's rate over a few tokens of the
    # offload run against the CPU expert path's rate on pool blobs, threshold 2.0x
    hybrid = None
    if args.mode != "offload" and wl.fmt != 0:
        hybrid = {"mode": "offload", "note": "no CPU expert path for this weight format"}
    if args.hybrid_rates and wl.fmt == 0:
        bc, bp = (int(v) for v in args.hybrid_rates.split(","))
        hybrid = {"mode": "hybrid", "cpu_expert_GBps": bc / 1e3, "offload_GBps": bp / 1e3,
                  "ratio": round(bc / bp, 3), "threshold": 2.0, "cpu_threads": args.cpu_threads,
                  "choice": "given"}
        wb.set_hybrid(bc, bp, args.cpu_threads)
        wb.reset()
        warm()
    elif args.mode != "offload" and wl.fmt == 0:
        moe_profile_enable(wb.handle, PROF_FILL)
        for t in range(8):
            token(t)
        pf = moe_profile_read(wb.handle)
        moe_profile_enable(wb.handle, 0)
        pcie = pf["fill_bytes"] / (pf["fill"]["ms"] / 1e3) / 1e9 if pf["fill"]["ms"] else 0.0
        cpu_rate = moe_cpu_expert_rate(wb.shape, wb.pool_addr, 48, args.cpu_threads, 2)
        use = args.mode == "hybrid" or choose_hybrid(cpu_rate, pcie)
        hybrid = {"mode": "hybrid" if use else "offload", "cpu_expert_GBps": round(cpu_rate, 2),
                  "offload_GBps": round(pcie, 2), "ratio": round(cpu_rate / pcie, 3) if pcie else None,
                  "threshold": 2.0, "cpu_threads": args.cpu_threads,
                  "choice": "forced" if args.mode == "hybrid" else "measured"}
        print(f"[bench] CPU expert path {cpu_rate:.1f} GB/s, fills {pcie:.1f} GB/s -> "
              f"{hybrid['mode']}", file=sys.stderr, flush=True)
        if use:
            wb.set_hybrid(int(cpu_rate * 1000), int(pcie * 1000), args.cpu_threads)
            wb.reset()  # from a cold cache again, now splitting misses
            h0 = moe_hybrid_read(wb.handle)
            warm()
            # the CPU path's rate re-measured on the warmup's own requests (the probe runs one
            # expert per call and reads lower): the split uses the rate the server sustained
            h1 = moe_hybrid_read(wb.handle)
            busy = h1["busy_s"] - h0["busy_s"]
            if busy > 0 and h1["experts"] > h0["experts"]:
                eff = (h1["experts"] - h0["experts"]) * wl.blob_bytes / busy / 1e9
                hybrid["cpu_rate_warmup_GBps"] = round(eff, 2)
                wb.set_hybrid(int(eff * 1000), int(pcie * 1000), args.cpu_threads)
                print(f"[bench] CPU path sustained {eff:.1f} GB/s over the warmup: split "
                      "recomputed with it", file=sys.stderr, flush=True)
    st0 = wb.stats()
    hy0 = moe_hybrid_read(wb.handle)
    if not args.no_profile:
        moe_profile_enable(wb.handle, PROF_GATE_UP, args.profile_every)
    # the timed tokens in windows (their rates give median / min / max); a cache resize at a
    # safe point inside the timed region is timed on its own and counted in the total
    n_win = 5
    bounds = [args.warmup + (args.steps * i) // n_win for i in range(n_win + 1)]
    segments, resize_s = [], None  # (tokens, seconds, "before" | "after" the resize)
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
            print(f"[bench] tokens {t}..{stop - 1}: {(stop - t) * wl.tokens_per_step / segments[-1][1]:.2f} "
                  "tok/s", file=sys.stderr, flush=True)
            t = stop
    wall = sum(dt for _, dt, _ in segments) + (resize_s or 0.0)
    prof = moe_profile_read(wb.handle) if not args.no_profile else None
    st1 = wb.stats()
    hy1 = moe_hybrid_read(wb.handle)
    if hybrid is not None and hybrid["mode"] == "hybrid":
        busy = hy1["busy_s"] - hy0["busy_s"]
        ex = hy1["experts"] - hy0["experts"]
        hybrid["cpu_busy_frac"] = round(busy / wall, 4) if wall > 0 else None
        hybrid["cpu_effective_GBps"] = round(ex * wl.blob_bytes / busy / 1e9, 2) if busy else None
        hybrid["requests"] = hy1["requests"] - hy0["requests"]
    brk = None
    if not args.no_profile and args.breakdown_steps > 0:
        moe_profile_enable(wb.handle, PROF_ALL)
        for t in range(n_tok, n_all):
            token(t)
        brk = moe_profile_read(wb.handle)
        moe_profile_enable(wb.handle, 0)
    hits = st1["hits"] - st0["hits"]
    misses = st1["misses"] - st0["misses"]
    cpu_misses = st1["cpu_misses"] - st0["cpu_misses"]
    if hybrid is not None and hybrid["mode"] == "hybrid" and not args.no_ablation:
        # ablation: the same tokens with every miss filled, from a cold cache
        wb.set_hybrid(0)
        wb.reset()
        warm()
        n_ab = min(96, args.steps)
        torch.cuda.synchronize()
        a0 = time.perf_counter()
        for t in range(args.warmup, args.warmup + n_ab):
            token(t)
        torch.cuda.synchronize()
        hybrid["offload_tok_s"] = round(n_ab * wl.tokens_per_step / (time.perf_counter() - a0), 3)
        hybrid["offload_tokens"] = n_ab
        print(f"[bench] offload ablation {hybrid['offload_tok_s']:.2f} tok/s", file=sys.stderr,
              flush=True)
    fill_bytes = st1["bytes_filled"] - st0["bytes_filled"]
    tokens = args.steps * wl.tokens_per_step
    tok_s = tokens / wall
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s -> {tok_s:.2f} tok/s; "
          f"miss rate {misses / max(1, hits + misses):.3f}", file=sys.stderr, flush=True)

    # pinned hipMemcpyAsync H2D on this machine (denominator of the fill bar)
    scratch = torch.empty(min(1 << 30, wl.capacity * wl.blob_bytes), dtype=torch.uint8,
                          device=wb.dev)
    h2d = h2d_memcpy_probe(wb.pool_addr, wb.pool_bytes, wl.blob_bytes, scratch.data_ptr(),
                           scratch.numel())
    del scratch

    roofline = None
    fill = {"bytes": fill_bytes, "link_GBps": fill_bytes / wall / 1e9,
            "h2d_memcpy_blob_GBps": h2d["blob_GBps"], "h2d_memcpy_1GiB_GBps": h2d["large_GBps"]}
    extra = {}
    if prof is not None:
        gu = prof["gate_up"]
        gu_bytes = prof["gate_up_timed_bytes"]  # expert bytes the timed launches were given
        gu_s = gu["ms"] / 1e3
        achieved = gu_bytes / gu_s / 1e9 if gu_s > 0 else 0.0
        fused = gu_bytes > 0 and prof["fused_timed_bytes"] == gu_bytes
        kname = "ffn_fused_kernel" if fused else "ffn_gate_up_kernel"
        ratio = _traffic_ratio_from_profile(
            f"{'ffn_fused' if fused else 'ffn_gate_up'}_{wl.name}_pmc.txt", kname)
        traffic = round(ratio * gu_bytes / max(1, gu["launches"])) if ratio else None
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic, "kernel": kname,
                    "launches": gu["launches"],
                    "avg_launch_us": round(gu["ms"] * 1e3 / max(1, gu["launches"]), 3),
                    "algorithmic_bytes_per_launch": round(gu_bytes / max(1, gu["launches"]))}
    if brk is not None:
        nb = args.breakdown_steps
        per = lambda k: round(brk[k]["ms"] * 1e3 / max(1, brk[k]["launches"]), 2)  # noqa: E731
        fk = brk["fill"]
        fill_kernel_gbps = brk["fill_bytes"] / (fk["ms"] / 1e3) / 1e9 if fk["ms"] else 0.0
        fill.update({"kernel_GBps": round(fill_kernel_gbps, 2),
                     "kernel_frac_of_memcpy": round(fill_kernel_gbps / h2d["blob_GBps"], 3)})
        extra["breakdown"] = {
            "tokens": nb, "note": "untimed tokens after the timed region, every launch timed",
            "route_us_per_launch": per("route"), "fill_us_per_launch": per("fill"),
            "gate_up_us_per_launch": per("gate_up"), "down_us_per_launch": per("down"),
            "route_ms_per_token": round(brk["route"]["ms"] / nb, 3),
            "fill_ms_per_token": round(fk["ms"] / nb, 3),
            "gate_up_ms_per_token": round(brk["gate_up"]["ms"] / nb, 3),
            "down_ms_per_token": round(brk["down"]["ms"] / nb, 3)}
    fill["link_frac_of_memcpy"] = round(fill["link_GBps"] / h2d["blob_GBps"], 3)
    T = wl.tokens_per_step
    rates = sorted(n * T / dt for n, dt, _ in segments if n > 0)
    extra["repeats"] = {"windows": len(rates), "tok_s": [round(r, 3) for r in rates],
                        "median": round(rates[len(rates) // 2], 3), "min": round(rates[0], 3),
                        "max": round(rates[-1], 3)}
    if resize_s is not None:
        side = {k: (sum(n for n, _, sd in segments if sd == k),
                    sum(dt for _, dt, sd in segments if sd == k)) for k in ("before", "after")}
        extra["resize"] = {
            "at_token_step": resize_at, "from_slots": wl.capacity,
            "to_slots": wl.resize_capacity, "latency_ms": round(resize_s * 1e3, 3),
            "tok_s_before": round(side["before"][0] * T / side["before"][1], 3)
            if side["before"][1] > 0 else None,
            "tok_s_after": round(side["after"][0] * T / side["after"][1], 3)
            if side["after"][1] > 0 else None}
    extra["hbm_stream"] = hbm_stream_probe(wb.dev)
    if roofline is not None:
        roofline["frac_of_measured_read"] = round(
            roofline["achieved"] / extra["hbm_stream"]["read_GBps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wb, args.cpu_tokens)
        print(f"[bench] oracle {cpu['value']:.4f} tok/s ({cpu['seconds']:.1f} s)", file=sys.stderr,
              flush=True)
    wb.close()

    dtype = {0: "bf16", 1: "fp8", 2: "mxfp4"}[wl.fmt]
    line = {
        "metric": "MoE decode tokens/s per layer stack + HBM GB/s fraction; miss-fill PCIe GB/s",
        "value": round(tok_s, 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "hidden": wl.hidden,
                   "experts": wl.experts, "top_k": wl.top_k, "inter": wl.inter,
                   "cache_slots": wl.capacity, "pool_bytes": wl.pool_bytes,
                   "tokens_per_step": wl.tokens_per_step, "fill_groups": args.groups,
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fill": fill,
        "miss_rate": round(misses / max(1, hits + misses), 4),
        "misses_per_token": round(misses / max(1, tokens), 2),
        "cpu_misses_per_token": round(cpu_misses / max(1, tokens), 2),
        "hybrid": hybrid,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
