"""Drives the layer step over a synthetic workload on one GPU (allocation and marshalling only).

A ``Workbench`` owns the device buffers of one workload: the pinned host expert pool
(filled in place by the seeded generator), router weights, activations, shared-expert
blobs, the slot arena, the workspace and two streams (compute and fill).  ``step(t, l)``
issues one ``moe_layer_step`` for token step t and layer l.  Every step of the method runs
in the HIP library; this module only allocates memory with PyTorch and passes pointers.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

import moe_inputs as mi

from . import (make_shape, moe_cache_create, moe_cache_destroy, moe_cache_resize,
               moe_cache_snapshot, moe_expert_ffn, moe_fill_misses, moe_host_pool_alloc,
               moe_host_pool_free, moe_layer_step, moe_plan_read, moe_pool_read, moe_route_classify,
               moe_set_hybrid, moe_set_prefetch, moe_stats, moe_workspace_bytes)


def pinned_view(addr: int, nbytes: int) -> np.ndarray:
    buf = (ctypes.c_uint8 * nbytes).from_address(addr)
    return np.frombuffer(buf, dtype=np.uint8)


class Workbench:
    def __init__(self, wl, device: str = "cuda:0", groups: int = 2, capacity: int | None = None,
                 max_capacity: int | None = None, gen_threads: int = 0, token_steps=None,
                 compute_stream=None, fill_stream=None, pool_file: str | None = None,
                 pool_threads: int = 8):
        self.wl = wl
        self.dev = torch.device(device)
        self.groups = groups
        self.T = wl.tokens_per_step
        self.n_tok = wl.token_steps if token_steps is None else token_steps
        L, E, H, I, K = wl.layers, wl.experts, wl.hidden, wl.inter, wl.top_k
        self.capacity = wl.capacity if capacity is None else capacity
        caps = [self.capacity]
        if wl.resize_at >= 0:
            caps.append(wl.resize_capacity)
        self.max_capacity = max(caps) if max_capacity is None else max_capacity
        self.shape = make_shape(L, E, K, H, I, wl.fmt, wl.has_shared, self.T)
        self.S = wl.blob_bytes
        # pinned host pool: generated in place, or read from a pool file in the runtime
        # layout by the library's parallel readers straight into the pinned memory
        self.pool_bytes = L * E * self.S
        self.pool_addr = moe_host_pool_alloc(self.pool_bytes)
        self.pool = pinned_view(self.pool_addr, self.pool_bytes)
        if pool_file:
            moe_pool_read(pool_file, self.shape, self.pool_addr, pool_threads)
        else:
            mi.fill_pool(wl.seed, wl.fmt, 0, L, E, H, I, self.pool_addr, gen_threads)
        # GPU-resident inputs
        self.router_np = mi.router_weights(wl.seed, 0, L, E, H, nthreads=gen_threads)
        self.router = torch.from_numpy(self.router_np.view(np.int16)).to(self.dev)
        if wl.kind == "decode":
            self.acts_np = mi.decode_acts(wl.seed, 0, L, self.T, self.n_tok, H,
                                          nthreads=gen_threads)
        else:
            self.acts_np = mi.prefill_acts(wl.seed, 0, L, self.T, H, nthreads=gen_threads)
        self.acts = torch.from_numpy(self.acts_np.view(np.int16)).to(self.dev)
        self.shared_np = None
        self.shared = None
        if wl.has_shared:
            self.shared_np = np.stack([mi.shared_blob(wl.seed, wl.fmt, l, H, I) for l in range(L)])
            self.shared = torch.from_numpy(self.shared_np).to(self.dev)
        self.arena = torch.empty(self.max_capacity * self.S, dtype=torch.uint8, device=self.dev)
        self.ws = torch.empty(moe_workspace_bytes(self.shape, self.max_capacity),
                              dtype=torch.uint8, device=self.dev)
        self.y = torch.zeros((L, self.T, H), dtype=torch.int16, device=self.dev)
        self.topk_idx = torch.zeros((L, self.T, K), dtype=torch.int32, device=self.dev)
        self.topk_w = torch.zeros((L, self.T, K), dtype=torch.float32, device=self.dev)
        self.compute = compute_stream or torch.cuda.Stream(device=self.dev)
        self.fill = fill_stream or torch.cuda.Stream(device=self.dev)
        torch.cuda.synchronize(self.dev)
        self.handle = moe_cache_create(self.shape, self.capacity, self.max_capacity, self.arena,
                                       self.ws, self.pool_addr, self.compute.cuda_stream)
        torch.cuda.synchronize(self.dev)

    # ---- pointers ----
    def x_ptr(self, t: int, l: int) -> int:
        if self.wl.kind == "decode":
            return self.acts[t, l].data_ptr()
        return self.acts[l].data_ptr()

    def shared_ptr(self, l: int):
        return None if self.shared is None else self.shared[l].data_ptr()

    # ---- steps ----
    def step(self, t: int, l: int, T: int | None = None) -> None:
        T = self.T if T is None else T
        moe_layer_step(self.handle, l, self.x_ptr(t, l), T, self.router[l].data_ptr(),
                       self.shared_ptr(l), self.y[l].data_ptr(), self.topk_idx[l].data_ptr(),
                       self.topk_w[l].data_ptr(), self.groups, self.compute.cuda_stream,
                       self.fill.cuda_stream)

    def step_parts(self, t: int, l: int) -> None:
        """The same step through the three separate calls."""
        moe_route_classify(self.handle, l, self.x_ptr(t, l), self.T, self.router[l].data_ptr(),
                           self.topk_idx[l].data_ptr(), self.topk_w[l].data_ptr(),
                           self.compute.cuda_stream)
        moe_fill_misses(self.handle, max(1, self.groups), self.fill.cuda_stream)
        moe_expert_ffn(self.handle, l, self.x_ptr(t, l), self.T, self.shared_ptr(l),
                       self.y[l].data_ptr(), self.compute.cuda_stream)

    def resize(self, new_capacity: int, new_arena=None) -> None:
        moe_cache_resize(self.handle, new_capacity, new_arena, self.compute.cuda_stream)
        if new_arena is not None:
            self.sync()  # the old arena is read by the copy before it may be released
            self.arena = new_arena
        self.capacity = new_capacity

    def reset(self) -> None:
        """Start again from an empty cache (a new handle over the same arena and workspace)."""
        self.sync()
        moe_cache_destroy(self.handle)
        self.handle = moe_cache_create(self.shape, self.capacity, self.max_capacity, self.arena,
                                       self.ws, self.pool_addr, self.compute.cuda_stream)
        self.sync()
        if getattr(self, "prefetch", False):
            moe_set_prefetch(self.handle, True)
        if getattr(self, "hybrid", None):
            moe_set_hybrid(self.handle, *self.hybrid)

    def set_prefetch(self, enable: bool) -> None:
        self.prefetch = bool(enable)
        moe_set_prefetch(self.handle, self.prefetch)

    def set_hybrid(self, b_cpu_mbps: int, b_pcie_mbps: int = 0, threads: int = 8) -> None:
        """Split decode misses between fills and the CPU (b_cpu_mbps 0: off)."""
        self.sync()
        self.hybrid = (int(b_cpu_mbps), int(b_pcie_mbps), int(threads)) if b_cpu_mbps else None
        moe_set_hybrid(self.handle, int(b_cpu_mbps), int(b_pcie_mbps), int(threads))

    def sync(self) -> None:
        torch.cuda.synchronize(self.dev)

    # ---- state readback (synchronous) ----
    def snapshot(self):
        return moe_cache_snapshot(self.handle, self.capacity, self.wl.n_keys)

    def plan(self):
        umax = min(self.T * self.wl.top_k, self.wl.experts)
        return moe_plan_read(self.handle, umax, self.T * self.wl.top_k)

    def stats(self):
        return moe_stats(self.handle)

    def y_f64(self, l: int) -> np.ndarray:
        u = self.y[l].cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)

    def slot_bytes(self, slot: int) -> np.ndarray:
        return self.arena[slot * self.S:(slot + 1) * self.S].cpu().numpy()

    def close(self) -> None:
        if getattr(self, "handle", None):
            self.sync()
            moe_cache_destroy(self.handle)
            self.handle = None
        if getattr(self, "pool_addr", None):
            self.pool = None
            moe_host_pool_free(self.pool_addr)
            self.pool_addr = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
