"""moe_cache_create_static (the library's static per-device workspace, no allocation) against
moe_cache_create (a caller workspace): the same steps over the same arena and pool give
bit-identical integer streams, cache state and layer outputs.  Two handles in a row, the second
on a smaller input, so the second starts from the first one's leftover array contents."""
import dataclasses
import sys

import numpy as np
import pytest

import moe_inputs as mi

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _record(wb, t, l):
    wb.sync()
    p = wb.plan()
    key_of, stamp, slot_of, n, step, cap = wb.snapshot()
    return {"y": wb.y[l].cpu().numpy().copy(), "idx": wb.topk_idx[l].cpu().numpy().copy(),
            "w": wb.topk_w[l].cpu().numpy().copy(), "plan": p, "key_of": key_of.copy(),
            "stamp": stamp.copy(), "slot_of": slot_of.copy(), "n": n, "step": step}


def _run(wb, tokens):
    out = []
    for t in range(tokens):
        for l in range(wb.wl.layers):
            wb.step(t, l)
            out.append(_record(wb, t, l))
    return out


def _same(a, b, ctx):
    for k in ("y", "idx", "w", "key_of", "stamp", "slot_of"):
        assert np.array_equal(a[k], b[k]), f"{ctx}: {k}"
    assert a["n"] == b["n"] and a["step"] == b["step"], ctx
    for k, v in a["plan"].items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b["plan"][k]), f"{ctx}: plan {k}"
        else:
            assert v == b["plan"][k], f"{ctx}: plan {k}"


def _compare(wl, tokens, groups):
    from expert_cache_offload_amd import (moe_cache_create_static, moe_cache_destroy)
    from expert_cache_offload_amd.runner import Workbench
    with Workbench(wl, groups=groups, token_steps=tokens) as wb:
        ref = _run(wb, tokens)           # caller workspace
        wb.sync()
        moe_cache_destroy(wb.handle)
        wb.handle = None
        wb.handle = moe_cache_create_static(wb.shape, wb.capacity, wb.max_capacity, wb.arena,
                                            wb.pool_addr, wb.compute.cuda_stream)
        got = _run(wb, tokens)           # static workspace
        for i, (a, b) in enumerate(zip(ref, got)):
            _same(a, b, f"{wl.name} step {i}")
    return len(ref)


def test_static_workspace_matches_caller_workspace_twice():
    big = dataclasses.replace(mi.WORKLOADS["qwen35b_decode"].with_layers(3), fixed_capacity=40)
    _log(f"case {big.name} static workspace, 6 tokens, one queue")
    n1 = _compare(big, 6, 0)
    small = mi.WORKLOADS["tiny"]
    _log(f"case {small.name} static workspace (smaller input, after the first), 12 tokens, "
         "fill groups 2")
    n2 = _compare(small, 12, 2)
    _log(f"static workspace: {n1} + {n2} layer steps bit-identical")


def test_static_workspace_refusals():
    import torch

    from expert_cache_offload_amd import (MOE_E_BUSY, MOE_E_SCRATCH, MoeError, make_shape,
                                          moe_cache_create_static, moe_cache_destroy,
                                          moe_host_pool_alloc, moe_host_pool_free)
    wl = mi.WORKLOADS["tiny"]
    shape = make_shape(wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.fmt, False, 1)
    big = make_shape(wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.fmt, False, 65536)
    pool = moe_host_pool_alloc(wl.pool_bytes)
    arena = torch.empty(16 * wl.blob_bytes, dtype=torch.uint8, device="cuda:0")
    try:
        with pytest.raises(MoeError) as ei:
            moe_cache_create_static(big, 8, 16, arena, pool)
        assert ei.value.status == MOE_E_SCRATCH
        h = moe_cache_create_static(shape, 8, 16, arena, pool)
        with pytest.raises(MoeError) as ei:
            moe_cache_create_static(shape, 8, 16, arena, pool)
        assert ei.value.status == MOE_E_BUSY
        torch.cuda.synchronize()
        moe_cache_destroy(h)
        h = moe_cache_create_static(shape, 8, 16, arena, pool)  # released by destroy
        torch.cuda.synchronize()
        moe_cache_destroy(h)
    finally:
        torch.cuda.synchronize()
        moe_host_pool_free(pool)
