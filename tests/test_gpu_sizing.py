"""Budget-driven cache sizing and pool files on the device (GPU).

The cache is sized from the device's free memory as hipMemGetInfo reports it
(moe_auto_capacity_device) and checked against the oracle's sizing arithmetic for the same
free byte count; the pool is written to a file in the runtime layout and read back by the
library's parallel readers into pinned memory; decode steps over that handle and pool match
the float64 oracle, whose expert weights come straight from the seeded generator (not from
the file).  Pages: "FreeToken vs vLLM on one RTX 3090", Runtime configurations (automatic
cache); "FreeToken: az VRAM ile büyük MoE modelleri", "KV cache" (KV floor reserved first);
"FreeToken：在消费级 NVIDIA GPU 上进行 MoE 推理" (--offload-ratio); FreeToken paper summary,
execution-layer paragraph (runtime-layout weights loaded into their final place)."""
import dataclasses
import sys

import numpy as np
import pytest

import moe_inputs as mi
from parity import compare_step

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_capacity(shape, wl, free, reserve, ratio):
    from expert_cache_offload_amd import moe_workspace_bytes
    from oracle.sizing import auto_capacity
    floor = min(wl.tokens_per_step * wl.top_k, wl.experts)
    return auto_capacity(free, reserve, wl.blob_bytes, wl.n_keys, floor, 4096,
                         lambda c: moe_workspace_bytes(shape, c),
                         None if ratio < 0 else ratio)


def test_device_sized_cache_over_a_pool_file(tmp_path):
    from expert_cache_offload_amd import (MOE_E_CAPACITY, MoeError, make_shape,
                                          moe_auto_capacity_device, moe_pool_write)
    from expert_cache_offload_amd.runner import Workbench
    from oracle.step import Oracle
    wl = mi.WORKLOADS["qwen35b_decode"].with_layers(2).with_steps(10)
    shape = make_shape(wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.fmt,
                       wl.has_shared, wl.tokens_per_step)
    # keep 30% of the experts on the device (offload ratio 0.7): the ratio binds on 288 GB
    cap, free = moe_auto_capacity_device(shape, 0, 0.7)
    assert cap == _oracle_capacity(shape, wl, free, 0, 0.7) == int(0.3 * wl.n_keys), (cap, free)
    # a reserve that leaves room for about 100 slots: the free-memory budget binds
    S = wl.blob_bytes
    reserve = free - 100 * S - (64 << 20)
    cap2, free2 = moe_auto_capacity_device(shape, reserve, -1.0)
    assert cap2 == _oracle_capacity(shape, wl, free2, reserve, -1.0), (cap2, free2)
    assert 90 <= cap2 <= 107, cap2
    with pytest.raises(MoeError) as ei:  # nothing left once the reserve is taken
        moe_auto_capacity_device(shape, free2 + (1 << 30), -1.0)
    assert ei.value.status == MOE_E_CAPACITY
    _log(f"auto capacity: {cap} slots (ratio 0.7), {cap2} slots (budget) of {free / 2**30:.1f} "
         f"GiB free")
    path = str(tmp_path / "qwen_L2.pool")
    with Workbench(wl, groups=0, capacity=8, token_steps=1) as gen:  # generated pool, saved
        moe_pool_write(path, shape, gen.pool_addr, 8)
    with Workbench(wl, groups=0, capacity=cap, pool_file=path) as wb:
        assert wb.capacity == cap
        blob = lambda key: mi.expert_blob(wl.seed, wl.fmt, mi.PURPOSE_EXPERT,  # noqa: E731
                                          key // wl.experts, key % wl.experts, wl.hidden,
                                          wl.inter)
        orc = Oracle(dataclasses.replace(wl, fixed_capacity=cap), blob, wb.router_np)
        errs = []
        for t in range(wl.token_steps):
            for l in range(wl.layers):
                wb.step(t, l)
                ref = orc.layer_step(t, l, wb.acts_np[t, l], True)
                errs.append(compare_step(wb, ref, f"auto-sized t={t} l={l}"))
        st = wb.stats()
    _log(f"auto-sized {cap} slots over the pool file: {len(errs)} layer steps, max rel-L2 "
         f"{max(errs):.2e}, misses {st['misses']}")
