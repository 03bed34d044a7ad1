"""The step counter and the stamps are 64-bit: a handle whose counter is set just below 2^32
(moe_cache_set_step on an empty cache) keeps matching the oracle, whose integers are unbounded,
across the 2^32 boundary - victims chosen by stamp order, a resize that keeps the most recently
used keys, and prefetch steps of a prefill chunk."""
import dataclasses
import sys

import pytest

import moe_inputs as mi
from parity import compare_step

pytestmark = pytest.mark.gpu

START = (1 << 32) - 5


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_decode_across_2_to_the_32_with_resize():
    from expert_cache_offload_amd import MOE_E_INVALID, MoeError, moe_cache_set_step
    from expert_cache_offload_amd.runner import Workbench
    from oracle.step import Oracle
    wl = mi.WORKLOADS["tiny"].with_steps(24)
    with Workbench(wl, groups=0, max_capacity=8) as wb:
        moe_cache_set_step(wb.handle, START)
        orc = Oracle(wl, wb.pool, wb.router_np)
        orc.s = START
        for t in range(wl.token_steps):
            if t == 16:  # a safe point after the crossing: keep the 4 most recently used
                orc.resize(4)
                wb.resize(4)
                key_of, stamp, slot_of, n, step, cap = wb.snapshot()
                assert list(key_of) == orc.cache.key_of and list(stamp) == orc.cache.stamp
            wb.step(t, 0)
            ref = orc.layer_step(t, 0, wb.acts_np[t, 0], True)
            compare_step(wb, ref, f"tiny s={ref.s}")
        key_of, stamp, slot_of, n, step, cap = wb.snapshot()
        assert step == START + wl.token_steps > (1 << 32)
        assert min(stamp) < (1 << 32) <= max(stamp) or min(stamp) >= (1 << 32)
        with pytest.raises(MoeError) as ei:  # the cache holds experts now
            moe_cache_set_step(wb.handle, 0)
        assert ei.value.status == MOE_E_INVALID
    _log(f"decode across 2^32: {wl.token_steps} steps from {START}, resize to 4 slots")


def test_prefill_prefetch_across_2_to_the_32():
    from expert_cache_offload_amd import moe_cache_set_step
    from expert_cache_offload_amd.runner import Workbench
    from oracle.step import Oracle
    base = dataclasses.replace(mi.WORKLOADS["tiny"], layers=5, fixed_capacity=40)
    wl = base.as_prefill(100)
    with Workbench(wl, groups=0) as wb:
        moe_cache_set_step(wb.handle, START)
        wb.set_prefetch(True)
        orc = Oracle(wl, wb.pool, wb.router_np)
        orc.s = START
        for l in range(wl.layers):
            wb.step(0, l)
            ref = orc.layer_step(0, l, wb.acts_np[l], True)
            compare_step(wb, ref, f"prefill s={ref.s}", check_state=False)
            if l + 1 < wl.layers:
                orc.prefetch(l + 1, l, ref.U)
            key_of, stamp, slot_of, n, step, cap = wb.snapshot()
            assert step == orc.s and n == orc.cache.n
            assert list(key_of) == orc.cache.key_of and list(stamp) == orc.cache.stamp, l
    _log(f"prefill with prefetch across 2^32: {wl.layers} layers from {START}")
