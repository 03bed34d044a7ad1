"""GPU parity of hybrid decode: each step's misses split between PCIe fills and in-place CPU
compute (the route kernel derives q, the host server computes the CPU experts from the pinned
pool, the combine adds them), against the float64 oracle with the same integer rates.

Integer results - including which misses went to the CPU - and the cache state are compared
bit-exactly every step; layer outputs within the bf16 relative-L2 tolerance per token."""
import sys

import numpy as np
import pytest

import moe_inputs as mi
from parity import compare_step

pytestmark = pytest.mark.gpu

RATES = (124_500, 56_000)  # CPU expert rate, PCIe fill rate (MB/s): 1-3 misses mostly to the CPU


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(wl, n_tok, groups, rates=RATES, threads=6, switch_off_at=None, ffn_every=1,
         state_every=1):
    from expert_cache_offload_amd.runner import Workbench
    from oracle.step import Oracle
    with Workbench(wl, groups=groups) as wb:
        orc = Oracle(wl, wb.pool, wb.router_np, split=rates)
        # the first step follows at once: the request may be posted before the server thread
        # has started
        wb.set_hybrid(rates[0], rates[1], threads)
        worst, n_cpu, n_miss = 0.0, 0, 0
        for t in range(n_tok):
            if switch_off_at is not None and t == switch_off_at:
                wb.set_hybrid(0)
                orc.split = None
            for l in range(wl.layers):
                wb.step(t, l)
                k = t * wl.layers + l
                ref = orc.layer_step(t, l, wb.acts_np[t, l], k % ffn_every == 0)
                err = compare_step(wb, ref, f"{wl.name} hybrid t={t} l={l}",
                                   check_state=k % state_every == 0)
                worst = max(worst, err or 0.0)
                n_cpu += len(ref.rec.cpu)
                n_miss += len(ref.rec.cpu) + len(ref.rec.misses)
        st = wb.stats()
        assert st["cpu_misses"] == n_cpu and st["misses"] == n_miss
        return worst, n_cpu, n_miss


def test_hybrid_tiny_every_step():
    wl = mi.WORKLOADS["tiny"].with_steps(48)
    worst, n_cpu, n_miss = _run(wl, wl.token_steps, groups=0, threads=12)
    _log(f"tiny hybrid: max rel-L2 {worst:.2e}, {n_cpu} of {n_miss} misses on the CPU")
    assert n_cpu > 0


@pytest.mark.parametrize("groups", [0, 2])
def test_hybrid_35b_shape(groups):
    wl = mi.WORKLOADS["qwen35b_decode"].with_layers(4).with_steps(16)
    worst, n_cpu, n_miss = _run(wl, wl.token_steps, groups=groups)
    _log(f"35B hybrid groups={groups}: max rel-L2 {worst:.2e}, {n_cpu} of {n_miss} misses on the CPU")
    assert n_cpu > 0 and n_cpu < n_miss


def test_hybrid_eight_streams_then_off():
    wl = mi.WORKLOADS["qwen35b_decode_b8"].with_layers(3).with_steps(8)
    worst, n_cpu, n_miss = _run(wl, wl.token_steps, groups=0, threads=8, switch_off_at=5)
    _log(f"8 streams hybrid: max rel-L2 {worst:.2e}, {n_cpu} of {n_miss} misses on the CPU")
    assert n_cpu > 0


def test_hybrid_cpu_slower_than_pcie():
    # CPU at 40 GB/s against 56: one miss is filled, two split one-one, five put two on the CPU
    wl = mi.WORKLOADS["qwen35b_decode"].with_layers(2).with_steps(12)
    worst, n_cpu, n_miss = _run(wl, wl.token_steps, groups=0, rates=(40_000, 56_000))
    _log(f"35B hybrid, slow CPU: max rel-L2 {worst:.2e}, {n_cpu} of {n_miss} misses on the CPU")
    assert 0 < n_cpu < n_miss


def test_full_size_hybrid_decode_sampled():
    """The 48-layer 35B-A3B decode stack at full size (58 GB pinned pool, 1,843 slots) in
    hybrid mode with 12 host threads: every integer result (CPU misses included) of 40 token
    steps (1,920 layer steps), cache state and outputs sampled."""
    wl = mi.WORKLOADS["qwen35b_decode"].with_steps(40)
    _log(f"case {wl.name} full size hybrid, 40 tokens")
    worst, n_cpu, n_miss = _run(wl, wl.token_steps, groups=0, rates=(160_000, 56_000),
                                threads=12, ffn_every=23, state_every=37)
    _log(f"full-size hybrid: max rel-L2 {worst:.2e}, {n_cpu} of {n_miss} misses on the CPU")
    assert 0 < n_cpu < n_miss


def test_hybrid_rejects_non_bf16():
    from expert_cache_offload_amd import MoeError
    from expert_cache_offload_amd.runner import Workbench
    wl = mi.WORKLOADS["dsv4_fp8_decode"].with_layers(1).with_steps(1)
    with Workbench(wl, groups=0) as wb:
        with pytest.raises(MoeError):
            wb.set_hybrid(*RATES, 4)


def test_hybrid_with_resize_at_a_safe_point():
    """Hybrid decode across an elastic resize (30% -> 12% of the pool at token step 6): CPU
    misses hold no slot, so the resize keeps the most recently used cached keys exactly as
    without the split."""
    from expert_cache_offload_amd.runner import Workbench
    from oracle.step import Oracle
    wl = mi.WORKLOADS["qwen35b_decode"].with_layers(2).with_steps(12)
    new_cap = int(0.12 * wl.n_keys)
    with Workbench(wl, groups=0) as wb:
        orc = Oracle(wl, wb.pool, wb.router_np, split=RATES)
        wb.set_hybrid(*RATES, 6)
        worst = 0.0
        for t in range(wl.token_steps):
            if t == 6:
                orc.resize(new_cap)
                wb.resize(new_cap)
                key_of, stamp, slot_of, n, step, cap = wb.snapshot()
                assert cap == new_cap and n == orc.cache.n
                assert list(key_of) == orc.cache.key_of and list(stamp) == orc.cache.stamp
            for l in range(wl.layers):
                wb.step(t, l)
                ref = orc.layer_step(t, l, wb.acts_np[t, l], True)
                worst = max(worst, compare_step(wb, ref, f"hybrid resize t={t} l={l}") or 0.0)
    _log(f"hybrid across a resize: max rel-L2 {worst:.2e}")


def test_hybrid_host_silence_is_bounded_and_reported():
    """Failure path, forced from the host: the server holds its answers, the combine gives up
    after the handle's (here 2 ms) timeout, the steps complete, and the next counter read
    reports MOE_E_HYBRID."""
    import time

    from expert_cache_offload_amd import (MOE_E_HYBRID, MoeError, moe_hybrid_hold,
                                          moe_set_hybrid_timeout)
    from expert_cache_offload_amd.runner import Workbench
    wl = mi.WORKLOADS["tiny"].with_steps(4)
    with Workbench(wl, groups=0) as wb:
        wb.set_hybrid(*RATES, 2)
        moe_set_hybrid_timeout(wb.handle, 2000)
        moe_hybrid_hold(wb.handle, True)
        t0 = time.perf_counter()
        for t in range(3):
            wb.step(t, 0)
        wb.sync()
        dt = time.perf_counter() - t0
        with pytest.raises(MoeError) as ei:
            wb.stats()
        assert ei.value.status == MOE_E_HYBRID
        moe_hybrid_hold(wb.handle, False)
    _log(f"host silence: 3 steps in {dt * 1e3:.1f} ms with a 2 ms bound each")
    assert dt < 2.0
