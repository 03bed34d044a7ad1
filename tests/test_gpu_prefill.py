"""GPU parity of steps with many tokens (prefill chunks): tiled router, one-workgroup plan,
scatter, matrix-core grouped GEMM FFN and combine, against the float64 oracle.

Integer results (top-k indices, distinct experts, hits, misses with slots and victims,
expert-sorted rows, key_of / stamp / slot_of) bit-exact; routing weights within 1e-6
relative; outputs within relative L2 2e-2 per token."""
import dataclasses
import sys

import numpy as np
import pytest

import moe_inputs as mi
from parity import TOL_REL_L2, compare_step, rel_l2_rows

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bench(wl, **kw):
    from expert_cache_offload_amd.runner import Workbench
    return Workbench(wl, **kw)


def _oracle(wb):
    from oracle.step import Oracle
    shared = (lambda l: wb.shared_np[l]) if wb.wl.has_shared else None
    return Oracle(wb.wl, wb.pool, wb.router_np, shared)


def _run_chunk(wb, ffn_layers=None, state=True):
    wl = wb.wl
    orc = _oracle(wb)
    errs = []
    for l in range(wl.layers):
        wb.step(0, l)
        with_ffn = ffn_layers is None or l in ffn_layers
        ref = orc.layer_step(0, l, wb.acts_np[l], with_ffn)
        err = compare_step(wb, ref, f"{wl.name} l={l}", check_state=state)
        if err is not None:
            errs.append(err)
    return errs


def _run_chunk_prefetch(wb):
    """Layer steps with prefetch of the next layer: every step against the oracle's step, the
    cache state after each call against the oracle after the step and the prefetch."""
    wl = wb.wl
    orc = _oracle(wb)
    wb.set_prefetch(True)
    errs = []
    for l in range(wl.layers):
        wb.step(0, l)
        ref = orc.layer_step(0, l, wb.acts_np[l], True)
        errs.append(compare_step(wb, ref, f"{wl.name} prefetch l={l}", check_state=False))
        if l > 0:
            assert not ref.rec.misses, "the prefetched layer should route to hits only"
        if l + 1 < wl.layers:
            orc.prefetch(l + 1, l, ref.U)
        key_of, stamp, slot_of, n, step, cap = wb.snapshot()
        assert n == orc.cache.n and step == orc.s, (l, n, orc.cache.n, step, orc.s)
        assert list(key_of) == orc.cache.key_of, l
        assert list(stamp) == orc.cache.stamp, l
        for sl, k in enumerate(orc.cache.key_of):
            if k >= 0:
                assert slot_of[k] == sl
    return [e for e in errs if e is not None]


@pytest.mark.parametrize("groups", [0, 3])
def test_prefill_prefetch_tiny(groups):
    """Prefetch of the next layer at the tiny shape with a shared expert: 100 tokens, 4 layers,
    40 slots (a layer's 16 experts plus the protected 16 of the step before fit)."""
    base = dataclasses.replace(mi.WORKLOADS["tiny"], layers=4, fixed_capacity=40, has_shared=True)
    wl = base.as_prefill(100)
    _log(f"case {wl.name} prefetch groups={groups}")
    with _bench(wl, groups=groups) as wb:
        errs = _run_chunk_prefetch(wb)
    _log(f"tiny prefetch: max rel-L2 {max(errs):.2e}")


def test_prefill_prefetch_qwen_shape():
    """Prefetch at the 35B expert shape: 300 tokens over 5 layers with 300 slots, so the
    prefetches evict (the protected keys of the step before are never taken)."""
    wl = dataclasses.replace(mi.WORKLOADS["qwen35b_prefill"].with_layers(5).with_tokens(300),
                             fixed_capacity=300)
    _log(f"case {wl.name} prefetch C={wl.capacity}")
    with _bench(wl, groups=0) as wb:
        errs = _run_chunk_prefetch(wb)
        st = wb.stats()
    _log(f"qwen prefetch: max rel-L2 {max(errs):.2e}, misses {st['misses']}")


@pytest.mark.parametrize("k,hidden,inter,cap", [(8, 2048, 768, 260), (2, 256, 128, 160)])
def test_prefetch_steps_smaller_than_a_layer(k, hidden, inter, cap):
    """Prefetch on handles whose steps hold fewer distinct experts than a layer has (128
    experts, max_tokens 9: at most 9*k distinct per step, while a prefetch plans all 128), 6
    layers.  With top-2 a prefetch group of ~110 keys stamped alike outlives its step and is
    evicted by the next prefetch; every step, and the state after each prefetch, against R8."""
    wl = mi.Workload(f"e128_k{k}_h{hidden}_prefill9", 6, hidden, 128, k, inter, 0, 0.0, 9, 1,
                     "prefill", fixed_capacity=cap)
    _log(f"case {wl.name} prefetch C={cap}")
    with _bench(wl, groups=0) as wb:
        errs = _run_chunk_prefetch(wb)
        st = wb.stats()
    _log(f"{wl.name}: max rel-L2 {max(errs):.2e}, misses {st['misses']}")


def test_prefetch_capacity_floor_refused():
    """Prefetch needs min(max_tokens*k, E) + E slots (the step's protected keys plus a whole
    layer): refused on the host below that, and a resize below it is refused while prefetch
    is on (no kernel runs for a refused call)."""
    from expert_cache_offload_amd import MOE_E_CAPACITY, MoeError
    wl = mi.Workload("e128_k8_prefill9_floor", 2, 256, 128, 8, 128, 0, 0.0, 9, 1, "prefill",
                     fixed_capacity=199)
    _log(f"case {wl.name}")
    with _bench(wl, groups=0, max_capacity=260) as wb:
        with pytest.raises(MoeError) as ei:
            wb.set_prefetch(True)
        assert ei.value.status == MOE_E_CAPACITY
        wb.prefetch = False
        wb.resize(200)
        wb.set_prefetch(True)
        with pytest.raises(MoeError) as ei:
            wb.resize(199)
        assert ei.value.status == MOE_E_CAPACITY
        wb.set_prefetch(False)
        wb.resize(199)
        key_of, stamp, slot_of, n, step, cap = wb.snapshot()
        assert cap == 199 and n == 0 and step == 0


def test_prefill_tiny_shape_with_shared_expert():
    """16 experts top-2 at hidden 256: 100 tokens (one full and one ragged 64-token block,
    row tiles far from full), three layers over 24 slots so the later layers evict."""
    base = dataclasses.replace(mi.WORKLOADS["tiny"], layers=3, fixed_capacity=24, has_shared=True)
    wl = base.as_prefill(100)
    for groups in (0, 3):
        _log(f"case {wl.name} groups={groups}")
        with _bench(wl, groups=groups) as wb:
            errs = _run_chunk(wb)
        _log(f"tiny prefill groups={groups}: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("tokens", [9, 64, 65, 130])
def test_prefill_block_edges(tokens):
    """The smallest many-token step (9), exactly one 64-token block, one past it, and two
    blocks plus two tokens, at the tiny shape over two layers (16 slots: the second layer
    evicts)."""
    base = dataclasses.replace(mi.WORKLOADS["tiny"], layers=2, fixed_capacity=16)
    wl = base.as_prefill(tokens)
    _log(f"case {wl.name}")
    with _bench(wl, groups=0) as wb:
        _run_chunk(wb)


def test_prefill_256_experts():
    """256 experts top-8 (16 experts per router thread), hidden 1024, intermediate 512, bf16,
    200 tokens over two layers with 300 slots."""
    wl = mi.Workload("e256_bf16", 2, 1024, 256, 8, 512, 0, 0.0, 200, 1, "prefill",
                     fixed_capacity=300)
    _log(f"case {wl.name} C={wl.capacity}")
    with _bench(wl, groups=2) as wb:
        errs = _run_chunk(wb)
    _log(f"256 experts: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("groups", [0, 4])
def test_prefill_qwen_shape_ragged_chunk(groups):
    """35B-A3B expert shape, 4 layers, a 300-token chunk (4 full blocks and a ragged one):
    every layer routes to nearly all 128 experts, the 30% cache (153 slots) evicts from the
    second layer on."""
    wl = mi.WORKLOADS["qwen35b_prefill"].with_layers(4).with_tokens(300)
    _log(f"case {wl.name} groups={groups} C={wl.capacity}")
    with _bench(wl, groups=groups) as wb:
        errs = _run_chunk(wb)
        st = wb.stats()
    _log(f"qwen prefill 300: max rel-L2 {max(errs):.2e}, misses {st['misses']}")


def test_prefill_separate_calls_match_layer_step():
    wl = dataclasses.replace(mi.WORKLOADS["qwen35b_prefill"].with_layers(3).with_tokens(200),
                             fixed_capacity=160)
    with _bench(wl, groups=2) as wb:
        orc = _oracle(wb)
        for l in range(wl.layers):
            wb.step_parts(0, l)
            ref = orc.layer_step(0, l, wb.acts_np[l], True)
            compare_step(wb, ref, f"{wl.name} parts l={l}")


def test_full_size_prefill_chunk_sampled():
    """16,384-token chunk at the 35B-A3B shape over 12 layers (cache 30% = 460 slots) in the
    configuration the bench times (the layer's own fills in stream order, prefetch of the next
    layer on the fill stream): every integer result of every layer step, the cache state after
    every third step and its prefetch; outputs of 4 sampled tokens on three layers."""
    from oracle.ffn import moe_output
    from oracle.formats import bf16_to_f64, decode_blob
    wl = mi.WORKLOADS["qwen35b_prefill"].with_layers(12)
    _log(f"case {wl.name} full chunk, C={wl.capacity}, prefetch, one queue for own fills")
    rng = np.random.default_rng(7)
    sample = np.sort(rng.choice(wl.tokens_per_step, 4, replace=False))
    with _bench(wl, groups=0) as wb:
        wb.set_prefetch(True)
        orc = _oracle(wb)
        worst = 0.0
        for l in range(wl.layers):
            wb.step(0, l)
            ref = orc.layer_step(0, l, wb.acts_np[l], False)
            compare_step(wb, ref, f"{wl.name} l={l}", check_state=False)
            if l > 0:
                assert not ref.rec.misses, "the prefetched layer should route to hits only"
            if l + 1 < wl.layers:
                orc.prefetch(l + 1, l, ref.U)
            if l % 3 == 2:
                key_of, stamp, slot_of, n, step, cap = wb.snapshot()
                assert n == orc.cache.n and step == orc.s, (l, n, orc.cache.n, step, orc.s)
                assert list(key_of) == orc.cache.key_of, l
                assert list(stamp) == orc.cache.stamp, l
            if l in (0, 5, 11):
                x = bf16_to_f64(wb.acts_np[l][sample]).reshape(len(sample), wl.hidden)
                cache = {}

                def weights_of(e, l=l):
                    if e not in cache:
                        cache[e] = decode_blob(orc.blob(l * wl.experts + e), wl.fmt, wl.hidden,
                                               wl.inter)
                    return cache[e]

                y_ref = moe_output(x, ref.topk_idx[sample], ref.topk_w[sample], weights_of)
                y_gpu = wb.y_f64(l)[sample]
                err = rel_l2_rows(y_gpu, y_ref)
                assert err <= TOL_REL_L2[wl.fmt], (l, err)
                worst = max(worst, err)
        st = wb.stats()
    _log(f"full prefill: worst sampled rel-L2 {worst:.2e}, misses {st['misses']}")
