"""GPU parity: the HIP path (through the C ABI) against the float64 oracle, step by step.

Integer results (expert indices, distinct experts, hit flags, miss slots, victims, per-expert
token lists, key_of / stamp / slot_of / occupancy) must match bit-exactly; routing weights within
1e-6 relative; layer outputs within relative L2 2e-2 (bf16) or 5e-2 (fp8, MXFP4)."""
import dataclasses
import sys

import numpy as np
import pytest

import moe_inputs as mi
from parity import compare_step, rel_l2

pytestmark = pytest.mark.gpu


def _bench(wl, **kw):
    from expert_cache_offload_amd.runner import Workbench
    return Workbench(wl, **kw)


def _oracle(wb):
    from oracle.step import Oracle
    shared = (lambda l: wb.shared_np[l]) if wb.wl.has_shared else None
    return Oracle(wb.wl, wb.pool, wb.router_np, shared)


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_parity(wb, n_tok, ffn_every=1, state_every=1, slot_bytes=False, parts=False):
    wl = wb.wl
    orc = _oracle(wb)
    errs = []
    for t in range(n_tok):
        if wl.resize_at >= 0 and t == wl.resize_at:
            moves = orc.resize(wl.resize_capacity)
            wb.resize(wl.resize_capacity)
            key_of, stamp, slot_of, n, step, cap = wb.snapshot()
            assert cap == wl.resize_capacity and n == orc.cache.n
            assert list(key_of) == orc.cache.key_of and list(stamp) == orc.cache.stamp
            for src, dst in moves:  # moved blobs arrived intact
                k = orc.cache.key_of[dst]
                assert np.array_equal(wb.slot_bytes(dst), orc.blob(k))
        for l in range(wl.layers):
            (wb.step_parts if parts else wb.step)(t, l)
            with_ffn = (t * wl.layers + l) % ffn_every == 0
            x = wb.acts_np[t, l] if wl.kind == "decode" else wb.acts_np[l]
            ref = orc.layer_step(t, l, x, with_ffn)
            err = compare_step(wb, ref, f"{wl.name} t={t} l={l}",
                               check_state=(t * wl.layers + l) % state_every == 0)
            if err is not None:
                errs.append(err)
            if slot_bytes:
                for sl, k in enumerate(ref.rec.key_of):
                    if k >= 0:
                        assert np.array_equal(wb.slot_bytes(sl), orc.blob(k)), (t, l, sl, k)
    return errs


def test_tiny_decode_every_step_and_slot_bytes():
    wl = mi.WORKLOADS["tiny"]
    _log(f"case {wl.name}")
    with _bench(wl) as wb:
        errs = run_parity(wb, wl.token_steps, slot_bytes=True)
        st = wb.stats()
    assert st["steps"] == wl.token_steps
    assert st["hits"] + st["misses"] > 0 and st["bytes_filled"] == st["misses"] * wl.blob_bytes
    _log(f"tiny: max rel-L2 {max(errs):.2e}, misses {st['misses']}")


def test_tiny_single_queue_mode():
    wl = mi.WORKLOADS["tiny"].with_steps(24)
    with _bench(wl, groups=0) as wb:
        run_parity(wb, 24, slot_bytes=True)


def test_tiny_through_separate_calls():
    wl = mi.WORKLOADS["tiny"].with_steps(24)
    with _bench(wl, groups=3) as wb:
        run_parity(wb, 24, parts=True)


@pytest.mark.parametrize("groups", [0, 1, 2, 8])
def test_bf16_decode_multilayer_evictions(groups):
    """35B-A3B expert shape (H 2048, 128 experts top-8, I 768) with 4 layers sharing a 30% cache."""
    wl = mi.WORKLOADS["qwen35b_decode"].with_layers(4).with_steps(24)
    _log(f"case {wl.name} groups={groups} C={wl.capacity}")
    with _bench(wl, groups=groups) as wb:
        errs = run_parity(wb, wl.token_steps, ffn_every=7)
    _log(f"bf16 4-layer: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("hidden,inter,groups", [(512, 256, 0), (1024, 384, 2), (4096, 256, 0)])
def test_bf16_one_token_hidden_sizes(hidden, inter, groups):
    """bf16 decode at one token across hidden sizes: 512 and 1024 take the fused one-token
    FFN with 2 and 4 WdT rows per thread (the workloads' 256 and 2048 take 1 and 8), 4096 the
    gate/up and down kernels."""
    wl = dataclasses.replace(mi.WORKLOADS["qwen35b_decode"], name=f"bf16_h{hidden}_i{inter}",
                             layers=2, hidden=hidden, inter=inter, experts=32, token_steps=12)
    _log(f"case {wl.name} groups={groups} C={wl.capacity}")
    with _bench(wl, groups=groups) as wb:
        errs = run_parity(wb, wl.token_steps)
    _log(f"bf16 H={hidden}: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("groups", [0, 3])
def test_bf16_decode_eight_streams(groups):
    """8 decode streams batched at the 35B shape: one dedup and one cache step for 8 tokens,
    experts shared by several tokens read once."""
    wl = mi.WORKLOADS["qwen35b_decode_b8"].with_layers(3).with_steps(10)
    _log(f"case {wl.name} groups={groups} C={wl.capacity}")
    with _bench(wl, groups=groups) as wb:
        errs = run_parity(wb, wl.token_steps, ffn_every=4)
    _log(f"bf16 8 streams: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("groups", [0, 2])
def test_fp8_decode_with_shared_expert(groups):
    """284B-like shape: H 4096, 256 experts top-8 + shared expert, fp8 e4m3 1x128 blocks."""
    wl = mi.WORKLOADS["dsv4_fp8_decode"].with_layers(2).with_steps(12)
    _log(f"case {wl.name} groups={groups} C={wl.capacity}")
    with _bench(wl, groups=groups) as wb:
        errs = run_parity(wb, wl.token_steps, ffn_every=5)
    _log(f"fp8: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("fmt,hidden,tokens,shared", [
    (2, 8192, 4, False),   # e2m1: 256 chunks per half-row in passes of 192, the second partial
    (2, 8192, 1, False),   # e2m1 at one token: activations in registers, the same passes
    (1, 6144, 2, True),    # fp8: 384 chunks in passes of 256, the second partial; shared expert
    (0, 3072, 4, False),   # bf16: 384 chunks in passes of 256, staged activations
    (0, 2048, 3, False),   # bf16, 3 tokens: kernels built for 4, the fourth masked
    (2, 6144, 6, False),   # e2m1, 6 tokens: kernels built for 8, two masked
])
def test_decode_rows_longer_than_one_pass(fmt, hidden, tokens, shared):
    """Decode steps whose gate/up rows take more than one pass of the weight stream (the last
    pass partial), at one and at several tokens, for each weight format, and token counts
    between the kernels' bounds (1, 2, 4, 8); 16 experts top-8, so the step's tokens share
    experts and their activations are staged in LDS."""
    base = mi.WORKLOADS["qwen35b_decode"]
    wl = dataclasses.replace(base, name=f"passes_f{fmt}_h{hidden}_t{tokens}", layers=2,
                             hidden=hidden, inter=256, experts=16, fmt=fmt, cache_frac=0.75,
                             tokens_per_step=tokens, token_steps=8, has_shared=shared)
    _log(f"case {wl.name} C={wl.capacity}")
    with _bench(wl, groups=0) as wb:
        errs = run_parity(wb, wl.token_steps)
    _log(f"{wl.name}: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("experts,top_k,tokens", [(128, 8, 1), (256, 8, 4), (320, 6, 2)])
def test_topk_ties_and_expert_counts(experts, top_k, tokens):
    """Decode top-k with exact ties: every odd expert's router row is a copy of the even
    expert's before it, so their logits are equal and the lower id must come first.  One token
    of 128 experts takes the rank-counting top-k; four tokens of 256 and two of 320 (not a
    multiple of 64) take the wave argmax."""
    import torch
    base = mi.WORKLOADS["qwen35b_decode"]
    wl = dataclasses.replace(base, name=f"ties_e{experts}_k{top_k}_t{tokens}", layers=2,
                             hidden=256, inter=128, experts=experts, top_k=top_k,
                             cache_frac=0.5, tokens_per_step=tokens, token_steps=8)
    _log(f"case {wl.name} C={wl.capacity}")
    with _bench(wl, groups=0) as wb:
        wb.router_np[:, 1::2, :] = wb.router_np[:, 0::2, :][:, : experts // 2, :]
        wb.router.copy_(torch.from_numpy(wb.router_np.view(np.int16)))
        wb.sync()
        errs = run_parity(wb, wl.token_steps)
    _log(f"{wl.name}: max rel-L2 {max(errs):.2e}")


@pytest.mark.parametrize("groups", [0, 2])
def test_mxfp4_four_streams_with_resize(groups):
    """753B-like shape: H 6144, 256 experts top-8, MXFP4, 4 streams per step with cross-request
    dedup; the cache shrinks from 40% to 15% of the pool at a safe point."""
    wl = dataclasses.replace(mi.WORKLOADS["glm_mxfp4_4stream"].with_layers(2), token_steps=16,
                             resize_at=8)
    _log(f"case {wl.name} groups={groups} C={wl.capacity}->{wl.resize_capacity}")
    with _bench(wl, groups=groups) as wb:
        errs = run_parity(wb, wl.token_steps, ffn_every=6)
    _log(f"mxfp4: max rel-L2 {max(errs):.2e}")


def test_capacity_at_floor_and_everything_fits():
    base = mi.WORKLOADS["qwen35b_decode"].with_layers(2).with_steps(10)
    for cap in (8, 2 * 128):  # C = top_k (every step evicts), C = all keys (only cold misses)
        wl = dataclasses.replace(base, fixed_capacity=cap)
        _log(f"case capacity {cap}")
        with _bench(wl) as wb:
            run_parity(wb, wl.token_steps, ffn_every=9)
            st = wb.stats()
        if cap == 256:
            assert st["misses"] <= 256


def test_empty_step_advances_counter_only():
    wl = mi.WORKLOADS["tiny"].with_steps(4)
    with _bench(wl) as wb:
        wb.step(0, 0)
        before = wb.snapshot()
        wb.step(1, 0, T=0)
        p = wb.plan()
        after = wb.snapshot()
        assert p["n_unique"] == 0 and p["n_miss"] == 0
        assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
        assert after[4] == before[4] + 1


def test_resize_into_new_arena_keeps_contents():
    import torch
    wl = mi.WORKLOADS["tiny"].with_steps(20)
    with _bench(wl, capacity=8, max_capacity=12) as wb:
        orc = _oracle(wb)
        for t in range(10):
            wb.step(t, 0)
            orc.layer_step(t, 0, wb.acts_np[t, 0], False)
        new = torch.empty(5 * wl.blob_bytes, dtype=torch.uint8, device=wb.dev)
        wb.sync()
        wb.resize(5, new)
        orc.resize(5)
        key_of, stamp, slot_of, n, step, cap = wb.snapshot()
        assert list(key_of) == orc.cache.key_of and n == orc.cache.n == 5
        for sl, k in enumerate(orc.cache.key_of):
            assert np.array_equal(wb.slot_bytes(sl), orc.blob(k))
        with pytest.raises(Exception):
            wb.resize(12)  # the 5-slot arena cannot grow in place
        bigger = torch.empty(12 * wl.blob_bytes, dtype=torch.uint8, device=wb.dev)
        wb.resize(12, bigger)
        orc.resize(12)
        for t in range(10, 20):
            wb.step(t, 0)
            ref = orc.layer_step(t, 0, wb.acts_np[t, 0], True)
            compare_step(wb, ref, f"after growth t={t}")
        for sl, k in enumerate(orc.cache.key_of):
            if k >= 0:
                assert np.array_equal(wb.slot_bytes(sl), orc.blob(k))


def test_full_size_bf16_decode_sampled():
    """The 48-layer 35B-A3B shape at full size (58 GB pinned pool, 1,843 slots), in the launch
    configuration the bench times (one queue): every integer result for the first 96 token
    steps (4,608 layer steps), outputs sampled."""
    wl = mi.WORKLOADS["qwen35b_decode"].with_steps(96)
    _log(f"case {wl.name} full size, 96 tokens, one queue")
    with _bench(wl, groups=0) as wb:
        errs = run_parity(wb, wl.token_steps, ffn_every=97, state_every=53)
        st = wb.stats()
    _log(f"full-size: max rel-L2 {max(errs):.2e}; miss rate {st['misses'] / (st['hits'] + st['misses']):.3f}")


def test_full_size_fp8_decode_sampled():
    """The 284B-like fp8 shape at full width (256 experts + shared, H 4096, I 2048, 24.75 MiB
    blobs) over 9 layers (the most a pinned host pool of this box holds), cache 17%, one queue
    as the bench runs it: every integer result of 48 token steps, outputs of every 47th layer
    step, sampled slot bytes."""
    wl = mi.WORKLOADS["dsv4_fp8_decode"].with_layers(9).with_steps(48)
    _log(f"case {wl.name} full width, 48 tokens, C={wl.capacity}, one queue")
    with _bench(wl, groups=0) as wb:
        errs = run_parity(wb, wl.token_steps, ffn_every=47, state_every=31)
        orc_blob = _oracle(wb).blob
        key_of = wb.snapshot()[0]
        for sl in range(0, len(key_of), 97):  # sampled slots hold their keys' pool bytes
            if key_of[sl] >= 0:
                assert np.array_equal(wb.slot_bytes(sl), orc_blob(int(key_of[sl]))), sl
    _log(f"full-size fp8: max rel-L2 {max(errs):.2e}")


def test_full_size_mxfp4_four_streams_with_resize():
    """The 753B-like MXFP4 shape at full size (8 layers, 256 experts, H 6144, 41 GB pool), 4
    streams per step for 1,024 steps with the 40% -> 15% resize before step 512, one queue as
    the bench runs it: every integer result of every layer step, outputs sampled on both sides
    of the resize."""
    wl = mi.WORKLOADS["glm_mxfp4_4stream"]
    _log(f"case {wl.name} full size, {wl.token_steps} steps, C={wl.capacity}->{wl.resize_capacity}")
    with _bench(wl, groups=0) as wb:
        errs = run_parity(wb, wl.token_steps, ffn_every=2731, state_every=257)
    _log(f"full-size mxfp4: max rel-L2 {max(errs):.2e}")
