"""GPU parity of captured layer steps: the C-ABI step calls captured once into a hipGraph on the
compute stream (fills included; with double buffering the fill stream joins the capture through
the library's events), then replayed step after step with new activations copied into the
captured input buffer between replays.

The step counter, the plan and the cache state live on the device, so each replay is one more
step of the method; every replay is checked against the float64 oracle exactly as an eager step
is: integer results bit-exact, routing weights within 1e-6, outputs within the format's
relative-L2 tolerance.  Eager host work (copies, plan and state read-back, synchronisation)
runs between the replays."""
import dataclasses
import sys

import numpy as np
import pytest

import moe_inputs as mi
from parity import TOL_REL_L2, TOL_TOPK_W, compare_step, rel_l2_rows

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _setup(wl, groups, hybrid=None):
    import torch
    from expert_cache_offload_amd.runner import Workbench
    from oracle.step import Oracle
    wb = Workbench(wl, groups=groups)
    shared = (lambda l: wb.shared_np[l]) if wl.has_shared else None
    orc = Oracle(wl, wb.pool, wb.router_np, shared, split=hybrid)
    if hybrid:
        wb.set_hybrid(hybrid[0], hybrid[1], 6)
    x_static = torch.zeros((wl.layers, wb.T, wl.hidden), dtype=torch.int16, device=wb.dev)
    return torch, wb, orc, x_static


def _capture(torch, wb, x_static, layers):
    """One graph whose body is the layer steps `layers` of a token, reading x_static."""
    from expert_cache_offload_amd import moe_layer_step
    g = torch.cuda.CUDAGraph()
    wb.sync()
    with torch.cuda.graph(g, stream=wb.compute):
        for l in layers:
            moe_layer_step(wb.handle, l, x_static[l].data_ptr(), wb.T, wb.router[l].data_ptr(),
                           wb.shared_ptr(l), wb.y[l].data_ptr(), wb.topk_idx[l].data_ptr(),
                           wb.topk_w[l].data_ptr(), wb.groups, wb.compute.cuda_stream,
                           wb.fill.cuda_stream)
    wb.sync()
    return g


def _replay(torch, wb, g, x_static, t):
    with torch.cuda.stream(wb.compute):
        x_static.copy_(wb.acts[t])  # eager work between the replays
        g.replay()
    wb.sync()


def _per_layer_graphs(wl, groups, n_tok, hybrid=None):
    """One captured graph per layer; every replay compared in full against the oracle."""
    torch, wb, orc, x_static = _setup(wl, groups, hybrid)
    try:
        graphs = [_capture(torch, wb, x_static, [l]) for l in range(wl.layers)]
        worst = 0.0
        for t in range(n_tok):
            with torch.cuda.stream(wb.compute):
                x_static.copy_(wb.acts[t])
            for l in range(wl.layers):
                with torch.cuda.stream(wb.compute):
                    graphs[l].replay()
                wb.sync()
                ref = orc.layer_step(t, l, wb.acts_np[t, l], True)
                err = compare_step(wb, ref, f"{wl.name} graph groups={groups} t={t} l={l}")
                worst = max(worst, err or 0.0)
        st = wb.stats()
        assert st["steps"] == n_tok * wl.layers
        return worst, st
    finally:
        wb.close()


def test_graph_tiny_every_replay():
    wl = mi.WORKLOADS["tiny"].with_steps(24)
    _log(f"case {wl.name} graph per layer step, 24 replays")
    worst, st = _per_layer_graphs(wl, 0, wl.token_steps)
    assert st["misses"] > 0
    _log(f"tiny graph: max rel-L2 {worst:.2e}, misses {st['misses']}")


@pytest.mark.parametrize("groups", [0, 2])
def test_graph_35b_shape_per_layer(groups):
    wl = mi.WORKLOADS["qwen35b_decode"].with_layers(3).with_steps(8)
    _log(f"case {wl.name} graph per layer step, groups={groups}")
    worst, _ = _per_layer_graphs(wl, groups, wl.token_steps)
    _log(f"35B graph groups={groups}: max rel-L2 {worst:.2e}")


def test_graph_hybrid_tiny():
    """Hybrid decode inside the graph: the route kernel's mailbox post and the combine's
    bounded wait for the host's answer are replayed like any other node."""
    wl = mi.WORKLOADS["tiny"].with_steps(16)
    _log(f"case {wl.name} hybrid graph")
    worst, st = _per_layer_graphs(wl, 0, wl.token_steps, hybrid=(124_500, 56_000))
    assert st["cpu_misses"] > 0
    _log(f"tiny hybrid graph: max rel-L2 {worst:.2e}, cpu misses {st['cpu_misses']}")


@pytest.mark.parametrize("groups", [0, 2])
def test_graph_whole_token(groups):
    """All layer steps of a token in one graph: per layer the top-k indices, weights and
    output; after each token the last layer's plan and the whole cache state."""
    wl = mi.WORKLOADS["qwen35b_decode"].with_layers(4).with_steps(8)
    _log(f"case {wl.name} whole-token graph, groups={groups}")
    torch, wb, orc, x_static = _setup(wl, groups)
    try:
        g = _capture(torch, wb, x_static, range(wl.layers))
        worst = 0.0
        for t in range(wl.token_steps):
            _replay(torch, wb, g, x_static, t)
            refs = [orc.layer_step(t, l, wb.acts_np[t, l], True) for l in range(wl.layers)]
            for l, ref in enumerate(refs[:-1]):
                ctx = f"whole-token graph t={t} l={l}"
                idx = wb.topk_idx[l].cpu().numpy()
                w = wb.topk_w[l].cpu().numpy().astype(np.float64)
                assert np.array_equal(idx, ref.topk_idx), ctx
                assert np.allclose(w, ref.topk_w, rtol=TOL_TOPK_W, atol=0), ctx
                err = rel_l2_rows(wb.y_f64(l), ref.y)
                assert err <= TOL_REL_L2[wl.fmt], (ctx, err)
                worst = max(worst, err)
            err = compare_step(wb, refs[-1], f"whole-token graph t={t} l={wl.layers - 1}")
            worst = max(worst, err or 0.0)
        assert wb.stats()["steps"] == wl.token_steps * wl.layers
    finally:
        wb.close()
    _log(f"whole-token graph groups={groups}: max rel-L2 {worst:.2e}")


@pytest.mark.parametrize("groups", [0, 3])
def test_graph_prefill_tiny(groups):
    """Steps of many tokens (tiled router, plan, scatter, matrix-core FFN, shared expert)
    captured one graph per layer: the 100-token chunk replayed twice through 3 layers of 24
    slots (cold, then warm), every replay against the oracle."""
    base = dataclasses.replace(mi.WORKLOADS["tiny"], layers=3, fixed_capacity=24, has_shared=True)
    wl = base.as_prefill(100)
    _log(f"case {wl.name} prefill graph per layer step, groups={groups}")
    torch, wb, orc, x_static = _setup(wl, groups)
    try:
        graphs = [_capture(torch, wb, x_static, [l]) for l in range(wl.layers)]
        with torch.cuda.stream(wb.compute):
            x_static.copy_(wb.acts)
        worst = 0.0
        for c in range(2):
            for l in range(wl.layers):
                with torch.cuda.stream(wb.compute):
                    graphs[l].replay()
                wb.sync()
                ref = orc.layer_step(c, l, wb.acts_np[l], True)
                err = compare_step(wb, ref, f"prefill graph groups={groups} c={c} l={l}")
                worst = max(worst, err or 0.0)
        assert wb.stats()["steps"] == 2 * wl.layers
    finally:
        wb.close()
    _log(f"prefill graph groups={groups}: max rel-L2 {worst:.2e}")
