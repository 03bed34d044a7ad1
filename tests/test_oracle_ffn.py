"""Pins for oracle/ffn.py and oracle/step.py: dense-MoE equivalence, linearity, zero input,
a 60-digit decimal cross-check, silu identities, and the composed layer step."""
from decimal import Decimal, getcontext

import numpy as np

import moe_inputs as mi
from oracle import formats as F
from oracle.dedup import dedup
from oracle.ffn import expert_ffn, moe_output, silu
from oracle.router import router_logits, topk_softmax
from oracle.step import Oracle


def _experts(rng, E, H, I):
    return [(rng.standard_normal((I, H)) * 0.1, rng.standard_normal((I, H)) * 0.1,
             rng.standard_normal((H, I)) * 0.1) for _ in range(E)]


def test_cached_moe_equals_dense_moe():
    """A dense loop over every expert with gate 0 outside the top-k equals the routed sum."""
    rng = np.random.default_rng(0)
    E, H, I, T, k = 8, 32, 16, 5, 2
    ex = _experts(rng, E, H, I)
    x = rng.standard_normal((T, H))
    Wr = rng.standard_normal((E, H)) * 0.3
    idx, w = topk_softmax(router_logits(x, Wr), k)
    y = moe_output(x, idx, w, lambda e: ex[e])
    dense = np.zeros((T, H))
    for t in range(T):
        for e in range(E):
            g = w[t, list(idx[t]).index(e)] if e in idx[t] else 0.0
            Wg, Wu, Wd = ex[e]
            h = np.array([sum(x[t, c] * Wg[i, c] for c in range(H)) for i in range(I)])
            u = np.array([sum(x[t, c] * Wu[i, c] for c in range(H)) for i in range(I)])
            a = h / (1 + np.exp(-h)) * u
            dense[t] += g * np.array([sum(Wd[o, i] * a[i] for i in range(I)) for o in range(H)])
    assert np.allclose(y, dense, rtol=1e-12, atol=1e-15)


def test_linearity_and_zero():
    rng = np.random.default_rng(1)
    E, H, I, T, k = 6, 16, 8, 3, 2
    ex = _experts(rng, E, H, I)
    x = rng.standard_normal((T, H))
    idx = np.array([[0, 3], [5, 1], [2, 4]])
    w = rng.random((T, k))
    y1 = moe_output(x, idx, w, lambda e: ex[e])
    y2 = moe_output(x, idx, 2.5 * w, lambda e: ex[e])
    assert np.allclose(y2, 2.5 * y1, rtol=1e-13)
    assert np.all(moe_output(np.zeros((T, H)), idx, w, lambda e: ex[e]) == 0)
    sh = _experts(rng, 1, H, I)[0]
    ys = moe_output(x, idx, w, lambda e: ex[e], shared=sh)
    assert np.allclose(ys - y1, expert_ffn(x, *sh), rtol=1e-12, atol=1e-15)


def test_silu_identities():
    z = np.linspace(-30, 30, 601)
    assert silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(silu(-z), silu(z) - z, atol=1e-13)
    assert np.allclose(silu(np.array([40.0])), 40.0, rtol=1e-15)


def test_expert_ffn_against_60_digit_decimal():
    getcontext().prec = 60
    rng = np.random.default_rng(2)
    H, I = 8, 4
    Wg, Wu, Wd = (rng.standard_normal((I, H)), rng.standard_normal((I, H)),
                  rng.standard_normal((H, I)))
    x = rng.standard_normal(H)
    D = lambda v: Decimal(float(v))  # noqa: E731
    a = []
    for i in range(I):
        g = sum(D(Wg[i, c]) * D(x[c]) for c in range(H))
        u = sum(D(Wu[i, c]) * D(x[c]) for c in range(H))
        a.append(g / (1 + (-g).exp()) * u)
    ref = [sum(D(Wd[o, i]) * a[i] for i in range(I)) for o in range(H)]
    y = expert_ffn(x[None], Wg, Wu, Wd)[0]
    for o in range(H):
        assert abs(D(y[o]) - ref[o]) <= Decimal("1e-13") * (1 + abs(ref[o]))


def test_layer_step_composition_tiny():
    wl = mi.WORKLOADS["tiny"]
    pool = np.empty(wl.pool_bytes, np.uint8)
    mi.fill_pool(wl.seed, wl.fmt, 0, wl.layers, wl.experts, wl.hidden, wl.inter, pool)
    router = mi.router_weights(wl.seed, 0, wl.layers, wl.experts, wl.hidden)
    acts = mi.decode_acts(wl.seed, 0, wl.layers, wl.tokens_per_step, wl.token_steps, wl.hidden)
    orc = Oracle(wl, pool, router)
    steps = list(orc.run(acts, with_ffn=lambda t, l: t % 8 == 0))
    assert len(steps) == wl.token_steps * wl.layers
    misses = 0
    for st in steps:
        x = F.bf16_to_f64(acts[st.token_step, st.layer])
        idx, w = topk_softmax(router_logits(x, F.bf16_to_f64(router[st.layer])), wl.top_k)
        assert np.array_equal(idx, st.topk_idx) and np.array_equal(w, st.topk_w)
        assert st.U == dedup(idx, wl.experts)[0]
        misses += len(st.rec.misses)
        if st.y is not None:
            # every slot's bytes are the pool blob of its key: FFN via the slot table equals
            # FFN via the pool
            def via_slot(e, st=st):
                slot = st.rec.slot[st.U.index(e)]
                key = st.rec.key_of[slot]
                S = wl.blob_bytes
                return F.decode_blob(pool[key * S:(key + 1) * S], wl.fmt, wl.hidden, wl.inter)
            y2 = moe_output(x, idx, w, via_slot)
            assert np.array_equal(st.y, y2)
    # the AR(1) stream keeps some routing locality: with 8 of 16 slots not every step misses
    assert 0 < misses < wl.token_steps * wl.top_k
