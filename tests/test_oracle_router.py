"""Pins for oracle/router.py and oracle/dedup.py: exact rational sums, brute-force top-k,
closed forms of the renormalised softmax, and set-based dedup."""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

from oracle.dedup import dedup
from oracle.formats import bf16_to_f64
from oracle.router import router_logits, topk_softmax


def _bf16(rng, shape, scale):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return u


def test_router_logits_within_fp64_bound_of_exact_rational_sum():
    rng = np.random.default_rng(1)
    H, E, T = 64, 8, 3
    xu, wu = _bf16(rng, (T, H), 1.0), _bf16(rng, (E, H), 0.02)
    x, W = bf16_to_f64(xu), bf16_to_f64(wu)
    z = router_logits(x, W)
    u = 2.0 ** -53
    gamma = H * u / (1 - H * u)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(W[e, h])) for h in range(H))
            bound = gamma * float(sum(abs(Fraction(float(x[t, h])) * Fraction(float(W[e, h])))
                                      for h in range(H)))
            assert abs(Fraction(float(z[t, e])) - exact) <= Fraction(bound)


def _brute_topk(z, k):
    return sorted(range(len(z)), key=lambda e: (-z[e], e))[:k]


@pytest.mark.parametrize("E,k", [(16, 2), (128, 8), (256, 8)])
def test_topk_matches_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E)
    z = np.round(rng.standard_normal((50, E)) * 4) / 4  # coarse grid: many exact ties
    idx, w = topk_softmax(z, k)
    for t in range(z.shape[0]):
        assert list(idx[t]) == _brute_topk(list(z[t]), k)
        sm = softmax(z[t])
        sel = sm[idx[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=1e-14, atol=0)


def test_topk_closed_forms():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((20, 16))
    _, w = topk_softmax(z, 8)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)  # descending logits give descending weights
    idx, w = topk_softmax(z, 16)  # k = E: the full softmax in descending order
    for t in range(20):
        assert np.allclose(w[t], softmax(z[t])[idx[t]], rtol=1e-14)
    idx, w = topk_softmax(z, 1)
    assert np.array_equal(idx[:, 0], np.argmax(z, 1)) and np.all(w == 1.0)
    idx, w = topk_softmax(np.zeros((2, 16)), 4)  # all equal: lowest ids, uniform weights
    assert np.array_equal(idx, [[0, 1, 2, 3]] * 2) and np.all(w == 0.25)


def test_dedup_against_sets():
    rng = np.random.default_rng(5)
    for T, E, k in [(1, 16, 2), (4, 256, 8), (300, 128, 8)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        U, count, offset, perm = dedup(idx, E)
        assert U == sorted(set(idx.ravel().tolist()))
        assert count.sum() == T * k and len(U) <= min(T * k, E)
        assert np.array_equal(offset[1:] - offset[:-1], count)
        for e in range(E):
            ids = perm[offset[e]:offset[e + 1]]
            toks = ids // k
            assert np.all(idx[toks, ids % k] == e)
            assert np.all(np.diff(toks) > 0)
            assert len(ids) == sum(1 for t in range(T) if e in idx[t])
        assert sorted(perm.tolist()) == list(range(T * k))
