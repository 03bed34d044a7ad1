"""Pins for oracle/split.py and the R9 rule of oracle/lru.py (hybrid decode).

* the pages' printed probe: bf16 52.4 vs 51.5 GB/s is 1.02x, below the 2.0x threshold, so
  offload; fp8 has no CPU path (tests/golden/mode_probe_ceilings.json);
* the split against the real equal-finish point m * b_cpu / (b_cpu + b_pcie): q is its
  floor or its ceiling; special cases (no CPU, no PCIe, equal rates with the tie rule);
  monotonicity in m and in either rate; hand-derived cases;
* R9 against an independent dictionary model of the cache, and its invariants.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle.lru import LRUCache
from oracle.split import hybrid_mode, miss_split

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mode_probe_ceilings.json")


def test_pages_probe_picks_offload():
    g = json.load(open(GOLDEN))
    for row in g["rows"]:
        cpu = row["cpu_GBps"] or 0.0
        got = hybrid_mode(cpu, row["offload_GBps"], g["threshold"])
        assert (got and row["mode"] == "hybrid") or (not got and row["mode"] == "offload")
        if row["ratio"] is not None:
            assert round(cpu / row["offload_GBps"], 2) == row["ratio"]
    assert hybrid_mode(2.0 * 51.5, 51.5)          # at the threshold: hybrid
    assert not hybrid_mode(1.99 * 51.5, 51.5)


def test_split_brackets_the_equal_finish_point():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        m = int(rng.integers(0, 65))
        bc = int(rng.integers(1, 300_000))
        bp = int(rng.integers(1, 300_000))
        q = miss_split(m, bc, bp)
        x = m * bc / (bc + bp)
        assert 0 <= q <= m
        assert math.floor(x) <= q <= math.ceil(x), (m, bc, bp, q, x)


def test_split_special_cases():
    for m in range(0, 20):
        assert miss_split(m, 0, 56_000) == 0          # no CPU path
        assert miss_split(m, 56_000, 0) == m          # no PCIe: everything on the CPU
        assert miss_split(m, 50_000, 50_000) == m // 2  # equal rates: halves, ties -> fewer
    assert miss_split(0, 124_500, 56_000) == 0


def test_split_monotone():
    for bc, bp in ((124_500, 56_000), (40_000, 56_000), (7, 3)):
        qs = [miss_split(m, bc, bp) for m in range(40)]
        assert all(b >= a for a, b in zip(qs, qs[1:]))
    for m in (1, 2, 3, 7, 16):
        qs = [miss_split(m, bc, 56_000) for bc in range(0, 400_000, 5_000)]
        assert all(b >= a for a, b in zip(qs, qs[1:]))
        qs = [miss_split(m, 124_500, bp) for bp in range(1, 400_000, 5_000)]
        assert all(b <= a for a, b in zip(qs, qs[1:]))


def test_split_hand_cases():
    # CPU 124.5 GB/s, PCIe 56 GB/s (the rates of a 16-thread EPYC host and a PCIe 5 link):
    # m = 1: fill 1/56 > CPU 1/124.5 -> the CPU takes it;
    # m = 2: one each finishes at 1/56 (fill), both on the CPU at 2/124.5 = 1/62.25 -> 2;
    # m = 3: (1 fill, 2 CPU) finishes at max(1/56, 2/124.5) = 1/56 vs all CPU 3/124.5 -> 2.
    assert [miss_split(m, 124_500, 56_000) for m in (1, 2, 3)] == [1, 2, 2]
    # CPU slower than PCIe (40 vs 56): m = 1 -> fill; m = 2 -> one each
    # (max(1/56, 1/40) = 1/40 < 2/56 = 1/28); m = 5 -> 2 on the CPU
    # (max(3/56, 2/40) = 3/56 beats 4/56 with one and 3/40 with three).
    assert [miss_split(m, 40_000, 56_000) for m in (1, 2, 5)] == [0, 1, 2]


def _dict_model(seq, C, E):
    """Independent model of R1-R6 + R9: key -> (stamp, slot); the last n_cpu misses of a
    step are not inserted and not stamped."""
    cache, free, out = {}, list(range(C)), []
    for s, (l, U, n_cpu) in enumerate(seq):
        keys = [l * E + e for e in U]
        hit = [k in cache for k in keys]
        allm = [k for k, h in zip(keys, hit) if not h]
        fill, cpu = allm[:len(allm) - n_cpu], allm[len(allm) - n_cpu:]
        need = max(0, len(fill) - len(free))
        cand = sorted((st, k) for k, (st, sl) in cache.items() if k not in set(keys))
        victims = [k for _, k in cand[:need]]
        fs = sorted(free)
        assigned = []
        for i, k in enumerate(fill):
            if i < len(fs):
                assigned.append((k, fs[i], -1))
            else:
                v = victims[i - len(fs)]
                assigned.append((k, cache[v][1], v))
        for v in victims:
            del cache[v]
        for k, sl, _ in assigned:
            if sl in free:
                free.remove(sl)
            cache[k] = (s, sl)
        for k in keys:
            if k in cache:
                cache[k] = (s, cache[k][1])
        out.append((hit, assigned, cpu, {k: sl for k, (st, sl) in cache.items()}))
    return out


def test_cpu_misses_against_dictionary_model():
    L, E = 3, 10
    for seed in range(6):
        rng = np.random.default_rng(200 + seed)
        for C in (8, 13, 25):
            c = LRUCache(C, L * E)
            seq = []
            # build the sequence step by step: n_cpu must not exceed the step's misses
            ref_cache = LRUCache(C, L * E)
            for s in range(40):
                l = s % L
                U = sorted(set(int(v) for v in rng.integers(0, E, size=5)))
                m = sum(1 for e in U if ref_cache.slot_of(l * E + e) < 0)
                n_cpu = int(rng.integers(0, m + 1))
                ref_cache.step(l, U, E, s, n_cpu=n_cpu)
                seq.append((l, U, n_cpu))
            ref = _dict_model(seq, C, E)
            for s, (l, U, n_cpu) in enumerate(seq):
                rec = c.step(l, U, E, s, n_cpu=n_cpu)
                hit, assigned, cpu, content = ref[s]
                assert rec.hit == hit, (seed, C, s)
                assert [tuple(x) for x in rec.misses] == assigned, (seed, C, s)
                assert rec.cpu == cpu
                got = {k: sl for sl, k in enumerate(rec.key_of) if k >= 0}
                assert got == content, (seed, C, s)
                assert not set(cpu) & set(got)                   # CPU keys are not cached
                assert all(rec.slot[i] == -1 for i, e in enumerate(U) if l * E + e in set(cpu))


def test_cpu_misses_take_no_slot():
    E = 8
    c = LRUCache(4, E)
    r = c.step(0, [1, 2, 3], E, 0, n_cpu=2)      # misses 1, 2, 3: 1 filled, 2 and 3 on the CPU
    assert r.misses == [(1, 0, -1)] and r.cpu == [2, 3] and r.n == 1
    r = c.step(0, [2, 3], E, 1, n_cpu=0)         # still misses: they were never cached
    assert r.hit == [False, False] and [k for k, _, _ in r.misses] == [2, 3]
    with pytest.raises(ValueError):
        c.step(0, [5], E, 2, n_cpu=2)


def test_oracle_hybrid_step_same_output_and_split():
    """With a split the layer output is the same sum over the selected experts; the number of
    CPU misses per step is the split of that step's misses; steps of more than 8 tokens
    never split."""
    import moe_inputs as mi
    from oracle.step import Oracle

    wl = mi.WORKLOADS["tiny"]
    pool = np.empty(wl.pool_bytes, np.uint8)
    mi.fill_pool(wl.seed, wl.fmt, 0, wl.layers, wl.experts, wl.hidden, wl.inter, pool)
    router = mi.router_weights(wl.seed, 0, wl.layers, wl.experts, wl.hidden)
    acts = mi.decode_acts(wl.seed, 0, wl.layers, wl.tokens_per_step, wl.token_steps, wl.hidden)
    plain = Oracle(wl, pool, router)
    hyb = Oracle(wl, pool, router, split=(124_500, 56_000))
    n_cpu_total = 0
    for t in range(12):
        a = plain.layer_step(t, 0, acts[t, 0], True)
        U = a.U
        m = sum(1 for e in U if hyb.cache.slot_of(int(e)) < 0)
        b = hyb.layer_step(t, 0, acts[t, 0], True)
        assert np.array_equal(a.topk_idx, b.topk_idx)
        assert np.allclose(a.y, b.y, rtol=0, atol=0)
        assert len(b.rec.cpu) == miss_split(m, 124_500, 56_000)
        assert len(b.rec.misses) + len(b.rec.cpu) == m
        n_cpu_total += len(b.rec.cpu)
    assert n_cpu_total > 0
    big = Oracle(wl, pool, router, split=(124_500, 56_000))
    x9 = np.repeat(acts[0, 0][None], 9, axis=0).reshape(9, -1)
    r = big.layer_step(0, 0, x9, False)
    assert r.rec.cpu == []
