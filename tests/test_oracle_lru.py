"""Pins for oracle/lru.py.

* a brute-force stack characterisation that shares nothing with the linked list:
  after step s the cache holds exactly the C keys with the largest (last use, key);
* LRU inclusion: hits with capacity C are hits with capacity C + 1;
* compulsory misses when every key fits;
* slot-table invariants (inverse maps, occupied prefix, no duplicates);
* resize-to-C' equals a cache that always had C' slots (flags after the resize);
* Belady's optimal replacement never misses more;
* a hand-derived 8-step trace (tests/golden/lru_hand_trace.json);
* the full-capacity prefill case in which layers 0-14 route every expert.
"""
import json
import os

import numpy as np
import pytest

from oracle.lru import CapacityError, LRUCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lru_hand_trace.json")


def random_trace(seed, steps, L, E, max_u):
    rng = np.random.default_rng(seed)
    out = []
    for s in range(steps):
        l = s % L
        nu = int(rng.integers(1, max_u + 1))
        # temporal locality: draw from a small moving window of experts
        base = int(rng.integers(0, E))
        pick = sorted({(base + int(v)) % E for v in rng.integers(0, max(2, E // 3), size=nu)})
        out.append((l, pick))
    return out


def run(trace, C, E, n_keys, resize=None):
    c = LRUCache(C, n_keys)
    recs = []
    for s, (l, U) in enumerate(trace):
        if resize is not None and s == resize[0]:
            c.resize(resize[1])
        recs.append(c.step(l, U, E, s))
    return recs


def test_stack_characterisation_brute_force():
    L, E = 3, 10
    for seed in range(6):
        trace = random_trace(seed, 60, L, E, 4)
        for C in (4, 6, 9, 15):
            recs = run(trace, C, E, L * E)
            last = {}
            for s, (l, U) in enumerate(trace):
                cached = sorted(last, key=lambda k: (last[k], k))[-C:]
                keys = [l * E + e for e in U]
                assert recs[s].hit == [k in cached for k in keys]
                for k in keys:
                    last[k] = s
                content = set(sorted(last, key=lambda k: (last[k], k))[-C:])
                assert set(x for x in recs[s].key_of if x >= 0) == content


def test_inclusion_property():
    L, E = 4, 12
    trace = random_trace(11, 200, L, E, 5)
    prev = None
    total = []
    for C in range(5, L * E + 1):
        recs = run(trace, C, E, L * E)
        flags = [r.hit for r in recs]
        if prev is not None:
            for a, b in zip(prev, flags):
                assert all((not x) or y for x, y in zip(a, b))
        total.append(sum(len(r.misses) for r in recs))
        prev = flags
    assert all(a >= b for a, b in zip(total, total[1:]))


def test_compulsory_misses_when_everything_fits():
    L, E = 3, 8
    trace = random_trace(2, 100, L, E, 4)
    distinct = {l * E + e for l, U in trace for e in U}
    recs = run(trace, L * E, E, L * E)
    assert sum(len(r.misses) for r in recs) == len(distinct)
    assert all(v == -1 for r in recs for _, _, v in r.misses)


def test_slot_table_invariants():
    L, E, C = 3, 10, 7
    trace = random_trace(4, 150, L, E, 5)
    c = LRUCache(C, L * E)
    seen = set()
    for s, (l, U) in enumerate(trace):
        r = c.step(l, U, E, s)
        seen |= {l * E + e for e in U}
        assert r.n == min(C, len(seen))
        occ = [k for k in r.key_of[:r.n]]
        assert all(k >= 0 for k in occ) and all(k == -1 for k in r.key_of[r.n:])
        assert len(set(occ)) == len(occ)
        for slot, k in enumerate(r.key_of[:r.n]):
            assert c.slot_of(k) == slot
        for e, sl in zip(U, r.slot):
            assert r.key_of[sl] == l * E + e and r.stamp[sl] == s
        # list order == ascending (stamp, key)
        order = list(c.order.keys())
        st = {k: r.stamp[c.order[k]] for k in order}
        assert order == sorted(order, key=lambda k: (st[k], k))


def test_resize_equals_smaller_cache_from_the_start():
    L, E = 3, 12
    for seed in range(4):
        trace = random_trace(100 + seed, 120, L, E, 4)
        for C0, C1, at in [(20, 6, 40), (9, 5, 70), (12, 12, 10)]:
            a = run(trace, C0, E, L * E, resize=(at, C1))
            b = run(trace, C1, E, L * E)
            for s in range(at, len(trace)):
                assert a[s].hit == b[s].hit
                assert set(a[s].key_of) - {-1} == set(b[s].key_of) - {-1}
        # growth: the grown cache holds the most recent keys it has room for, so its content
        # (and its hits) stay inside those of a cache that always had the larger capacity
        a = run(trace, 6, E, L * E, resize=(50, 14))
        b = run(trace, 14, E, L * E)
        for s in range(50, len(trace)):
            assert set(a[s].key_of) - {-1} <= set(b[s].key_of) - {-1}
            assert all((not x) or y for x, y in zip(a[s].hit, b[s].hit))


def test_resize_compaction_moves():
    c = LRUCache(6, 100)
    for s, U in enumerate([[0, 1, 2], [3, 4], [5]]):
        c.step(0, U, 10, s)
    # order (LRU first): 0 1 2 3 4 5 in slots 0..5; shrink to 3 keeps keys 3, 4, 5 (slots 3-5)
    moves = c.resize(3)
    assert moves == [(3, 0), (4, 1), (5, 2)]
    assert c.key_of == [3, 4, 5] and c.stamp == [1, 1, 2] and c.n == 3


def belady_misses(trace, C, E):
    """Optimal replacement on the request sequence serialised step by step (keys of a
    step consecutive): evict the cached key, not requested in this step, whose next use is
    farthest in the future."""
    seq = [(s, l * E + e) for s, (l, U) in enumerate(trace) for e in U]
    cache, misses = set(), 0
    for i, (s, key) in enumerate(seq):
        if key in cache:
            continue
        misses += 1
        if len(cache) >= C:
            now = {k for t, k in seq if t == s}

            def next_use(k):
                for j in range(i + 1, len(seq)):
                    if seq[j][1] == k:
                        return j
                return 10 ** 9

            cand = [k for k in cache if k not in now]
            cache.remove(max(cand, key=lambda k: (next_use(k), k)))
        cache.add(key)
    return misses


def test_belady_never_worse():
    L, E = 2, 8
    for seed in range(5):
        trace = random_trace(seed, 40, L, E, 3)
        for C in (3, 5, 8):
            lru = sum(len(r.misses) for r in run(trace, C, E, L * E))
            assert belady_misses(trace, C, E) <= lru


def test_capacity_floor():
    c = LRUCache(2, 10)
    with pytest.raises(CapacityError):
        c.step(0, [0, 1, 2], 10, 0)


def test_hand_derived_trace():
    """Tables derived by hand from rules R1-R7 (derivation in the fixture's notes)."""
    g = json.load(open(GOLDEN))
    E = g["E"]
    c = LRUCache(g["C"], g["L"] * E)
    for ev in g["events"]:
        if "resize" in ev:
            moves = c.resize(ev["resize"])
            assert [list(m) for m in moves] == ev["moves"]
        else:
            r = c.step(ev["layer"], ev["U"], E, ev["s"])
            assert r.hit == ev["hit"], ev
            assert [list(m) for m in r.misses] == ev["misses"], ev
        assert c.key_of == ev["key_of"], ev
        assert c.stamp == ev["stamp"], ev
        assert c.n == ev["n"], ev


def test_prefill_full_capacity_case():
    """48 layers x 128 experts, 1,843 slots, every expert routed in each layer (a prefill
    chunk): layer 14 finds 1843 - 14*128 = 51 free slots for experts 0..50 and evicts the
    layer-0 keys 0..76 from slots 0..76 for experts 51..127."""
    E, C = 128, 1843
    c = LRUCache(C, 48 * E)
    for l in range(14):
        r = c.step(l, list(range(E)), E, l)
        assert not any(r.hit)
    r = c.step(14, list(range(E)), E, 14)
    assert r.misses[:51] == [(14 * E + e, 14 * E + e, -1) for e in range(51)]
    assert r.misses[51:] == [(14 * E + 51 + i, i, i) for i in range(77)]
    assert r.n == C


def _brute_force_protected(seq, C, E):
    """Independent model of R1-R6 + R8: the cache is a dict key -> (stamp, slot); victims are
    the `need` smallest (stamp, key) outside U and the protected keys."""
    cache = {}
    free = list(range(C))
    out = []
    for s, (l, U, prot) in enumerate(seq):
        keys = [l * E + e for e in U]
        hit = [k in cache for k in keys]
        misses = [k for k, h in zip(keys, hit) if not h]
        n_free = len(free)
        need = max(0, len(misses) - n_free)
        skip = set(keys) | set(prot)
        cand = sorted((st, k) for k, (st, sl) in cache.items() if k not in skip)
        victims = [k for _, k in cand[:need]]
        assert len(victims) == need
        assigned = []
        free_sorted = sorted(free)
        for i, k in enumerate(misses):
            if i < n_free:
                assigned.append((k, free_sorted[i], -1))
            else:
                v = victims[i - n_free]
                assigned.append((k, cache[v][1], v))
        for v in victims:
            del cache[v]
        for k, sl, _ in assigned:
            if sl in free:
                free.remove(sl)
            cache[k] = (s, sl)
        for k in keys:
            cache[k] = (s, cache[k][1])
        out.append((hit, assigned, {k: sl for k, (st, sl) in cache.items()}))
    return out


def test_prefetch_steps_against_brute_force():
    """R8: route steps alternating with prefetch steps of the next layer (every expert, the
    previous step's keys protected) against an independent dictionary model."""
    L, E = 4, 6
    for seed in range(5):
        rng = np.random.default_rng(100 + seed)
        for C in (2 * E, 2 * E + 3, 3 * E):
            seq = []
            prev = None
            for rep in range(3):
                for l in range(L):
                    if prev is not None:
                        seq.append((l, list(range(E)), [prev[0] * E + e for e in prev[1]]))
                    U = sorted(set(int(x) for x in rng.integers(0, E, size=4)))
                    seq.append((l, U, []))
                    prev = (l, U)
            c = LRUCache(C, L * E)
            ref = _brute_force_protected(seq, C, E)
            for s, (l, U, prot) in enumerate(seq):
                rec = c.step(l, U, E, s, protected=prot)
                hit, assigned, content = ref[s]
                assert rec.hit == hit, (seed, C, s)
                assert [tuple(m) for m in rec.misses] == assigned, (seed, C, s)
                got = {k: sl for sl, k in enumerate(rec.key_of) if k >= 0}
                assert got == content, (seed, C, s)
                assert not any(v in set(prot) for _, _, v in rec.misses)


def test_prefetch_makes_the_next_step_all_hits_and_protects():
    L, E = 3, 8
    c = LRUCache(2 * E, L * E)
    c.step(0, [1, 2, 5], E, 0)
    pf = c.step(1, list(range(E)), E, 1, protected=[0 * E + e for e in (1, 2, 5)])
    assert sum(not h for h in pf.hit) == E  # every expert of layer 1 fetched
    r = c.step(1, [0, 3, 7], E, 2)
    assert all(r.hit) and not r.misses
    # the next prefetch must evict the oldest unprotected keys: layer 0's keys go first,
    # layer 1's routed keys (protected) stay
    pf2 = c.step(2, list(range(E)), E, 3, protected=[1 * E + e for e in (0, 3, 7)])
    victims = [v for _, _, v in pf2.misses if v >= 0]
    assert set(victims).isdisjoint({E + 0, E + 3, E + 7})
    assert {0 * E + e for e in (1, 2, 5)} <= set(victims)


def test_prefetch_capacity_error_when_protected_fill_the_cache():
    E = 4
    c = LRUCache(E + 2, 2 * E)
    c.step(0, [0, 1, 2, 3], E, 0)
    with pytest.raises(CapacityError):
        c.step(1, list(range(E)), E, 1, protected=[0, 1, 2, 3])


def test_stamps_beyond_32_bits_change_nothing_but_the_stamps():
    """The rule depends only on the order of stamps: the same accesses from a counter that
    starts just below 2^32 (so that it crosses it) give the same hits, victims, slots and
    occupancy as from 0, with every stamp shifted by the offset."""
    import random
    rng = random.Random(5)
    E, L, C = 16, 3, 10
    trace = [(s % L, sorted(rng.sample(range(E), rng.randint(1, 4)))) for s in range(300)]
    off = (1 << 32) - 7
    a, b = LRUCache(C, L * E), LRUCache(C, L * E)
    for s, (l, U) in enumerate(trace):
        if s == 150:
            assert a.resize(6) == b.resize(6)
        ra, rb = a.step(l, U, E, s), b.step(l, U, E, s + off)
        assert (ra.hit, ra.slot, ra.misses, ra.key_of, ra.n) == (rb.hit, rb.slot, rb.misses,
                                                                 rb.key_of, rb.n)
        assert [x + off if x >= 0 else -1 for x in ra.stamp] == rb.stamp
    assert max(b.stamp) > (1 << 32)
