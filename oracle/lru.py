"""Linked-list LRU simulator of the shared (layer, expert) slot cache (test oracle only).

Follows:
* FreeToken paper summary, memory-architecture paragraph: one elastic GPU expert
  cache shared by every MoE layer, its slots managed by the logical id
  (layer, expert).
* FreeToken paper summary, execution-layer paragraph: per layer, hit
  classification and LRU victim selection after routing dedup; when the VRAM
  budget changes the cache is rebuilt at a scheduler safe point without
  restarting the engine.
* FreeToken paper summary, attribution paragraph, and the "FreeToken vs vLLM on
  one RTX 3090" report (Runtime configurations; "FreeToken exploits MoE
  sparsity"): the replacement policy is a global LRU.

The pages name the policy but not its granularity, tie order or slot
assignment.  The rule implemented here (the GPU path implements the same rule
independently):

R1  key = layer * E + expert.
R2  a key of the step's distinct set U is a hit iff it is cached.
R3  misses are taken in ascending expert id; free slots are exactly [n, C)
    (occupied slots always form the prefix [0, n)).
R4  need = max(0, #misses - (C - n)); the victims are the first `need` keys met
    walking from the LRU end, skipping keys of U.
R5  miss i takes free slot n + i while free slots last, then the slots of the
    victims in walk order.
R6  victims leave; every key of U (hits and misses) moves to the MRU end in
    ascending expert id with stamp = s, the global step counter.  The list order
    is therefore always ascending (stamp, key).
R8  prefetch (steps of many tokens only): before layer l' is routed, a prefetch step of
    layer l' is an R1-R6 step whose U is every expert of l', except that the victims also
    skip the keys of a protected set (the distinct keys of the layer step just before it,
    whose expert FFN may still be reading their slots).  It takes its own value of the
    step counter.  (FreeToken paper summary, problem paragraph: a long prefill's routing
    union covers nearly every expert of every layer; "FreeToken：在消费级 NVIDIA GPU 上进行
    MoE 推理", "FreeToken 解决的问题": experts are streamed ahead so that transfers overlap
    compute - so layer l' can be fetched while layer l computes.)
R9  hybrid decode (CPU in-place compute of some misses): of the step's m misses, in
    ascending expert id, the first m - q are filled as R3-R6 and the last q are computed
    by the CPU straight from the host pool: they take no slot, evict nothing and are not
    stamped (they are not cached), so need = max(0, m - q - (C - n)).  q comes from the
    miss split (oracle/split.py).  (FreeToken paper summary: a decode miss is either moved
    over PCIe or computed in place by the CPU; q is derived in the fused routing kernel.)
R7  resize to C': if n <= C' nothing moves.  Otherwise the C' keys nearest the
    MRU end survive; holes in [0, C') are filled, in ascending slot order, by the
    survivors that sit in slots >= C', taken in ascending old-slot order; stamps
    are kept and n = C'.  Growing adds empty slots [C, C').
"""
from __future__ import annotations

from collections import OrderedDict
from dataclasses import dataclass, field


class CapacityError(ValueError):
    pass


@dataclass
class StepRecord:
    step: int
    layer: int
    U: list                  # distinct experts, ascending
    hit: list                # bool per entry of U
    slot: list               # cache slot per entry of U after the step
    misses: list             # (key, slot, victim_key or -1) in ascending expert id, filled
    cpu: list = field(default_factory=list)  # keys computed in place by the CPU (R9)
    key_of: list = field(default_factory=list)
    stamp: list = field(default_factory=list)
    n: int = 0


class LRUCache:
    def __init__(self, capacity: int, n_keys: int):
        if capacity <= 0:
            raise CapacityError("capacity must be positive")
        self.C = capacity
        self.n_keys = n_keys
        self.order: "OrderedDict[int, int]" = OrderedDict()  # key -> slot, LRU end first
        self.key_of = [-1] * capacity
        self.stamp = [-1] * capacity
        self.n = 0

    def slot_of(self, key: int) -> int:
        return self.order.get(key, -1)

    def step(self, layer: int, U, E: int, s: int, protected=(), n_cpu: int = 0) -> StepRecord:
        """R1-R6; `protected` keys are never victims either (R8); the last `n_cpu` misses
        are computed by the CPU and not cached (R9)."""
        keys = [layer * E + int(e) for e in U]                          # R1 (U ascending)
        if len(keys) > self.C:
            raise CapacityError(f"{len(keys)} distinct experts exceed capacity {self.C}")
        hit = [key in self.order for key in keys]                       # R2
        all_misses = [key for key, h in zip(keys, hit) if not h]         # R3
        if not 0 <= n_cpu <= len(all_misses):
            raise ValueError("n_cpu out of range")
        misses = all_misses[:len(all_misses) - n_cpu]                    # R9
        cpu = all_misses[len(all_misses) - n_cpu:]
        n_free = self.C - self.n
        need = max(0, len(misses) - n_free)                              # R4
        in_step = set(keys) | set(protected)
        victims = []
        for key in self.order:
            if len(victims) == need:
                break
            if key in in_step:
                continue
            victims.append(key)
        if len(victims) < need:
            raise CapacityError("not enough evictable slots")
        assigned = []                                                    # R5
        for i, key in enumerate(misses):
            if i < n_free:
                assigned.append((key, self.n + i, -1))
            else:
                v = victims[i - n_free]
                assigned.append((key, self.order[v], v))
        for v in victims:                                                # R6
            del self.order[v]
        slot_of_new = {key: slot for key, slot, _ in assigned}
        cpu_set = set(cpu)
        for key in keys:
            if key in cpu_set:
                continue
            slot = self.order.pop(key) if key in self.order else slot_of_new[key]
            self.order[key] = slot
            self.key_of[slot] = key
            self.stamp[slot] = s
        self.n = min(self.C, self.n + len(misses))
        return StepRecord(step=s, layer=layer, U=[int(e) for e in U], hit=hit,
                          slot=[self.order.get(key, -1) for key in keys], misses=assigned,
                          cpu=cpu, key_of=list(self.key_of), stamp=list(self.stamp), n=self.n)

    def resize(self, new_capacity: int):
        """R7.  Returns the list of (old_slot, new_slot) moves, in ascending new slot."""
        if new_capacity <= 0:
            raise CapacityError("capacity must be positive")
        if new_capacity >= self.C:
            self.key_of += [-1] * (new_capacity - self.C)
            self.stamp += [-1] * (new_capacity - self.C)
            self.C = new_capacity
            return []
        if self.n <= new_capacity:
            self.key_of = self.key_of[:new_capacity]
            self.stamp = self.stamp[:new_capacity]
            self.C = new_capacity
            return []
        lru_first = list(self.order.keys())
        evicted = lru_first[: self.n - new_capacity]
        evicted_slots = [self.order[k] for k in evicted]
        for k in evicted:
            del self.order[k]
        holes = sorted(sl for sl in evicted_slots if sl < new_capacity)
        movers = sorted(sl for sl in self.order.values() if sl >= new_capacity)
        assert len(holes) == len(movers)
        moves = list(zip(movers, holes))
        key_at = {sl: k for k, sl in self.order.items()}
        for src, dst in moves:
            key = key_at[src]
            self.order[key] = dst
            self.key_of[dst] = key
            self.stamp[dst] = self.stamp[src]
        self.key_of = self.key_of[:new_capacity]
        self.stamp = self.stamp[:new_capacity]
        self.C = new_capacity
        self.n = new_capacity
        return moves
