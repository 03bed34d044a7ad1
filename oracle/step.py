"""One MoE layer step, and whole workloads, composed from the oracle parts (test oracle only).

Order of one layer step (FreeToken paper summary, execution-layer paragraph;
"FreeToken vs vLLM on one RTX 3090", section "FreeToken exploits MoE sparsity"):
router -> top-k -> per-step dedup -> hit classification -> LRU victims and slot
update -> fills of the missed experts -> expert FFN and combine.  Fills are a
byte copy of pool[key] into the slot, so the FFN reads the pool blob directly.

Step counter: s increments once per layer step; decode visits token step t
outer and layer l inner (s = t * L + l); a prefill chunk visits layers in order.
With prefetch (R8), a prefetch step of layer l + 1 follows the step of layer l and takes
the next counter value.
With a miss split (R9, decode steps of at most 8 tokens only), the last q of a step's misses
are computed by the CPU and not cached, q = miss_split(m, b_cpu, b_pcie); the layer output is
the same sum over the selected experts whichever device computes each.
At decode all streams of a step (T tokens) share one dedup and one cache step.
The resize happens at the safe point before token step ``resize_at``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .dedup import dedup
from .ffn import moe_output
from .formats import bf16_to_f64, decode_blob
from .lru import LRUCache, StepRecord
from .router import router_logits, topk_softmax
from .split import miss_split


@dataclass
class LayerStep:
    token_step: int
    layer: int
    s: int
    topk_idx: np.ndarray
    topk_w: np.ndarray
    U: list
    count: np.ndarray
    offset: np.ndarray
    perm: np.ndarray
    rec: StepRecord
    y: np.ndarray | None = None


class Oracle:
    """Float64 oracle over one workload.

    pool      - uint8 array of L*E blobs (layer-major), or a callable key -> blob bytes
    router    - uint16 (bf16) array [L, E, H]
    shared    - optional callable layer -> shared-expert blob bytes
    split     - optional (b_cpu, b_pcie) integer rates: hybrid decode (R9)
    """

    DECODE_MAX_TOKENS = 8

    def __init__(self, wl, pool, router, shared=None, split=None):
        self.wl = wl
        self.pool = pool
        self.router = router
        self.shared = shared
        self.split = split
        self.cache = LRUCache(wl.capacity, wl.n_keys)
        self.s = 0

    def blob(self, key: int) -> np.ndarray:
        if callable(self.pool):
            return self.pool(key)
        S = self.wl.blob_bytes
        return self.pool[key * S:(key + 1) * S]

    def expert_weights(self, layer: int, e: int):
        wl = self.wl
        return decode_blob(self.blob(layer * wl.experts + e), wl.fmt, wl.hidden, wl.inter)

    def layer_step(self, token_step: int, layer: int, x_bf16: np.ndarray, with_ffn: bool) -> LayerStep:
        wl = self.wl
        x = bf16_to_f64(x_bf16).reshape(-1, wl.hidden)
        z = router_logits(x, bf16_to_f64(self.router[layer]))
        idx, w = topk_softmax(z, wl.top_k)
        U, count, offset, perm = dedup(idx, wl.experts)
        n_cpu = 0
        if self.split is not None and x.shape[0] <= self.DECODE_MAX_TOKENS:
            m = sum(1 for e in U if self.cache.slot_of(layer * wl.experts + int(e)) < 0)
            n_cpu = miss_split(m, *self.split)
        rec = self.cache.step(layer, U, wl.experts, self.s, n_cpu=n_cpu)
        y = None
        if with_ffn:
            decoded = {}

            def weights_of(e):
                if e not in decoded:
                    decoded[e] = self.expert_weights(layer, e)
                return decoded[e]

            sh = None
            if wl.has_shared:
                sh = decode_blob(self.shared(layer), wl.fmt, wl.hidden, wl.inter)
            y = moe_output(x, idx, w, weights_of, sh)
        out = LayerStep(token_step, layer, self.s, idx, w, U, count, offset, perm, rec, y)
        self.s += 1
        return out

    def prefetch(self, layer: int, protected_layer: int, protected_U) -> StepRecord:
        """R8: fetch every expert of `layer` before it is routed; the keys of the previous
        layer step (`protected_layer`, its distinct experts `protected_U`) are not evicted."""
        E = self.wl.experts
        prot = [protected_layer * E + int(e) for e in protected_U]
        rec = self.cache.step(layer, list(range(E)), E, self.s, protected=prot)
        self.s += 1
        return rec

    def resize(self, new_capacity: int):
        return self.cache.resize(new_capacity)

    def run(self, acts, with_ffn=lambda t, l: False, token_steps=None):
        """Yield LayerStep for every layer step of the workload, in order.

        acts: decode - uint16 [ntok, L, T, H]; prefill - uint16 [L, T, H] (one chunk)."""
        wl = self.wl
        n_t = wl.token_steps if token_steps is None else token_steps
        for t in range(n_t):
            if wl.resize_at >= 0 and t == wl.resize_at:
                self.resize(wl.resize_capacity)
            for l in range(wl.layers):
                x = acts[t, l] if wl.kind == "decode" else acts[l]
                yield self.layer_step(t, l, x, with_ffn(t, l))
