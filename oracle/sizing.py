"""Budget-driven cache sizing (test oracle only).

Pages: "FreeToken vs vLLM on one RTX 3090" (Runtime configurations: an automatic cache of
2,486 slots with the whole routed-expert bank kept in host memory); "FreeToken: az VRAM ile
büyük MoE modelleri" ("KV cache": a KV floor is reserved before the expert cache is filled;
"Dilim küçülünce ne kaybediliyor": the expert cache gets the usable VRAM left after the KV
reserve); "FreeToken：在消费级 NVIDIA GPU 上进行 MoE 推理" (--offload-ratio r keeps the
fraction 1 - r of the experts on the GPU).

Reading: slots = the largest C with C * S + workspace(C) <= free - reserve (reserve = the KV
floor plus whatever else must stay resident), limited to floor((1 - r) * L * E) when an
offload ratio r is given, to L * E, and to the handle's slot limit; below the capacity floor
min(max_tokens * top_k, E) there is no valid cache.  The pages' own numbers do not reconcile
(the 18 GB slice's cached fraction is printed inverted), so only the arithmetic is pinned.
"""
from __future__ import annotations

import math


def auto_capacity(free_bytes: int, reserve_bytes: int, blob_bytes: int, n_keys: int,
                  floor: int, slot_limit: int, workspace, offload_ratio: float | None = None):
    """Largest admissible capacity, or None when even the floor does not fit.

    workspace(C) -> device bytes of the handle's workspace for C slots."""
    budget = free_bytes - reserve_bytes
    top = min(n_keys, slot_limit)
    if offload_ratio is not None:
        top = min(top, math.floor((1.0 - offload_ratio) * n_keys))
    best = None
    for c in range(floor, top + 1):
        if c * blob_bytes + workspace(c) <= budget:
            best = c
    return best
