"""Workload shapes for the expert-offload MoE layer step (synthetic, seed 0).

Each workload is one model shape plus a cache budget and a token schedule:

* ``tiny`` - 1 layer, hidden 256, 16 experts top-2, SwiGLU intermediate 128,
  bf16, 8 cache slots, 64 decode tokens at batch 1.
* ``qwen35b_decode`` - 48 layers, hidden 2048, 128 experts top-8, intermediate
  768, bf16 (9 MiB per expert), cache = 30% of the pool (1,843 slots), 512 decode
  tokens at batch 1.
* ``qwen35b_prefill`` - the same shape, one 16,384-token prefill chunk with
  i.i.d. N(0,1) activations, cache 30% of the pool.
* ``qwen35b_decode_b8`` - the 35B shape with 8 concurrent decode streams batched (8 tokens per
  layer step, one cache step and one dedup for all of them).
* ``dsv4_fp8_decode`` - 43 layers, hidden 4096, 256 routed experts top-8 plus one
  GPU-resident shared expert, intermediate 2048, fp8-e4m3 with a fp32 scale per
  1x128 block (24.75 MiB per expert), cache = 17% of the pool, 512 decode tokens.
* ``glm_mxfp4_4stream`` - 8 layers at hidden 6144, 256 experts top-8,
  intermediate 2048, MXFP4 (19.125 MiB per expert); 4 decode streams batched
  (4 tokens per step) for 1,024 steps; the cache budget shrinks from 40% to 15%
  of the pool before token step 512.

Capacities are floor(fraction * layers * experts) slots.
"""
from __future__ import annotations

import dataclasses
import math


def blob_bytes(fmt: int, H: int, I: int) -> int:
    if fmt == 0:
        return 6 * I * H
    if fmt == 1:
        return 3 * I * H + 4 * (2 * I * (H // 128)) + 4 * ((I // 128) * H)
    if fmt == 2:
        return 3 * I * H // 2 + 2 * I * (H // 32) + (I // 32) * H
    raise ValueError(fmt)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    hidden: int
    experts: int
    top_k: int
    inter: int
    fmt: int                 # 0 bf16, 1 fp8-e4m3 1x128, 2 mxfp4
    cache_frac: float
    tokens_per_step: int     # T: tokens in one layer step (streams at decode, chunk at prefill)
    token_steps: int         # token steps (decode) or chunks (prefill)
    kind: str                # "decode" or "prefill"
    has_shared: bool = False
    resize_at: int = -1      # token step before which the cache is resized
    resize_frac: float = 0.0
    fixed_capacity: int = 0  # overrides cache_frac when > 0
    seed: int = 0

    @property
    def blob_bytes(self) -> int:
        return blob_bytes(self.fmt, self.hidden, self.inter)

    @property
    def n_keys(self) -> int:
        return self.layers * self.experts

    @property
    def pool_bytes(self) -> int:
        return self.n_keys * self.blob_bytes

    @property
    def capacity(self) -> int:
        if self.fixed_capacity:
            return self.fixed_capacity
        return int(math.floor(self.cache_frac * self.n_keys + 1e-9))

    @property
    def resize_capacity(self) -> int:
        return int(math.floor(self.resize_frac * self.n_keys + 1e-9))

    def with_layers(self, layers: int) -> "Workload":
        """Same shape and cache fraction with fewer layers (capacity rescaled)."""
        return dataclasses.replace(self, name=f"{self.name}_L{layers}", layers=layers)

    def with_steps(self, token_steps: int) -> "Workload":
        return dataclasses.replace(self, token_steps=token_steps)

    def with_tokens(self, tokens: int) -> "Workload":
        """Same shape with a different number of tokens per layer step."""
        return dataclasses.replace(self, name=f"{self.name}_T{tokens}", tokens_per_step=tokens)

    def as_prefill(self, tokens: int) -> "Workload":
        """One chunk of `tokens` i.i.d. activations through the same layers and cache."""
        return dataclasses.replace(self, name=f"{self.name}_prefill{tokens}", kind="prefill",
                                   tokens_per_step=tokens, token_steps=1, resize_at=-1)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 16, 2, 128, 0, 0.0, 1, 64, "decode", fixed_capacity=8),
    "qwen35b_decode": Workload("qwen35b_decode", 48, 2048, 128, 8, 768, 0, 0.30, 1, 512, "decode"),
    "qwen35b_prefill": Workload("qwen35b_prefill", 48, 2048, 128, 8, 768, 0, 0.30, 16384, 1,
                                "prefill"),
    "qwen35b_decode_b8": Workload("qwen35b_decode_b8", 48, 2048, 128, 8, 768, 0, 0.30, 8, 512,
                                  "decode"),
    "dsv4_fp8_decode": Workload("dsv4_fp8_decode", 43, 4096, 256, 8, 2048, 1, 0.17, 1, 512,
                                "decode", has_shared=True),
    "glm_mxfp4_4stream": Workload("glm_mxfp4_4stream", 8, 6144, 256, 8, 2048, 2, 0.40, 4, 1024,
                                  "decode", resize_at=512, resize_frac=0.15),
}
