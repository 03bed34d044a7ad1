"""Float64 CPU oracle for the expert-offload MoE layer step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what one MoE layer step computes, used to check the GPU path.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the GPU library never calls into it and shares no
code with it (the two sides only read the same seeded input bytes produced by
``moe_inputs``).

Sources (the FreeToken pages):
* FreeToken paper summary (agihunt.info, arXiv 2608.16157): the memory
  architecture paragraph (full expert pool in host memory, one elastic GPU
  cache shared by all MoE layers, slots keyed by (layer, expert)); the
  execution-layer paragraph (one kernel doing routing dedup, hit
  classification and LRU victim selection; cache rebuilt at a scheduler safe
  point when the VRAM budget changes); the attribution paragraph (global LRU).
* "FreeToken vs vLLM on one RTX 3090" report, section "FreeToken exploits MoE
  sparsity" (eight routed experts chosen per token, an LRU expert cache,
  fetching selected experts on demand) and its Summary (only missed experts
  cross PCIe).

Modules:
* ``formats`` - exact float64 decoding of bf16, e4m3fn, e2m1, e8m0 and of an
  expert blob.
* ``router``  - router logits, renormalised softmax top-k.
* ``dedup``   - per-step distinct experts and per-expert token lists.
* ``lru``     - linked-list LRU simulator for the shared slot cache, with
  elastic resize.
* ``ffn``     - SwiGLU expert FFN and the weighted combine.
* ``step``    - one layer step and whole workloads composed from the above.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, library routines or hand-derived traces.
"""
