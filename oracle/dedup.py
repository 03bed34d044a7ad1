"""Per-step routing dedup (test oracle only).

Follows the FreeToken paper summary, execution-layer paragraph (routing dedup
is the first job of the fused per-layer kernel), and the batching observation
of "FreeToken: az VRAM ile büyük MoE modelleri", section "Eş zamanlı istekler"
(one fetched expert serves every request of the batch).  The scope of one dedup
is one layer step: every token of the step, all streams of a batched decode,
the whole chunk of a prefill.
"""
from __future__ import annotations

import numpy as np


def dedup(idx: np.ndarray, E: int):
    """Distinct experts of a step and the tokens routed to each.

    Returns (U, count, offset, perm):
      U      - ascending list of distinct expert ids;
      count  - count[e] = number of (token, j) assignments to expert e, length E;
      offset - exclusive prefix sum of count, length E + 1;
      perm   - assignment ids a = t * k + j grouped by expert (ascending e), with
               ascending token inside an expert; perm[offset[e]:offset[e+1]]
               are the assignments of expert e.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    U = sorted({int(e) for e in flat})
    count = np.bincount(flat, minlength=E).astype(np.int64)
    offset = np.concatenate([[0], np.cumsum(count)]).astype(np.int64)
    # A stable sort of the assignment ids a = t*k + j by expert keeps ascending a, hence
    # ascending token, inside each expert (a token selects an expert at most once).
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    return U, count, offset, perm
