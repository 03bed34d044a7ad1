"""Router logits and renormalised softmax top-k in float64 (test oracle only).

Follows the "FreeToken vs vLLM on one RTX 3090" report, section "FreeToken
exploits MoE sparsity": each token selects a fixed number k of its routed
experts (eight of 256 there).  The pages give no gating formula; the reading
used here (and by the GPU path) is the renormalised softmax: the k experts with
the largest logits z_e = x . W_r[e], ordered by descending logit with ties going
to the lower expert id, weighted w_j = exp(z_j - z_max) / sum_{i in top-k}
exp(z_i - z_max).  This equals softmax over all experts renormalised over the
selected ones.
"""
from __future__ import annotations

import numpy as np


def router_logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] * Wr[e, h] (float64)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64).T


def topk_softmax(z: np.ndarray, k: int):
    """Per token: indices of the k largest logits (descending, lower id on ties)
    and their renormalised softmax weights.  Returns (idx int32 [T,k], w float64 [T,k])."""
    z = np.asarray(z, dtype=np.float64)
    T, E = z.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    ids = np.arange(E)
    for t in range(T):
        order = np.lexsort((ids, -z[t]))  # primary key -z (descending z), then ascending id
        sel = order[:k]
        idx[t] = sel
        zs = z[t, sel]
        ex = np.exp(zs - zs[0])
        w[t] = ex / ex.sum()
    return idx, w
