"""SwiGLU expert FFN and weighted combine in float64 (test oracle only).

The pages say selected experts run on the GPU after they are fetched ("FreeToken
vs vLLM on one RTX 3090", section "FreeToken exploits MoE sparsity") but never
give the expert form.  The form used here, and by the GPU path, is the SwiGLU
expert: FFN_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x)), silu(z) = z / (1 + e^-z), and
the layer output y_t = sum_j w_{t,j} FFN_{e_{t,j}}(x_t) (+ FFN_shared(x_t) with
weight 1 when the model has a GPU-resident shared expert).
"""
from __future__ import annotations

import numpy as np


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """x [n, H] -> [n, H] in float64."""
    x = np.asarray(x, dtype=np.float64)
    return (silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T


def moe_output(x: np.ndarray, idx: np.ndarray, w: np.ndarray, weights_of, shared=None) -> np.ndarray:
    """y[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x[t]) (+ FFN_shared(x[t])).

    weights_of(e) returns (Wg, Wu, Wd) of routed expert e; shared is (Wg, Wu, Wd) or None."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    y = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for j in range(idx.shape[1]):
            Wg, Wu, Wd = weights_of(int(idx[t, j]))
            y[t] += w[t, j] * expert_ffn(x[t:t + 1], Wg, Wu, Wd)[0]
        if shared is not None:
            y[t] += expert_ffn(x[t:t + 1], *shared)[0]
    return y
