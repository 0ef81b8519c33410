"""Decode attention of N agents against the shared pool, in fp64.

PolyKV, Abstract: one compressed pool is handed to N separate agent contexts, all of
which read it at the same time. One decode step of one agent is
ordinary softmax attention of each of its query heads over every token of the shared
pool (all pool tokens precede the query, so there is no mask). Query head j reads KV
head floor(j / G) when G query heads share a KV head.
"""

import numpy as np


def attention_weights(q, k_hat, scale: float) -> np.ndarray:
    """q [R][d], k_hat [T][d] -> softmax(scale * q k^T) [R][T] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    s = scale * (q @ np.asarray(k_hat, dtype=np.float64).T)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    return p / np.sum(p, axis=-1, keepdims=True)


def attention_rows(q, k_hat, v_hat, scale: float) -> np.ndarray:
    """q [R][d], k_hat [T][d], v_hat [T][d] -> [R][d]; softmax(scale * q k^T) v in fp64."""
    return attention_weights(q, k_hat, scale) @ np.asarray(v_hat, dtype=np.float64)


def shared_pool_decode(q, k_hat, v_hat, gqa: int, scale: float, layers=None) -> np.ndarray:
    """All agents' query rows against the dequantised pool.

    q: [L][A][H*G][d]; k_hat, v_hat: [L][H][T][d] (fp64 per-token reconstructions).
    Returns fp64 [L'][A][H*G][d] for the chosen layers (default: all).
    """
    q = np.asarray(q)
    L, A, HG, d = q.shape
    H = HG // gqa
    layers = range(L) if layers is None else layers
    out = np.zeros((len(layers), A, HG, d), dtype=np.float64)
    for li, l in enumerate(layers):
        for h in range(H):
            rows = q[l, :, h * gqa:(h + 1) * gqa, :].reshape(A * gqa, d)
            o = attention_rows(rows, k_hat[l, h], v_hat[l, h], scale)
            out[li, :, h * gqa:(h + 1) * gqa, :] = o.reshape(A, gqa, d)
    return out
