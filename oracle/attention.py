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


def attention_lse(q, k_hat, scale: float) -> np.ndarray:
    """q [R][d], k_hat [T][d] -> [R]: ln sum_t exp(scale * q . k_t) in fp64 (the
    normaliser of the softmax, kept so that results over disjoint token sets can be
    combined)."""
    s = scale * (np.asarray(q, dtype=np.float64) @ np.asarray(k_hat, dtype=np.float64).T)
    m = np.max(s, axis=-1)
    return m + np.log(np.sum(np.exp(s - m[:, None]), axis=-1))


def shared_pool_lse(q, k_hat, gqa: int, scale: float, layers=None) -> np.ndarray:
    """ln sum over the pool's tokens of exp(scale q . k) for every row of q [L][A][H*G][d];
    k_hat [L][H][T][d]. Returns fp64 [L'][A][H*G]."""
    q = np.asarray(q)
    L, A, HG, d = q.shape
    H = HG // gqa
    layers = range(L) if layers is None else layers
    out = np.zeros((len(layers), A, HG), dtype=np.float64)
    for li, l in enumerate(layers):
        for h in range(H):
            rows = q[l, :, h * gqa:(h + 1) * gqa, :].reshape(A * gqa, d)
            out[li, :, h * gqa:(h + 1) * gqa] = attention_lse(rows, k_hat[l, h], scale).reshape(A, gqa)
    return out


def pool_and_tail_decode(q, k_hat, v_hat, tail_k, tail_v, tail_len, gqa: int, scale: float,
                         layers=None) -> np.ndarray:
    """Decode with private tails: every query row of agent a attends over the shared
    pool's tokens followed by the first tail_len[a] tokens of its own tail, as one softmax
    over the union (the definition; nothing is merged).

    q: [L][A][H*G][d]; k_hat, v_hat: [L][H][T][d] (pool, dequantised);
    tail_k, tail_v: [A][L][H][cap][d]; tail_len: [A]. Returns fp64 [L'][A][H*G][d] for the
    chosen layers, with the tails indexed by the same layer order.
    """
    q = np.asarray(q)
    L, A, HG, d = q.shape
    H = HG // gqa
    layers = range(L) if layers is None else layers
    out = np.zeros((len(layers), A, HG, d), dtype=np.float64)
    for li, l in enumerate(layers):
        for a in range(A):
            n = int(tail_len[a])
            for h in range(H):
                keys = np.concatenate([np.asarray(k_hat[l, h], dtype=np.float64),
                                       np.asarray(tail_k[a, li, h, :n], dtype=np.float64)])
                vals = np.concatenate([np.asarray(v_hat[l, h], dtype=np.float64),
                                       np.asarray(tail_v[a, li, h, :n], dtype=np.float64)])
                rows = q[l, a, h * gqa:(h + 1) * gqa, :]
                out[li, a, h * gqa:(h + 1) * gqa, :] = attention_rows(rows, keys, vals, scale)
    return out
