"""K/V projection of a prefill chunk, the input of the fused projection + compression.

TEST INFRASTRUCTURE ONLY (see the package docstring).

PolyKV, Abstract: the shared cache is compressed a single time, when it is written. K and
V of a chunk are the layer's projections of its input rows, held by an fp16 cache as
fp16 values; the pool is the compression of those values. Here: K = RNE16(x W^T) with the
product in fp64 (a library matmul) and one round-to-nearest-even to binary16, arranged
head-major [n_heads][n_tok][head_dim] (output j of W is dim j % head_dim of head
j // head_dim).
"""

import numpy as np


def project_fp64(x, w, n_heads: int, head_dim: int) -> np.ndarray:
    """x [n][hidden], w [n_heads*head_dim][hidden] -> fp64 [n_heads][n][head_dim]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if w.shape != (n_heads * head_dim, x.shape[1]):
        raise ValueError("weight shape does not match")
    y = x @ w.T                                   # [n][n_heads*head_dim]
    return y.reshape(x.shape[0], n_heads, head_dim).transpose(1, 0, 2).copy()


def project_fp16(x, w, n_heads: int, head_dim: int) -> np.ndarray:
    """The fp16 projection an fp16 cache holds: RNE16 of project_fp64."""
    return project_fp64(x, w, n_heads, head_dim).astype(np.float16)
