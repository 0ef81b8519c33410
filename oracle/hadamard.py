"""Walsh-Hadamard transform in natural (Sylvester) order.

PolyKV, Abstract: values pass through a fast Walsh-Hadamard rotation before they are
quantised.
The pages name no ordering, normalisation or random signs, so the plain reading is
used: the Sylvester matrix H with H[i][j] = (-1)^popcount(i & j), no sign
randomisation and no permutation. The orthonormal transform is H / sqrt(d).
"""

import numpy as np


def hadamard_matrix(d: int) -> np.ndarray:
    """Explicit d x d Sylvester Hadamard matrix (fp64), entries +-1."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    parity = np.zeros_like(bits)
    while np.any(bits):
        parity ^= bits & 1
        bits >>= 1
    return np.where(parity == 1, -1.0, 1.0)


def fwht(x) -> np.ndarray:
    """Unnormalised FWHT along the last axis, in fp64: returns x @ H (H is symmetric).

    The butterfly: for h = 1, 2, 4, ..., d/2, within each block of 2h entries the pair
    (a, b) at offsets (i, i + h) becomes (a + b, a - b).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        blocks = y.reshape(lead + (d // (2 * h), 2, h))
        a = blocks[..., 0, :].copy()
        b = blocks[..., 1, :].copy()
        blocks[..., 0, :] = a + b
        blocks[..., 1, :] = a - b
        h *= 2
    return y
