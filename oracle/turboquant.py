"""TurboQuant-MSE value compression.

PolyKV, Abstract: values are compressed with TurboQuant MSE, which rotates each vector
with a fast Walsh-Hadamard transform and then applies a 3-bit Lloyd-Max quantiser
fitted to N(0,1). Steps used, per value head vector v of length d:
1. n = ||v||_2;
2. u = v / n * sqrt(d) (so the coordinates of the rotated vector are ~N(0,1));
3. y = H u / sqrt(d), the orthonormal Sylvester FWHT;
4. code_i = #{k : y_i > b_k}: code 0 is the most negative centroid and a coordinate
   lying exactly on a boundary takes the lower code;
5. stored: the d codes and fp16(n), rounded to nearest even.
A zero vector (n = 0) is stored as y = 0, which gives code 3 everywhere (the middle
boundary is exactly 0 and ties go down), and norm 0.
Decoding inverts steps 3 and 2 with the stored fp16 norm: v_hat = n16/sqrt(d) * H c[code] / sqrt(d).
"""

import math

import numpy as np

from .hadamard import fwht


def rotated_coordinates(v) -> np.ndarray:
    """Steps 1-3 in fp64: y [..., d] for fp16 v [..., d]."""
    x = np.asarray(v).astype(np.float64)
    d = x.shape[-1]
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n > 0, x / safe * math.sqrt(d), 0.0)
    return fwht(u) / math.sqrt(d)


def tq_mse_encode(v, boundaries):
    """v: fp16 [..., d]; boundaries: 7 ascending float32 values.

    Returns (codes uint8 [..., d] in 0..7, norms fp16 [...]).
    """
    v = np.asarray(v)
    if v.dtype != np.float16:
        raise TypeError("values must be fp16")
    x = v.astype(np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1))
    y = rotated_coordinates(v)
    b = np.asarray(boundaries, dtype=np.float32).astype(np.float64)
    codes = np.zeros(y.shape, dtype=np.uint8)
    for bk in b:
        codes += (y > bk).astype(np.uint8)
    return codes, n.astype(np.float16)


def tq_mse_decode(codes, norms, centroids) -> np.ndarray:
    """fp64 v_hat [..., d] from codes, fp16 norms and float32 centroids."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    y_hat = c[codes.astype(np.intp)]
    u_hat = fwht(y_hat) / math.sqrt(d)
    n = np.asarray(norms).astype(np.float64)[..., None]
    return u_hat * n / math.sqrt(d)
