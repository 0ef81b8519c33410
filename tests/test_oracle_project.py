"""Pins of the oracle projection: brute-force sums, exact integer products, head order."""

import math

import numpy as np

from oracle import project_fp16, project_fp64


def test_brute_force_small():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 8)).astype(np.float16)
    w = rng.standard_normal((4, 8)).astype(np.float16)      # 2 heads of dim 2
    got = project_fp64(x, w, 2, 2)
    for h in range(2):
        for t in range(3):
            for i in range(2):
                want = math.fsum(float(x[t, k]) * float(w[h * 2 + i, k]) for k in range(8))
                assert abs(got[h, t, i] - want) <= 1e-12 * max(1.0, abs(want))


def test_integer_products_are_exact_and_rounded_once():
    # small integers: the fp64 sums are exact; 2049 is a tie between 2048 and 2050 in fp16
    x = np.array([[1, 2048, 1]], dtype=np.float16)
    w = np.array([[1, 1, 0], [0, 1, 1], [1, 0, 0]], dtype=np.float16)
    y = project_fp16(x, w, 3, 1)
    assert [float(v) for v in y.reshape(-1)] == [2048.0, 2048.0, 1.0]   # 2049 -> 2048 (even)
    x = np.array([[3, 2048, 0]], dtype=np.float16)
    y = project_fp16(x, w, 3, 1)
    assert float(y[0, 0, 0]) == 2052.0                                   # 2051 -> 2052 (even)


def test_head_major_order():
    # W = identity: head h, dim i of token t is x[t, h*d + i]
    n, H, d = 5, 3, 4
    x = np.arange(n * H * d, dtype=np.float16).reshape(n, H * d) / 8
    y = project_fp16(x, np.eye(H * d, dtype=np.float16), H, d)
    for h in range(H):
        assert np.array_equal(y[h], x[:, h * d:(h + 1) * d])
