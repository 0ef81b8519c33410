"""Pins of the oracle's decode attention: brute force and special cases."""

import math

import numpy as np
import pytest

from oracle import (attention_rows, attention_weights, codebook_fp32, compress_pool, dequant_pool,
                    shared_pool_decode)


def _brute(q, k, v, scale):
    out = []
    for qr in q:
        s = [scale * sum(float(a) * float(b) for a, b in zip(qr, kt)) for kt in k]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        out.append([sum(e[t] / z * float(v[t][i]) for t in range(len(k))) for i in range(len(v[0]))])
    return np.array(out)


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_brute_force_small(T):
    rng = np.random.default_rng(T)
    q, k, v = rng.standard_normal((3, 16)), rng.standard_normal((T, 16)), rng.standard_normal((T, 16))
    assert np.allclose(attention_rows(q, k, v, 0.25), _brute(q, k, v, 0.25), atol=1e-13)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((1, 32))
    o = attention_rows(rng.standard_normal((4, 32)) * 100, rng.standard_normal((1, 32)), v, 1.0)
    assert np.allclose(o, np.repeat(v, 4, axis=0), atol=1e-14)


def test_zero_query_or_identical_keys_average_values():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((9, 32))
    o = attention_rows(np.zeros((2, 32)), rng.standard_normal((9, 32)), v, 1.0)
    assert np.allclose(o, v.mean(axis=0), atol=1e-14)
    k = np.repeat(rng.standard_normal((1, 32)), 9, axis=0)
    o = attention_rows(rng.standard_normal((2, 32)), k, v, 1.0)
    assert np.allclose(o, v.mean(axis=0), atol=1e-13)


def test_large_scale_selects_argmax_token():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((1, 32)), rng.standard_normal((20, 32)), rng.standard_normal((20, 32))
    o = attention_rows(q, k, v, 1e4)
    assert np.allclose(o[0], v[np.argmax(k @ q[0])], atol=1e-12)


def test_agent_permutation_and_gqa_head_mapping():
    c32, b32 = codebook_fp32()
    rng = np.random.default_rng(4)
    L, H, T, d, A, G = 2, 2, 40, 64, 3, 2
    k = rng.standard_normal((L, H, T, d)).astype(np.float16)
    v = rng.standard_normal((L, H, T, d)).astype(np.float16)
    kh, vh = dequant_pool(compress_pool(k, v, b32), c32)
    q = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    o = shared_pool_decode(q, kh, vh, G, 0.125)
    perm = [2, 0, 1]
    assert np.allclose(shared_pool_decode(q[:, perm], kh, vh, G, 0.125), o[:, perm], atol=1e-14)
    # query head j reads KV head j // G
    for j in range(H * G):
        want = attention_rows(q[1, :, j, :], kh[1, j // G], vh[1, j // G], 0.125)
        assert np.allclose(o[1, :, j, :], want, atol=1e-14)


def test_weights_brute_force_and_normalised():
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((3, 16)), rng.standard_normal((6, 16))
    w = attention_weights(q, k, 0.3)
    assert np.allclose(w.sum(axis=-1), 1.0, atol=1e-15)
    for r in range(3):
        s = [0.3 * sum(float(a) * float(b) for a, b in zip(q[r], kt)) for kt in k]
        e = [math.exp(x - max(s)) for x in s]
        assert np.allclose(w[r], [x / sum(e) for x in e], atol=1e-15)
