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


# ---- log-sum-exp and private tails ------------------------------------------------------

from oracle import attention_lse, pool_and_tail_decode, shared_pool_lse  # noqa: E402


def test_lse_special_cases_and_brute_force():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 8))
    k1 = rng.standard_normal((1, 8))
    # one token: the score itself
    np.testing.assert_allclose(attention_lse(q, k1, 0.3), 0.3 * (q @ k1.T)[:, 0], rtol=0, atol=1e-14)
    # T identical keys: score + ln T
    kT = np.repeat(k1, 5, axis=0)
    np.testing.assert_allclose(attention_lse(q, kT, 0.3), 0.3 * (q @ k1.T)[:, 0] + math.log(5), rtol=0, atol=1e-13)
    # brute force with scalar loops
    k = rng.standard_normal((6, 8))
    for r in range(3):
        s = [0.7 * sum(float(a) * float(b) for a, b in zip(q[r], kt)) for kt in k]
        want = math.log(math.fsum(math.exp(x) for x in s))
        assert abs(attention_lse(q[r:r + 1], k, 0.7)[0] - want) < 1e-12
    # no overflow for large scores
    big = attention_lse(np.array([[1000.0]]), np.array([[1.0], [1.0]]), 1.0)
    assert abs(big[0] - (1000.0 + math.log(2))) < 1e-9


def test_pool_and_tail_matches_brute_force_union():
    rng = np.random.default_rng(11)
    L, A, H, G, d, T, cap = 2, 3, 2, 2, 4, 3, 4
    q = rng.standard_normal((L, A, H * G, d))
    kh, vh = rng.standard_normal((L, H, T, d)), rng.standard_normal((L, H, T, d))
    tk, tv = rng.standard_normal((A, L, H, cap, d)), rng.standard_normal((A, L, H, cap, d))
    tl = np.array([0, 2, 4])
    got = pool_and_tail_decode(q, kh, vh, tk, tv, tl, G, 0.5)
    for l in range(L):
        for a in range(A):
            for j in range(H * G):
                h = j // G
                keys = [list(kh[l, h, t]) for t in range(T)] + [list(tk[a, l, h, t]) for t in range(tl[a])]
                vals = [list(vh[l, h, t]) for t in range(T)] + [list(tv[a, l, h, t]) for t in range(tl[a])]
                want = _brute([q[l, a, j]], keys, vals, 0.5)[0]
                np.testing.assert_allclose(got[l, a, j], want, rtol=1e-12, atol=1e-12)


def test_empty_tails_give_the_pool_result_and_lse_merges_disjoint_sets():
    rng = np.random.default_rng(12)
    L, A, H, G, d, T, cap = 1, 2, 2, 2, 8, 5, 3
    q = rng.standard_normal((L, A, H * G, d))
    kh, vh = rng.standard_normal((L, H, T, d)), rng.standard_normal((L, H, T, d))
    tk, tv = rng.standard_normal((A, L, H, cap, d)), rng.standard_normal((A, L, H, cap, d))
    none = pool_and_tail_decode(q, kh, vh, tk, tv, np.zeros(A, int), G, 0.4)
    np.testing.assert_allclose(none, shared_pool_decode(q, kh, vh, G, 0.4), rtol=1e-13, atol=1e-13)
    # union = log-sum-exp weighted combination of the two disjoint partials
    full = pool_and_tail_decode(q, kh, vh, tk, tv, np.full(A, cap), G, 0.4)
    lp = shared_pool_lse(q, kh, G, 0.4)[0]
    op = shared_pool_decode(q, kh, vh, G, 0.4)[0]
    for a in range(A):
        for j in range(H * G):
            h = j // G
            rows = q[0, a, j:j + 1]
            ot = attention_rows(rows, tk[a, 0, h], tv[a, 0, h], 0.4)[0]
            lt = attention_lse(rows, tk[a, 0, h], 0.4)[0]
            wp, wt = math.exp(lp[a, j]), math.exp(lt)
            np.testing.assert_allclose(full[0, a, j], (wp * op[a, j] + wt * ot) / (wp + wt), rtol=1e-12, atol=1e-12)
