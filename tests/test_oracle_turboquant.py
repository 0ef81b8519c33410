"""Pins of the oracle's TurboQuant-MSE value codec: closed forms, brute force, statistics."""

import math

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook_fp32, tq_mse_decode, tq_mse_encode
from oracle.codebook import cell_probabilities

C32, B32 = codebook_fp32()


def _sylvester(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("j", [0, 1, 37])
@pytest.mark.parametrize("alpha", [1.0, -3.5, 0.125])
def test_one_hot(d, j, alpha):
    v = np.zeros(d, dtype=np.float16)
    v[j] = alpha
    codes, norm = tq_mse_encode(v, B32)
    col = _sylvester(d)[:, j] * np.sign(alpha)
    # rotated vector is column j of H (+-1): +1 -> code 5, -1 -> code 2
    assert np.array_equal(codes, np.where(col > 0, 5, 2).astype(np.uint8))
    assert float(norm) == abs(alpha)
    vhat = tq_mse_decode(codes, norm, C32)
    want = np.zeros(d)
    want[j] = np.float64(C32[5]) * alpha
    assert np.count_nonzero(vhat) == 1
    assert np.allclose(vhat, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("beta", [1.0, -0.5, 2.0])
def test_constant_vector_pins_ordering_and_ties(d, beta):
    v = np.full(d, beta, dtype=np.float16)
    codes, norm = tq_mse_encode(v, B32)
    want = np.full(d, 3, dtype=np.uint8)
    want[0] = 7 if beta > 0 else 0
    assert np.array_equal(codes, want)
    n16 = np.float64(np.float16(abs(beta) * math.sqrt(d)))
    assert float(norm) == n16
    vhat = tq_mse_decode(codes, norm, C32)
    c_first, c_mid = np.float64(C32[want[0]]), np.float64(C32[3])
    # H (c_first e0 + c_mid (1 - e0)) = c_mid d e0 + (c_first - c_mid) 1
    assert vhat[0] == pytest.approx(n16 / d * (c_mid * d + c_first - c_mid), rel=1e-14)
    assert np.allclose(vhat[1:], n16 / d * (c_first - c_mid), rtol=1e-14)
    if d == 128 and beta == 1.0:
        assert vhat[0] == pytest.approx(-2.5611, abs=1e-3)
        assert vhat[1] == pytest.approx(0.2119, abs=1e-3)


def test_zero_vector():
    codes, norm = tq_mse_encode(np.zeros((3, 128), dtype=np.float16), B32)
    assert np.all(codes == 3) and np.all(norm.astype(np.float32) == 0)
    assert np.all(tq_mse_decode(codes, norm, C32) == 0)


@pytest.mark.parametrize("d", [4, 8, 16])
def test_brute_force_nearest_centroid(d):
    rng = np.random.default_rng(d)
    v = rng.standard_normal((200, d)).astype(np.float16)
    codes, norms = tq_mse_encode(v, B32)
    h = _sylvester(d)
    c = C32.astype(np.float64)
    for r in range(v.shape[0]):
        x = [float(a) for a in v[r]]
        n = math.sqrt(sum(a * a for a in x))
        u = [a / n * math.sqrt(d) for a in x]
        y = [sum(h[i][j] * u[j] for j in range(d)) / math.sqrt(d) for i in range(d)]
        want = [min(range(8), key=lambda k: abs(yi - c[k])) for yi in y]
        assert list(codes[r]) == want
        assert float(norms[r]) == float(np.float16(n))
        yhat = [c[k] for k in want]
        vhat = [float(norms[r]) / math.sqrt(d) * sum(h[i][j] * yhat[j] for j in range(d)) / math.sqrt(d)
                for i in range(d)]
        assert np.allclose(tq_mse_decode(codes[r], norms[r], C32), vhat, atol=1e-12)


def _sphere_marginal_mse(d):
    """E[(x - Q(x))^2] for one coordinate of a uniform point on the sphere of radius sqrt(d)."""
    rt = math.sqrt(d)
    f = lambda x: (1.0 - x * x / d) ** ((d - 3) / 2.0)
    z = integrate.quad(f, -rt, rt)[0]
    edges = [-rt] + [float(b) for b in B32] + [rt]
    tot = 0.0
    for k in range(8):
        ck = float(C32[k])
        tot += integrate.quad(lambda x: (x - ck) ** 2 * f(x), edges[k], edges[k + 1], epsabs=1e-13)[0]
    return tot / z


@pytest.mark.parametrize("d", [64, 128])
def test_round_trip_mse_matches_sphere_marginal_integral(d):
    rng = np.random.default_rng(100 + d)
    v = rng.standard_normal((20000, d)).astype(np.float16)
    codes, norms = tq_mse_encode(v, B32)
    vhat = tq_mse_decode(codes, norms, C32)
    x = v.astype(np.float64)
    rel = np.mean(np.sum((x - vhat) ** 2, axis=-1) / np.sum(x * x, axis=-1))
    want = _sphere_marginal_mse(d)
    assert 0.033 < want < 0.0345
    assert rel == pytest.approx(want, rel=0.01)


def test_round_trip_mse_student_t():
    rng = np.random.default_rng(9)
    v = rng.standard_t(4.0, size=(20000, 128)).astype(np.float16)
    codes, norms = tq_mse_encode(v, B32)
    vhat = tq_mse_decode(codes, norms, C32)
    x = v.astype(np.float64)
    rel = np.mean(np.sum((x - vhat) ** 2, axis=-1) / np.sum(x * x, axis=-1))
    assert 0.0332 * 0.97 < rel < 0.0332 * 1.03


def test_code_histogram_follows_cell_probabilities():
    v = np.random.default_rng(21).standard_normal((20000, 128)).astype(np.float16)
    codes, _ = tq_mse_encode(v, B32)
    hist = np.bincount(codes.ravel(), minlength=8) / codes.size
    assert np.allclose(hist, cell_probabilities(B32), atol=2e-3)
    assert np.allclose(hist, hist[::-1], atol=2e-3)
