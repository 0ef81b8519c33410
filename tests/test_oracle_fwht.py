"""Pins of the oracle's Walsh-Hadamard transform."""

import numpy as np
import pytest

from oracle import fwht, hadamard_matrix


def _sylvester(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_explicit_matrix_is_sylvester_recursion(d):
    assert np.array_equal(hadamard_matrix(d), _sylvester(d))


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16])
def test_butterfly_equals_brute_force_matrix_product(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d))
    h = _sylvester(d)
    brute = np.array([[sum(x[r, j] * h[j, i] for j in range(d)) for i in range(d)] for r in range(5)])
    assert np.allclose(fwht(x), brute, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_involution_and_parseval(d):
    x = np.random.default_rng(3).standard_normal((7, d))
    y = fwht(x)
    assert np.allclose(fwht(y), d * x, atol=1e-10)
    assert np.allclose(np.sum(y * y, axis=-1), d * np.sum(x * x, axis=-1), rtol=1e-12)
    assert np.allclose(y, x @ _sylvester(d), atol=1e-10)


def test_unit_vectors():
    d = 128
    e0 = np.zeros(d)
    e0[0] = 1.0
    assert np.array_equal(fwht(e0), np.ones(d))
    assert np.array_equal(fwht(np.ones(d)), d * e0)
    # natural ordering: H e_j is column j, whose entry i is (-1)^popcount(i & j)
    ej = np.zeros(d)
    ej[5] = 1.0
    col = fwht(ej)
    assert col[0] == 1 and col[1] == -1 and col[4] == -1 and col[5] == 1 and col[2] == 1


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        fwht(np.ones(12))
