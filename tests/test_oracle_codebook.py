"""Pins of the oracle's Lloyd-Max codebook against textbook values and closed forms."""

import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook as cbm
from oracle import codebook_fp32, lloyd_max_gaussian, quantizer_mse_gaussian


def _read_golden(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = [float(v) for v in vals]
    return out


def test_cell_moment_helpers_match_numerical_integration():
    # The closed-form cell mass and moments against scipy quadrature of the density.
    for a, b in [(-math.inf, -1.7), (-1.7, -0.4), (-0.4, 0.0), (0.0, 0.5), (0.5, 2.2), (2.2, math.inf)]:
        m0 = integrate.quad(stats.norm.pdf, a, b)[0]
        m1 = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b)[0]
        m2 = integrate.quad(lambda x: x * x * stats.norm.pdf(x), a, b)[0]
        assert cbm._cell_mass(a, b) == pytest.approx(m0, rel=1e-10, abs=1e-14)
        assert cbm._cell_first_moment(a, b) == pytest.approx(m1, rel=1e-10, abs=1e-14)
        assert cbm._cell_second_moment(a, b) == pytest.approx(m2, rel=1e-10, abs=1e-14)


def test_matches_max_1960_table(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "max1960_gaussian_8level.txt"))
    c32, b32 = codebook_fp32()
    # printed to four significant digits; Max's own values can be off by one unit in the
    # last printed place (0.500550 is printed as 0.5006), so allow one unit
    for printed, ours in zip(g["outputs"], c32[4:]):
        assert abs(printed - ours) <= 10 ** (math.floor(math.log10(printed)) - 3) + 1e-12
    for printed, ours in zip(g["endpoints"], b32[3:]):
        if printed == 0.0:
            assert ours == 0.0
        else:
            assert abs(printed - ours) <= 10 ** (math.floor(math.log10(printed)) - 3) + 1e-12
    assert quantizer_mse_gaussian(c32, b32) == pytest.approx(g["mse"][0], abs=1e-4)


def test_centroid_condition_fp64():
    c, _ = lloyd_max_gaussian()
    t = [-math.inf] + [(c[k] + c[k + 1]) / 2 for k in range(7)] + [math.inf]
    for k in range(8):
        # conditional mean by quadrature, independent of the helpers
        num = integrate.quad(lambda x: x * stats.norm.pdf(x), t[k], t[k + 1], epsabs=1e-14)[0]
        den = integrate.quad(stats.norm.pdf, t[k], t[k + 1], epsabs=1e-14)[0]
        assert c[k] == pytest.approx(num / den, abs=1e-9)


def test_symmetry_midpoints_and_zero_boundary():
    c32, b32 = codebook_fp32()
    assert c32.dtype == np.float32 and b32.dtype == np.float32
    assert np.array_equal(c32, -c32[::-1])
    assert np.array_equal(b32, -b32[::-1])
    assert b32[3] == 0.0
    assert np.all(np.diff(c32) > 0) and np.all(np.diff(b32) > 0)
    for k in range(7):
        assert b32[k] == np.float32((np.float64(c32[k]) + np.float64(c32[k + 1])) / 2)
        assert c32[k] < b32[k] < c32[k + 1]


def test_mse_value():
    c32, b32 = codebook_fp32()
    assert quantizer_mse_gaussian(c32, b32) == pytest.approx(0.0345478, abs=2e-7)


def test_fixed_point_unique_from_other_start():
    c_a, _ = lloyd_max_gaussian()
    c_b, _ = lloyd_max_gaussian(init=np.linspace(-3.0, 3.0, 8))
    c_c, _ = lloyd_max_gaussian(init=[-0.9, -0.5, -0.2, -0.1, 0.1, 0.3, 0.6, 4.0])
    assert np.allclose(c_a, c_b, atol=1e-12) and np.allclose(c_a, c_c, atol=1e-12)


def test_monte_carlo_mse():
    c32, b32 = codebook_fp32()
    z = np.random.default_rng(7).standard_normal(2_000_000)
    idx = np.searchsorted(b32.astype(np.float64), z, side="left")  # count of boundaries < z
    mse = np.mean((z - c32.astype(np.float64)[idx]) ** 2)
    assert mse == pytest.approx(0.0345478, rel=0.01)


def test_mse_is_lower_than_a_perturbed_codebook():
    # optimality: any small move of a centroid or boundary raises the distortion
    c32, b32 = codebook_fp32()
    base = quantizer_mse_gaussian(c32, b32)
    for k in range(8):
        for eps in (-1e-3, 1e-3):
            c = c32.astype(np.float64).copy()
            c[k] += eps
            assert quantizer_mse_gaussian(c, b32) > base
    for k in range(7):
        for eps in (-1e-3, 1e-3):
            b = b32.astype(np.float64).copy()
            b[k] += eps
            assert quantizer_mse_gaussian(c32, b) > base
