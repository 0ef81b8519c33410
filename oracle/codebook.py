"""3-bit Lloyd-Max codebook for N(0,1).

PolyKV, Abstract: after the rotation, values get 3-bit Lloyd-Max codes whose centroids
are fitted to the standard normal distribution. Lloyd's method (Lloyd 1957/1982; Max 1960) alternates two
optimality conditions until a fixed point:
- each boundary is the midpoint of its two neighbouring centroids;
- each centroid is the mean of N(0,1) restricted to its cell.
For a log-concave density the fixed point is unique (Fleischer 1964), so the result does
not depend on the starting point.
"""

import math
from statistics import NormalDist

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _pdf(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _upper_tail(x: float) -> float:
    """P(Z > x) for Z ~ N(0,1), via erfc so that tails keep full precision."""
    return 0.5 * math.erfc(x / _SQRT2)


def _cell_mass(a: float, b: float) -> float:
    """P(a < Z < b). Uses whichever tail form avoids cancellation."""
    if b <= 0.0:
        return _cell_mass(-b, -a)
    return _upper_tail(a) - _upper_tail(b)


def _cell_first_moment(a: float, b: float) -> float:
    """Integral of x*phi(x) over (a, b) = phi(a) - phi(b)."""
    return _pdf(a) - _pdf(b)


def _cell_second_moment(a: float, b: float) -> float:
    """Integral of x^2*phi(x) over (a, b) = mass + a*phi(a) - b*phi(b)."""
    ta = 0.0 if math.isinf(a) else a * _pdf(a)
    tb = 0.0 if math.isinf(b) else b * _pdf(b)
    return _cell_mass(a, b) + ta - tb


def _edges(centroids):
    n = len(centroids)
    return [-math.inf] + [0.5 * (centroids[k] + centroids[k + 1]) for k in range(n - 1)] + [math.inf]


def lloyd_max_gaussian(levels: int = 8, tol: float = 1e-15, max_iter: int = 100000, init=None):
    """Run Lloyd's iteration on N(0,1) in fp64.

    Start: centroids at the N(0,1) quantiles of (k + 1/2)/levels, or ``init`` (any
    ascending list) when given. Step: boundaries at
    centroid midpoints, then centroids at the conditional means of their cells. Stop
    when no centroid moves by ``tol`` or more. Returns (centroids as a list of floats,
    iterations taken).
    """
    if init is None:
        nd = NormalDist()
        c = [nd.inv_cdf((k + 0.5) / levels) for k in range(levels)]
    else:
        c = [float(x) for x in init]
    for it in range(1, max_iter + 1):
        t = _edges(c)
        new = [_cell_first_moment(t[k], t[k + 1]) / _cell_mass(t[k], t[k + 1])
               for k in range(levels)]
        delta = max(abs(a - b) for a, b in zip(new, c))
        c = new
        if delta < tol:
            return c, it
    raise RuntimeError("Lloyd iteration did not converge")


def codebook_fp32(levels: int = 8):
    """The stored codebook: float32 centroids (ascending) and float32 boundaries.

    The fp64 fixed point is made exactly symmetric (c_k = (c_k - c_{L-1-k}) / 2) and
    rounded to float32. Boundary k is the fp64 midpoint of float32 centroids k and k+1,
    rounded to float32; the middle boundary is then exactly 0.
    Returns (centroids float32 [levels], boundaries float32 [levels-1]).
    """
    c, _ = lloyd_max_gaussian(levels)
    sym = [(c[k] - c[levels - 1 - k]) / 2.0 for k in range(levels)]
    c32 = np.array(sym, dtype=np.float32)
    c64 = c32.astype(np.float64)
    b32 = ((c64[:-1] + c64[1:]) / 2.0).astype(np.float32)
    return c32, b32


def quantizer_mse_gaussian(centroids, boundaries) -> float:
    """E[(Z - Q(Z))^2] for Z ~ N(0,1), where Q maps a cell to its centroid.

    Closed form per cell (a, b) with centroid c: M2 - 2c*M1 + c^2*M0, where M0, M1, M2
    are the cell's mass, first and second moments under phi.
    """
    c = [float(x) for x in centroids]
    t = [-math.inf] + [float(x) for x in boundaries] + [math.inf]
    total = 0.0
    for k, ck in enumerate(c):
        a, b = t[k], t[k + 1]
        total += (_cell_second_moment(a, b) - 2.0 * ck * _cell_first_moment(a, b)
                  + ck * ck * _cell_mass(a, b))
    return total


def cell_probabilities(boundaries):
    t = [-math.inf] + [float(x) for x in boundaries] + [math.inf]
    return np.array([_cell_mass(t[k], t[k + 1]) for k in range(len(t) - 1)])
