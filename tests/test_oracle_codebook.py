"""Pins for the oracle's Lloyd-Max codebook on the rotated-coordinate law."""
import functools
import math
import os

import numpy as np
import pytest
from scipy import integrate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _max_table():
    rows = {}
    with open(os.path.join(GOLDEN, "max1960_gaussian.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            n, ys, xs, mse = [p.strip() for p in line.split("|")]
            rows[int(n)] = ([float(v) for v in ys.split()],
                            [float(v) for v in xs.split()], float(mse))
    return rows


@functools.lru_cache(None)
def _cb(d, b):
    import oracle
    return oracle.codebook(d, b)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_large_d_limit_is_max_gaussian_table(b):
    """As d grows the coordinate law tends to N(0,1); Max's table is the limit."""
    ys, xs, mse = _max_table()[1 << b]
    c64, _, _, got_mse, _ = _cb(1 << 20, b)
    pos = c64[len(c64) // 2:]
    assert np.allclose(pos, ys, atol=6e-4, rtol=6e-4)
    mids = 0.5 * (pos[:-1] + pos[1:])
    assert np.allclose(mids, xs, atol=6e-4, rtol=6e-4)
    assert abs(got_mse - mse) < 6e-4 * max(mse, 0.01) + 5e-6


@pytest.mark.parametrize("d", [64, 128, 256])
def test_one_bit_closed_form(d):
    """With one bit the centroid is E|t| = sqrt(d) G(d/2) / (sqrt(pi) G((d+1)/2))."""
    c64 = _cb(d, 1)[0]
    want = math.sqrt(d) * math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c64[1] - want) < 1e-9 and c64[0] == -c64[1]


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_lloyd_fixed_point_by_independent_quadrature(d, b):
    """Each centroid is the conditional mean of its cell (adaptive quadrature),
    and the cells are bounded by centroid midpoints."""
    c64 = _cb(d, b)[0]
    w = lambda t: (1 - t * t / d) ** ((d - 3) / 2)
    edges = [-math.sqrt(d)] + list(0.5 * (c64[:-1] + c64[1:])) + [math.sqrt(d)]
    for k in range(len(c64)):
        a, c = edges[k], edges[k + 1]
        m0 = integrate.quad(w, a, c, epsabs=0, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda t: t * w(t), a, c, epsabs=0, epsrel=1e-13, limit=200)[0]
        assert abs(m1 / m0 - c64[k]) < 1e-9


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp16_centroids_are_far_from_rounding_ties(d, b):
    """fp16 rounding of the centroids is stable: no fp64 centroid lies within
    1e-7 of an fp16 rounding tie, so any implementation accurate to 1e-8
    stores the same fp16 bits."""
    c64, c16, bounds, _, _ = _cb(d, b)
    v16 = c16.view(np.float16).astype(np.float64)
    assert np.array_equal(c16, c64.astype(np.float16).view(np.uint16))
    ulp = np.spacing(np.abs(v16).astype(np.float16)).astype(np.float64)
    assert np.all(ulp / 2 - np.abs(c64 - v16) > 1e-7)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_codebook_symmetric_sorted_with_exact_midpoints(b):
    c64, c16, bounds, _, _ = _cb(128, b)
    L = 1 << b
    v = c16.view(np.float16).astype(np.float64)
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(v, -v[::-1])
    assert np.array_equal(bounds.astype(np.float64), (v[:-1] + v[1:]) / 2)
    assert bounds[L // 2 - 1] == 0.0


def test_marginal_density_is_sphere_coordinate_law():
    """The density used is that of sqrt(d)*u_1 for u uniform on the sphere:
    its variance is 1 (E t^2 = d * E u_1^2 = 1)."""
    import oracle
    d = 128
    m0 = oracle.marginal_mass(d, 0.0, math.sqrt(d))
    m2 = integrate.quad(lambda t: t * t * (1 - t * t / d) ** ((d - 3) / 2), 0, math.sqrt(d),
                        epsrel=1e-13)[0]
    assert abs(m2 / m0 - 1.0) < 1e-9
    # Monte-Carlo: mean |t| for random unit vectors matches the 1-bit centroid
    rng = np.random.default_rng(3)
    g = rng.standard_normal((20000, d))
    t = math.sqrt(d) * g[:, 0] / np.linalg.norm(g, axis=1)
    assert abs(np.abs(t).mean() - _cb(d, 1)[0][1]) < 4 * t.std() / math.sqrt(t.size)
