"""Pins for the oracle's rotation, radius/angle quantiser and q8 blocks."""
import functools
import math

import numpy as np
import pytest
from scipy.linalg import hadamard


@functools.lru_cache(None)
def _cb(d, b):
    import oracle
    return oracle.codebook(d, b)


@pytest.mark.parametrize("d", [2, 4, 8, 16])
def test_fwht_equals_dense_sylvester_small(orc, d):
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    rng = np.random.default_rng(d)
    for _ in range(20):
        x = rng.integers(-50, 50, d).astype(np.float64)
        want = H @ x
        assert np.array_equal(orc.fwht_f32(x.astype(np.float32)), want.astype(np.float32))
        assert np.array_equal(orc.fwht_f64(x), want)


@pytest.mark.parametrize("d", [32, 128, 256])
def test_fwht_integer_exact_and_involution(orc, d):
    H = hadamard(d).astype(np.float64)
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1000, d).astype(np.float64)
    assert np.array_equal(orc.fwht_f64(x), H @ x)
    assert np.array_equal(orc.fwht_f32(x.astype(np.float32)).astype(np.float64), H @ x)
    assert np.array_equal(orc.fwht_f64(orc.fwht_f64(x)), d * x)   # H H = d I


def test_fwht_preserves_norm_up_to_sqrt_d(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(128).astype(np.float32)
    y = orc.fwht_f32(x).astype(np.float64)
    assert abs(np.sum(y * y) / (128 * np.sum(x.astype(np.float64) ** 2)) - 1) < 1e-6


def test_tree_sum_of_squares(orc):
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float32)
        exact = math.fsum(float(v) * float(v) for v in x)
        got = orc.tree_sumsq(x)
        assert abs(got - exact) <= 4 * np.spacing(exact)


def _brute_codes(x, D, c16, d):
    """Nearest fp16 centroid of t = (H D x)_i / |x|, in fp64, lower index on ties."""
    y = hadamard(d).astype(np.float64) @ (D.astype(np.float64) * x.astype(np.float64))
    n = np.linalg.norm(x.astype(np.float64))
    t = y / n
    C = c16.view(np.float16).astype(np.float64)
    return np.argmin(np.abs(t[:, None] - C[None, :]), axis=1), t


@pytest.mark.parametrize("b", [2, 3, 4])
def test_polar_codes_are_nearest_centroids(orc, b):
    d = 128
    _, c16, bounds, _, _ = _cb(d, b)
    D = orc.signs(7, 0, 0, d)
    rng = np.random.default_rng(b)
    mism = total = 0
    for _ in range(300):
        x = (rng.standard_normal(d) * rng.uniform(0.1, 10)).astype(np.float32)
        x[rng.integers(0, d, 2)] *= 10
        r = orc.quantize_polar(x, D, c16, bounds, b)
        want, t = _brute_codes(x, D, c16, d)
        bad = r["codes"] != want
        mism += bad.sum()
        total += d
        # a disagreement may only happen right at a cell boundary
        assert np.all(r["tmargin"][bad] < 1e-5)
        n16 = np.float32(np.sqrt(np.sum(x.astype(np.float64) ** 2))).astype(np.float16).view(np.uint16)
        assert abs(int(r["n16"]) - int(n16)) <= 1
    assert mism <= 1e-4 * total


@pytest.mark.parametrize("b,lloyd_mse_tol", [(2, 0.03), (3, 0.03), (4, 0.03)])
def test_polar_mse_matches_lloyd_mse(orc, b, lloyd_mse_tol):
    """Mean squared error of the standardised coordinate equals the Lloyd MSE
    (the rotated coordinates follow the assumed law)."""
    d = 128
    _, c16, bounds, mse, _ = _cb(d, b)
    D = orc.signs(11, 0, 0, d)
    C = c16.view(np.float16).astype(np.float64)
    rng = np.random.default_rng(5)
    errs = []
    for _ in range(1500):
        x = rng.standard_normal(d).astype(np.float32)
        r = orc.quantize_polar(x, D, c16, bounds, b)
        _, t = _brute_codes(x, D, c16, d)
        errs.append(np.mean((t - C[r["codes"]]) ** 2))
    assert abs(np.mean(errs) / mse - 1) < lloyd_mse_tol


@pytest.mark.parametrize("b", [3, 4])
def test_qjl_residual_norm_and_signs(orc, b):
    d = m = 128
    _, c16, bounds, _, _ = _cb(d, b)
    D = orc.signs(13, 0, 0, d)
    S = orc.sketch(13, 0, m, d)
    rng = np.random.default_rng(9)
    Hd = hadamard(d).astype(np.float64)
    bad_signs = 0
    for _ in range(200):
        x = (rng.standard_normal(d) * 3).astype(np.float32)
        r = orc.quantize_polar(x, D, c16, bounds, b, m, S)
        xhat = orc.dequant_polar(D, c16, r["codes"], r["n16"])
        rho = np.linalg.norm(x.astype(np.float64) - xhat)
        rho16 = np.float32(rho).astype(np.float16).view(np.uint16)
        assert abs(int(r["rho16"]) - int(rho16)) <= 1
        # residual in the rotated frame, independently: r_rot = H D (x - x_hat)
        rrot = Hd @ (D.astype(np.float64) * (x.astype(np.float64) - xhat))
        z = S.astype(np.float64) @ rrot
        want = (z >= 0).astype(np.uint8)
        diff = r["signs"] != want
        assert np.all(np.abs(z[diff]) < 1e-5 * np.linalg.norm(rrot))
        bad_signs += diff.sum()
    assert bad_signs <= 1e-4 * 200 * m


def test_zero_vector(orc):
    d = m = 128
    _, c16, bounds, _, _ = _cb(d, 3)
    r = orc.quantize_polar(np.zeros(d, np.float32), orc.signs(1, 0, 0, d), c16, bounds, 3, m,
                           orc.sketch(1, 0, m, d))
    assert r["n16"] == 0 and r["rho16"] == 0
    assert np.all(r["codes"] == 0) and np.all(r["signs"] == 1)


def test_norm_saturates_at_fp16_max(orc):
    d = 128
    _, c16, bounds, _, _ = _cb(d, 2)
    x = np.full(d, 1e4, np.float32)
    r = orc.quantize_polar(x, orc.signs(1, 0, 0, d), c16, bounds, 2)
    assert r["n16"] == 0x7bff


def test_q8_exact_multiples_round_trip(orc):
    rng = np.random.default_rng(4)
    for _ in range(100):
        s16 = np.float16(rng.uniform(1e-3, 10)).astype(np.float32)
        k = rng.integers(-127, 128, 128)
        k[rng.integers(0, 32)] = 127 * rng.choice([-1, 1])       # amax in each block
        for blk in range(4):
            k[blk * 32 + rng.integers(0, 32)] = 127 * rng.choice([-1, 1])
        x = (k * s16).astype(np.float32)
        k8, sc, _ = orc.quantize_q8(x)
        assert np.array_equal(k8.astype(np.int64), k)
        assert np.all(sc == np.float16(s16).view(np.uint16))


def test_q8_properties(orc):
    rng = np.random.default_rng(5)
    for _ in range(200):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 50)).astype(np.float32)
        k8, sc, _ = orc.quantize_q8(x)
        s = sc.view(np.float16).astype(np.float64).repeat(32)
        xh = orc.dequant_q8(k8, sc)
        assert np.array_equal(xh, s * k8)
        assert np.all(np.abs(x - xh) <= s / 2 + 1e-12 + np.abs(x) * 2 ** -10)
        for blk in range(4):
            i = blk * 32 + np.argmax(np.abs(x[blk * 32:(blk + 1) * 32]))
            assert abs(int(k8[i])) == 127
    k8, sc, _ = orc.quantize_q8(np.zeros(128, np.float32))
    assert np.all(k8 == 0) and np.all(sc == 0)
