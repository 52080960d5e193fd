"""Statistical pins for the QJL-corrected inner-product estimator.

The estimate of <q, x> is <q, x_tilde> with x_tilde the QJL-corrected key
(dequant_polar_qjl); it must equal <q, x> on average over the random
rotation and sketch, with the variance the Gaussian sign-sketch gives."""
import math

import numpy as np
import pytest


def _setup(orc, b=3, d=128):
    _, c16, bounds, _, _ = orc.codebook(d, b)
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(d) * 2).astype(np.float32)
    x[[3, 77]] *= 8
    # q with cos(q, x) = 0.4
    u = x.astype(np.float64) / np.linalg.norm(x)
    w = rng.standard_normal(d)
    w -= w.dot(u) * u
    w /= np.linalg.norm(w)
    q = (0.4 * u + math.sqrt(1 - 0.16) * w) * 3.0
    return c16, bounds, x, q.astype(np.float32)


@pytest.mark.slow
def test_estimator_unbiased_over_seeds(orc):
    d = m = 128
    c16, bounds, x, q = _setup(orc)
    true = float(np.dot(q.astype(np.float64), x.astype(np.float64)))
    est = []
    for seed in range(10_000):
        D = orc.signs(seed, 0, 0, d)
        S = orc.sketch(seed, 0, m, d)
        r = orc.quantize_polar(x, D, c16, bounds, 3, m, S)
        xt = orc.dequant_polar_qjl(D, c16, S, r["codes"], r["n16"], r["signs"], r["rho16"])
        est.append(float(np.dot(q.astype(np.float64), xt)))
    est = np.array(est)
    err = est.mean() - true
    se = est.std() / math.sqrt(est.size)
    assert abs(err) < 1e-2 * abs(true)
    assert abs(err) < 5 * se + 2e-4 * abs(true)   # fp16 radius rounding is the only bias


@pytest.mark.slow
def test_sketch_term_mean_and_variance_closed_form(orc):
    """For a fixed rotation the correction term is a mean of m i.i.d. terms
    rho sqrt(pi/2) sign(<s, r>) <s, q'> with E = <q', r_bar> and
    Var = (pi/2 rho^2 |q'|^2 - <q', r_bar>^2) / m  (q' = R q, r_bar = r_rot/sqrt d)."""
    d = m = 128
    c16, bounds, x, _ = _setup(orc)
    D = orc.signs(5, 0, 0, d)
    S0 = orc.sketch(5, 0, m, d)
    r0 = orc.quantize_polar(x, D, c16, bounds, 3, m, S0)      # codes do not depend on S
    xhat = orc.dequant_polar(D, c16, r0["codes"], r0["n16"])
    res = x.astype(np.float64) - xhat                         # input-frame residual
    rng = np.random.default_rng(8)
    for qdir in ("residual", "random"):
        if qdir == "residual":
            q = res / np.linalg.norm(res) * 2.0
        else:
            q = rng.standard_normal(d)
        terms = []
        for seed in range(1000, 9000):
            S = orc.sketch(seed, 0, m, d)
            r = orc.quantize_polar(x, D, c16, bounds, 3, m, S)
            assert np.array_equal(r["codes"], r0["codes"])
            xt = orc.dequant_polar_qjl(D, c16, S, r["codes"], r["n16"], r["signs"], r["rho16"])
            terms.append(float(np.dot(q, xt - xhat)))
        terms = np.array(terms)
        rho = float(np.float16(np.uint16(r0["rho16"]).view(np.float16)))
        rho_true = np.linalg.norm(res)
        mean_want = np.dot(q, res) * rho / rho_true           # stored radius is fp16
        var_want = (math.pi / 2 * rho ** 2 * np.dot(q, q) - (np.dot(q, res) * rho / rho_true) ** 2) / m
        se = math.sqrt(var_want / terms.size)
        assert abs(terms.mean() - mean_want) < 5 * se
        assert abs(terms.var() / var_want - 1) < 0.08
