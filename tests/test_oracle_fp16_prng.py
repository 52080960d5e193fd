"""Pins for the oracle's fp16 conversion and its random streams."""
import os

import numpy as np
import pytest
from scipy import stats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [int(l) for l in f if l.strip() and not l.startswith("#")]


def test_f16_to_f32_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_matches_numpy_rne(orc):
    rng = np.random.default_rng(0)
    mags = np.exp(rng.uniform(np.log(1e-9), np.log(1e6), 200_000)).astype(np.float32)
    x = mags * rng.choice([-1, 1], mags.size).astype(np.float32)
    # exact ties: fp16 values plus half an ulp, both parities, incl. subnormals
    h = rng.integers(0, 0x7bff, 50_000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    special = np.array([0.0, -0.0, 65504, 65519.99, 65520, 1e30, -1e30, np.inf, -np.inf,
                        2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 6.1e-5], np.float32)
    x = np.concatenate([x, ties, -ties, special])
    got = orc.f32_to_f16(x)
    with np.errstate(over="ignore"):   # the specials past 65520 overflow to infinity on purpose
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    assert orc.f32_to_f16(np.array([np.nan], np.float32))[0] & 0x7c00 == 0x7c00


def test_splitmix64_reference_outputs(orc):
    want = _golden_ints("splitmix64_seed1234567.txt")
    got = [orc.splitmix64_at(1234567, k) for k in range(len(want))]
    assert got == want


def test_sign_stream_balanced_and_distinct(orc):
    D = np.concatenate([orc.signs(42, layer, 0, 4096) for layer in range(4)])
    assert set(np.unique(D)) == {-1.0, 1.0}
    assert abs(D.mean()) < 4 / np.sqrt(D.size)
    a = orc.signs(42, 0, 0, 4096)
    b = orc.signs(42, 0, 1, 4096)
    c = orc.signs(42, 1, 0, 4096)
    assert abs((a * b).mean()) < 0.1 and abs((a * c).mean()) < 0.1


def test_sketch_is_standard_gaussian(orc):
    S = orc.sketch(42, 0, 128, 128).astype(np.float64).ravel()
    assert abs(S.mean()) < 4 / np.sqrt(S.size)
    assert abs(S.var() - 1) < 0.05
    assert abs(stats.kurtosis(S, fisher=False) - 3) < 0.15
    assert stats.kstest(S, "norm").pvalue > 1e-3
    S2 = orc.sketch(42, 1, 128, 128).astype(np.float64).ravel()
    assert abs(np.corrcoef(S, S2)[0, 1]) < 0.05
