"""Pins of the Lloyd-Max codebooks the Octave format indexes.

vLLM rocm_octave docs (module text): every code indexes a Lloyd-Max codebook
for N(0, 1) stored as int8; no calibration.  The integers are not printed;
the oracle derives them (a READING), and these tests pin the derivation to
the textbook quantizer (Max 1960), the closed form of the 1-bit case, the
centroid / midpoint conditions, and numpy's searchsorted for the code rule.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.stats

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _max1960():
    levels, mse = {}, {}
    with open(os.path.join(GOLDEN, "lloyd_max_gaussian.txt")) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "mse":
                mse[int(t[1])] = float(t[2])
            else:
                levels[int(t[0])] = [float(v) for v in t[1:]]
    return levels, mse


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_levels_match_max_1960(bits):
    levels, _ = _max1960()
    L = O.lloyd_max(bits)
    assert L.shape == (1 << bits,)
    np.testing.assert_allclose(L, -L[::-1], atol=1e-12)  # symmetric
    np.testing.assert_allclose(L[len(L) // 2:], levels[bits], atol=1e-3, rtol=0)


def test_one_bit_closed_form():
    L = O.lloyd_max(1)
    assert abs(L[1] - math.sqrt(2.0 / math.pi)) < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_centroid_and_midpoint_conditions(bits):
    L = O.lloyd_max(bits)
    edges = np.concatenate([[-np.inf], (L[1:] + L[:-1]) / 2, [np.inf]])
    for k in range(len(L)):
        a, b = edges[k], edges[k + 1]
        mass = scipy.stats.norm.cdf(b) - scipy.stats.norm.cdf(a)
        num, _ = scipy.integrate.quad(lambda x: x * scipy.stats.norm.pdf(x), a, b)
        assert abs(num / mass - L[k]) < 1e-8


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_distortion_matches_max_1960(bits):
    _, mse = _max1960()
    L = O.lloyd_max(bits)
    edges = np.concatenate([[-np.inf], (L[1:] + L[:-1]) / 2, [np.inf]])
    d = 0.0
    for k in range(len(L)):
        v, _ = scipy.integrate.quad(lambda x: (x - L[k]) ** 2 * scipy.stats.norm.pdf(x),
                                    edges[k], edges[k + 1])
        d += v
    assert abs(d - mse[bits]) / mse[bits] < 2e-3


def test_integer_codebooks():
    lut3, m3 = O.codebook(3)
    lut4, m4 = O.codebook(4)
    assert (m3, m4) == (59, 46)
    assert lut3.tolist() == [-127, -79, -45, -14, 14, 45, 79, 127]
    assert lut4.tolist() == [-126, -95, -74, -58, -43, -30, -18, -6, 6, 18, 30, 43, 58, 74, 95, 126]
    for bits, lut, m in ((3, lut3, m3), (4, lut4, m4)):
        L = O.lloyd_max(bits)
        np.testing.assert_array_equal(lut, np.round(L * m).astype(int))
        assert np.abs(lut).max() <= 127
        assert np.abs(np.round(L * (m + 1))).max() > 127  # the multiplier is the largest
        # rounding margins: far from .5, so the integers are robust
        frac = np.abs(L * m - np.round(L * m))
        assert frac.max() < 0.47    # at least 0.03 away from a rounding tie
    assert O.lut_one() == 64


@pytest.mark.parametrize("bits", [3, 4])
def test_bucket_rule_is_searchsorted_left(bits):
    lut, _ = O.codebook(bits)
    mids = ((lut[1:] + lut[:-1]) / 2).astype(np.float32)
    ys = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                         np.nextafter(mids, np.float32(-np.inf)),
                         np.linspace(-200, 200, 4001, dtype=np.float32),
                         np.array([0.0, -0.0, 1e30, -1e30], np.float32)]).astype(np.float32)
    want = np.searchsorted(mids, ys, side="left")
    got = np.array([O.bucket(float(y), bits) for y in ys])
    np.testing.assert_array_equal(got, want)
    # a value exactly on a midpoint takes the lower code
    for k, m in enumerate(mids):
        assert O.bucket(float(m), bits) == k
