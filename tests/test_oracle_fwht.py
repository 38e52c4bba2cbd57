"""Pins of the oracle's rotation: Walsh-Hadamard transform and sign pattern.

Pinned against: the Sylvester Hadamard matrix from scipy (closed form),
exactness on small-integer inputs, H.H = I, <Hq, Hk> = <q, k> (Strata PR #21,
"Verification"), the published SplitMix64 test vector, and the definition
of sign_bits (vLLM rocm_octave docs, "sign_bits").
"""
import os

import numpy as np
import pytest
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("B", [2, 8, 64, 128, 256])
def test_fwht_matches_sylvester_closed_form(B):
    rng = np.random.default_rng(B)
    x = rng.standard_normal((5, B))
    H = scipy.linalg.hadamard(B).astype(np.float64) / np.sqrt(B)
    want = x @ H.T
    got64 = O.fwht(x, B)
    np.testing.assert_allclose(got64, want, rtol=0, atol=1e-12)
    got32 = O.fwht(x.astype(np.float32), B)
    np.testing.assert_allclose(got32, want, rtol=0, atol=2e-5 * np.abs(x).max() * np.log2(B))


@pytest.mark.parametrize("B", [64, 256])
def test_fwht_exact_on_small_integers(B):
    rng = np.random.default_rng(7)
    x = rng.integers(-100, 101, (16, B)).astype(np.float32)
    H = scipy.linalg.hadamard(B).astype(np.int64)
    exact = (x.astype(np.int64) @ H.T).astype(np.float64) / np.sqrt(B)
    got = O.fwht(x, B)
    assert np.array_equal(got.astype(np.float64), exact)
    # H . H . x == x, bitwise ("Verification": Hadamard self-inverse)
    assert np.array_equal(O.fwht(got, B), x)


@pytest.mark.parametrize("B", [64, 128, 256])
def test_fwht_self_inverse_and_isometry(B):
    rng = np.random.default_rng(B + 1)
    x = rng.standard_normal((64, B)).astype(np.float32)
    back = O.fwht(O.fwht(x, B), B)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-5)
    q = rng.standard_normal((64, B)).astype(np.float32)
    hq, hk = O.fwht(q, B).astype(np.float64), O.fwht(x, B).astype(np.float64)
    ip = np.einsum("ij,ij->i", q.astype(np.float64), x.astype(np.float64))
    np.testing.assert_allclose(np.einsum("ij,ij->i", hq, hk), ip, rtol=0, atol=1e-4)


@pytest.mark.parametrize("B", [64, 256])
def test_fwht_unit_vector(B):
    e0 = np.zeros(B, np.float32)
    e0[0] = 1.0
    assert np.array_equal(O.fwht(e0, B), np.full(B, 1.0 / np.sqrt(B), np.float32))


def test_fwht_blocks_are_independent():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 192)).astype(np.float32)
    got = O.fwht(x, 64)
    for b in range(3):
        assert np.array_equal(got[:, 64 * b:64 * (b + 1)], O.fwht(x[:, 64 * b:64 * (b + 1)], 64))


def test_fwht_norm_constant_for_128_is_fp32_rounded():
    # The normalisation 1/sqrt(128) is applied as one fp32 multiply by the
    # fp32-rounded constant (0x3DB504F3).
    e0 = np.zeros(128, np.float32)
    e0[0] = 1.0
    got = O.fwht(e0, 128)
    assert got.view(np.uint32)[0] == 0x3DB504F3
    assert np.all(got == got[0])


@pytest.mark.parametrize("B", [64, 128, 256])
def test_fwht_xor_partner_form_is_bitwise_identical(B):
    # A data-parallel butterfly in which the element with bit h set computes
    # (partner - mine) and the other (mine + partner), stages ascending, then
    # one fp32 multiply, gives the same bits as the oracle.
    rng = np.random.default_rng(B)
    y = rng.standard_normal((32, B)).astype(np.float32) * np.float32(7.3)
    ref = O.fwht(y, B)
    idx = np.arange(B)
    h = 1
    while h < B:
        partner = y[:, idx ^ h]
        y = np.where((idx & h) == 0, y + partner, partner - y).astype(np.float32)
        h *= 2
    y = (y * np.float32(1.0 / np.sqrt(B))).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def _golden_splitmix():
    vals = []
    with open(os.path.join(GOLDEN, "splitmix64_seed0.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(int(line, 16))
    return vals


def test_splitmix64_published_vector():
    want = _golden_splitmix()
    assert O.splitmix64(0, len(want)) == want


@pytest.mark.parametrize("n", [64, 128, 192, 256])
def test_signs_follow_generator_words(n):
    s = O.signs(n)
    words = O.splitmix64(n, (n + 63) // 64)
    for i in range(n):
        bit = (words[i // 64] >> (i % 64)) & 1
        assert s[i] == (-1.0 if bit else 1.0)


@pytest.mark.parametrize("n", [64, 128, 256])
def test_sign_bits_definition(n):
    s = O.signs(n)
    w = O.sign_bits(n)
    assert w.dtype == np.int32 and w.shape == (n // 32,)
    u = w.view(np.uint32)
    for i in range(n):
        assert ((int(u[i // 32]) >> (i % 32)) & 1) == int(s[i] < 0)


def test_signs_are_balanced():
    s = O.signs(4096)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(float((s < 0).mean()) - 0.5) < 0.04
