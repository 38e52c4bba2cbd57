"""Pins of the oracle's block-sum order and of the Octave scale placement.

The quantizer's two block sums (vLLM API docs "vllm.v1.attention.ops.
rocm_octave", _quantize_lut: the sum of squares and the dot product with the
codebook values) have an order the page leaves open; the oracle's reading is
fixed by hand-derived values on crafted inputs in
tests/golden/block_sum_order.txt, each of which another plausible order
(sequential, halving the whole block, pieces summed on their own first,
pieces left to right, adjacent pairs) gets wrong.  The scale words' order
(reference_quantize: K scales, RoPE blocks then NoPE blocks, then V) is
pinned by blocks of very different magnitudes.
"""
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "block_sum_order.txt")
B = np.float32(2 ** 24)


def _entries(kind):
    with open(GOLD) as f:
        for line in f:
            parts = line.split()
            if parts and parts[0] == kind:
                yield parts[1:]


def _bits(x):
    return int(np.float32(x).view(np.uint32))


# The alternative orders a mistake could take, in plain fp32 numpy loops
# (not the oracle): each must give a different result on the pinned inputs.
def _seq(t):
    s = np.float32(t[0])
    for v in t[1:]:
        s = np.float32(s + v)
    return s


def _halving(t):
    t = [np.float32(v) for v in t]
    while len(t) > 1 and len(t) % 2 == 0:
        h = len(t) // 2
        t = [np.float32(t[i] + t[i + h]) for i in range(h)]
    return _seq(t)


def _pieces_first(t):
    return _seq([_halving(t[64 * b:64 * b + 64]) for b in range(len(t) // 64)])


def _pieces_left_to_right(t):
    acc = [np.float32(v) for v in t[:64]]
    for b in range(1, len(t) // 64):
        acc = [np.float32(acc[i] + t[64 * b + i]) for i in range(64)]
    return _halving(acc)


def _adjacent(t):
    t = [np.float32(v) for v in t]
    while len(t) > 1:
        t = [np.float32(t[2 * i] + t[2 * i + 1]) for i in range(len(t) // 2)]
    return t[0]


ALTERNATIVES = {64: (_seq, _adjacent),
                128: (_seq, _pieces_first, _adjacent),
                192: (_seq, _halving, _pieces_first),
                256: (_seq, _pieces_first, _pieces_left_to_right, _adjacent)}


@pytest.mark.parametrize("n,i,j,want", [(int(a), int(b), int(c), int(d, 16))
                                        for a, b, c, d in _entries("sum")])
def test_block_sum_order_pinned(n, i, j, want):
    t = np.zeros(n, np.float32)
    t[0], t[i], t[j] = B, 1.0, 1.0
    assert _bits(O.block_sum(t)) == want
    for alt in ALTERNATIVES[n]:
        assert _bits(alt(list(t))) != want, alt.__name__


@pytest.mark.parametrize("n,bits,i,j,want", [(int(a), int(b), int(c), int(d), int(e, 16))
                                             for a, b, c, d, e in _entries("scale")])
def test_quantizer_scale_pins_sum_of_squares_order(n, bits, i, j, want):
    x = np.zeros(n, np.float32)
    x[0], x[i], x[j] = 4096.0, 1.0, 1.0
    codes, scale = O.quantize_lut(x, bits)
    top, small, zero = (15, 8, 7) if bits == 4 else (7, 4, 3)
    assert codes[0] == top and codes[i] == small and codes[j] == small
    assert all(codes[k] == zero for k in range(n) if k not in (0, i, j))
    assert _bits(scale) == want


@pytest.mark.parametrize("entry", list(_entries("dotscale")))
def test_quantizer_scale_pins_dot_order(entry):
    n, bits, big_i, big_x, small_x, small_ix, want = entry
    n, bits, big_i = int(n), int(bits), int(big_i)
    x = np.zeros(n, np.float32)
    x[big_i] = float(big_x)
    idx = [int(k) for k in small_ix.split(",")]
    x[idx] = float(small_x)
    codes, scale = O.quantize_lut(x, bits)
    assert codes[big_i] == 7 and all(codes[k] == 4 for k in idx)
    assert _bits(scale) == int(want, 16)
    # summed left to right, the small products are lost and the scale differs
    lut, _ = O.codebook(bits)
    prods = [np.float32(x[k] * np.float32(lut[codes[k]])) for k in range(n)]
    alt = np.float32(np.float32(x @ x) / _seq(prods)) * np.float32(64)
    assert _bits(alt) != int(want, 16)


# ---------------------------------------------------------------------------
# Scale placement: reference_quantize stores the K scales (RoPE blocks, then
# NoPE blocks; one scale for compact K) and then the V scale, as fp16 words
# from off_scales.  Each block is built as 2^(4 b) times the same rotated
# 64-vector u (the sign pattern is undone first, so that the rotation of
# block b is exactly 2^(4 b) H u), so scale word b must equal
# fp16(2^(4 b) * scale(H u)) with block b's bit width -- a swapped order puts
# a factor of 16 in the wrong word.
@pytest.mark.parametrize("dtype,D,rope", [("octave_k3v4", 128, 64), ("octave_k3v3", 128, 64),
                                          ("octave_k3v4", 192, 64), ("octave_k3v4", 256, 128),
                                          ("octave_k3v3_compact", 256, 0)])
def test_octave_scale_placement(dtype, D, rope):
    f = O.format_init(dtype, D, rope)
    rng = np.random.default_rng(11)
    s = O.signs(D)
    u = rng.standard_normal(64).astype(np.float32)
    nkb = D // 64
    key = np.concatenate([np.float32(2.0 ** (4 * b)) * u for b in range(nkb)]) * s
    vmag = np.float32(2.0 ** (4 * nkb + 2))
    w = rng.standard_normal(D).astype(np.float32)
    value = (vmag * w) * s
    slots = O.quantize(f, key.reshape(1, 1, D).astype(np.float32),
                       value.reshape(1, 1, D).astype(np.float32))[0, 0]
    words = slots[f.off_scales:f.off_scales + 2 * f.num_scales].view(np.uint16)
    assert f.num_scales == (2 if f.compact else nkb + 1)
    if f.compact:
        kr = O.fwht((key * s).astype(np.float32).reshape(1, D), D)[0]
        _, ks = O.quantize_lut(kr, 3)
        want_k = [O.f32_to_f16_bits(ks)]
    else:
        hu = O.fwht(u.reshape(1, 64), 64)[0]
        want_k = []
        for b in range(nkb):
            bits = 4 if b < rope // 64 else 3
            _, sc = O.quantize_lut(hu, bits)
            want_k.append(O.f32_to_f16_bits(np.float32(2.0 ** (4 * b)) * np.float32(sc)))
    vr = O.fwht(w.reshape(1, D), f.v_block)[0]
    _, sv = O.quantize_lut(vr, f.v_bits)
    want_v = O.f32_to_f16_bits(vmag * np.float32(sv))
    assert [int(x) for x in words[:-1]] == want_k
    assert int(words[-1]) == want_v
    # the words differ pairwise by the planted magnitudes (a swap would show)
    assert len(set(int(x) for x in words)) == len(words)
