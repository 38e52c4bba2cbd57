"""GPU parity of hkv_hadamard (blockwise Walsh-Hadamard rotation of rows)
against the oracle's fwht_blocks: bitwise, for blocks 64/128/256, f32 and f16
input, with and without a sign pattern, rotate and unrotate, in place, and
block counts that leave a ragged last wave."""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_amd import hkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _ref(x32, block, bits, inverse):
    n = x32.shape[-1]
    if bits is None:
        return O.fwht(x32, block)
    s = (1 - 2 * ((bits.view(np.uint32)[np.arange(n) // 32] >> (np.arange(n) % 32)) & 1)).astype(np.float32)
    if inverse:
        return O.fwht(x32, block) * s
    return O.fwht(x32 * s, block)


@pytest.mark.parametrize("rows,n,block", [(37, 128, 128), (5, 384, 128), (9, 1024, 64),
                                          (3, 512, 256), (1001, 128, 128), (2, 64, 64),
                                          (700, 256, 256)])
@pytest.mark.parametrize("in_dtype", [np.float32, np.float16])
@pytest.mark.parametrize("signs,inverse", [(False, False), (True, False), (True, True)])
def test_hadamard_matches_oracle(rows, n, block, in_dtype, signs, inverse):
    rng = np.random.default_rng(rows * 7 + n + block)
    x = (rng.standard_normal((rows, n)) * rng.uniform(0.01, 30, (rows, 1))).astype(in_dtype)
    x[0, :block] = 0
    bits = rng.integers(-2**31, 2**31, n // 32, dtype=np.int64).astype(np.int32) if signs else None
    y = hkv.hadamard(torch.from_numpy(x).to(DEV), block,
                     None if bits is None else torch.from_numpy(bits).to(DEV), inverse)
    ref = _ref(x.astype(np.float32), block, bits, inverse)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_hadamard_in_place_and_round_trip():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((333, 256)).astype(np.float32)
    bits = O.sign_bits(256)
    t = torch.from_numpy(x).to(DEV)
    sb = torch.from_numpy(bits).to(DEV)
    y = hkv.hadamard(t, 128, sb, False, out=t)        # in place
    assert y.data_ptr() == t.data_ptr()
    assert np.array_equal(t.cpu().numpy().view(np.uint32), _ref(x, 128, bits, False).view(np.uint32))
    z = hkv.hadamard(t, 128, sb, True)                 # unrotate: back to x up to rounding
    assert np.allclose(z.cpu().numpy(), x, atol=1e-5, rtol=1e-5)


def test_hadamard_is_the_cache_rotation():
    """Unrotating the oracle's rotated dequantized Octave K (64-blocks, then
    the signs) with hkv_hadamard gives the oracle's unrotated dequantized K,
    bit for bit: the op is the cache formats' own rotation."""
    f = O.format_init("octave_k3v4", 128, 64)
    rng = np.random.default_rng(11)
    k = rng.standard_normal((40, 1, 128)).astype(np.float32)
    v = rng.standard_normal((40, 1, 128)).astype(np.float32)
    slots = O.quantize(f, k, v)
    kr, vr = O.dequantize(f, slots, rotated=True)
    ku, vu = O.dequantize(f, slots, rotated=False)
    bits = torch.from_numpy(O.sign_bits(128)).to(DEV)
    got = hkv.hadamard(torch.from_numpy(np.ascontiguousarray(kr.reshape(40, 128))).to(DEV), 64,
                       bits, True)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ku.reshape(40, 128).view(np.uint32))


@pytest.mark.parametrize("in_dtype", [np.float32, np.float16])
def test_hadamard_many_blocks(in_dtype):
    """More blocks than one grid pass (2048 workgroups x 16 blocks): every
    wave runs several loop iterations with two groups of loads in flight,
    and the last group is ragged."""
    rng = np.random.default_rng(77)
    rows, n, block = 40001, 128, 64                   # 80002 blocks
    x = rng.standard_normal((rows, n)).astype(in_dtype)
    bits = rng.integers(-2**31, 2**31, n // 32, dtype=np.int64).astype(np.int32)
    y = hkv.hadamard(torch.from_numpy(x).to(DEV), block, torch.from_numpy(bits).to(DEV), False)
    ref = _ref(x.astype(np.float32), block, bits, False)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
