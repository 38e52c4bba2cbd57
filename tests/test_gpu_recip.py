"""The quantizers' block reciprocal (v_rcp_f32 and one Newton step) and
their x / 127 (Markstein's quotient with RN(1/127)), each with the division
outside 2^-100 <= |x| <= 2^100, equal the IEEE quotients 1/x and x/127 bit
for bit for every float on this GPU; the bytes of the Q4_0, Q8_0 and Octave
caches depend on them.  The check runs in the probe library (all 2^32 bit
patterns, about a second)."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_recip_and_div127_equal_ieee_division_for_every_float():
    path = os.path.join(ROOT, "decode_attention_amd", "libhkv_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the extension first")
    L = ctypes.CDLL(path)
    L.hkv_probe_recip_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.hkv_probe_recip_check.restype = ctypes.c_int
    out = torch.zeros(18, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    assert L.hkv_probe_recip_check(out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().tolist()
    for name, o in (("1/x", 0), ("x/127", 9)):
        bad = [hex(v & 0xFFFFFFFF) for v in got[o + 1:o + 1 + min(got[o], 8)]]
        assert got[o] == 0, f"{name}: {got[o]} mismatches, e.g. {bad}"


def test_sqrt_large_equals_sqrtf_for_every_large_float():
    """The square root the Octave many-row quantizer takes for fp16 rows
    (v_sqrt_f32 and a residual correction, no argument scaling) equals sqrtf
    for +0 and every finite float from 2^-96 up; the block RMS of an fp16
    row is zero or at least 2^-64."""
    path = os.path.join(ROOT, "decode_attention_amd", "libhkv_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the extension first")
    L = ctypes.CDLL(path)
    L.hkv_probe_sqrt_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.hkv_probe_sqrt_check.restype = ctypes.c_int
    out = torch.zeros(9, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    assert L.hkv_probe_sqrt_check(out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().tolist()
    bad = [hex(v & 0xFFFFFFFF) for v in got[1:1 + min(got[0], 8)]]
    assert got[0] == 0, f"sqrt: {got[0]} mismatches, e.g. {bad}"
