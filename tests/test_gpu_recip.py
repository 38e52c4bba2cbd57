"""The quantizers' block reciprocal (v_rcp_f32 and one Newton step, the
division outside 2^-100 <= |x| <= 2^100) equals the IEEE quotient 1/x bit
for bit for every float on this GPU; the bytes of the Q4_0 and Q8_0 caches
depend on it.  The check runs in the probe library (all 2^32 bit patterns,
about half a second)."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_recip_rn_equals_ieee_division_for_every_float():
    path = os.path.join(ROOT, "decode_attention_amd", "libhkv_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the extension first")
    L = ctypes.CDLL(path)
    L.hkv_probe_recip_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.hkv_probe_recip_check.restype = ctypes.c_int
    out = torch.zeros(9, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    assert L.hkv_probe_recip_check(out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().tolist()
    bad = [hex(v & 0xFFFFFFFF) for v in got[1:1 + min(got[0], 8)]]
    assert got[0] == 0, f"{got[0]} mismatches, e.g. {bad}"
