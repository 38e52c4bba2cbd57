"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/hkv.h declares, builds the same format descriptor
as the oracle, and refuses bad arguments before anything is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from decode_attention_amd import hkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "hkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hkv_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(hkv.EXPORTS)
    L = hkv.lib()
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in hkv.version()


@pytest.mark.parametrize("dtype,D,R", [("q4_0", 256, 0), ("q4_0", 128, 0), ("q4_0", 64, 0),
                                       ("octave_k3v4", 128, 64), ("octave_k3v3", 128, 64),
                                       ("octave_k3v3_compact", 256, 64), ("octave_k3v4", 192, 64),
                                       ("octave_k3v4", 256, 128), ("octave_k3v3_compact", 64, 0),
                                       ("q8_0", 256, 0), ("q8_0", 64, 0)])
def test_format_matches_oracle(dtype, D, R):
    f = hkv.format_init(dtype, D, R, 16)
    g = O.format_init(dtype, D, R)
    for name in ("kind", "head_size", "v_bits", "compact", "k_block", "v_block", "k_wide_dim",
                 "off_k_nope", "off_v", "off_scales", "num_k_scales", "num_scales", "slot_bytes",
                 "kernel_code"):
        assert getattr(f, name) == getattr(g, name), name
    words = np.array(list(f.sign_bits), np.uint32)[:(D + 31) // 32]
    if g.use_signs:
        assert np.array_equal(words, O.sign_bits(D).view(np.uint32))
    else:
        assert not words.any()


@pytest.mark.parametrize("args", [("octave_k3v3_compact", 192, 64, 16), ("octave_k3v4", 128, 32, 16),
                                  ("octave_k3v4", 96, 0, 16), ("octave_k3v4", 128, 192, 16),
                                  ("octave_k5v5", 128, 64, 16), ("q4_0", 96, 0, 16),
                                  ("q4_0", 256, 0, 0), ("q4_0", 256, 0, 2048), ("q8_0", 96, 0, 16),
                                  ("q8_0", 512, 0, 16)])
def test_format_validation(args):
    with pytest.raises(hkv.HkvError) as e:
        hkv.format_init(*args)
    assert e.value.status == hkv.HKV_ERR_INVALID_ARG


def test_format_too_wide_is_unsupported():
    with pytest.raises(hkv.HkvError) as e:
        hkv.format_init("octave_k3v4", 512, 64, 16)
    assert e.value.status == hkv.HKV_ERR_UNSUPPORTED


FAKE = 1 << 20   # a non-null, aligned address; never dereferenced by these calls


def _fmt(*a):
    return hkv.format_init(*a)


def test_quantize_append_host_errors():
    L = hkv.lib()
    f = _fmt("q4_0", 256, 0, 16)
    q = lambda **kw: L.hkv_quantize_append(ctypes.byref(kw.get("f", f)), kw.get("k", FAKE),
                                           kw.get("v", FAKE), kw.get("dt", 1), kw.get("T", 4),
                                           kw.get("H", 2), kw.get("sm", FAKE),
                                           kw.get("cache", FAKE), None)
    assert q(T=0) == hkv.HKV_OK                       # nothing to do, nothing enqueued
    assert q(k=None) == hkv.HKV_ERR_INVALID_ARG
    assert q(sm=None) == hkv.HKV_ERR_INVALID_ARG
    assert q(cache=FAKE + 4) == hkv.HKV_ERR_INVALID_ARG   # misaligned
    assert q(dt=7) == hkv.HKV_ERR_INVALID_ARG
    assert q(H=0) == hkv.HKV_ERR_INVALID_ARG
    assert q(T=-1) == hkv.HKV_ERR_INVALID_ARG
    bad = _fmt("q4_0", 256, 0, 16)
    bad.slot_bytes = 300                               # inconsistent descriptor
    assert q(f=bad) == hkv.HKV_ERR_INVALID_ARG
    assert b"inconsistent" in L.hkv_last_error()


def test_dequantize_host_errors():
    L = hkv.lib()
    f = _fmt("octave_k3v4", 128, 64, 16)
    d = lambda **kw: L.hkv_dequantize(ctypes.byref(f), kw.get("cache", FAKE), kw.get("H", 2),
                                      kw.get("ids", FAKE), kw.get("T", 3), 0, kw.get("k", FAKE),
                                      kw.get("v", FAKE), None)
    assert d(T=0) == hkv.HKV_OK
    assert d(ids=None) == hkv.HKV_ERR_INVALID_ARG
    assert d(v=None) == hkv.HKV_ERR_INVALID_ARG
    assert d(cache=FAKE + 8) == hkv.HKV_ERR_INVALID_ARG
    assert d(H=-1) == hkv.HKV_ERR_INVALID_ARG


def test_decode_host_errors_and_workspace():
    L = hkv.lib()
    f = _fmt("q4_0", 256, 0, 16)
    need = hkv.decode_workspace_bytes(f, 4, 16, 2, 131072, 1)
    assert need > 0
    assert hkv.decode_workspace_bytes(f, 4, 16, 3, 131072, 1) == 0      # Hq % Hkv != 0
    assert hkv.decode_workspace_bytes(f, 6, 16, 2, 1000, 4) == 0        # 6 % 4 != 0

    def call(**kw):
        return L.hkv_decode_attention(
            ctypes.byref(kw.get("f", f)), kw.get("q", FAKE), kw.get("dt", 1), kw.get("Q", 4),
            kw.get("Hq", 16), kw.get("Hkv", 2), kw.get("cache", FAKE), kw.get("bt", FAKE),
            kw.get("mp", 8192), kw.get("qr", FAKE), kw.get("ql", FAKE), kw.get("mk", 131072),
            kw.get("nq", 1), kw.get("scale", 0.0625), kw.get("flags", 0), kw.get("out", FAKE),
            kw.get("ws", FAKE), kw.get("wsb", need), None)
    assert call(Q=0) == hkv.HKV_OK
    assert call(Hkv=3) == hkv.HKV_ERR_INVALID_ARG
    assert call(nq=3) == hkv.HKV_ERR_INVALID_ARG
    assert call(nq=17, Q=17) == hkv.HKV_ERR_INVALID_ARG
    assert call(q=None) == hkv.HKV_ERR_INVALID_ARG
    assert call(out=None) == hkv.HKV_ERR_INVALID_ARG
    assert call(mk=-1) == hkv.HKV_ERR_INVALID_ARG
    assert call(scale=float("inf")) == hkv.HKV_ERR_INVALID_ARG
    assert call(flags=2) == hkv.HKV_ERR_INVALID_ARG             # unknown flag bit
    assert call(wsb=need - 1) == hkv.HKV_ERR_WORKSPACE
    assert call(ws=None) == hkv.HKV_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == hkv.HKV_ERR_INVALID_ARG
    assert call(cache=FAKE + 2) == hkv.HKV_ERR_INVALID_ARG
    assert call(Hq=64, Hkv=1) == hkv.HKV_ERR_UNSUPPORTED      # 64 rows per KV head


def test_decode_noalloc_host_errors():
    """The no-allocation decode checks what hkv_decode_attention checks and
    refuses sizes whose partial records exceed the static scratch, before it
    touches a device."""
    L = hkv.lib()
    f = _fmt("octave_k3v3_compact", 256, 64, 16)

    def call(**kw):
        return L.hkv_decode_attention_noalloc(
            ctypes.byref(kw.get("f", f)), kw.get("q", FAKE), 1, kw.get("Q", 256),
            kw.get("Hq", 32), kw.get("Hkv", 4), kw.get("cache", FAKE), FAKE, 2048, FAKE, FAKE,
            kw.get("mk", 32768), kw.get("nq", 4), 0.0625, kw.get("flags", 1), kw.get("out", FAKE),
            None)
    need = hkv.decode_workspace_bytes(f, 256, 32, 4, 32768, 4)
    assert need > hkv.DECODE_SCRATCH_BYTES                  # 65 MiB of partial records
    assert call() == hkv.HKV_ERR_WORKSPACE
    assert b"hkv_decode_attention with a workspace" in L.hkv_last_error()
    assert call(Q=0) == hkv.HKV_OK
    assert call(nq=3) == hkv.HKV_ERR_INVALID_ARG
    assert call(q=None) == hkv.HKV_ERR_INVALID_ARG
    assert call(out=None) == hkv.HKV_ERR_INVALID_ARG
    assert call(mk=-1) == hkv.HKV_ERR_INVALID_ARG
    assert call(flags=4) == hkv.HKV_ERR_INVALID_ARG
    assert call(cache=FAKE + 2) == hkv.HKV_ERR_INVALID_ARG
    assert call(Hq=256, Hkv=1, Q=4, nq=1) == hkv.HKV_ERR_UNSUPPORTED
    assert "HKV_DECODE_SCRATCH_BYTES ((size_t)64 << 20)" in open(
        os.path.join(ROOT, "include", "hkv.h")).read()
    assert hkv.DECODE_SCRATCH_BYTES == 64 << 20


def test_hadamard_host_errors():
    L = hkv.lib()
    h = lambda **kw: L.hkv_hadamard(kw.get("x", FAKE), kw.get("dt", 0), kw.get("y", FAKE + (1 << 24)),
                                    kw.get("rows", 4), kw.get("n", 256), kw.get("block", 128),
                                    kw.get("sb", None), 0, None)
    assert h(rows=0) == hkv.HKV_OK
    assert h(block=96) == hkv.HKV_ERR_INVALID_ARG
    assert h(n=192) == hkv.HKV_ERR_INVALID_ARG                  # not a multiple of 128
    assert h(n=0) == hkv.HKV_ERR_INVALID_ARG
    assert h(x=None) == hkv.HKV_ERR_INVALID_ARG
    assert h(dt=5) == hkv.HKV_ERR_INVALID_ARG
    assert h(x=FAKE + 8) == hkv.HKV_ERR_INVALID_ARG             # f32 input not 16-byte aligned
    assert h(y=FAKE + (1 << 24) + 4) == hkv.HKV_ERR_INVALID_ARG
    assert h(sb=FAKE + 2) == hkv.HKV_ERR_INVALID_ARG
    assert h(y=FAKE + 1024) == hkv.HKV_ERR_INVALID_ARG          # partial overlap
    assert h(dt=1, y=FAKE) == hkv.HKV_ERR_INVALID_ARG           # f16 input cannot be in place


@pytest.mark.parametrize("dtype,D,R,Q,Hq,Hkv,klen,qps,rows_pad,splits,groups", [
    ("q4_0", 256, 0, 4, 16, 2, 131072, 1, 8, 32, 4),             # 8 rows, 4096-token splits
    ("q8_0", 256, 0, 4, 16, 2, 131072, 1, 8, 32, 4),             # Q8_0 matrix-core kernel
    ("q8_0", 128, 0, 4, 16, 2, 131072, 1, 8, 128, 4),            # generic kernel: 1024-token splits
    ("octave_k3v3_compact", 256, 64, 256, 32, 4, 32768, 4, 32, 8, 64),  # one pass for 32 rows
    ("octave_k3v4", 192, 64, 16, 16, 4, 32768, 1, 8, 8, 16),     # 4 rows in the 8-row mode
    ("octave_k3v3", 128, 64, 32, 32, 8, 32768, 1, 8, 8, 32),
    ("q4_0", 256, 0, 128, 16, 2, 32768, 8, 8, 8, 128),           # 64 rows -> 8-row sub-groups
])
def test_decode_plan_workspace(dtype, D, R, Q, Hq, Hkv, klen, qps, rows_pad, splits, groups):
    """The workspace a plan asks for is one partial record (m, l, two pad
    words, o[D]) per (query group, KV head, split, padded row): the row
    padding, split count and sub-grouping the planner picks for these shapes."""
    f = _fmt(dtype, D, R, 16)
    want = 4 * (4 + D) * rows_pad * splits * groups * Hkv
    assert hkv.decode_workspace_bytes(f, Q, Hq, Hkv, klen, qps) == want


def _decode_args(**over):
    """Well-shaped host tensors for config-2-like decode arguments."""
    import torch
    f = hkv.format_init("q4_0", 256, 0, 16)
    a = dict(fmt=f, query=torch.zeros((2, 16, 256)), cache=torch.zeros((8, 2, 16, 288),
             dtype=torch.uint8), block_table=torch.zeros((2, 4), dtype=torch.int32),
             q_to_req=torch.zeros(2, dtype=torch.int32), q_to_klen=torch.zeros(2, dtype=torch.int32),
             max_klen=64)
    a.update(over)
    return a


@pytest.mark.parametrize("bad,match", [
    ({"query": "q128"}, "head size"),
    ({"cache": "page8"}, "cache shape"),
    ({"cache": "slot"}, "cache shape"),
    ({"q_to_req": "short"}, "entries"),
    ({"q_to_klen": "short"}, "entries"),
    ({"out": "shape"}, "out must be"),
])
def test_decode_binding_rejects_mismatched_shapes(bad, match):
    import torch
    make = {"q128": lambda: torch.zeros((2, 16, 128)),
            "page8": lambda: torch.zeros((8, 2, 8, 288), dtype=torch.uint8),
            "slot": lambda: torch.zeros((8, 2, 16, 272), dtype=torch.uint8),
            "short": lambda: torch.zeros(1, dtype=torch.int32),
            "shape": lambda: torch.zeros((2, 16, 128))}
    (k, v), = bad.items()
    a = _decode_args(**{k: make[v]()})
    with pytest.raises(ValueError, match=match):
        hkv.decode_attention(**a)


def test_decode_binding_needs_device_tensors():
    with pytest.raises(ValueError, match="device tensor"):
        hkv.decode_attention(**_decode_args())


def test_dequantize_binding_rejects_mismatched_cache():
    import torch
    f = hkv.format_init("q4_0", 256, 0, 16)
    with pytest.raises(ValueError, match="does not match the format"):
        hkv.dequantize(f, torch.zeros((8, 2, 16, 272), dtype=torch.uint8),
                       torch.zeros(4, dtype=torch.int64))
