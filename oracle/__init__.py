"""CPU oracle for the FWHT-rotated low-bit paged KV cache (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the
oracle never loads the GPU library.  The arithmetic lives in
``hkv_oracle.c``; this module only marshals numpy arrays through ctypes.
"""
import ctypes
import os
import threading

import numpy as np

from . import build as _build

_lock = threading.Lock()
_lib = None


class Format(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kind", "head_size", "rope_dim", "v_bits", "compact", "k_block",
        "v_block", "use_signs", "k_wide_dim", "off_k_nope", "off_v",
        "off_scales", "num_k_scales", "num_scales", "slot_bytes",
        "kernel_code")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_build.LIB):
                _build.build()
            L = ctypes.CDLL(_build.LIB)
            i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
            P = ctypes.POINTER
            L.orc_format_init.argtypes = [P(Format), ctypes.c_char_p, i32, i32]
            L.orc_format_init.restype = ctypes.c_int
            L.orc_f32_to_f16.argtypes = [f32]
            L.orc_f32_to_f16.restype = ctypes.c_uint16
            L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
            L.orc_f16_to_f32.restype = f32
            L.orc_fwht_f32.argtypes = [P(f32), i32, i32]
            L.orc_fwht_f64.argtypes = [P(f64), i32, i32]
            L.orc_splitmix64_next.argtypes = [P(ctypes.c_uint64)]
            L.orc_splitmix64_next.restype = ctypes.c_uint64
            L.orc_signs.argtypes = [i32, P(f32)]
            L.orc_sign_bits.argtypes = [i32, P(i32)]
            L.orc_lloyd_max.argtypes = [i32, P(f64)]
            L.orc_codebook.argtypes = [i32, P(i32)]
            L.orc_codebook.restype = i32
            L.orc_lut_one.restype = i32
            L.orc_bucket.argtypes = [f32, i32]
            L.orc_bucket.restype = i32
            L.orc_block_sum.argtypes = [P(f32), i32]
            L.orc_block_sum.restype = f32
            L.orc_quantize_lut.argtypes = [P(f32), i32, i32, P(ctypes.c_uint8), P(f32)]
            L.orc_q4_0_block.argtypes = [P(f32), P(ctypes.c_uint8), P(ctypes.c_uint16)]
            L.orc_q8_0_block.argtypes = [P(f32), P(ctypes.c_int8), P(ctypes.c_uint16)]
            L.orc_pack.argtypes = [P(ctypes.c_uint8), i32, i32, P(ctypes.c_uint8)]
            L.orc_unpack.argtypes = [P(ctypes.c_uint8), i32, i32, P(ctypes.c_uint8)]
            L.orc_quantize.argtypes = [P(Format), P(f32), P(f32), i64, i32, P(ctypes.c_uint8)]
            L.orc_dequantize.argtypes = [P(Format), P(ctypes.c_uint8), i64, i32, i32, P(f32), P(f32)]
            L.orc_dequantize_f64.argtypes = [P(Format), P(ctypes.c_uint8), i64, i32, P(f64), P(f64)]
            L.orc_attention.argtypes = [P(Format), P(f32), i32, i32, P(ctypes.c_uint8), i32, i32,
                                        P(i32), i32, P(i32), P(i32), f64, P(f64)]
            L.orc_attention_lse.argtypes = [P(Format), P(f32), i32, i32, P(ctypes.c_uint8), i32,
                                            i32, P(i32), i32, P(i32), P(i32), f64, P(f64),
                                            P(f64)]
            _lib = L
    return _lib


def format_init(cache_dtype: str, head_size: int, rope_dim: int = 0) -> Format:
    f = Format()
    rc = lib().orc_format_init(ctypes.byref(f), cache_dtype.encode(), head_size, rope_dim)
    if rc != 0:
        raise ValueError(f"invalid format {cache_dtype!r} head_size={head_size} rope_dim={rope_dim}")
    return f


def f32_to_f16_bits(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().orc_f16_to_f32(int(h)))


def fwht(x: np.ndarray, block: int) -> np.ndarray:
    """Blockwise orthonormal FWHT over the last dim (fp32 or fp64 as given)."""
    y = np.ascontiguousarray(x).copy()
    n = y.shape[-1]
    rows = y.reshape(-1, n)
    for r in rows:
        if y.dtype == np.float32:
            lib().orc_fwht_f32(_p(r, ctypes.c_float), n, block)
        elif y.dtype == np.float64:
            lib().orc_fwht_f64(_p(r, ctypes.c_double), n, block)
        else:
            raise TypeError(y.dtype)
    return rows.reshape(y.shape)


def splitmix64(seed: int, count: int) -> list:
    st = ctypes.c_uint64(seed)
    return [int(lib().orc_splitmix64_next(ctypes.byref(st))) for _ in range(count)]


def signs(n: int) -> np.ndarray:
    s = np.empty(n, np.float32)
    lib().orc_signs(n, _p(s, ctypes.c_float))
    return s


def sign_bits(n: int) -> np.ndarray:
    w = np.empty((n + 31) // 32, np.int32)
    lib().orc_sign_bits(n, _p(w, ctypes.c_int32))
    return w


def lloyd_max(bits: int) -> np.ndarray:
    L = np.empty(1 << bits, np.float64)
    lib().orc_lloyd_max(bits, _p(L, ctypes.c_double))
    return L


def codebook(bits: int):
    lut = np.empty(1 << bits, np.int32)
    mult = lib().orc_codebook(bits, _p(lut, ctypes.c_int32))
    return lut, int(mult)


def lut_one() -> int:
    return int(lib().orc_lut_one())


def bucket(y: float, bits: int) -> int:
    return int(lib().orc_bucket(float(np.float32(y)), bits))


def block_sum(x: np.ndarray) -> float:
    """fp32 sum of a block in the quantizer's order (64-value pieces added
    position by position, then folded in halves)."""
    x = np.ascontiguousarray(x, np.float32)
    return float(np.float32(lib().orc_block_sum(_p(x, ctypes.c_float), x.shape[-1])))


def quantize_lut(x: np.ndarray, bits: int):
    x = np.ascontiguousarray(x, np.float32)
    codes = np.empty(x.shape[-1], np.uint8)
    sc = ctypes.c_float()
    lib().orc_quantize_lut(_p(x, ctypes.c_float), x.shape[-1], bits, _p(codes, ctypes.c_uint8),
                           ctypes.byref(sc))
    return codes, float(sc.value)


def q4_0_block(x: np.ndarray):
    x = np.ascontiguousarray(x, np.float32)
    assert x.shape == (32,)
    codes = np.empty(32, np.uint8)
    d16 = ctypes.c_uint16()
    lib().orc_q4_0_block(_p(x, ctypes.c_float), _p(codes, ctypes.c_uint8), ctypes.byref(d16))
    return codes, int(d16.value)



def q8_0_block(x: np.ndarray):
    """Q8_0 block (READING, the GGML block type): int8 codes and fp16 bits of d."""
    x = np.ascontiguousarray(x, np.float32)
    assert x.shape == (32,)
    codes = np.empty(32, np.int8)
    d16 = ctypes.c_uint16()
    lib().orc_q8_0_block(_p(x, ctypes.c_float), _p(codes, ctypes.c_int8), ctypes.byref(d16))
    return codes, int(d16.value)

def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, np.uint8)
    n = c.shape[-1]
    out = np.zeros(n * bits // 8, np.uint8)
    lib().orc_pack(_p(c, ctypes.c_uint8), n, bits, _p(out, ctypes.c_uint8))
    return out


def unpack(packed: np.ndarray, n: int, bits: int) -> np.ndarray:
    b = np.ascontiguousarray(packed, np.uint8)
    out = np.zeros(n, np.uint8)
    lib().orc_unpack(_p(b, ctypes.c_uint8), n, bits, _p(out, ctypes.c_uint8))
    return out


def quantize(fmt: Format, key: np.ndarray, value: np.ndarray) -> np.ndarray:
    """(T, H, D) K and V -> (T, H, slot_bytes) uint8."""
    k = np.ascontiguousarray(key, np.float32)
    v = np.ascontiguousarray(value, np.float32)
    T, H, D = k.shape
    assert D == fmt.head_size and v.shape == k.shape
    out = np.zeros((T, H, fmt.slot_bytes), np.uint8)
    lib().orc_quantize(ctypes.byref(fmt), _p(k, ctypes.c_float), _p(v, ctypes.c_float), T, H,
                       _p(out, ctypes.c_uint8))
    return out


def dequantize(fmt: Format, slots: np.ndarray, rotated: bool = False):
    s = np.ascontiguousarray(slots, np.uint8)
    T, H, S = s.shape
    assert S == fmt.slot_bytes
    k = np.empty((T, H, fmt.head_size), np.float32)
    v = np.empty_like(k)
    lib().orc_dequantize(ctypes.byref(fmt), _p(s, ctypes.c_uint8), T, H, int(rotated),
                         _p(k, ctypes.c_float), _p(v, ctypes.c_float))
    return k, v


def dequantize_f64(fmt: Format, slots: np.ndarray):
    s = np.ascontiguousarray(slots, np.uint8)
    T, H, S = s.shape
    k = np.empty((T, H, fmt.head_size), np.float64)
    v = np.empty_like(k)
    lib().orc_dequantize_f64(ctypes.byref(fmt), _p(s, ctypes.c_uint8), T, H,
                             _p(k, ctypes.c_double), _p(v, ctypes.c_double))
    return k, v


def attention(fmt: Format, query: np.ndarray, cache: np.ndarray, block_table: np.ndarray,
              q_to_req: np.ndarray, q_to_klen: np.ndarray, sm_scale: float) -> np.ndarray:
    """Paged decode attention in fp64.  query (Q, Hq, D); cache (pages, Hkv, page, slot)."""
    q = np.ascontiguousarray(query, np.float32)
    c = np.ascontiguousarray(cache, np.uint8)
    bt = np.ascontiguousarray(block_table, np.int32)
    qr = np.ascontiguousarray(q_to_req, np.int32)
    ql = np.ascontiguousarray(q_to_klen, np.int32)
    Q, Hq, D = q.shape
    _, Hkv, page, S = c.shape
    assert S == fmt.slot_bytes and D == fmt.head_size and Hq % Hkv == 0
    out = np.zeros((Q, Hq, D), np.float64)
    lib().orc_attention(ctypes.byref(fmt), _p(q, ctypes.c_float), Q, Hq, _p(c, ctypes.c_uint8),
                        Hkv, page, _p(bt, ctypes.c_int32), bt.shape[1], _p(qr, ctypes.c_int32),
                        _p(ql, ctypes.c_int32), float(sm_scale), _p(out, ctypes.c_double))
    return out


def attention_lse(fmt: Format, query: np.ndarray, cache: np.ndarray, block_table: np.ndarray,
                  q_to_req: np.ndarray, q_to_klen: np.ndarray, sm_scale: float):
    """attention() and, per (query, head), the natural log of the softmax
    denominator over the row's scaled scores (-inf for a row with no tokens):
    attention over disjoint token ranges merges exactly with these weights."""
    q = np.ascontiguousarray(query, np.float32)
    c = np.ascontiguousarray(cache, np.uint8)
    bt = np.ascontiguousarray(block_table, np.int32)
    qr = np.ascontiguousarray(q_to_req, np.int32)
    ql = np.ascontiguousarray(q_to_klen, np.int32)
    Q, Hq, D = q.shape
    _, Hkv, page, S = c.shape
    assert S == fmt.slot_bytes and D == fmt.head_size and Hq % Hkv == 0
    out = np.zeros((Q, Hq, D), np.float64)
    lse = np.zeros((Q, Hq), np.float64)
    lib().orc_attention_lse(ctypes.byref(fmt), _p(q, ctypes.c_float), Q, Hq,
                            _p(c, ctypes.c_uint8), Hkv, page, _p(bt, ctypes.c_int32),
                            bt.shape[1], _p(qr, ctypes.c_int32), _p(ql, ctypes.c_int32),
                            float(sm_scale), _p(out, ctypes.c_double), _p(lse, ctypes.c_double))
    return out, lse
