"""Thin Python binding of libhkv (include/hkv.h): argument marshalling only.

Every step of the path runs in the HIP kernels of ``libhkv.so``; torch is
used for device memory and streams.  There is no CPU fallback: if the
library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhkv.so")

HKV_OK, HKV_ERR_INVALID_ARG, HKV_ERR_UNSUPPORTED, HKV_ERR_WORKSPACE, HKV_ERR_HIP = range(5)
HKV_F32, HKV_F16 = 0, 1
HKV_DECODE_DETERMINISTIC = 1
HKV_KIND_Q4_0, HKV_KIND_OCTAVE, HKV_KIND_Q8_0 = 0, 1, 2
HKV_MAX_HEAD = 256
DECODE_SCRATCH_BYTES = 64 << 20  # HKV_DECODE_SCRATCH_BYTES

# Names of the exported entry points (include/hkv.h).
EXPORTS = ("hkv_format_init", "hkv_quantize_append", "hkv_dequantize",
           "hkv_decode_workspace_bytes", "hkv_decode_attention",
           "hkv_decode_attention_noalloc", "hkv_hadamard",
           "hkv_last_error", "hkv_version")


class HkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hkv status {status}: {message}")
        self.status = status


class HkvFormat(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kind", "head_size", "rope_dim", "v_bits", "compact", "page_size", "k_block",
        "v_block", "k_wide_dim", "off_k_nope", "off_v", "off_scales", "num_k_scales",
        "num_scales", "slot_bytes", "kernel_code")] + [
        ("sign_bits", ctypes.c_uint32 * (HKV_MAX_HEAD // 32))]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_ if n != "sign_bits"}
        d["sign_bits"] = list(self.sign_bits)
        return d


_lock = threading.Lock()
_lib = None


def lib():
    """Load libhkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -c 'import __graft_entry__ as g; g.build()'`")
            L = ctypes.CDLL(LIB_PATH)
            i32, i64, vp, P = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER
            L.hkv_format_init.argtypes = [P(HkvFormat), ctypes.c_char_p, i32, i32, i32]
            L.hkv_format_init.restype = ctypes.c_int
            L.hkv_quantize_append.argtypes = [P(HkvFormat), vp, vp, i32, i64, i32, vp,
                                              vp, vp]
            L.hkv_quantize_append.restype = ctypes.c_int
            L.hkv_dequantize.argtypes = [P(HkvFormat), vp, i32, vp, i64, i32, vp, vp, vp]
            L.hkv_dequantize.restype = ctypes.c_int
            L.hkv_decode_workspace_bytes.argtypes = [P(HkvFormat), i32, i32, i32, i32, i32]
            L.hkv_decode_workspace_bytes.restype = ctypes.c_size_t
            L.hkv_decode_attention.argtypes = [P(HkvFormat), vp, i32, i32, i32, i32, vp,
                                               vp, i32, vp, vp, i32, i32, ctypes.c_float,
                                               ctypes.c_uint32, vp, vp, ctypes.c_size_t, vp]
            L.hkv_decode_attention.restype = ctypes.c_int
            L.hkv_decode_attention_noalloc.argtypes = [P(HkvFormat), vp, i32, i32, i32, i32,
                                                       vp, vp, i32, vp, vp, i32, i32,
                                                       ctypes.c_float, ctypes.c_uint32, vp, vp]
            L.hkv_decode_attention_noalloc.restype = ctypes.c_int
            L.hkv_hadamard.argtypes = [vp, i32, vp, i64, i32, i32, vp, i32, vp]
            L.hkv_hadamard.restype = ctypes.c_int
            L.hkv_last_error.restype = ctypes.c_char_p
            L.hkv_version.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(status: int):
    if status != HKV_OK:
        raise HkvError(status, lib().hkv_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HKV_F32
    if t.dtype == torch.float16:
        return HKV_F16
    raise TypeError(f"unsupported dtype {t.dtype}; need float32 or float16")


def _need(t: torch.Tensor, name: str, dtype=None, dims=None, device: bool = True):
    """Type, layout, dtype and rank checks; the device check comes last (and
    can be left to a later _on_device call, so that shape errors are reported
    the same way for host tensors)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device:
        _on_device(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {tuple(t.shape)}")


def _on_device(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def format_init(cache_dtype: str, head_size: int, rope_dim: int = 0,
                page_size: int = 16) -> HkvFormat:
    f = HkvFormat()
    _check(lib().hkv_format_init(ctypes.byref(f), cache_dtype.encode(), head_size, rope_dim,
                                 page_size))
    return f


def new_cache(fmt: HkvFormat, num_pages: int, num_kv_heads: int,
              device="cuda") -> torch.Tensor:
    """Zeroed (num_pages, Hkv, page_size, slot_bytes) uint8 cache tensor."""
    return torch.zeros((num_pages, num_kv_heads, fmt.page_size, fmt.slot_bytes),
                       dtype=torch.uint8, device=device)


def quantize_append(fmt: HkvFormat, key: torch.Tensor, value: torch.Tensor,
                    slot_mapping: torch.Tensor, cache: torch.Tensor, stream=None) -> None:
    _need(key, "key", dims=3)
    _need(value, "value", dtype=key.dtype, dims=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, dims=1)
    _need(cache, "cache", dtype=torch.uint8, dims=4)
    T, H, D = key.shape
    if value.shape != key.shape or D != fmt.head_size or slot_mapping.shape[0] != T:
        raise ValueError("quantize_append: shape mismatch")
    if cache.shape[1] != H or cache.shape[2] != fmt.page_size or cache.shape[3] != fmt.slot_bytes:
        raise ValueError("quantize_append: cache shape does not match the format")
    _check(lib().hkv_quantize_append(ctypes.byref(fmt), _ptr(key), _ptr(value), _dtype_code(key),
                                     T, H, _ptr(slot_mapping), _ptr(cache), _stream(stream)))


def dequantize(fmt: HkvFormat, cache: torch.Tensor, slot_ids: torch.Tensor, rotated: bool = False,
               k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
               stream=None):
    _need(cache, "cache", dtype=torch.uint8, dims=4, device=False)
    _need(slot_ids, "slot_ids", dtype=torch.int64, dims=1, device=False)
    H = cache.shape[1]
    T = slot_ids.shape[0]
    if cache.shape[2] != fmt.page_size or cache.shape[3] != fmt.slot_bytes:
        raise ValueError("dequantize: cache shape does not match the format")
    _on_device(cache, "cache")
    _on_device(slot_ids, "slot_ids")
    shape = (T, H, fmt.head_size)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.float32, device=cache.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=torch.float32, device=cache.device)
    for t, n in ((k_out, "k_out"), (v_out, "v_out")):
        _need(t, n, dtype=torch.float32, dims=3)
        if tuple(t.shape) != shape:
            raise ValueError(f"{n} must be {shape}")
    _check(lib().hkv_dequantize(ctypes.byref(fmt), _ptr(cache), H, _ptr(slot_ids), T,
                                int(bool(rotated)), _ptr(k_out), _ptr(v_out), _stream(stream)))
    return k_out, v_out


def decode_workspace_bytes(fmt: HkvFormat, num_queries: int, num_q_heads: int, num_kv_heads: int,
                           max_klen: int, queries_per_seq: int = 1) -> int:
    return int(lib().hkv_decode_workspace_bytes(ctypes.byref(fmt), num_queries, num_q_heads,
                                                num_kv_heads, max_klen, queries_per_seq))


def decode_attention(fmt: HkvFormat, query: torch.Tensor, cache: torch.Tensor,
                     block_table: torch.Tensor, q_to_req: torch.Tensor, q_to_klen: torch.Tensor,
                     max_klen: int, queries_per_seq: int = 1, sm_scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None, deterministic: bool = False) -> torch.Tensor:
    """Decode attention; see include/hkv.h (one call at a time per workspace;
    deterministic=True: bitwise reproducible, a few percent slower)."""
    _need(query, "query", dims=3, device=False)
    _need(cache, "cache", dtype=torch.uint8, dims=4, device=False)
    _need(block_table, "block_table", dtype=torch.int32, dims=2, device=False)
    _need(q_to_req, "q_to_req", dtype=torch.int32, dims=1, device=False)
    _need(q_to_klen, "q_to_klen", dtype=torch.int32, dims=1, device=False)
    Q, Hq, D = query.shape
    Hkv = cache.shape[1]
    if D != fmt.head_size:
        raise ValueError(f"decode_attention: query head size {D} != format head_size "
                         f"{fmt.head_size}")
    if cache.shape[2] != fmt.page_size or cache.shape[3] != fmt.slot_bytes:
        raise ValueError("decode_attention: cache shape does not match the format "
                         f"(page_size {fmt.page_size}, slot_bytes {fmt.slot_bytes})")
    if q_to_req.shape[0] != Q or q_to_klen.shape[0] != Q:
        raise ValueError(f"decode_attention: q_to_req and q_to_klen need {Q} entries")
    if out is not None:
        _need(out, "out", dtype=torch.float32, dims=3, device=False)
        if tuple(out.shape) != (Q, Hq, D):
            raise ValueError(f"decode_attention: out must be {(Q, Hq, D)}, "
                             f"got {tuple(out.shape)}")
    if workspace is not None:
        _need(workspace, "workspace", device=False)
    for t, n in ((query, "query"), (cache, "cache"), (block_table, "block_table"),
                 (q_to_req, "q_to_req"), (q_to_klen, "q_to_klen"), (out, "out"),
                 (workspace, "workspace")):
        if t is not None:
            _on_device(t, n)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((Q, Hq, D), dtype=torch.float32, device=query.device)
    if workspace is None:  # a caller's workspace is size-checked by the library
        need = decode_workspace_bytes(fmt, Q, Hq, Hkv, max_klen, queries_per_seq)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hkv_decode_attention(
        ctypes.byref(fmt), _ptr(query), _dtype_code(query), Q, Hq, Hkv, _ptr(cache),
        _ptr(block_table), block_table.shape[1], _ptr(q_to_req), _ptr(q_to_klen), int(max_klen),
        int(queries_per_seq), float(sm_scale), HKV_DECODE_DETERMINISTIC if deterministic else 0,
        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def decode_attention_noalloc(fmt: HkvFormat, query: torch.Tensor, cache: torch.Tensor,
                             block_table: torch.Tensor, q_to_req: torch.Tensor,
                             q_to_klen: torch.Tensor, max_klen: int, queries_per_seq: int,
                             sm_scale: float, out: torch.Tensor, stream=None,
                             deterministic: bool = False) -> torch.Tensor:
    """Decode attention into a caller's `out` with the library's static scratch
    in place of a workspace; allocates nothing (include/hkv.h).  Calls that
    overlap in time on one device race on the scratch."""
    _need(query, "query", dims=3, device=False)
    _need(cache, "cache", dtype=torch.uint8, dims=4, device=False)
    _need(block_table, "block_table", dtype=torch.int32, dims=2, device=False)
    _need(q_to_req, "q_to_req", dtype=torch.int32, dims=1, device=False)
    _need(q_to_klen, "q_to_klen", dtype=torch.int32, dims=1, device=False)
    _need(out, "out", dtype=torch.float32, dims=3, device=False)
    Q, Hq, D = query.shape
    if D != fmt.head_size:
        raise ValueError(f"decode_attention_noalloc: query head size {D} != format head_size "
                         f"{fmt.head_size}")
    if cache.shape[2] != fmt.page_size or cache.shape[3] != fmt.slot_bytes:
        raise ValueError("decode_attention_noalloc: cache shape does not match the format")
    if q_to_req.shape[0] != Q or q_to_klen.shape[0] != Q:
        raise ValueError(f"decode_attention_noalloc: q_to_req and q_to_klen need {Q} entries")
    if tuple(out.shape) != (Q, Hq, D):
        raise ValueError(f"decode_attention_noalloc: out must be {(Q, Hq, D)}")
    for t, n in ((query, "query"), (cache, "cache"), (block_table, "block_table"),
                 (q_to_req, "q_to_req"), (q_to_klen, "q_to_klen"), (out, "out")):
        _on_device(t, n)
    _check(lib().hkv_decode_attention_noalloc(
        ctypes.byref(fmt), _ptr(query), _dtype_code(query), Q, Hq, cache.shape[1], _ptr(cache),
        _ptr(block_table), block_table.shape[1], _ptr(q_to_req), _ptr(q_to_klen), int(max_klen),
        int(queries_per_seq), float(sm_scale), HKV_DECODE_DETERMINISTIC if deterministic else 0,
        _ptr(out), _stream(stream)))
    return out


def hadamard(x: torch.Tensor, block: int = 128, sign_bits: Optional[torch.Tensor] = None,
             inverse: bool = False, out: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """Blockwise orthonormal Walsh-Hadamard rotation over the last dim of x
    (f32 or f16), fp32 result; sign_bits: None or an int32 device tensor of
    n/32 words (bit set = element negated), applied before the transform, or
    after it when inverse.  out may be x itself for f32 input."""
    _need(x, "x")
    n = x.shape[-1] if x.dim() else 0
    rows = x.numel() // n if n else 0
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _need(out, "out", dtype=torch.float32)
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError("hadamard: out must have the shape of x")
    if sign_bits is not None:
        _need(sign_bits, "sign_bits", dtype=torch.int32, dims=1)
        if sign_bits.numel() * 32 < n:
            raise ValueError("hadamard: sign_bits needs n/32 words")
    _check(lib().hkv_hadamard(_ptr(x), _dtype_code(x), _ptr(out), rows, n, int(block),
                              _ptr(sign_bits), int(bool(inverse)), _stream(stream)))
    return out


def version() -> str:
    return lib().hkv_version().decode()
