"""decode_attention_amd: FWHT-rotated low-bit paged KV cache and decode
attention for AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libhkv.so`` (include/hkv.h) built from the
HIP sources in ``csrc/``; ``hkv`` is its thin Python binding and ``workloads``
the seeded synthetic inputs.
"""
from . import hkv  # noqa: F401

__all__ = ["hkv"]
