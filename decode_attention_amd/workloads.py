"""Seeded synthetic workloads for the rotated low-bit paged KV cache.

This module only draws random inputs and builds index tables; it holds none
of the method's arithmetic.  Both the GPU tests/benchmark and the CPU oracle
consume the arrays it returns.

Recipe (numpy PCG64, seed = 1000 + config number unless given):
  * outlier channels: drawn first from the main stream (PCG64(seed)),
    without replacement, shared by every token and head, multiplied by 20;
  * sequence lengths (config 5): uniform integers in [1024, 32768], next
    from the main stream;
  * K, V and the query (tensors 0, 1, 2): standard normal in fp32, in chunks
    of whole rows (the largest multiple of the head size not above 2^22
    values) in row-major order; chunk c of tensor k comes from its
    own stream PCG64(SeedSequence(seed, spawn_key=(k, c))), so the chunks
    are drawn in parallel and the values do not depend on the thread count;
    outlier channels scaled, then rounded to fp16 (round-to-nearest-even)
    where the config says fp16 (the fp16 values are what both sides see,
    widened exactly);
  * pages: every sequence gets ceil(L / page) pages; physical page ids are a
    random permutation of all pages from the main stream (identity for
    config 1);
  * queries: n_q per sequence; query j of a sequence of length L attends to
    the first L - n_q + j + 1 tokens (causal among the new tokens).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    cache_dtype: str          # "q4_0" | "q8_0" | "octave_k3v4" | "octave_k3v3" | "octave_k3v3_compact"
    head_size: int
    rope_dim: int
    batch: int
    seq_len: int              # fixed length, or the upper bound when lengths vary
    num_q_heads: int
    num_kv_heads: int
    in_dtype: str             # "f32" | "f16"
    n_q: int = 1              # query tokens per sequence (causal among them)
    n_outliers: int = 0
    outlier_frac: float = 0.0
    outliers_on_query: bool = False
    page_size: int = 16
    shuffle_pages: bool = True
    min_len: Optional[int] = None   # lengths uniform in [min_len, seq_len] when set
    n_append: int = 0         # tokens appended per sequence by each step

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS = {
    1: Config(1, "tiny_q4_0", "q4_0", 256, 0, 1, 256, 4, 2, "f32", n_outliers=4,
              outliers_on_query=True, shuffle_pages=False),
    2: Config(2, "q4_0_paged_8k", "q4_0", 256, 0, 1, 8192, 16, 2, "f16",
              outlier_frac=0.01),
    3: Config(3, "q4_0_long_128k", "q4_0", 256, 0, 4, 131072, 16, 2, "f16",
              outlier_frac=0.01, n_append=4),
    4: Config(4, "octave_k3v4_32k", "octave_k3v4", 128, 64, 32, 32768, 32, 8, "f16"),
    5: Config(5, "octave_k3v3_compact_verify", "octave_k3v3_compact", 256, 64, 64, 32768,
              32, 4, "f16", n_q=4, min_len=1024, n_append=4),
    # Shapes beyond the five above, for the widened paths: a verify window of
    # 8 query tokens (64 query rows per KV head), the non-compact 3-bit V
    # format, and a head size that is not a power of two.
    6: Config(6, "q4_0_window8_32k", "q4_0", 256, 0, 16, 32768, 16, 2, "f16", n_q=8,
              outlier_frac=0.01),
    7: Config(7, "octave_k3v3_32k", "octave_k3v3", 128, 64, 32, 32768, 32, 8, "f16"),
    8: Config(8, "octave_k3v4_d192_32k", "octave_k3v4", 192, 64, 16, 32768, 16, 4, "f16"),
    # the shape of config 3 in the int8 (Q8_0) mode
    9: Config(9, "q8_0_long_128k", "q8_0", 256, 0, 4, 131072, 16, 2, "f16",
              outlier_frac=0.01, n_append=4),
}


@dataclasses.dataclass
class Workload:
    cfg: Config
    lengths: np.ndarray        # (B,) int64, tokens in each sequence (incl. new ones)
    key: np.ndarray            # (T_total, Hkv, D) f32 or f16, tokens of all sequences
    value: np.ndarray          # same
    query: np.ndarray          # (Q, Hq, D) f32 or f16
    seq_start: np.ndarray      # (B+1,) offsets of each sequence in key/value
    block_table: np.ndarray    # (B, max_pages) int32
    num_pages: int
    q_to_req: np.ndarray       # (Q,) int32
    q_to_klen: np.ndarray      # (Q,) int32
    slot_mapping: np.ndarray   # (T_total,) int64: page * page_size + offset
    outlier_channels: np.ndarray

    @property
    def max_klen(self) -> int:
        return int(self.q_to_klen.max()) if len(self.q_to_klen) else 0

    def append_rows(self) -> np.ndarray:
        """Indices (into key/value/slot_mapping) of the tokens one step appends."""
        n = self.cfg.n_append
        if n == 0:
            return np.zeros(0, np.int64)
        return np.concatenate([np.arange(self.seq_start[b + 1] - n, self.seq_start[b + 1])
                               for b in range(len(self.lengths))]).astype(np.int64)


_CHUNK = 1 << 22


def _draw(seed: int, tensor: int, shape, scale_ch: Optional[np.ndarray], dtype: str) -> np.ndarray:
    """Standard normals of `shape` (last dim = channels), outliers x20, cast.
    Chunk c (whole rows, at most 2^22 values) comes from PCG64(SeedSequence(seed,
    spawn_key=(tensor, c))); chunks are filled by a thread pool (numpy
    releases the GIL while it draws)."""
    out_dtype = np.float16 if dtype == "f16" else np.float32
    total = int(np.prod(shape))
    D = shape[-1]
    out = np.empty(total, out_dtype)
    scale = scale_ch is not None and len(scale_ch) > 0
    step = max(D, (_CHUNK // D) * D)

    def fill(c: int) -> None:
        s = c * step
        n = min(step, total - s)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, c))))
        x = g.standard_normal(n, dtype=np.float32)
        if scale:
            x = x.reshape(-1, D)
            x[:, scale_ch] *= np.float32(20.0)
        out[s:s + n] = x.reshape(-1).astype(out_dtype)

    n_chunks = (total + step - 1) // step
    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with concurrent.futures.ThreadPoolExecutor(min(n_chunks, os.cpu_count() or 1, 16)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def make_workload(cfg: Config, seed: Optional[int] = None, batch: Optional[int] = None,
                  seq_len: Optional[int] = None, min_len: Optional[int] = None) -> Workload:
    """Build the seeded workload of `cfg`; batch / seq_len / min_len may be
    changed for tests (min_len makes the lengths vary)."""
    if seed is None:
        seed = 1000 + cfg.index
    rng = np.random.Generator(np.random.PCG64(seed))
    B = cfg.batch if batch is None else batch
    Lmax = cfg.seq_len if seq_len is None else seq_len
    D, Hkv, Hq, P = cfg.head_size, cfg.num_kv_heads, cfg.num_q_heads, cfg.page_size

    n_out = cfg.n_outliers if cfg.n_outliers else int(math.ceil(cfg.outlier_frac * D))
    chans = np.sort(rng.choice(D, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)

    lo_len = cfg.min_len if min_len is None else min_len
    if lo_len is not None:
        lo = min(lo_len, Lmax)
        lengths = rng.integers(lo, Lmax + 1, size=B).astype(np.int64)
    else:
        lengths = np.full(B, Lmax, np.int64)
    lengths = np.maximum(lengths, cfg.n_q)
    seq_start = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(seq_start[-1])

    key = _draw(seed, 0, (T, Hkv, D), chans, cfg.in_dtype)
    value = _draw(seed, 1, (T, Hkv, D), chans, cfg.in_dtype)
    Q = B * cfg.n_q
    query = _draw(seed, 2, (Q, Hq, D), chans if cfg.outliers_on_query else None, cfg.in_dtype)

    pages_per_seq = (lengths + P - 1) // P
    num_pages = int(pages_per_seq.sum())
    phys = rng.permutation(num_pages) if cfg.shuffle_pages else np.arange(num_pages)
    max_pages = int(pages_per_seq.max())
    block_table = np.zeros((B, max_pages), np.int32)
    slot_mapping = np.empty(T, np.int64)
    off = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        block_table[b, :n] = phys[off:off + n]
        off += n
        pos = np.arange(lengths[b])
        slot_mapping[seq_start[b]:seq_start[b + 1]] = (
            block_table[b, pos // P].astype(np.int64) * P + pos % P)

    q_to_req = np.repeat(np.arange(B, dtype=np.int32), cfg.n_q)
    q_to_klen = np.concatenate([
        lengths[b] - cfg.n_q + np.arange(cfg.n_q) + 1 for b in range(B)]).astype(np.int32)
    return Workload(cfg, lengths, key, value, query, seq_start, block_table, num_pages,
                    q_to_req, q_to_klen, slot_mapping, chans)


def default_sm_scale(head_size: int) -> float:
    """1/sqrt(D), rounded to fp32 (the softmax scale the configs imply)."""
    return float(np.float32(1.0 / math.sqrt(head_size)))


def packed_bytes(w: Workload, slot_bytes: int) -> int:
    """Packed K/V bytes one decode call reads: sum over (sequence, KV head) of
    the longest klen among its queries times the slot size."""
    total = 0
    for b in range(len(w.lengths)):
        kl = w.q_to_klen[w.q_to_req == b]
        if len(kl):
            total += int(max(0, kl.max())) * w.cfg.num_kv_heads * slot_bytes
    return total


def subset(w: Workload, seqs: List[int]) -> Workload:
    """The workload restricted to some sequences (re-indexed, same pages)."""
    seqs = list(seqs)
    rows = np.concatenate([np.arange(w.seq_start[b], w.seq_start[b + 1]) for b in seqs])
    qsel = np.concatenate([np.nonzero(w.q_to_req == b)[0] for b in seqs])
    lengths = w.lengths[seqs]
    seq_start = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    remap = {b: i for i, b in enumerate(seqs)}
    return Workload(w.cfg, lengths, w.key[rows], w.value[rows], w.query[qsel], seq_start,
                    w.block_table[seqs], w.num_pages,
                    np.array([remap[int(r)] for r in w.q_to_req[qsel]], np.int32),
                    w.q_to_klen[qsel], w.slot_mapping[rows], w.outlier_channels)
