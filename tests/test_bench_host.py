"""Host side of the benchmark: its CPU baseline cuts each (query, KV head)
into page-aligned token ranges and merges them by log-sum-exp; the merged
output must be the oracle's attention of the whole workload."""
import os
import sys

import numpy as np
import pytest

import oracle as O
from decode_attention_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.parametrize("ci,sizes,threads", [(3, dict(batch=2, seq_len=300), 7),
                                              (5, dict(batch=2, seq_len=90, min_len=40), 16),
                                              (4, dict(batch=1, seq_len=64), 1)])
def test_cpu_baseline_merge_is_the_oracle(ci, sizes, threads):
    cfg = W.CONFIGS[ci]
    w = W.make_workload(cfg, **sizes)
    scale = W.default_sm_scale(cfg.head_size)
    got = []
    rec = bench.cpu_baseline(cfg, w, threads, scale, min_seconds=0.0, outputs=got)
    assert rec["cores"] == min(threads, rec["cores"]) and rec["value"] > 0
    fo = O.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim)
    slots = O.quantize(fo, w.key.astype(np.float32), w.value.astype(np.float32))
    P = cfg.page_size
    cache = np.zeros((w.num_pages, cfg.num_kv_heads, P, fo.slot_bytes), np.uint8)
    cache[w.slot_mapping // P, :, w.slot_mapping % P] = slots
    ref = O.attention(fo, w.query.astype(np.float32), cache, w.block_table, w.q_to_req,
                      w.q_to_klen, scale)
    np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-12)
