"""The seeded input recipe: determinism, shapes, page tables, causal lengths."""
import numpy as np

from decode_attention_amd import workloads as W


def test_deterministic_and_shaped():
    cfg = W.CONFIGS[5]
    a = W.make_workload(cfg, batch=3, seq_len=200)
    b = W.make_workload(cfg, batch=3, seq_len=200)
    assert np.array_equal(a.key, b.key) and np.array_equal(a.block_table, b.block_table)
    assert a.key.dtype == np.float16 and a.key.shape == (int(a.lengths.sum()), 4, 256)
    assert a.query.shape == (12, 32, 256)
    # causal among the 4 new tokens of each sequence
    for s in range(3):
        kl = a.q_to_klen[a.q_to_req == s]
        L = a.lengths[s]
        assert kl.tolist() == [L - 3, L - 2, L - 1, L]


def test_page_tables_are_a_permutation():
    cfg = W.CONFIGS[3]
    w = W.make_workload(cfg, seq_len=1000)
    used = np.concatenate([w.block_table[b, :(w.lengths[b] + 15) // 16] for b in range(cfg.batch)])
    assert sorted(used.tolist()) == list(range(w.num_pages))
    # slot mapping: distinct, consistent with the table
    assert len(np.unique(w.slot_mapping)) == len(w.slot_mapping)
    pos = np.arange(w.lengths[1])
    sm = w.slot_mapping[w.seq_start[1]:w.seq_start[2]]
    assert np.array_equal(sm // 16, w.block_table[1, pos // 16]) and np.array_equal(sm % 16, pos % 16)
    assert len(w.append_rows()) == 4 * cfg.batch


def test_outlier_channels():
    w = W.make_workload(W.CONFIGS[1])
    assert len(w.outlier_channels) == 4 and w.key.dtype == np.float32
    std = w.key.reshape(-1, 256).std(0)
    assert np.all(std[w.outlier_channels] > 10) and np.median(std) < 1.5
    assert w.query.reshape(-1, 256)[:, w.outlier_channels].std() > 5  # config 1: query too
    w2 = W.make_workload(W.CONFIGS[2], seq_len=256)
    assert len(w2.outlier_channels) == 3                              # 1% of 256, rounded up
    assert np.array_equal(w.block_table[0], np.arange(16))            # identity pages, config 1
