"""A step captured in a HIP graph (quantize-append of the new tokens, then
decode attention) replays to the eager result.

Each replay is checked on its own, with eager work of the program and a
synchronization between replays: the cache bytes exactly, and the attention
output of the deterministic decode mode bit for bit.  The graph holds only the library's kernels
(no memset nodes).  The eager result is itself checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_amd import hkv
from decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("ci,sizes", [(3, dict(batch=2, seq_len=1537)),
                                      (4, dict(batch=3, seq_len=700, min_len=300)),
                                      (5, dict(batch=3, seq_len=1300, min_len=200)),
                                      (9, dict(batch=2, seq_len=1537))])
def test_graph_replay_matches_eager(ci, sizes):
    cfg = W.CONFIGS[ci]
    w = W.make_workload(cfg, **sizes)
    f = hkv.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim, cfg.page_size)
    fo = O.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim)
    scale = W.default_sm_scale(cfg.head_size)
    Hq, D = cfg.num_q_heads, cfg.head_size
    key = torch.from_numpy(w.key).to(DEV)
    value = torch.from_numpy(w.value).to(DEV)
    sm = torch.from_numpy(w.slot_mapping).to(DEV)
    rows = torch.from_numpy(w.append_rows()).to(DEV)
    new_k, new_v, new_sm = key[rows].contiguous(), value[rows].contiguous(), sm[rows].contiguous()
    query = torch.from_numpy(w.query).to(DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    q2r = torch.from_numpy(w.q_to_req).to(DEV)
    q2k = torch.from_numpy(w.q_to_klen).to(DEV)
    nq = len(w.q_to_req)
    ws = torch.empty(max(hkv.decode_workspace_bytes(f, nq, Hq, cfg.num_kv_heads, w.max_klen,
                                                    cfg.n_q), 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((nq, Hq, D), dtype=torch.float32, device=DEV)
    cache = hkv.new_cache(f, w.num_pages, cfg.num_kv_heads, DEV)
    # the cache before the step: every token except the appended ones
    old = torch.ones(key.shape[0], dtype=torch.bool, device=DEV)
    old[rows] = False
    hkv.quantize_append(f, key[old].contiguous(), value[old].contiguous(), sm[old].contiguous(),
                        cache)
    before = cache.clone()

    def step():
        hkv.quantize_append(f, new_k, new_v, new_sm, cache)
        hkv.decode_attention(f, query, cache, bt, q2r, q2k, w.max_klen, cfg.n_q, scale,
                             out=out, workspace=ws, deterministic=True)

    step()
    torch.cuda.synchronize()
    eager_out, eager_cache = out.clone(), cache.clone()

    # eager result against the oracle (full cache, all queries)
    slots = O.quantize(fo, w.key.astype(np.float32), w.value.astype(np.float32))
    ref_cache = np.zeros(tuple(cache.shape), np.uint8)
    P = cfg.page_size
    ref_cache[w.slot_mapping // P, :, w.slot_mapping % P] = slots
    assert np.array_equal(eager_cache.cpu().numpy(), ref_cache)
    ref = O.attention(fo, w.query.astype(np.float32), ref_cache, w.block_table, w.q_to_req,
                      w.q_to_klen, scale)
    err = np.abs(eager_out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 2e-3 + 1e-3 * np.abs(ref)), f"max abs err {err.max():.3e}"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    other = torch.empty_like(out)
    for rep in range(4):
        # eager work of the program between replays: reset the state the
        # step reads and writes, run an unrelated decode into another buffer
        cache.copy_(before)
        out.fill_(float("nan"))
        hkv.decode_attention(f, query, cache, bt, q2r, q2k, w.max_klen, cfg.n_q, scale,
                             out=other, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache, eager_cache), f"replay {rep}: cache bytes differ"
        # the deterministic mode sums in a fixed order: every replay gives the
        # eager bits (a replay that did not run leaves NaN)
        assert torch.equal(out.view(torch.int32), eager_out.view(torch.int32)), (
            f"replay {rep}: {(out != eager_out).sum().item()} values differ")
