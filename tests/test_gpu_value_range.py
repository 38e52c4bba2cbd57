"""Decode parity when the value magnitudes of one stream span five decades.

Every 32-token unit of a sequence takes one of three value scales in turn
(x2000, x1, x0.05), so each wave of a split sees all three.  In the
"masked" mode the x2000 tokens' keys point away from every query of the
group (scores about -50), so the output comes from the small values alone
and any loss of precision that the large values force on the others would
show; in the "mixed" mode all keys are random and the large values dominate.
The pages' reference attention is plain fp32 over the dequantized cache
(vLLM API docs, "vllm.v1.attention.ops.rocm_octave", reference_attention),
so the tolerance does not depend on the value scale.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_amd import hkv
from decode_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-3
DEV = "cuda:0"

KERNELS = [  # dtype, D, rope_dim, Hq, Hkv, queries_per_seq
    ("q4_0", 256, 0, 16, 2, 1),
    ("q4_0", 256, 0, 16, 2, 4),
    ("q8_0", 256, 0, 16, 2, 1),
    ("octave_k3v4", 128, 64, 32, 8, 1),
    ("octave_k3v4", 128, 64, 32, 4, 2),
    ("octave_k3v3_compact", 256, 64, 32, 4, 1),
    ("octave_k3v3_compact", 256, 64, 32, 4, 4),
    ("q8_0", 128, 0, 8, 2, 1),
]


def _case(D, Hq, Hkv, qps, mode, seed):
    lens = [2300, 1100, 45]
    P = 16
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    T = sum(lens)
    nq = len(lens) * qps
    # one direction per (sequence, KV head) shared by its query heads
    u = rng.standard_normal((len(lens), Hkv, D))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    q = np.repeat(u, qps, axis=0)[:, :, None, :] * 4.0 + 0.3 * rng.standard_normal((nq, Hkv, G, D))
    q = q.reshape(nq, Hq, D)
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    t0 = 0
    for b, L in enumerate(lens):
        unit = np.arange(L) // 32
        big = unit % 3 == 0
        small = unit % 3 == 2
        v[t0:t0 + L][big] *= 2000.0
        v[t0:t0 + L][small] *= 0.05
        if mode == "masked":
            # scores of the large-value tokens: about -4 x 200 x scale = -50
            k[t0:t0 + L][big] = -200.0 * u[b][None]
        t0 += L
    pages = [(L + P - 1) // P for L in lens]
    perm = rng.permutation(sum(pages))
    bt = np.zeros((len(lens), max(pages)), np.int32)
    sm = np.empty(T, np.int64)
    off = t0 = 0
    for b, L in enumerate(lens):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
        pos = np.arange(L)
        sm[t0:t0 + L] = bt[b, pos // P].astype(np.int64) * P + pos % P
        t0 += L
    q_to_req = np.arange(len(lens), dtype=np.int32).repeat(qps)
    q_to_klen = np.array([[L - qps + 1 + i for i in range(qps)] for L in lens],
                         np.int32).reshape(-1)
    return (k.astype(np.float16), v.astype(np.float16), sm, bt, q_to_req, q_to_klen,
            q.astype(np.float32))


@pytest.mark.parametrize("mode", ["masked", "mixed"])
@pytest.mark.parametrize("dtype,D,R,Hq,Hkv,qps", KERNELS)
def test_decode_value_range(dtype, D, R, Hq, Hkv, qps, mode):
    print(f"value range {mode}: {dtype} D={D} Hq={Hq} Hkv={Hkv} qps={qps}", flush=True)
    k, v, sm, bt, q_to_req, q_to_klen, q = _case(D, Hq, Hkv, qps, mode, seed=3 * D + Hq + qps)
    P = 16
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    cache = hkv.new_cache(f, int(bt.max()) + 1, Hkv, DEV)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    ref_cache = np.zeros(tuple(cache.shape), np.uint8)
    ref_cache[sm // P, :, sm % P] = slots
    assert np.array_equal(cache.cpu().numpy(), ref_cache)
    scale = W.default_sm_scale(D)
    ref = O.attention(fo, q, ref_cache, bt, q_to_req, q_to_klen, scale)
    for det in (False, True):
        got = hkv.decode_attention(f, torch.from_numpy(q).to(DEV), cache,
                                   torch.from_numpy(bt).to(DEV),
                                   torch.from_numpy(q_to_req).to(DEV),
                                   torch.from_numpy(q_to_klen).to(DEV), int(q_to_klen.max()), qps,
                                   scale, deterministic=det).cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        bad = err > ATOL + RTOL * np.abs(ref)
        assert not bad.any(), (f"{dtype} {mode} det={det}: {bad.sum()} of {bad.size} outside "
                               f"tolerance; max abs err {err.max():.3e}, max |ref| "
                               f"{np.abs(ref).max():.3e}")
