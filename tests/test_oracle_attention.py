"""Pins of the oracle's paged attention (vLLM rocm_octave docs,
"reference_attention"; Strata PR #21 on query/output rotation).

Pinned against torch's scaled_dot_product_attention in fp64 (a library
routine) on the oracle's own dequantized cache, closed-form special cases,
page relabelling, and the rotated-space evaluation that the GPU path uses
(<Rq, Rk> = <q, k>; output rotated back once).
"""
import numpy as np
import pytest
import torch

import oracle as O

FORMATS = [("q4_0", 256, 0), ("octave_k3v4", 128, 64), ("octave_k3v3_compact", 256, 64),
           ("octave_k3v3", 128, 64), ("octave_k3v4", 192, 64), ("q8_0", 128, 0)]


def _setup(dtype, D, R, lens, Hq, Hkv, page=16, seed=0, shuffle=True):
    rng = np.random.default_rng(seed)
    f = O.format_init(dtype, D, R)
    B = len(lens)
    T = sum(lens)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    slots = O.quantize(f, k, v)
    pages = [(L + page - 1) // page for L in lens]
    npages = sum(pages)
    perm = rng.permutation(npages) if shuffle else np.arange(npages)
    bt = np.zeros((B, max(pages)), np.int32)
    cache = np.zeros((npages, Hkv, page, f.slot_bytes), np.uint8)
    off = t0 = 0
    for b, L in enumerate(lens):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
        for t in range(L):
            cache[bt[b, t // page], :, t % page] = slots[t0 + t]
        t0 += L
    return f, slots, cache, bt


@pytest.mark.parametrize("dtype,D,R", FORMATS)
def test_attention_matches_torch_sdpa_fp64(dtype, D, R):
    lens = [37, 5, 64]
    Hq, Hkv = 8, 2
    f, slots, cache, bt = _setup(dtype, D, R, lens, Hq, Hkv)
    rng = np.random.default_rng(1)
    Q = 6
    q = rng.standard_normal((Q, Hq, D)).astype(np.float32)
    q_to_req = np.array([0, 0, 1, 2, 2, 2], np.int32)
    q_to_klen = np.array([37, 20, 5, 64, 1, 33], np.int32)
    scale = 1.0 / np.sqrt(D)
    out = O.attention(f, q, cache, bt, q_to_req, q_to_klen, scale)
    kd, vd = O.dequantize_f64(f, slots)
    starts = np.concatenate([[0], np.cumsum(lens)])
    for i in range(Q):
        b, L = q_to_req[i], q_to_klen[i]
        K = torch.from_numpy(kd[starts[b]:starts[b] + L]).permute(1, 0, 2)[None]
        V = torch.from_numpy(vd[starts[b]:starts[b] + L]).permute(1, 0, 2)[None]
        qq = torch.from_numpy(q[i].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, K, V, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(out[i], ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dtype,D,R", FORMATS[:3])
def test_attention_special_cases(dtype, D, R):
    lens = [48]
    Hq, Hkv = 4, 2
    f, slots, cache, bt = _setup(dtype, D, R, lens, Hq, Hkv, seed=3)
    kd, vd = O.dequantize_f64(f, slots)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, Hq, D)).astype(np.float32)
    q[2] = 0.0
    q_to_req = np.zeros(4, np.int32)
    q_to_klen = np.array([1, 0, 48, -3], np.int32)
    out = O.attention(f, q, cache, bt, q_to_req, q_to_klen, 0.1)
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], vd[0, h // G], rtol=0, atol=1e-12)   # klen = 1
        np.testing.assert_allclose(out[2, h], vd[:, h // G].mean(0), rtol=0, atol=1e-12)  # q = 0
    assert np.all(out[1] == 0) and np.all(out[3] == 0)                        # klen <= 0


def test_attention_identical_keys_average_values():
    D, Hkv, Hq = 256, 1, 2
    f = O.format_init("q4_0", D)
    rng = np.random.default_rng(5)
    k = np.repeat(rng.standard_normal((1, Hkv, D)).astype(np.float32), 32, axis=0)
    v = rng.standard_normal((32, Hkv, D)).astype(np.float32)
    slots = O.quantize(f, k, v)
    cache = slots.reshape(2, 16, Hkv, -1).transpose(0, 2, 1, 3).copy()
    bt = np.array([[0, 1]], np.int32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = O.attention(f, q, cache, bt, np.zeros(1, np.int32), np.array([32], np.int32), 0.5)
    _, vd = O.dequantize_f64(f, slots)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], vd[:, 0].mean(0), rtol=0, atol=1e-12)


def test_attention_page_relabel_invariance():
    lens = [70, 33]
    f, slots, cache, bt = _setup("octave_k3v4", 128, 64, lens, 8, 4, seed=6)
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 8, 128)).astype(np.float32)
    qr, ql = np.array([0, 1], np.int32), np.array([70, 33], np.int32)
    a = O.attention(f, q, cache, bt, qr, ql, 0.09)
    perm = rng.permutation(cache.shape[0])          # new id of each page
    cache2 = np.empty_like(cache)
    cache2[perm] = cache
    b = O.attention(f, q, cache2, perm[bt].astype(np.int32), qr, ql, 0.09)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype,D,R", FORMATS)
def test_rotated_space_evaluation_agrees(dtype, D, R):
    # Scores in the rotated space with the query rotated like K, output
    # rotated back once with the inverse V rotation (module text).
    lens = [40]
    Hq, Hkv = 4, 2
    f, slots, cache, bt = _setup(dtype, D, R, lens, Hq, Hkv, seed=8)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    scale = 0.07
    out = O.attention(f, q, cache, bt, np.zeros(1, np.int32), np.array([40], np.int32), scale)
    kr, vr = O.dequantize(f, slots, rotated=True)      # exact values
    s = O.signs(D).astype(np.float64) if f.use_signs else np.ones(D)
    G = Hq // Hkv
    for h in range(Hq):
        qr = O.fwht(q[0, h].astype(np.float64) * s, f.k_block)
        sc = kr[:, h // G].astype(np.float64) @ qr * scale
        p = np.exp(sc - sc.max())
        p /= p.sum()
        o_rot = p @ vr[:, h // G].astype(np.float64)
        o = O.fwht(o_rot, f.v_block) * s
        np.testing.assert_allclose(out[0, h], o, rtol=0, atol=1e-10)


def test_attention_lse_is_log_sum_exp_and_leaves_output_alone():
    # lse against scipy's logsumexp of the fp64 scores on the oracle's own
    # dequantized cache; the output equals attention() bit for bit.
    from scipy.special import logsumexp
    lens = [45, 16]
    Hq, Hkv, D = 6, 2, 128
    f, slots, cache, bt = _setup("q8_0", D, 0, lens, Hq, Hkv, seed=10)
    kd, _ = O.dequantize_f64(f, slots)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, Hq, D)).astype(np.float32)
    qr = np.array([0, 0, 1, 1], np.int32)
    ql = np.array([45, 17, 0, 16], np.int32)
    scale = 0.11
    out, lse = O.attention_lse(f, q, cache, bt, qr, ql, scale)
    assert np.array_equal(out, O.attention(f, q, cache, bt, qr, ql, scale))
    starts = [0, 45]
    G = Hq // Hkv
    for i in range(4):
        for h in range(Hq):
            if ql[i] <= 0:
                assert lse[i, h] == -np.inf and np.all(out[i, h] == 0)
                continue
            k = kd[starts[qr[i]]:starts[qr[i]] + ql[i], h // G]
            s = k @ q[i, h].astype(np.float64) * scale
            np.testing.assert_allclose(lse[i, h], logsumexp(s), rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype,D,R", FORMATS[:3])
def test_attention_token_ranges_merge_to_whole(dtype, D, R):
    # Attention over page-aligned token ranges (a shifted block table and the
    # range's length) merged with the lse weights gives the whole-range row.
    lens = [150]
    Hq, Hkv, P = 4, 2, 16
    f, slots, cache, bt = _setup(dtype, D, R, lens, Hq, Hkv, page=P, seed=12)
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    L, scale = 150, 1.0 / np.sqrt(D)
    whole = O.attention(f, q, cache, bt, np.zeros(1, np.int32), np.array([L], np.int32), scale)
    cuts = [0, 3, 4, 8, 10]                  # page boundaries; last range ragged
    outs, lses = [], []
    for p0, p1 in zip(cuts[:-1], cuts[1:]):
        n = min(L, p1 * P) - p0 * P
        o, s = O.attention_lse(f, q, cache, np.ascontiguousarray(bt[:, p0:]),
                               np.zeros(1, np.int32), np.array([n], np.int32), scale)
        outs.append(o)
        lses.append(s)
    lse = np.logaddexp.reduce(np.stack(lses), axis=0)
    merged = sum(np.exp(s - lse)[..., None] * o for o, s in zip(outs, lses))
    np.testing.assert_allclose(merged, whole, rtol=0, atol=1e-12)
