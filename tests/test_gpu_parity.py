"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: packed cache bytes and dequantized values bit-exact; attention within
|gpu - oracle| <= 2e-3 + 1e-3 * |oracle| elementwise (fp32 path vs the fp64
definition).  Inputs come from the seeded workload generator; the oracle
never sees anything the GPU produced.
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


def _gpu_cache(f, w):
    cfg = w.cfg
    cache = hkv.new_cache(f, w.num_pages, cfg.num_kv_heads, DEV)
    hkv.quantize_append(f, torch.from_numpy(w.key).to(DEV), torch.from_numpy(w.value).to(DEV),
                        torch.from_numpy(w.slot_mapping).to(DEV), cache)
    return cache


def _oracle_cache(fo, w, shape):
    slots = O.quantize(fo, w.key.astype(np.float32), w.value.astype(np.float32))
    ref = np.zeros(shape, np.uint8)
    P = w.cfg.page_size
    ref[w.slot_mapping // P, :, w.slot_mapping % P] = slots
    return ref, slots


def _decode(f, w, cache, scale, qps=None, deterministic=False):
    cfg = w.cfg
    return hkv.decode_attention(f, torch.from_numpy(w.query).to(DEV), cache,
                                torch.from_numpy(w.block_table).to(DEV),
                                torch.from_numpy(w.q_to_req).to(DEV),
                                torch.from_numpy(w.q_to_klen).to(DEV), w.max_klen,
                                cfg.n_q if qps is None else qps, scale,
                                deterministic=deterministic)


def _assert_close(got, ref, what):
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                           f"max abs err {err.max():.3e}")
    return float(err.max())


SMALL = {   # config -> reduced sizes that still span several tiles, splits and a ragged tail
    1: dict(),
    2: dict(seq_len=2100),
    3: dict(batch=2, seq_len=1537),
    4: dict(batch=3, seq_len=700, min_len=300),
    5: dict(batch=3, seq_len=1300, min_len=200),
}


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
def test_quantize_append_bit_exact(ci):
    cfg = W.CONFIGS[ci]
    w = W.make_workload(cfg, **SMALL[ci])
    f = hkv.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim, cfg.page_size)
    fo = O.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim)
    got = _gpu_cache(f, w).cpu().numpy()
    ref, _ = _oracle_cache(fo, w, got.shape)
    diff = got != ref
    assert not diff.any(), f"config {ci}: {diff.sum()} bytes differ"


@pytest.mark.parametrize("dtype,D,R", [("q4_0", 256, 0), ("q4_0", 128, 0), ("q4_0", 64, 0),
                                       ("octave_k3v4", 128, 64), ("octave_k3v3", 128, 64),
                                       ("octave_k3v3_compact", 256, 64), ("octave_k3v4", 192, 64),
                                       ("octave_k3v4", 256, 128), ("octave_k3v3_compact", 64, 0),
                                       ("octave_k3v4", 128, 0), ("octave_k3v4", 128, 128),
                                       ("q8_0", 256, 0), ("q8_0", 128, 0), ("q8_0", 64, 0)])
@pytest.mark.parametrize("in_dtype", [np.float32, np.float16])
def test_quantize_and_dequantize_formats(dtype, D, R, in_dtype):
    rng = np.random.default_rng(D + R)
    T, H, P = 50, 3, 16
    k = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(in_dtype)
    v = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(in_dtype)
    k[3] = 0
    v[4, 1] = 0
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    pages = (T + P - 1) // P
    sm = rng.permutation(pages * P)[:T].astype(np.int64)
    sm[7] = -1                                         # skipped token
    cache = hkv.new_cache(f, pages, H, DEV)
    cache.fill_(0xA5)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    got = cache.cpu().numpy()
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    keep = sm >= 0
    assert np.array_equal(got[sm[keep] // P, :, sm[keep] % P], slots[keep])
    untouched = np.ones(pages * P, bool)
    untouched[sm[keep]] = False
    flat = got.transpose(0, 2, 1, 3).reshape(pages * P, H, -1)
    assert np.all(flat[untouched] == 0xA5)             # nothing else written
    for rotated in (True, False):
        ids = torch.from_numpy(sm).to(DEV)
        kd, vd = hkv.dequantize(f, cache, ids, rotated=rotated)
        kr, vr = O.dequantize(fo, slots, rotated=rotated)
        kd, vd = kd.cpu().numpy(), vd.cpu().numpy()
        assert np.array_equal(kd[keep].view(np.uint32), kr[keep].view(np.uint32))
        assert np.array_equal(vd[keep].view(np.uint32), vr[keep].view(np.uint32))
        assert np.all(kd[~keep] == 0) and np.all(vd[~keep] == 0)


MANY_ROW_FORMATS = [("q4_0", 64, 0), ("q4_0", 128, 0), ("q4_0", 256, 0),
                    ("q8_0", 64, 0), ("q8_0", 128, 0), ("q8_0", 256, 0),
                    ("octave_k3v4", 128, 64), ("octave_k3v3", 128, 64),
                    ("octave_k3v3_compact", 256, 64), ("octave_k3v3_compact", 64, 0),
                    ("octave_k3v4", 192, 64), ("octave_k3v4", 256, 128),
                    ("octave_k3v4", 128, 0), ("octave_k3v4", 128, 128)]


@pytest.mark.parametrize("dtype,D,R", MANY_ROW_FORMATS)
@pytest.mark.parametrize("in_dtype", [np.float32, np.float16])
@pytest.mark.parametrize("misaligned", [False, True])
def test_quantize_many_rows(dtype, D, R, in_dtype, misaligned):
    """Row counts that take the many-rows kernels (16 lanes per row, four
    rows per wave; a ragged last wave, skipped slots); a key/value pointer
    off its 8/16-byte alignment takes the one-row-per-wave kernel instead.
    Both must give the oracle's bytes."""
    rng = np.random.default_rng(7 * D + R + (3 if misaligned else 0) + len(dtype))
    T, H, P = 1501, 3, 16                              # 4503 rows = 281 waves of 16 + 7
    k = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(in_dtype)
    v = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(in_dtype)
    k[5] = 0
    v[9, 2] = 0
    k[11, 1, :32] = -np.abs(k[11, 1, :32]).max()     # max-abs ties inside one block
    k[11, 1, 3] = -k[11, 1, 3]
    k[13, 0] = (rng.standard_normal(D) * 3e-6).astype(in_dtype)  # fp16 subnormals
    v[13, 2] = (rng.standard_normal(D) * 3e-6).astype(in_dtype)
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    pages = (T + P - 1) // P + 2
    sm = rng.permutation(pages * P)[:T].astype(np.int64)
    sm[[0, 17, T - 1]] = -1
    cache = hkv.new_cache(f, pages, H, DEV)
    cache.fill_(0xA5)

    def dev(a):
        t = torch.from_numpy(a).to(DEV)
        if not misaligned:
            return t
        buf = torch.empty(a.size + 1, dtype=t.dtype, device=DEV)
        buf[1:] = t.reshape(-1)
        return buf[1:].view(a.shape)
    kt, vt = dev(k), dev(v)
    assert (kt.data_ptr() % 16 != 0) == misaligned
    hkv.quantize_append(f, kt, vt, torch.from_numpy(sm).to(DEV), cache)
    got = cache.cpu().numpy()
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    keep = sm >= 0
    assert np.array_equal(got[sm[keep] // P, :, sm[keep] % P], slots[keep])
    untouched = np.ones(pages * P, bool)
    untouched[sm[keep]] = False
    flat = got.transpose(0, 2, 1, 3).reshape(pages * P, H, -1)
    assert np.all(flat[untouched] == 0xA5)


@pytest.mark.parametrize("dtype,D,R,scales", [
    ("q4_0", 256, 0, (1e35, 1e-30, 1e20, 1e-20)), ("q4_0", 128, 0, (1e35, 1e-30, 1e20, 1e-20)),
    ("q8_0", 256, 0, (1e35, 1e-30, 1e20, 1e-20)),
    ("octave_k3v4", 128, 64, (1e15, 1e-15, 1e8, 1e-8)),
    ("octave_k3v3_compact", 256, 64, (1e15, 1e-15, 1e8, 1e-8))])
def test_quantize_many_rows_fp32_magnitudes(dtype, D, R, scales):
    """fp32 rows far outside the fp16 range through the many-rows kernels:
    whole rows, and single 32-value blocks, scaled up or down by the given
    factors beside plain rows.  Blocks whose scale falls outside the range
    where the reciprocal's fast form is exact send their wave to the per-lane
    reciprocal (Q4_0, Q8_0); the Octave kernels keep every range test on fp32
    rows.  Bytes equal the oracle's."""
    rng = np.random.default_rng(17 * D + R + len(dtype))
    T, H, P = 1400, 3, 16                              # 4200 rows
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    for t in range(0, T, 5):
        f_ = scales[(t // 5) % len(scales)]
        for a in (k, v):
            h = rng.integers(H)
            if (t // 5) % 2:
                a[t, h] *= np.float32(f_)
            else:
                b0 = 32 * rng.integers(D // 32)
                a[t, h, b0:b0 + 32] *= np.float32(f_)
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    pages = (T + P - 1) // P + 1
    sm = rng.permutation(pages * P)[:T].astype(np.int64)
    cache = hkv.new_cache(f, pages, H, DEV)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    got = cache.cpu().numpy()
    slots = O.quantize(fo, k, v)
    assert np.array_equal(got[sm // P, :, sm % P], slots)


@pytest.mark.parametrize("dtype,D,R", [("q4_0", 256, 0), ("q4_0", 128, 0), ("q8_0", 256, 0),
                                       ("octave_k3v4", 128, 64), ("octave_k3v3", 128, 64),
                                       ("octave_k3v3_compact", 256, 64), ("octave_k3v4", 192, 64)])
def test_quantize_many_rows_fp16_extremes(dtype, D, R):
    """fp16 rows at the ends of the fp16 range through the many-rows kernels,
    whose fp16 paths rest on the range of a transformed fp16 row (every
    nonzero value between 2^-28 and 2^20): rows of +-65504, rows of the
    smallest subnormals, rows mixing both, rows with a single nonzero value
    and zero rows, beside plain N(0, 1) rows.  Bytes equal the oracle's."""
    rng = np.random.default_rng(31 * D + R + len(dtype))
    T, H, P = 1400, 3, 16                              # 4200 rows
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    tiny = np.float16(2.0 ** -24)
    big = np.float16(65504.0)
    sgn = lambda *shape: np.where(rng.random(shape) < 0.5, -1, 1).astype(np.float16)
    for t in range(0, T, 7):
        kind = (t // 7) % 6
        for a in (k, v):
            h = rng.integers(H)
            if kind == 0:
                a[t, h] = big * sgn(D)
            elif kind == 1:
                a[t, h] = tiny * sgn(D)
            elif kind == 2:
                a[t, h] = np.where(rng.random(D) < 0.5, big, tiny) * sgn(D)
            elif kind == 3:
                a[t, h] = 0
                a[t, h, rng.integers(D)] = big if rng.random() < 0.5 else tiny
            elif kind == 4:
                a[t, h] = 0
            else:
                a[t, h] = (rng.standard_normal(D) * 1e3).astype(np.float16)
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    pages = (T + P - 1) // P + 1
    sm = rng.permutation(pages * P)[:T].astype(np.int64)
    cache = hkv.new_cache(f, pages, H, DEV)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    got = cache.cpu().numpy()
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    assert np.array_equal(got[sm // P, :, sm % P], slots)


@pytest.mark.parametrize("dtype,D,R", [("q4_0", 256, 0), ("q8_0", 128, 0), ("octave_k3v4", 128, 64),
                                       ("octave_k3v3_compact", 256, 64)])
@pytest.mark.parametrize("P", [12, 48, 1000])
def test_quantize_many_rows_page_sizes(dtype, D, R, P):
    """The many-rows kernels with page sizes that are not powers of two (the
    slot's page and offset then come from divisions, not a shift and a
    mask), five KV heads, a ragged last wave and skipped slots: the
    oracle's bytes, nothing else written."""
    rng = np.random.default_rng(5 * D + P + len(dtype))
    T, H = 1003, 5                                     # 5015 rows
    k = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(np.float16)
    v = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(np.float16)
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    pages = (T + P - 1) // P + 2
    sm = rng.permutation(pages * P)[:T].astype(np.int64)
    sm[[1, T // 2, T - 1]] = -1
    cache = hkv.new_cache(f, pages, H, DEV)
    cache.fill_(0xA5)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    got = cache.cpu().numpy()
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    keep = sm >= 0
    assert np.array_equal(got[sm[keep] // P, :, sm[keep] % P], slots[keep])
    untouched = np.ones(pages * P, bool)
    untouched[sm[keep]] = False
    flat = got.transpose(0, 2, 1, 3).reshape(pages * P, H, -1)
    assert np.all(flat[untouched] == 0xA5)


@pytest.mark.parametrize("dtype,D", [("q4_0", 256), ("q4_0", 128), ("q4_0", 64), ("q8_0", 256)])
@pytest.mark.parametrize("in_dtype", [np.float32, np.float16])
@pytest.mark.parametrize("T", [3, 512, 513, 1000])
def test_quantize_row_count_paths(dtype, D, in_dtype, T):
    """Q4_0 / Q8_0 appends of 6, 1024, 1026 and 2000 (token, head) rows: up to
    1024 rows each row's K and V halves go to separate waves, above that one
    wave takes a whole row.  Both give the oracle's bytes, with skipped
    slots, zero rows and max-abs ties, and write nothing else."""
    rng = np.random.default_rng(11 * D + T + len(dtype) + (1 if in_dtype == np.float16 else 0))
    H, P = 2, 16
    k = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(in_dtype)
    v = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(in_dtype)
    k[T // 2] = 0
    v[T - 1, 1] = 0
    k[0, 1, :32] = -np.abs(k[0, 1, :32]).max()     # max-abs ties inside one block
    k[0, 1, 3] = -k[0, 1, 3]
    f = hkv.format_init(dtype, D, 0, P)
    fo = O.format_init(dtype, D, 0)
    pages = (T + P - 1) // P + 2
    sm = rng.permutation(pages * P)[:T].astype(np.int64)
    sm[T // 3] = -1
    cache = hkv.new_cache(f, pages, H, DEV)
    cache.fill_(0xA5)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    got = cache.cpu().numpy()
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    keep = sm >= 0
    assert np.array_equal(got[sm[keep] // P, :, sm[keep] % P], slots[keep])
    untouched = np.ones(pages * P, bool)
    untouched[sm[keep]] = False
    flat = got.transpose(0, 2, 1, 3).reshape(pages * P, H, -1)
    assert np.all(flat[untouched] == 0xA5)


@pytest.mark.parametrize("dtype,R", [("q4_0", 0), ("q8_0", 0), ("octave_k3v3_compact", 64),
                                     ("octave_k3v4", 128)])
def test_quantize_many_rows_several_passes(dtype, R):
    """More rows than one grid pass of the 16-lanes-per-row kernel (2048
    workgroups x 16 rows): waves loop, loading the next rows during the
    current ones; ragged end."""
    rng = np.random.default_rng(88)
    T, H, P, D = 17003, 2, 16, 256                     # 34006 rows
    k = (rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30, (T, H, 1))).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    pages = (T + P - 1) // P
    sm = rng.permutation(pages * P)[:T].astype(np.int64)
    cache = hkv.new_cache(f, pages, H, DEV)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    got = cache.cpu().numpy()
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    assert np.array_equal(got[sm // P, :, sm % P], slots)


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
def test_decode_matches_oracle(ci):
    cfg = W.CONFIGS[ci]
    w = W.make_workload(cfg, **SMALL[ci])
    f = hkv.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim, cfg.page_size)
    fo = O.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim)
    cache = _gpu_cache(f, w)
    ref_cache, _ = _oracle_cache(fo, w, tuple(cache.shape))
    scale = W.default_sm_scale(cfg.head_size)
    got = _decode(f, w, cache, scale).cpu().numpy()
    ref = O.attention(fo, w.query.astype(np.float32), ref_cache, w.block_table, w.q_to_req,
                      w.q_to_klen, scale)
    _assert_close(got, ref, f"config {ci}")


@pytest.mark.parametrize("dtype,D,R,Hq,Hkv,n_q", [("q4_0", 256, 0, 16, 2, 8),
                                                  ("q4_0", 256, 0, 16, 2, 16),
                                                  ("octave_k3v3_compact", 256, 64, 32, 4, 8),
                                                  ("octave_k3v3_compact", 256, 64, 32, 4, 3),
                                                  ("octave_k3v3_compact", 256, 64, 34, 2, 1),
                                                  ("octave_k3v3_compact", 256, 64, 32, 2, 2),
                                                  ("octave_k3v4", 128, 64, 32, 8, 16),
                                                  ("octave_k3v4", 128, 64, 32, 8, 6),
                                                  ("q4_0", 128, 0, 32, 1, 4),
                                                  ("octave_k3v3", 128, 64, 8, 1, 12),
                                                  ("octave_k3v4", 192, 64, 16, 2, 2),
                                                  ("octave_k3v4", 192, 64, 12, 4, 5),
                                                  ("q8_0", 256, 0, 16, 2, 4)])
def test_decode_long_query_windows(dtype, D, R, Hq, Hkv, n_q):
    """Query windows beyond 4 tokens (verify / multi-token prediction): more
    query rows per KV head than one kernel pass takes, so the window's
    queries run as sub-groups; causal among the window's tokens."""
    cfg = W.Config(90, "window", dtype, D, R, 3, 900, Hq, Hkv, "f16", n_q=n_q, min_len=300)
    w = W.make_workload(cfg)
    f = hkv.format_init(dtype, D, R, cfg.page_size)
    fo = O.format_init(dtype, D, R)
    cache = _gpu_cache(f, w)
    ref_cache, _ = _oracle_cache(fo, w, tuple(cache.shape))
    scale = W.default_sm_scale(D)
    got = _decode(f, w, cache, scale).cpu().numpy()
    ref = O.attention(fo, w.query.astype(np.float32), ref_cache, w.block_table, w.q_to_req,
                      w.q_to_klen, scale)
    _assert_close(got, ref, f"{dtype} D={D} G={Hq // Hkv} n_q={n_q}")


@pytest.mark.parametrize("dtype,D,R,Hq,Hkv", [("q4_0", 256, 0, 16, 2), ("q4_0", 256, 0, 8, 2),
                                              ("q4_0", 128, 0, 4, 4),
                                              ("q4_0", 64, 0, 6, 3),
                                              ("octave_k3v4", 128, 64, 32, 8),
                                              ("octave_k3v4", 128, 64, 32, 4),
                                              ("octave_k3v3", 128, 64, 8, 1),
                                              ("octave_k3v3_compact", 256, 64, 32, 4),
                                              ("octave_k3v4", 192, 64, 4, 2),
                                              ("q8_0", 256, 0, 16, 2), ("q8_0", 128, 0, 4, 4),
                                              ("q8_0", 64, 0, 6, 3)])
def test_decode_edge_lengths(dtype, D, R, Hq, Hkv):
    # klen 0, 1, one page, page +- 1, 1024 and 2048 +- 1 (split boundaries for
    # the split sizes these shapes get: multiples of 64 that divide them) and a
    # long ragged one; with two queries per sequence the second query sees one
    # token less, so for the lengths 1025 and 2049 it has no token in the last
    # split that the first query uses.
    lens = [1, 15, 16, 17, 1023, 1024, 1025, 2047, 2049, 2500, 3]
    rng = np.random.default_rng(D + Hq)
    P = 16
    T = sum(lens)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float16)
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
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    cache = hkv.new_cache(f, sum(pages), Hkv, DEV)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    ref_cache = np.zeros(tuple(cache.shape), np.uint8)
    ref_cache[sm // P, :, sm % P] = slots
    q_to_req = np.arange(len(lens), dtype=np.int32).repeat(2)
    q_to_klen = np.array([[L, L - 1] for L in lens], np.int32).reshape(-1)
    q_to_klen[1] = 0                 # klen 0 -> zero row
    q_to_klen[-1] = -5               # negative -> zero row
    q = rng.standard_normal((len(q_to_req), Hq, D)).astype(np.float32)
    scale = W.default_sm_scale(D)
    for qps in (1, 2):
        got = hkv.decode_attention(f, torch.from_numpy(q).to(DEV), cache,
                                   torch.from_numpy(bt).to(DEV), torch.from_numpy(q_to_req).to(DEV),
                                   torch.from_numpy(q_to_klen).to(DEV), int(q_to_klen.max()), qps,
                                   scale).cpu().numpy()
        ref = O.attention(fo, q, ref_cache, bt, q_to_req, q_to_klen, scale)
        _assert_close(got, ref, f"{dtype} qps={qps}")
        assert np.all(got[1] == 0) and np.all(got[-1] == 0)


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (24, 4), (17, 1)])
@pytest.mark.parametrize("dtype,R", [("octave_k3v3_compact", 64), ("q4_0", 0)])
def test_decode_one_pass_window_edge_lengths(dtype, R, Hq, Hkv):
    """The one-pass kernels for up to 32 query rows per KV head (Octave k3v3
    compact from 17 rows, Q4_0 from 9): four queries per sequence (causal:
    klen L-3 .. L), so with queries_per_seq 4 a pass holds 4 G rows (G = 8:
    all 32 rows live; G = 6: 24 rows and 8 padding rows; G = 17: one query
    per pass, 17 rows); lengths at the tile, page and split edges; a query
    with no tokens and one with a negative length give zero rows."""
    D, P = 256, 16
    lens = [4, 5, 16, 19, 20, 35, 1027, 2051, 2500, 7]
    rng = np.random.default_rng(Hq * 7 + Hkv)
    T = sum(lens)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float16)
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
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    cache = hkv.new_cache(f, sum(pages), Hkv, DEV)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    ref_cache = np.zeros(tuple(cache.shape), np.uint8)
    ref_cache[sm // P, :, sm % P] = slots
    q_to_req = np.arange(len(lens), dtype=np.int32).repeat(4)
    q_to_klen = np.array([[L - 3, L - 2, L - 1, L] for L in lens], np.int32).reshape(-1)
    q_to_klen[2] = 0                 # klen 0 -> zero row
    q_to_klen[-4] = -5               # negative -> zero row
    # small and large query magnitudes in one pass (each row's query operand
    # follows its own scale; larger magnitudes are covered in
    # test_gpu_query_magnitude.py)
    q = (rng.standard_normal((len(q_to_req), Hq, D)) *
         rng.choice([0.01, 1.0, 4.0], size=(len(q_to_req), Hq, 1))).astype(np.float32)
    scale = W.default_sm_scale(D)
    got = hkv.decode_attention(f, torch.from_numpy(q).to(DEV), cache,
                               torch.from_numpy(bt).to(DEV), torch.from_numpy(q_to_req).to(DEV),
                               torch.from_numpy(q_to_klen).to(DEV), int(q_to_klen.max()), 4,
                               scale).cpu().numpy()
    ref = O.attention(fo, q, ref_cache, bt, q_to_req, q_to_klen, scale)
    _assert_close(got, ref, f"{dtype} Hq={Hq} Hkv={Hkv}")
    assert np.all(got[2] == 0) and np.all(got[-4] == 0)


def test_decode_is_deterministic_and_page_relabel_invariant():
    cfg = W.CONFIGS[2]
    w = W.make_workload(cfg, seq_len=3000)
    f = hkv.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim, cfg.page_size)
    cache = _gpu_cache(f, w)
    scale = W.default_sm_scale(cfg.head_size)
    a = _decode(f, w, cache, scale, deterministic=True).cpu().numpy()
    b = _decode(f, w, cache, scale, deterministic=True).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # relabel physical pages: identical result
    perm = torch.randperm(cache.shape[0], generator=torch.Generator().manual_seed(0))
    cache2 = torch.empty_like(cache)
    cache2[perm.to(DEV)] = cache
    w2 = W.Workload(**{**w.__dict__, "block_table": perm.numpy()[w.block_table].astype(np.int32)})
    c = _decode(f, w2, cache2, scale, deterministic=True).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_requantize_reproduces_bytes():
    cfg = W.CONFIGS[5]
    w = W.make_workload(cfg, batch=2, seq_len=600)
    f = hkv.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim, cfg.page_size)
    a = _gpu_cache(f, w).cpu().numpy()
    b = _gpu_cache(f, w).cpu().numpy()
    assert np.array_equal(a, b)


def _full_size_check(ci, seqs, n_slot_samples=4096):
    """A workload at its full size, decoded in the launch configuration the
    benchmark times; the oracle checks sampled slots bit for bit and every
    output row of the sequences in `seqs` (it quantizes those sequences
    itself: nothing it uses comes from the GPU).

    The deterministic mode is the race detector of the waves' shared LDS
    work: two of its calls must agree bit for bit over the whole output
    (every wave, every split and the merge run in a fixed order), and agree
    with the default mode to rounding."""
    cfg = W.CONFIGS[ci]
    w = W.make_workload(cfg)
    f = hkv.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim, cfg.page_size)
    fo = O.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim)
    cache = _gpu_cache(f, w)
    scale = W.default_sm_scale(cfg.head_size)
    got = _decode(f, w, cache, scale).cpu().numpy()
    det1 = _decode(f, w, cache, scale, deterministic=True).cpu().numpy()
    det2 = _decode(f, w, cache, scale, deterministic=True).cpu().numpy()
    assert np.array_equal(det1.view(np.uint32), det2.view(np.uint32)), (
        f"deterministic mode: {(det1 != det2).sum()} of {det1.size} values differ between calls")
    P = cfg.page_size
    # sampled slots, bit-exact
    rng = np.random.default_rng(7)
    rows = rng.choice(w.key.shape[0], size=min(n_slot_samples, w.key.shape[0]), replace=False)
    slots = O.quantize(fo, w.key[rows].astype(np.float32), w.value[rows].astype(np.float32))
    sm = w.slot_mapping[rows]
    gpu_slots = cache[torch.from_numpy(sm // P).to(DEV), :, torch.from_numpy(sm % P).to(DEV)]
    assert np.array_equal(gpu_slots.cpu().numpy(), slots)
    # the decode rows of the chosen sequences against the oracle's own cache
    sub = W.subset(w, seqs)
    ref_cache = np.zeros(tuple(cache.shape), np.uint8)
    for b in range(len(seqs)):
        r0, r1 = sub.seq_start[b], sub.seq_start[b + 1]
        sl = O.quantize(fo, sub.key[r0:r1].astype(np.float32), sub.value[r0:r1].astype(np.float32))
        sm_b = sub.slot_mapping[r0:r1]
        ref_cache[sm_b // P, :, sm_b % P] = sl
    ref = O.attention(fo, sub.query.astype(np.float32), ref_cache, sub.block_table, sub.q_to_req,
                      sub.q_to_klen, scale)
    qsel = np.concatenate([np.nonzero(w.q_to_req == b)[0] for b in seqs])
    e_def = _assert_close(got[qsel], ref, f"config {ci} full size, sequences {seqs}")
    e_det = _assert_close(det1[qsel], ref, f"config {ci} full size, deterministic, sequences {seqs}")
    # the two modes differ only in summation order: far inside the oracle bar
    d = np.abs(det1.astype(np.float64) - got)
    bad = d > ATOL / 10 + RTOL / 10 * np.abs(got)
    where = np.unravel_index(int(np.argmax(d)), d.shape)
    assert not bad.any(), (f"modes differ at {bad.sum()} of {bad.size} values; max {d.max():.3e} at "
                           f"{where} ({got[where]:.6e} vs {det1[where]:.6e}); oracle errors "
                           f"default {e_def:.3e}, deterministic {e_det:.3e}")


def test_decode_full_size_q4_0_128k():
    _full_size_check(3, [0, 3])


@pytest.mark.parametrize("ci,seqs", [(4, [0, 31]), (5, [0, 37, 63])])
def test_decode_full_size_octave(ci, seqs):
    _full_size_check(ci, seqs)


@pytest.mark.parametrize("ci,seqs", [(6, [0, 15]), (7, [0, 31]), (8, [0, 15]), (9, [1])])
def test_decode_full_size_wider_formats(ci, seqs):
    """Query windows of 8 tokens (Q4_0), 3-bit V at head size 128, head size
    192 and the Q8_0 mode, each at its benchmark size."""
    _full_size_check(ci, seqs)


@pytest.mark.parametrize("P", [32, 64, 24, 1])
@pytest.mark.parametrize("dtype,D,R,Hq,Hkv,qps", [("q4_0", 256, 0, 16, 2, 1),
                                                  ("q4_0", 256, 0, 16, 2, 4),
                                                  ("q8_0", 256, 0, 16, 2, 1),
                                                  ("octave_k3v4", 128, 64, 32, 8, 1),
                                                  ("octave_k3v3", 128, 64, 16, 4, 4),
                                                  ("octave_k3v4", 192, 64, 8, 2, 1),
                                                  ("octave_k3v3_compact", 256, 64, 32, 4, 4)])
def test_decode_page_sizes(P, dtype, D, R, Hq, Hkv, qps):
    """Pages other than 16 tokens: 32 and 64 (the matrix-core kernels' tiles
    start inside a page), and 24 and 1 (not a multiple of the 16-token tile:
    the generic kernel)."""
    lens = [5, 100, 700, 2049]
    rng = np.random.default_rng(P * 31 + D + Hq)
    T = sum(lens)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float16)
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
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    cache = hkv.new_cache(f, sum(pages), Hkv, DEV)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm).to(DEV), cache)
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    ref_cache = np.zeros(tuple(cache.shape), np.uint8)
    ref_cache[sm // P, :, sm % P] = slots
    assert np.array_equal(cache.cpu().numpy(), ref_cache)
    q_to_req = np.arange(len(lens), dtype=np.int32).repeat(qps)
    q_to_klen = np.array([[L - qps + 1 + j for j in range(qps)] for L in lens], np.int32).reshape(-1)
    q = rng.standard_normal((len(q_to_req), Hq, D)).astype(np.float32)
    scale = W.default_sm_scale(D)
    got = hkv.decode_attention(f, torch.from_numpy(q).to(DEV), cache, torch.from_numpy(bt).to(DEV),
                               torch.from_numpy(q_to_req).to(DEV),
                               torch.from_numpy(q_to_klen).to(DEV), int(q_to_klen.max()), qps,
                               scale).cpu().numpy()
    ref = O.attention(fo, q, ref_cache, bt, q_to_req, q_to_klen, scale)
    _assert_close(got, ref, f"{dtype} D={D} page {P}")


@pytest.mark.parametrize("dtype,D,R,Hq,Hkv,qps,num_pages", [("q4_0", 256, 0, 16, 2, 1, 600_000),
                                                            ("q4_0", 256, 0, 16, 2, 4, 600_000),
                                                            ("q8_0", 256, 0, 16, 2, 1, 300_000),
                                                            ("octave_k3v3_compact", 256, 64, 32, 4, 4, 350_000),
                                                            ("octave_k3v4", 128, 64, 32, 8, 1, 300_000)])
def test_decode_cache_beyond_4gib(dtype, D, R, Hq, Hkv, qps, num_pages):
    """A cache of more than 4 GiB with the sequences' pages near its end, so
    every slot address needs 64 bits.  The oracle sees the same pages at low
    ids in a small cache of its own (nothing it uses comes from the GPU)."""
    P = 16
    lens = [300, 1500]
    rng = np.random.default_rng(D + Hkv)
    T = sum(lens)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    pages = [(L + P - 1) // P for L in lens]
    n_used = sum(pages)
    low = rng.permutation(n_used)                    # the oracle's page ids
    high = (num_pages - n_used - 7) + low            # the GPU's page ids, near the end
    bt_low = np.zeros((len(lens), max(pages)), np.int32)
    sm_low = np.empty(T, np.int64)
    off = t0 = 0
    for b, L in enumerate(lens):
        bt_low[b, :pages[b]] = low[off:off + pages[b]]
        off += pages[b]
        pos = np.arange(L)
        sm_low[t0:t0 + L] = bt_low[b, pos // P].astype(np.int64) * P + pos % P
        t0 += L
    shift = num_pages - n_used - 7
    bt_high = np.where(np.arange(bt_low.shape[1])[None, :] < np.array(pages)[:, None],
                       bt_low + shift, 0).astype(np.int32)
    sm_high = sm_low + shift * P
    f = hkv.format_init(dtype, D, R, P)
    fo = O.format_init(dtype, D, R)
    cache = hkv.new_cache(f, num_pages, Hkv, DEV)
    assert cache.numel() > (1 << 32)
    hkv.quantize_append(f, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.from_numpy(sm_high).to(DEV), cache)
    slots = O.quantize(fo, k.astype(np.float32), v.astype(np.float32))
    ref_cache = np.zeros((n_used, Hkv, P, f.slot_bytes), np.uint8)
    ref_cache[sm_low // P, :, sm_low % P] = slots
    got_pages = cache[torch.from_numpy(np.arange(n_used) + shift).to(DEV)].cpu().numpy()
    assert np.array_equal(got_pages, ref_cache)
    q_to_req = np.arange(len(lens), dtype=np.int32).repeat(qps)
    q_to_klen = np.array([[L - qps + 1 + j for j in range(qps)] for L in lens], np.int32).reshape(-1)
    q = rng.standard_normal((len(q_to_req), Hq, D)).astype(np.float32)
    scale = W.default_sm_scale(D)
    got = hkv.decode_attention(f, torch.from_numpy(q).to(DEV), cache,
                               torch.from_numpy(bt_high).to(DEV),
                               torch.from_numpy(q_to_req).to(DEV),
                               torch.from_numpy(q_to_klen).to(DEV), int(q_to_klen.max()), qps,
                               scale).cpu().numpy()
    ref = O.attention(fo, q, ref_cache, bt_low, q_to_req, q_to_klen, scale)
    _assert_close(got, ref, f"{dtype} cache of {cache.numel() / 2**30:.1f} GiB")
    del cache
    torch.cuda.empty_cache()
