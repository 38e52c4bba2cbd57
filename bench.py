#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

A step is one pass of the whole path over one batch: quantize-append of the
new tokens of every sequence (FWHT + quantize + pack into the paged cache),
then decode attention of the query tokens over the quantized cache (query
rotation, in-register dequantization inside an online softmax, split merge,
output rotated back).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is packed-KV bytes the decode reads per step
divided by the step time (GB/s); `roofline` rates the decode call (split
kernel + merge kernel) against the 8 TB/s HBM peak; `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config 3]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = ("decode-attn packed-KV GB/s (% HBM peak) at 128K ctx; "
          "quantize-append tokens/s")
INFINITY_CACHE_BYTES = 256 << 20
WARM_SECONDS = 0.3
DIST_BLOCKS = 20    # blocks of 10 decode calls for the median / p10 / p90


def arith_label(cfg) -> str:
    """What the decode kernel this workload runs on computes in: the matrix
    cores' operand types (the query enters as exact multi-part splits: three
    int8 planes, or an fp16 leading part and residual), then fp32 softmax and
    accumulation.  A query window wider than one kernel pass runs as
    sub-groups of whole queries on the same kernel."""
    group = cfg.num_q_heads // cfg.num_kv_heads
    rows = group * cfg.n_q
    i8 = "i8 MFMA scores (3 query planes) + f16 MFMA P.V, f32 softmax/accumulate"
    f16 = "f16 MFMA scores (lead + residual query) and P.V, f32 softmax/accumulate"
    if cfg.cache_dtype == "q4_0" and cfg.head_size == 256 and group <= 8:
        return f16
    if cfg.cache_dtype == "q8_0" and cfg.head_size == 256 and group <= 8:
        return i8
    if cfg.cache_dtype == "octave_k3v3_compact" and rows > 16 and group <= 32:
        return f16
    if cfg.cache_dtype.startswith("octave") and group <= 16:
        return i8
    return "f32"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--deterministic", action="store_true",
                   help="decode in the bitwise-reproducible mode (fixed unit order)")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--copies", type=int, default=0,
                   help="cache copies rotated between steps (0: enough to exceed the "
                        "256 MB Infinity Cache twice)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="replay the step from HIP graphs (one per cache copy) instead of "
                        "launching it from Python")
    p.add_argument("--cpu-threads", type=int, default=0)
    p.add_argument("--profile", action="store_true",
                   help="short run for a profiler: no CPU baseline")
    p.add_argument("--op", choices=["decode", "hadamard"], default="decode",
                   help="decode: the quantize-append + decode step (default); hadamard: the "
                        "standalone blockwise rotation on an activation-shaped tensor")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of 256 MiB (calibrates the HBM "
                        "byte counters of rocprofv3)")
    return p.parse_args()


def copy_calibration():
    import torch
    n = (256 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}))


# Sources of the decode kernels a cache format runs on: the format's
# split-K kernel, the planner, merge and generic kernel, and their headers.
DECODE_SOURCES = {
    "q4_0": ("hkv_decode_q4.hip", "hkv_decode_q4w.hip"),
    "q8_0": ("hkv_decode_q8.hip",),
    "octave": ("hkv_decode_oct.hip",),
}
SHARED_SOURCES = ("hkv_decode.hip", "hkv_decode_common.h", "hkv_device.h", "hkv_internal.h")


def source_hash(cache_dtype=None) -> str:
    """Hash of the kernel sources: all of csrc, or only those the decode of
    `cache_dtype` runs on."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "decode_attention_amd", "csrc")
    names = sorted(os.listdir(d))
    if cache_dtype is not None:
        own = DECODE_SOURCES["octave" if cache_dtype.startswith("octave") else cache_dtype]
        names = sorted(own + SHARED_SOURCES)
    for n in names:
        with open(os.path.join(d, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, cache_dtype: str):
    """HBM traffic per decode call from committed rocprofv3 counter runs, if
    they were taken on the current sources of this format's decode kernels."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_source_hash") != source_hash(cache_dtype):
        return None
    return t


CPU_WORKERS = 16   # host threads a GPU job may use on the benchmark machines


def gpu_info(torch) -> dict:
    """The device the run used: name, architecture, compute units, and its
    peak engine clock (hipDeviceGetAttribute, hipDeviceAttributeClockRate =
    5 in hip_runtime_api.h of this ROCm)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:
            info["peak_clock_mhz"] = v.value // 1000
    except OSError:
        pass
    return info


def host_cpus() -> int:
    """CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, w, threads: int, scale: float, min_seconds: float = 10.0,
                 outputs: list = None):
    """The oracle, as it is, on the host cores: quantize the appended rows,
    then the fp64 attention of every query.  Attention is independent per
    (query, KV head), and within one such sub-problem per token range: the
    oracle runs on each page-aligned range (a shifted block-table row and the
    range's length) and the ranges merge with their log-sum-exp weights.
    Every (query, KV head) is cut into as many ranges as it takes to give
    each thread at least one, and the threads take the pieces in turn.
    If outputs is a list, the merged attention of the last pass, shaped
    (queries, Hq, D), is appended to it."""
    import oracle as O
    from decode_attention_amd import workloads as W

    fo = O.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim)
    S = fo.slot_bytes
    P = cfg.page_size
    Hkv, G = cfg.num_kv_heads, cfg.num_q_heads // cfg.num_kv_heads
    # Oracle cache of the whole workload (setup, not timed), built in parallel.
    T = w.key.shape[0]
    slots = np.zeros((T, Hkv, S), np.uint8)
    chunks = np.array_split(np.arange(T), max(1, threads))

    def qwork(ix):
        if len(ix):
            slots[ix[0]:ix[-1] + 1] = O.quantize(fo, w.key[ix[0]:ix[-1] + 1].astype(np.float32),
                                                 w.value[ix[0]:ix[-1] + 1].astype(np.float32))
    th = [threading.Thread(target=qwork, args=(c,)) for c in chunks]
    [t.start() for t in th]
    [t.join() for t in th]
    # One cache per KV head, (pages, 1, page_size, S).
    head_cache = []
    for h in range(Hkv):
        c = np.zeros((w.num_pages, 1, P, S), np.uint8)
        c[w.slot_mapping // P, 0, w.slot_mapping % P] = slots[:, h]
        head_cache.append(c)
    rows = w.append_rows()
    qf = w.query.astype(np.float32)
    kf = w.key[rows].astype(np.float32)
    vf = w.value[rows].astype(np.float32)
    subs = [(i, h) for i in range(len(w.q_to_req)) for h in range(Hkv)]
    n_ranges = max(1, -(-threads // len(subs)))
    pieces = []                                   # (sub index, first page, tokens)
    for k, (i, h) in enumerate(subs):
        L = int(w.q_to_klen[i])
        pages = -(-L // P)
        cuts = np.unique(np.linspace(0, pages, n_ranges + 1).round().astype(int))
        for p0, p1 in zip(cuts[:-1], cuts[1:]):
            pieces.append((k, int(p0), min(L, int(p1) * P) - int(p0) * P))
    n_threads = max(1, min(threads, len(pieces)))
    results = [None] * len(pieces)

    def awork(j0):
        for j in range(j0, len(pieces), n_threads):
            k, p0, n = pieces[j]
            i, h = subs[k]
            r = int(w.q_to_req[i])
            results[j] = O.attention_lse(
                fo, np.ascontiguousarray(qf[i:i + 1, h * G:(h + 1) * G]), head_cache[h],
                np.ascontiguousarray(w.block_table[r:r + 1, p0:]), np.zeros(1, np.int32),
                np.array([n], np.int32), scale)

    def merge():
        out = np.zeros((len(subs), G, cfg.head_size))
        lse = np.full((len(subs), G), -np.inf)
        for (k, _, _), (_, s) in zip(pieces, results):
            lse[k] = np.logaddexp(lse[k], s[0])
        for (k, _, _), (o, s) in zip(pieces, results):
            out[k] += np.exp(s[0] - lse[k])[:, None] * o[0]
        return out
    # One pass = the whole step; passes repeat until min_seconds have elapsed.
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.quantize(fo, kf, vf)
        th = [threading.Thread(target=awork, args=(j,)) for j in range(n_threads)]
        [t.start() for t in th]
        [t.join() for t in th]
        merged = merge()
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    total = time.perf_counter() - t0
    dt = total / reps
    if outputs is not None:
        outputs.append(merged.reshape(len(w.q_to_req), Hkv * G, cfg.head_size))
    nbytes = W.packed_bytes(w, S)
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": n_threads,
            "kind": "oracle", "host_cpus": host_cpus(), "cpu_model": cpu_model(),
            "sample": (f"the full step of the workload, {reps} passes: quantize of {len(rows)} "
                       f"appended token rows and fp64 attention of {len(w.q_to_req)} queries over "
                       f"{nbytes} packed-KV bytes, as {len(pieces)} oracle calls over "
                       f"page-aligned token ranges of the {len(subs)} (query, KV head) pairs, "
                       f"merged by log-sum-exp; {dt:.3f} s per pass, {total:.1f} s wall on "
                       f"{n_threads} threads ({host_cpus()} host CPUs available)")}


def stream_read_gbs(torch, dev, nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Read rate of the streaming-read probe (libhkv_probe.so, a measurement
    aid built beside the library) over nbytes, after a short warm-up."""
    import ctypes
    path = os.path.join(ROOT, "decode_attention_amd", "libhkv_probe.so")
    L = ctypes.CDLL(path)
    L.hkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]
    L.hkv_probe_stream_read.restype = ctypes.c_int
    blocks = 8192
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    run = lambda: L.hkv_probe_stream_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream)
    for _ in range(3):
        if run() != 0:
            raise RuntimeError("stream-read probe launch failed")
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    return nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9


HAD_ROWS, HAD_N, HAD_BLOCK = 16384, 4096, 128


def hadamard_bench(args):
    """One step = hkv_hadamard (block 128, sign pattern, rotate) over a
    (16384, 4096) f16 activation tensor into fp32."""
    import torch
    from decode_attention_amd import hkv
    rng = np.random.default_rng(4242)
    x = rng.standard_normal((HAD_ROWS, HAD_N), dtype=np.float32).astype(np.float16)
    bits = rng.integers(-2**31, 2**31, HAD_N // 32, dtype=np.int64).astype(np.int32)
    dev = torch.device("cuda:0")
    xt, bt = torch.from_numpy(x).to(dev), torch.from_numpy(bits).to(dev)
    y = torch.empty((HAD_ROWS, HAD_N), dtype=torch.float32, device=dev)
    step = lambda: hkv.hadamard(xt, HAD_BLOCK, bt, False, out=y)
    warm = 0.0 if args.profile else WARM_SECONDS
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm:
            break
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    nbytes = HAD_ROWS * HAD_N * (2 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    rec = {"metric": "hadamard rotation GB/s (f16 in + fp32 out)", "value": round(gbs, 3),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"hadamard_b{HAD_BLOCK}_{HAD_ROWS}x{HAD_N}", "rows": HAD_ROWS,
                      "n": HAD_N, "block": HAD_BLOCK, "in": "f16", "out": "f32", "signs": True},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 3), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "hkv_hadamard", "bytes_per_call": nbytes,
                        "us_per_call": round(ms * 1e3, 3)}}
    if not args.no_cpu_baseline and not args.profile:
        import oracle as O
        n_rows, reps = 256, 0
        xs = x[:n_rows].astype(np.float32)
        s = (1 - 2 * ((bits.view(np.uint32)[np.arange(HAD_N) // 32] >> (np.arange(HAD_N) % 32)) & 1)
             ).astype(np.float32)
        t0 = time.perf_counter()
        while True:
            O.fwht(xs * s, HAD_BLOCK)
            reps += 1
            if time.perf_counter() - t0 >= 10.0:
                break
        dt = (time.perf_counter() - t0) / reps
        rec["cpu_baseline"] = {"value": round(n_rows * HAD_N * 6 / dt / 1e9, 6), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{n_rows} of the {HAD_ROWS} rows, {reps} passes, "
                                         f"{dt * 1e3:.1f} ms per pass, one thread"}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not built).", file=sys.stderr)
        sys.exit(2)

    if args.op == "hadamard":
        hadamard_bench(args)
        return

    import torch

    from decode_attention_amd import hkv
    from decode_attention_amd import workloads as W

    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[args.config]
    w = W.make_workload(cfg)
    f = hkv.format_init(cfg.cache_dtype, cfg.head_size, cfg.rope_dim, cfg.page_size)
    scale = W.default_sm_scale(cfg.head_size)
    B, Hkv, Hq, D = len(w.lengths), cfg.num_kv_heads, cfg.num_q_heads, cfg.head_size

    key = torch.from_numpy(w.key).to(dev)
    value = torch.from_numpy(w.value).to(dev)
    slot_mapping = torch.from_numpy(w.slot_mapping).to(dev)
    rows = torch.from_numpy(w.append_rows()).to(dev)
    new_k = key[rows].contiguous()
    new_v = value[rows].contiguous()
    new_sm = slot_mapping[rows].contiguous()
    query = torch.from_numpy(w.query).to(dev)
    block_table = torch.from_numpy(w.block_table).to(dev)
    q_to_req = torch.from_numpy(w.q_to_req).to(dev)
    q_to_klen = torch.from_numpy(w.q_to_klen).to(dev)
    out = torch.empty((len(w.q_to_req), Hq, D), dtype=torch.float32, device=dev)
    ws_bytes = hkv.decode_workspace_bytes(f, len(w.q_to_req), Hq, Hkv, w.max_klen, cfg.n_q)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    cache_bytes = w.num_pages * Hkv * cfg.page_size * f.slot_bytes
    copies = args.copies or max(2, -(-2 * INFINITY_CACHE_BYTES // cache_bytes))
    caches = [hkv.new_cache(f, w.num_pages, Hkv, dev) for _ in range(copies)]

    # Build every cache copy (quantize-append of all tokens; untimed here).
    for c in caches:
        hkv.quantize_append(f, key, value, slot_mapping, c)
    torch.cuda.synchronize()
    total_tokens = key.shape[0]

    def step(i):
        c = caches[i % copies]
        hkv.quantize_append(f, new_k, new_v, new_sm, c)
        hkv.decode_attention(f, query, c, block_table, q_to_req, q_to_klen, w.max_klen, cfg.n_q,
                             scale, out=out, workspace=workspace, deterministic=args.deterministic)

    def decode_call(i):
        hkv.decode_attention(f, query, caches[i % copies], block_table, q_to_req, q_to_klen,
                             w.max_klen, cfg.n_q, scale, out=out, workspace=workspace,
                             deterministic=args.deterministic)

    run_step, run_decode = step, decode_call
    if args.graph:
        # One HIP graph per cache copy for the step and for the decode call
        # alone; each replay is checked against the eager call (to the last
        # bits: the split kernels' wave-level work queue can change how a
        # split's tokens are grouped between calls).
        for i in range(copies):
            step(i)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g_step, g_dec = [], []
        for i in range(copies):
            for fn, lst in ((step, g_step), (decode_call, g_dec)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn(i)
                lst.append(g)
        torch.cuda.synchronize()
        for i in range(copies):
            decode_call(i)
            ref = out.clone()
            for g in (g_dec[i], g_step[i]):
                out.fill_(float("nan"))
                g.replay()
                torch.cuda.synchronize()
                err = (out - ref).abs().max().item()
                if not err <= 1e-4 * (1.0 + ref.abs().max().item()):
                    raise RuntimeError(f"graph replay differs from the eager call ({err})")
        run_step = lambda i: g_step[i % copies].replay()
        run_decode = lambda i: g_dec[i % copies].replay()

    # Clock warm-up: the GPU takes several milliseconds of load to reach its
    # steady clocks, so untimed steps run for WARM_SECONDS first (not under
    # --profile, where every dispatch is recorded); then the --warmup steps,
    # then exactly --steps timed steps.
    warm = 0.0 if args.profile else WARM_SECONDS
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < warm:
        for _ in range(10):
            run_step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        run_step(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # Average duration of one decode call (its split-K kernel and merge
    # kernel) on the stream it runs on (torch's current stream): one event
    # pair around back-to-back calls.  The append's device cost is the rest
    # of the step.
    n_t = max(args.steps, 20)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for i in range(n_t):
        run_decode(i)
    d1.record()
    torch.cuda.synchronize()
    decode_ms = d0.elapsed_time(d1) / n_t
    append_ms = max(ms_per_step - decode_ms, 0.0)

    # Spread of the decode call: blocks of 10 calls in one back-to-back run,
    # an event between blocks (per-call events would add their own gaps, and
    # a synchronisation per block would let the clocks drop); median, p10 and
    # p90 of the block averages.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(DIST_BLOCKS + 1)]
    evs[0].record()
    for b in range(DIST_BLOCKS):
        for i in range(10):
            run_decode(10 * b + i)
        evs[b + 1].record()
    torch.cuda.synchronize()
    blk = [evs[b].elapsed_time(evs[b + 1]) / 10 * 1e3 for b in range(DIST_BLOCKS)]
    dist = {"median": round(float(np.median(blk)), 3), "p10": round(float(np.percentile(blk, 10)), 3),
            "p90": round(float(np.percentile(blk, 90)), 3), "blocks": DIST_BLOCKS,
            "calls_per_block": 10}

    # Achievable read bandwidth beside the 8 TB/s peak: a plain streaming-read
    # probe (nontemporal 16-byte loads, eight in flight per thread) over 1 GiB.
    read_gbs = stream_read_gbs(torch, dev)

    # Bulk quantize-append of every token into every copy (same bytes again),
    # timed while the clocks are up.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for c in caches:
        hkv.quantize_append(f, key, value, slot_mapping, c)
    e1.record()
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1) / copies

    packed = W.packed_bytes(w, f.slot_bytes)
    bulk_gbs = (2 * total_tokens * Hkv * D * w.key.itemsize +
                total_tokens * Hkv * f.slot_bytes) / (bulk_ms * 1e-3) / 1e9
    value = packed / (ms_per_step * 1e-3) / 1e9
    achieved = packed / (decode_ms * 1e-3) / 1e9
    traffic = load_traffic(cfg.name, cfg.cache_dtype)
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith_label(cfg),
        "data": "synthetic",
        "config": {"workload": cfg.name, "cache_dtype": cfg.cache_dtype, "batch": B,
                   "context": int(w.max_klen), "head_size": D, "q_heads": Hq, "kv_heads": Hkv,
                   "page_size": cfg.page_size, "queries_per_seq": cfg.n_q,
                   "append_tokens_per_seq": cfg.n_append, "cache_copies_rotated": copies,
                   "launch": "hip_graph" if args.graph else "eager",
                   "deterministic": bool(args.deterministic)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_call"],
                     "kernel": "hkv_decode_attention (split-K kernel + merge kernel)",
                     "bytes_per_call": packed, "us_per_call": round(decode_ms * 1e3, 3)},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "achievable_read": {"gbs": round(read_gbs, 1),
                            "probe": "nontemporal 16-byte streaming reads of 1 GiB, "
                                     "8192 x 256 threads, 8 loads in flight each",
                            "decode_frac": round(achieved / read_gbs, 4)},
        "decode_us_dist": dist,
        "append_us": round(append_ms * 1e3, 3),
        "append_tokens_per_s": (round(len(rows) / (append_ms * 1e-3), 1)
                                if append_ms > 0 else None),
        "bulk_quantize_tokens_per_s": round(total_tokens / (bulk_ms * 1e-3), 1),
        "bulk_quantize_gbps": round(bulk_gbs, 3),
        "bulk_quantize_hbm_frac": round(bulk_gbs / HBM_PEAK_GBS, 4),
        "gpu": gpu_info(torch),
    }
    if not args.no_cpu_baseline and not args.profile:
        threads = args.cpu_threads or min(CPU_WORKERS, host_cpus())
        rec["cpu_baseline"] = cpu_baseline(cfg, w, threads, scale)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
