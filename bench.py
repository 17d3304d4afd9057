#!/usr/bin/env python3
"""Benchmark of the ring all-reduce on one MI355X.

Headline workload (one "step" = one all-reduce): N = 8 simulated ranks, each a separate HBM buffer of
134,217,728 bf16 gradients (256 MiB), values bf16(z * 1e-3) with z ~ N(0, 1); sum in fp32 in ring order
(chunk c folded from rank c), divided by 8, rounded once to bf16 and written to all 8 rank buffers.

Reported: busbw (the JSON "value") = algbw * 2(N-1)/N with algbw = S / t and S the per-rank bytes
(astro-wiki "AllReduce", section 通信量分析: each GPU sends 2(N-1)/N of its data); achieved HBM bandwidth
of the kernel = algorithmic bytes (N reads + N writes of S) / kernel time, against the 8 TB/s peak; the
CPU oracle timed on this host on the same inputs; and, beside the headline, every other step of the path
(rank-order and halving-doubling one-pass kernels, the round-per-launch schedules, bucketing with 25 MiB
buckets over 300 tensors, the fp8 codec and compressed ring, the owner's epilogue on its own) with its own
algorithmic-bytes roofline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--fp8-only] [--copy-calibration]
                       [--ring-bytes-per-rank S] [--per-rank-offsets-only] [--sweep OUT.jsonl]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "busbw & achieved HBM GB/s (% of peak) vs message size, N=8 ranks, fp32/bf16"
PEAK_HBM_GBPS = 8000.0
N_RANKS = 8
COUNT = 134_217_728
GB = 1e9


def _sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "all_reduce_reduction_ring_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _load_traffic(kernel_key, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on this exact
    kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("sources_sha256") != _sources_digest(sources):
        return None
    return ent.get("hbm_bytes_per_launch")


class Timer:
    """Per-call kernel time with HIP events recorded on the stream the library launches on."""

    def __init__(self, torch):
        self.torch = torch
        self.ms = []

    def run(self, fn, reps):
        torch = self.torch
        stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        self.ms = [a.elapsed_time(b) for a, b in evs]
        return self.ms


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _gen_parallel(fn, items, workers=16):
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def _upload(torch, arrays, dtype, dev):
    out = []
    for a in arrays:
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        out.append(t.to(dev, non_blocking=False).view(dtype))
    return out


def stats_us(ms):
    a = np.array(ms) * 1e3
    return {"p50": float(np.percentile(a, 50)), "p95": float(np.percentile(a, 95)),
            "p99": float(np.percentile(a, 99)), "mean": float(a.mean())}


def bus_factor(n):
    return 2.0 * (n - 1) / n


def headline(torch, ar, inputs, args, dev):
    """Generate the 8 rank buffers, warm up, time exactly K steps."""
    log("generating the headline inputs")
    host = _gen_parallel(lambda r: inputs.normal_bf16((2, r), COUNT), range(N_RANKS))
    ins = _upload(torch, host, torch.bfloat16, dev)
    log("timing the headline")
    outs = [torch.empty_like(t) for t in ins]
    step = lambda: ar.ar_allreduce(ins, outs, ar.AR_AVG, ar.AR_ALGO_RING)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    timer.run(step, args.steps)  # synchronises at the end
    wall = time.perf_counter() - t0
    return host, ins, outs, timer.ms, wall


def copy_ceiling(torch, ins, outs, reps=10):
    """A plain device copy moving the same bytes (N*S read + N*S written)."""
    src = torch.cat([t.view(-1) for t in ins])
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = Timer(torch).run(lambda: dst.copy_(src), reps)
    nbytes = 2 * src.numel() * src.element_size()
    del src, dst
    torch.cuda.empty_cache()  # later rank buffers must not be carved out of these segments (see sweep_points)
    return nbytes / (np.mean(ms) * 1e-3) / GB


def write_ceiling(torch, ins, reps=10):
    """Context for the roofline on this GPU: a plain write (torch fill_) of the headline's N*S bytes, median of
    10 after warm-up calls. Beside the copy above it brackets the all-reduce, which mixes reads and writes half
    and half."""
    dst = torch.empty(sum(t.numel() for t in ins) * ins[0].element_size() // 4, dtype=torch.float32,
                      device=ins[0].device)
    write = lambda: dst.fill_(0.5)
    for _ in range(3):  # first calls load the kernel
        write()
    ms = Timer(torch).run(write, reps)
    nbytes = dst.numel() * dst.element_size()
    del dst
    torch.cuda.empty_cache()
    return nbytes / (np.median(ms) * 1e-3) / GB


def fold_halves(torch, ins, outs, reps=10):
    """The headline fold's two halves on their own, with its launch shape and access order (libar_ceiling.so, the
    benchmark's measurement kernels): reading the N rank buffers with nothing written, and writing N buffers with
    nothing read, each N*S bytes; with the fold's large launch shape (the headline's) and its small one; and the
    fastest plain write pattern measured for these bytes (one-shot blocks, 16 KiB of one buffer each). Median of 10
    after warm-up calls. Returns {name: GB/s}, or None when the measurement library is not built."""
    path = os.path.join(ROOT, "all_reduce_reduction_ring_amd", "libar_ceiling.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.arc_read.argtypes = [vp, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint32, vp, ctypes.c_int, vp]
    L.arc_write.argtypes = [vp, ctypes.c_int, ctypes.c_size_t, ctypes.c_int, vp]
    n = len(ins)
    nbytes = ins[0].numel() * ins[0].element_size()
    rin = (ctypes.c_void_p * n)(*[t.data_ptr() for t in ins])
    rout = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    sink = torch.zeros(1, dtype=torch.int32, device=ins[0].device)
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"libar_ceiling call failed ({rc})")

    calls = {"read_fold_large": lambda: check(L.arc_read(rin, n, nbytes, 0x9E3779B9, sink.data_ptr(), 1, stream())),
             "read_fold_small": lambda: check(L.arc_read(rin, n, nbytes, 0x9E3779B9, sink.data_ptr(), 0, stream())),
             "write_fold_large": lambda: check(L.arc_write(rout, n, nbytes, 1, stream())),
             "write_fold_small": lambda: check(L.arc_write(rout, n, nbytes, 0, stream())),
             "write_blocks": lambda: check(L.arc_write(rout, n, nbytes, 2, stream()))}
    rates = {}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        ms = Timer(torch).run(fn, reps)
        rates[name] = n * nbytes / (np.median(ms) * 1e-3) / GB
    return rates


def mix_bound(read_gbps, write_gbps, read_bytes, write_bytes):
    """The rate a kernel moving read_bytes and write_bytes could reach if its reads and writes cost what they cost
    alone (the plain read and plain write ceilings above) and mixing them cost nothing: bytes / (R/r + W/w)."""
    return (read_bytes + write_bytes) / (read_bytes / read_gbps + write_bytes / write_gbps)


def cpu_baseline(host, budget_s=10.0, max_reps=5):
    """The oracle's literal ring on the headline inputs, repeated until ~budget_s of CPU time."""
    import oracle as _o
    reps, t_total = 0, 0.0
    while reps < max_reps and (t_total < budget_s or reps == 0):
        t0 = time.perf_counter()
        _o.ring_allreduce(host, _o.BF16, _o.AVG)
        t_total += time.perf_counter() - t0
        reps += 1
    t = t_total / reps
    S = COUNT * 2
    return {"value": S / t / GB * bus_factor(N_RANKS), "unit": "GB/s", "cores": _o.num_threads(), "kind": "oracle",
            "sample": f"the full headline workload (8 ranks x {COUNT} bf16, avg), literal ring rounds in C, "
                      f"{reps} repetition(s), {t:.2f} s each"}


def host_info(host, frac=8):
    """The host the oracle ran on, and the oracle on one thread over a 1/frac prefix of every headline rank."""
    import oracle as _o
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    m = COUNT // frac
    sample = [np.ascontiguousarray(h[:m]) for h in host]
    default_threads = _o.num_threads()
    _o.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        _o.ring_allreduce(sample, _o.BF16, _o.AVG)
        t = time.perf_counter() - t0
    finally:
        _o.set_num_threads(0)
    S = m * 2
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)),
            "oracle_threads": default_threads,
            "oracle_one_thread": {"s": t, "busbw_GBps": S / t / GB * bus_factor(N_RANKS),
                                  "sample": f"first {m} elements of each of the {N_RANKS} headline ranks"}}


def ring_bytes(n, count, es):
    return 2 * n * count * es


def stepwise_ring_bytes(n, count, es, acc):
    """Reduce-scatter round s: every rank reads the incoming partial and its own chunk and writes the new
    partial (inputs at s = 0, outputs at the last round); all-gather: read + write a chunk per rank."""
    chunk = count / n
    total = 0.0
    for s in range(n - 1):
        msg = es if s == 0 else acc
        dst = es if s == n - 2 else acc
        total += n * chunk * (msg + es + dst)
    total += (n - 1) * n * chunk * 2 * es
    return total


def stepwise_rhd_bytes(n, count, es, acc):
    k = int(np.log2(n))
    total = 0.0
    for j in range(k):
        part = count / 2 ** (j + 1)
        rd = es if j == 0 else acc
        wr = es if j == k - 1 else acc
        total += n * part * (2 * rd + wr)
    for j in range(k):
        total += n * (count / 2 ** (j + 1)) * 2 * es
    return total


def stepwise_tree_bytes(n, count, es, acc):
    """Binomial levels: each receiving pair reads the sender's value and its own and writes a partial (inputs
    where nothing has been received yet, the output at the last level); broadcast: read + write per pair."""
    k = int(np.ceil(np.log2(n)))
    total = 0.0
    for j in range(k):
        for i in range(0, n, 2 << j):
            src = i + (1 << j)
            if src >= n:
                continue
            msg = es if (j == 0 or src + 1 >= n) else acc
            own = es if j == 0 else acc
            wr = es if j == k - 1 else acc
            total += count * (msg + own + wr)
    for j in range(k):
        total += sum(1 for i in range(0, n, 2 << j) if i + (1 << j) < n) * count * 2 * es
    return total


def row_entry(name, ms, alg_bytes, S, n, extra=None, factor=None):
    """factor: busbw / algbw; 2(N-1)/N for an all-reduce (default), (N-1)/N for reduce-scatter and all-gather."""
    t = float(np.mean(ms)) * 1e-3
    f = bus_factor(n) if factor is None else factor
    e = {"us": stats_us(ms), "algbw_GBps": S / t / GB, "busbw_GBps": S / t / GB * f,
         "hbm_GBps": alg_bytes / t / GB, "frac_of_peak": alg_bytes / t / GB / PEAK_HBM_GBPS,
         "alg_bytes": alg_bytes}
    if extra:
        e.update(extra)
    return e


def oracle_time(fn, *args):
    """Wall time of one call of an oracle routine (its OpenMP threads on this host's cores)."""
    t0 = time.perf_counter()
    fn(*args)
    return time.perf_counter() - t0


def cpu_row(t, S, n, sample):
    """The oracle's rate for a row, in the row's own units (algbw and busbw from S per-rank bytes)."""
    import oracle as _o
    return {"s": t, "algbw_GBps": S / t / GB, "busbw_GBps": S / t / GB * bus_factor(n), "cores": _o.num_threads(),
            "sample": sample}


def other_rows(torch, ar, inputs, ins, outs, dev, reps, host):
    """Every other step of the path, timed beside the headline, each with the oracle timed on this host."""
    import oracle as _o
    rows = {}
    S = COUNT * 2
    timer = Timer(torch)
    log("timing the other rows")
    for name, algo, ofn in (("fused_reduce_broadcast", ar.AR_ALGO_FUSED, _o.fused_allreduce),
                            ("rhd_tree", ar.AR_ALGO_RHD, _o.rhd_allreduce),
                            ("binomial_tree", ar.AR_ALGO_TREE, _o.tree_allreduce)):
        fn = lambda: ar.ar_allreduce(ins, outs, ar.AR_AVG, algo)
        fn()
        rows[name] = row_entry(name, timer.run(fn, reps), ring_bytes(N_RANKS, COUNT, 2), S, N_RANKS)
        rows[name]["cpu_oracle"] = cpu_row(oracle_time(ofn, host, _o.BF16, _o.AVG), S, N_RANKS,
                                           "the full headline workload, one call")
    # the ring on views that do not start on a 16-byte boundary: the same offset in every buffer (a head of
    # elements, then 256-byte aligned slots), and rank r at an offset of r elements (element by element)
    # (bf16 at even per-rank offsets: 4-byte aligned, so 16-byte slots from element 0 that straddle cache lines)
    for name, offs in (("ring_common_offset", [1] * N_RANKS), ("ring_per_rank_offsets", list(range(N_RANKS))),
                       ("ring_per_rank_even_offsets", [2 * r for r in range(N_RANKS)])):
        pad = max(offs)
        vin = [torch.empty(COUNT + pad, dtype=torch.bfloat16, device=dev)[o:o + COUNT] for o in offs]
        vout = [torch.empty(COUNT + pad, dtype=torch.bfloat16, device=dev)[o:o + COUNT] for o in offs]
        for v, t in zip(vin, ins):
            v.copy_(t)
        fn = lambda: ar.ar_allreduce(vin, vout, ar.AR_AVG, ar.AR_ALGO_RING)
        fn()
        rows[name] = row_entry(name, timer.run(fn, reps), ring_bytes(N_RANKS, COUNT, 2), S, N_RANKS,
                               {"offsets_elements": offs})
        del vin, vout, fn
    torch.cuda.empty_cache()
    # the two halves on their own: reduce-scatter (N reads + 1 write per element) and all-gather (1 read + N writes)
    lo = ar.chunk_bounds(COUNT, N_RANKS)
    parts = [torch.empty(lo[c + 1] - lo[c], dtype=torch.bfloat16, device=dev) for c in range(N_RANKS)]
    fn = lambda: ar.ar_reduce_scatter(ins, parts, ar.AR_AVG)
    fn()
    rows["reduce_scatter"] = row_entry("reduce_scatter", timer.run(fn, reps), (N_RANKS + 1) * S, S, N_RANKS,
                                       factor=(N_RANKS - 1) / N_RANKS)
    rows["reduce_scatter"]["cpu_oracle"] = cpu_row(oracle_time(_o.reduce_scatter, host, _o.BF16, _o.AVG), S, N_RANKS,
                                                   "the full headline workload, one call")
    fn = lambda: ar.ar_all_gather(parts, outs)
    fn()
    rows["all_gather"] = row_entry("all_gather", timer.run(fn, reps), (N_RANKS + 1) * S, S, N_RANKS,
                                   factor=(N_RANKS - 1) / N_RANKS)
    del parts
    # the owner's epilogue on its own (ar_epilogue): one rank's count of fp32 partials -> avg by N -> bf16, 4 bytes
    # read and 2 written per element; no link traffic, so no busbw
    acc = ins[0].float()
    fn = lambda: ar.ar_epilogue(acc, outs[0], ar.AR_AVG, N_RANKS)
    fn()
    rows["epilogue"] = row_entry("epilogue", timer.run(fn, reps), 6 * COUNT, S, 1, {"count": COUNT}, factor=0.0)
    n_s = COUNT // N_RANKS
    acc_h = _o.bf16_to_f32(host[0][:n_s])
    rows["epilogue"]["cpu_oracle"] = cpu_row(oracle_time(_o.epilogue, acc_h, _o.BF16, _o.AVG, N_RANKS), n_s * 2, 1,
                                             f"the first {n_s:,} fp32 partials of one rank, one call")
    del acc, acc_h
    ws = torch.empty(ar.ar_allreduce_workspace_size(N_RANKS, COUNT, ar.AR_BF16, ar.AR_AVG, ar.AR_ALGO_RING_STEPWISE),
                     dtype=torch.uint8, device=dev)
    levels = int(np.ceil(np.log2(N_RANKS)))
    for name, algo, fb, launches in (
            ("ring_stepwise", ar.AR_ALGO_RING_STEPWISE, stepwise_ring_bytes, 2 * (N_RANKS - 1)),
            ("rhd_stepwise", ar.AR_ALGO_RHD_STEPWISE, stepwise_rhd_bytes, 2 * levels),
            ("tree_stepwise", ar.AR_ALGO_TREE_STEPWISE, stepwise_tree_bytes, 2 * levels)):
        fn = lambda: ar.ar_allreduce_ws(ins, outs, ar.AR_AVG, algo, ws)
        fn()
        rows[name] = row_entry(name, timer.run(fn, max(3, reps // 2)), fb(N_RANKS, COUNT, 2, 4), S, N_RANKS,
                               {"launches": launches,
                                "cpu_oracle": "same computation as the ring (cpu_baseline), rhd_tree and "
                                              "binomial_tree oracle timings: the oracle executes the rounds "
                                              "literally"})
    del ws
    torch.cuda.empty_cache()

    log("fp8 rows")
    # fp8 compressed ring: 8 ranks x 67,108,864 bf16 with 0.1% outliers x100, blocks of 128
    n8 = 67_108_864
    h8 = _gen_parallel(lambda r: inputs.outlier_bf16((5, r), n8), range(N_RANKS))
    i8 = _upload(torch, h8, torch.bfloat16, dev)
    o8 = [torch.empty_like(t) for t in i8]
    fn = lambda: ar.ar_allreduce(i8, o8, ar.AR_SUM, ar.AR_ALGO_RING_FP8)
    fn()
    rows["fp8_ring"] = row_entry("fp8_ring", timer.run(fn, reps), ring_bytes(N_RANKS, n8, 2), n8 * 2, N_RANKS,
                                 {"count": n8, "wire_bytes_per_element": 1 + 4 / 128})
    rows["fp8_ring"]["cpu_oracle"] = cpu_row(oracle_time(_o.fp8_ring_allreduce, h8, _o.BF16, _o.SUM), n8 * 2, N_RANKS,
                                             "the full 8 x 67,108,864 bf16 workload, one call")
    codes = torch.empty(n8, dtype=torch.uint8, device=dev)
    scales = torch.empty(n8 // 128, dtype=torch.float32, device=dev)
    fn = lambda: ar.ar_fp8_quant(i8[0], codes, scales)
    fn()
    qb = n8 * 2 + n8 + n8 // 128 * 4
    # the codec kernels run shorter than a host call: timed as 20 calls in one HIP graph, per-call events beside
    rows["fp8_quant"] = row_entry("fp8_quant", graph_ms(torch, fn), qb, n8 * 2, 1,
                                  {"count": n8, "timing": "HIP graph of 20 calls",
                                   "us_per_call_events": stats_us(timer.run(fn, reps))})
    rows["fp8_quant"]["cpu_oracle"] = cpu_row(oracle_time(_o.fp8_quant, h8[0], _o.BF16), n8 * 2, 1,
                                              "one rank's 67,108,864 bf16, one call")
    fn = lambda: ar.ar_fp8_dequant(codes, scales, o8[0])
    fn()
    rows["fp8_dequant"] = row_entry("fp8_dequant", graph_ms(torch, fn), qb, n8 * 2, 1,
                                    {"count": n8, "timing": "HIP graph of 20 calls",
                                     "us_per_call_events": stats_us(timer.run(fn, reps))})
    del i8, o8, codes, scales, h8
    torch.cuda.empty_cache()

    log("bucket row")
    # bucketing: 300 fp32 tensors per rank, log-uniform sizes in [1K, 16M], 25 MiB buckets, sum then /8.
    sizes = inputs.bucket_sizes()
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    bins = [[torch.randn(int(s), generator=g, device=dev, dtype=torch.float32).mul_(1e-2) for s in sizes]
            for _ in range(N_RANKS)]
    bouts = [[torch.empty_like(t) for t in r] for r in bins]
    bar = ar.BucketedAllReduce(bins, bouts, op=ar.AR_AVG, cap_bytes=25 << 20)
    bar()
    torch.cuda.synchronize()
    s_tot = int(np.sum(sizes)) * 4
    b_tot = int(np.sum(bar.bucket_count)) * 4
    phases = {}
    for name, fn in (("pack", bar.pack), ("allreduce", bar.reduce), ("unpack", bar.unpack)):
        phases[name] = stats_us(timer.run(fn, max(3, reps // 2)))
    ms = timer.run(bar, max(3, reps // 2))
    # pack: read the tensors, write the buckets with pads; ring: N reads + N writes of every bucket;
    # unpack: read and write the tensor elements
    alg = N_RANKS * (s_tot + b_tot) + 2 * N_RANKS * b_tot + 2 * N_RANKS * s_tot
    rows["buckets"] = row_entry("buckets", ms, alg, s_tot, N_RANKS,
                                {"tensors": len(sizes), "buckets": bar.nbuckets, "bytes_per_rank": s_tot,
                                 "launches": 3, "phases_us": phases,
                                 "data": "torch GPU generator, normal(0, 1e-2)"})
    # the same bucketed all-reduce read and written in place of the buckets: N reads + N writes per element
    bar.fused()
    torch.cuda.synchronize()
    rows["buckets_fused"] = row_entry("buckets_fused", timer.run(bar.fused, max(3, reps // 2)), 2 * N_RANKS * s_tot,
                                      s_tot, N_RANKS, {"tensors": len(sizes), "launches": 1,
                                                       "same_bits_as": "buckets (pack + per-bucket ring + unpack)"})
    del bins, bouts, bar
    torch.cuda.empty_cache()
    k = 60  # oracle sample: the first 60 tensors of every rank, drawn as in the tests
    hb = _gen_parallel(lambda r: inputs.bucket_tensors(r, sizes[:k]), range(N_RANKS))
    s_k = int(np.sum(sizes[:k])) * 4
    rows["buckets"]["cpu_oracle"] = cpu_row(oracle_time(_o.bucketed_allreduce, hb, _o.F32, _o.AVG, 25 << 20), s_k,
                                            N_RANKS, f"the first {k} of the 300 tensors ({s_k} bytes per rank): "
                                                     "plan, pack, per-bucket literal rings, unpack")
    return rows


def graph_ms(torch, call, calls=20, replays=5):
    """Per-call device times (ms, one per replay) of `calls` back-to-back calls captured in one HIP graph: for
    kernels shorter than the host's cost of a call, whose per-call events would time the launch gaps."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            call()
    g.replay()
    torch.cuda.synchronize()
    return [m / calls for m in Timer(torch).run(g.replay, replays)]


def graph_time_us(torch, call, calls, replays=5):
    """Per-call device time of `calls` back-to-back calls captured in one HIP graph (no host launch cost)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            call()
    g.replay()
    torch.cuda.synchronize()
    ms = Timer(torch).run(g.replay, replays)
    return float(np.median(ms)) * 1e3 / calls


def overlap_rows(torch, ar, ins, outs, dev, reps=5):
    """The headline all-reduce on a stream of its own beside another kernel on a second stream ([V]
    "communicationとcomputeを重ねる条件": overlap hides waiting only if the two do not compete for the same memory
    bandwidth or compute units; measure it end to end). Partners: an HBM-bound 2 GiB device copy (the same
    bytes as the all-reduce) and an MFMA-bound 8192^3 bf16 GEMM. All streams keep the default priority."""
    s_ar, s_p = torch.cuda.Stream(), torch.cuda.Stream()
    src = torch.empty(1 << 30, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)
    partners = {"hbm_copy_2GiB": lambda: dst.copy_(src), "gemm_bf16_8192": lambda: torch.mm(a, b, out=c)}
    run_ar = lambda: ar.ar_allreduce(ins, outs, ar.AR_AVG, ar.AR_ALGO_RING, stream=s_ar)

    def on(stream, fn):
        with torch.cuda.stream(stream):
            fn()

    def timed(work):
        """work: list of (stream, fn) started together; returns (wall us, per-stream us)."""
        cur = torch.cuda.current_stream()
        res_wall, res_each = [], []
        for _ in range(reps + 1):
            start = torch.cuda.Event(enable_timing=True)
            start.record(cur)
            ends = []
            for st, fn in work:
                st.wait_event(start)
                on(st, fn)
                e = torch.cuda.Event(enable_timing=True)
                e.record(st)
                ends.append(e)
            for e in ends:
                cur.wait_event(e)
            end = torch.cuda.Event(enable_timing=True)
            end.record(cur)
            torch.cuda.synchronize()
            res_wall.append(start.elapsed_time(end) * 1e3)
            res_each.append([start.elapsed_time(e) * 1e3 for e in ends])
        return float(np.median(res_wall[1:])), [float(np.median([r[k] for r in res_each[1:]])) for k in range(len(work))]

    out = {}
    ar_alone, _ = timed([(s_ar, run_ar)])
    for name, fn in partners.items():
        p_alone, _ = timed([(s_p, fn)])
        both, each = timed([(s_ar, run_ar), (s_p, fn)])
        out[name] = {"allreduce_alone_us": ar_alone, "partner_alone_us": p_alone, "together_us": both,
                     "allreduce_in_overlap_us": each[0], "partner_in_overlap_us": each[1],
                     "serial_us": ar_alone + p_alone, "gain_vs_serial": (ar_alone + p_alone) / both}
    del src, dst, a, b, c
    torch.cuda.empty_cache()
    return out


def alpha_beta_fit(lines, n):
    """Least-squares fit of time = rounds * alpha + bytes / beta to the one-level-per-launch schedules' HIP-graph
    device times (the pages' cost tables), and the tree/ring switch point of the same table with that alpha and
    one xGMI link's bandwidth (the AR_ALGO_AUTO rule)."""
    levels = int(np.ceil(np.log2(n)))
    rounds = {"ring_stepwise": 2 * (n - 1), "rhd_stepwise": 2 * levels, "tree_stepwise": 2 * levels}
    fb = {"ring_stepwise": stepwise_ring_bytes, "rhd_stepwise": stepwise_rhd_bytes,
          "tree_stepwise": stepwise_tree_bytes}
    a, y = [], []
    for r in lines:
        if r["algo"] in rounds and r.get("graph_us_per_call"):
            a.append([rounds[r["algo"]], fb[r["algo"]](n, r["bytes_per_rank"] // 4, 4, 4)])
            y.append(r["graph_us_per_call"] * 1e-6)
    if len(y) < 2:
        return None
    (alpha, inv_beta), *_ = np.linalg.lstsq(np.array(a), np.array(y), rcond=None)
    link = 153e9
    return {"fit": "steps * alpha + bytes / beta, stepwise schedules, HIP-graph device time", "points": len(y),
            "alpha_us": float(alpha) * 1e6, "beta_GBps": float(1.0 / inv_beta) / GB,
            "tree_below_bytes_at_153GBps_link": float(n * max(0, n - 1 - levels) * alpha * link)}


SWEEP_ALGOS = ("ring", "rhd", "fused", "tree", "ring_stepwise", "rhd_stepwise", "tree_stepwise")


def sweep_points(torch, ar, dev, S, names, reps=20, graph_max=16 << 20):
    """One message size of the sweep: N = 8 fp32 ranks of S bytes each, uniform [-1, 1), sum. Below 1 GiB of total
    traffic, ceil(1 GiB / (2 N S)) buffer sets (at most 64) are rotated so that no call finds its data in the
    256 MB last-level cache. Returns one record per algorithm (median of `reps` event-timed calls; sizes up to
    graph_max also get the per-call device time of 100 calls in one HIP graph)."""
    codes = {"ring": ar.AR_ALGO_RING, "rhd": ar.AR_ALGO_RHD, "fused": ar.AR_ALGO_FUSED, "tree": ar.AR_ALGO_TREE,
             "ring_stepwise": ar.AR_ALGO_RING_STEPWISE, "rhd_stepwise": ar.AR_ALGO_RHD_STEPWISE,
             "tree_stepwise": ar.AR_ALGO_TREE_STEPWISE}
    n = N_RANKS
    count = S // 4
    sets = int(min(64, max(1, -(-(1 << 30) // (2 * n * S)))))
    # Every rank buffer its own allocation, as separate tensors normally are: rank buffers cut from one large cached
    # segment sit at fixed physical strides, which measured 4-13% slower on MI355X (N = 8, 256 MiB fp32 per rank:
    # 784-800 us separate, 815-820 us at a 256 MiB stride in one allocation, 890-896 us at 256 MiB + 2 MiB).
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev)
    g.manual_seed(4000 + int(np.log2(S)))
    bufs = [([torch.rand(count, generator=g, device=dev).mul_(2).sub_(1) for _ in range(n)],
             [torch.empty(count, device=dev) for _ in range(n)]) for _ in range(sets)]
    recs = []
    for name in names:
        algo = codes[name]
        k = [0]

        def call():
            i, o = bufs[k[0] % sets]
            k[0] += 1
            ar.ar_allreduce(i, o, ar.AR_SUM, algo)

        for _ in range(3):
            call()
        ms = Timer(torch).run(call, reps)
        t = float(np.median(ms)) * 1e-3
        graph_us = graph_time_us(torch, call, 100) if S <= graph_max else None
        alg = {"ring_stepwise": stepwise_ring_bytes, "rhd_stepwise": stepwise_rhd_bytes,
               "tree_stepwise": stepwise_tree_bytes}.get(name, lambda n_, c_, e_, a_: ring_bytes(n_, c_, e_))(
            n, count, 4, 4)
        recs.append({"bytes_per_rank": S, "algo": name, "us_p50": t * 1e6, "us": stats_us(ms),
                     "algbw_GBps": S / t / GB, "busbw_GBps": S / t / GB * bus_factor(n),
                     "hbm_GBps": alg / t / GB, "frac_of_peak": alg / t / GB / PEAK_HBM_GBPS, "buffer_sets": sets,
                     "graph_us_per_call": graph_us})
    del bufs
    torch.cuda.empty_cache()
    return recs


def sweep(torch, ar, dev, out_path, reps=20, max_log2=30):
    """Message-size sweep: N = 8 fp32 ranks, sum, 8 B ... 1 GiB per rank, ring vs halving-doubling vs rank order
    vs the binomial tree vs the round-per-launch schedules. One JSON line per point, then the alpha-beta fit."""
    lines = []
    with open(out_path, "w") as f:
        for lg in range(3, max_log2 + 1):
            for rec in sweep_points(torch, ar, dev, 1 << lg, SWEEP_ALGOS, reps):
                f.write(json.dumps(rec) + "\n")
                f.flush()
                lines.append(rec)
            log(f"sweep {1 << lg} B done")
        fit = alpha_beta_fit(lines, N_RANKS)
        if fit:
            f.write(json.dumps(fit) + "\n")
    return lines


def compact_sweep(torch, ar, dev, reps=20):
    """The size curve of the metric in the default run: N = 8 fp32 sum, 64 KiB ... 1 GiB per rank, the four
    one-pass orders (the round-per-launch schedules and the sizes in between are in --sweep)."""
    out = []
    for S in (64 << 10, 1 << 20, 16 << 20, 64 << 20, 256 << 20, 1 << 30):
        for rec in sweep_points(torch, ar, dev, S, ("ring", "fused", "rhd", "tree"), reps, graph_max=1 << 20):
            out.append({k: rec[k] for k in ("bytes_per_rank", "algo", "us_p50", "algbw_GBps", "busbw_GBps",
                                            "hbm_GBps", "frac_of_peak", "buffer_sets", "graph_us_per_call")})
        log(f"compact sweep {S} B done")
    return out


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--headline-only", action="store_true", help="time the headline only (for profiler runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 2 GiB device copy, the reference for HBM counter scaling")
    p.add_argument("--fp8-only", action="store_true",
                   help="time only the compressed ring on its workload (8 x 67,108,864 bf16, 0.1%% outliers; for "
                        "profiler runs)")
    p.add_argument("--fp8-extra", type=int, default=0, metavar="E",
                   help="with --fp8-only: E more elements per rank (a count off the multiples of 8 N puts chunk "
                        "starts inside 16-byte slots, the compressed ring's shifted path)")
    p.add_argument("--ring-bytes-per-rank", type=int, metavar="S",
                   help="time only the ring on N = 8 fp32 ranks of S bytes each, sum (for profiler runs at one size)")
    p.add_argument("--per-rank-offsets-only", action="store_true",
                   help="time only the headline workload with rank r's buffers r elements past an aligned address "
                        "(the skewed kernel; for profiler runs)")
    p.add_argument("--sweep", metavar="OUT.jsonl", help="run only the message-size sweep, one JSON line per point")
    p.add_argument("--sweep-max-log2", type=int, default=30)
    args = p.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library runs all N ranks as separate buffers "
              "on one MI355X, so only --gpus 1 is measured", file=sys.stderr)
        sys.exit(2)

    import torch

    import all_reduce_reduction_ring_amd as ar
    from all_reduce_reduction_ring_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    ar.lib()

    if args.sweep:
        sweep(torch, ar, dev, args.sweep, max_log2=args.sweep_max_log2)
        return

    if args.per_rank_offsets_only:
        g = torch.Generator(device=dev)
        g.manual_seed(2)
        vin = [torch.empty(COUNT + N_RANKS, dtype=torch.bfloat16, device=dev)[r:r + COUNT] for r in range(N_RANKS)]
        vout = [torch.empty(COUNT + N_RANKS, dtype=torch.bfloat16, device=dev)[r:r + COUNT] for r in range(N_RANKS)]
        for v in vin:
            v.copy_(torch.randn(COUNT, generator=g, device=dev).mul_(1e-3))
        step = lambda: ar.ar_allreduce(vin, vout, ar.AR_AVG, ar.AR_ALGO_RING)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ms = Timer(torch).run(step, args.steps)
        t = float(np.mean(ms)) * 1e-3
        print(json.dumps({"ring_per_rank_offsets": {"kernel_us": stats_us(ms),
                                                    "hbm_GBps": ring_bytes(N_RANKS, COUNT, 2) / t / GB,
                                                    "steps": args.steps, "warmup": args.warmup}}))
        return

    if args.ring_bytes_per_rank:
        S = args.ring_bytes_per_rank
        g = torch.Generator(device=dev)
        g.manual_seed(4000)
        rin = [torch.rand(S // 4, generator=g, device=dev).mul_(2).sub_(1) for _ in range(N_RANKS)]
        rout = [torch.empty_like(t) for t in rin]
        step = lambda: ar.ar_allreduce(rin, rout, ar.AR_SUM, ar.AR_ALGO_RING)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ms = Timer(torch).run(step, args.steps)
        t = float(np.mean(ms)) * 1e-3
        print(json.dumps({"ring_f32": {"bytes_per_rank": S, "kernel_us": stats_us(ms),
                                       "hbm_GBps": ring_bytes(N_RANKS, S // 4, 4) / t / GB,
                                       "steps": args.steps, "warmup": args.warmup}}))
        return

    if args.fp8_only:
        n8 = 67_108_864 + args.fp8_extra
        log("generating the compressed-ring inputs")
        h8 = _gen_parallel(lambda r: inputs.outlier_bf16((5, r), n8), range(N_RANKS))
        i8 = _upload(torch, h8, torch.bfloat16, dev)
        o8 = [torch.empty_like(t) for t in i8]
        step = lambda: ar.ar_allreduce(i8, o8, ar.AR_SUM, ar.AR_ALGO_RING_FP8)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ms = Timer(torch).run(step, args.steps)
        t = float(np.mean(ms)) * 1e-3
        print(json.dumps({"fp8_ring": {"count": n8, "kernel_us": stats_us(ms),
                                       "hbm_GBps": ring_bytes(N_RANKS, n8, 2) / t / GB,
                                       "busbw_GBps": n8 * 2 / t / GB * bus_factor(N_RANKS),
                                       "steps": args.steps, "warmup": args.warmup}}))
        return

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_launch": 2 << 30, "bytes_written_per_launch": 2 << 30,
                                               "launches": args.warmup + args.steps}}))
        return

    host, ins, outs, ms, wall = headline(torch, ar, inputs, args, dev)
    S = COUNT * 2
    t_kernel = float(np.mean(ms)) * 1e-3
    algbw = S / t_kernel / GB
    alg_bytes = ring_bytes(N_RANKS, COUNT, 2)
    achieved = alg_bytes / t_kernel / GB
    sources = ["ar_collapsed.hip", "ar_device.h"]
    traffic = _load_traffic("ring_front_kernel<bf16,avg,8>", sources)
    traffic_source = (f"profiles/hbm_counters.json: rocprofv3 FETCH_SIZE and WRITE_SIZE of this kernel, taken in an "
                      f"earlier profiled run of the same sources (sha256 {_sources_digest(sources)[:16]}), not "
                      f"measured in this run") if traffic else None
    result = {
        "metric": METRIC,
        "value": algbw * bus_factor(N_RANKS),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ring all-reduce, N=8 simulated ranks (separate HBM buffers), 134,217,728 bf16 "
                               "per rank (256 MiB), fp32 sum in ring order, /8, bf16 out to all 8",
                   "nranks": N_RANKS, "count_per_rank": COUNT, "storage": "bf16", "accumulate": "fp32",
                   "op": "avg", "algo": "ring"},
        "algbw_GBps": algbw,
        "busbw_GBps": algbw * bus_factor(N_RANKS),
        "hbm_GBps": achieved,
        "kernel_us": stats_us(ms),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "traffic_source": traffic_source},
        # the counted HBM bytes of one launch over the same measured time (null while the counters are stale)
        "hbm_counter_GBps": traffic / (float(np.mean(ms)) * 1e-3) / GB if traffic else None,
    }
    if not args.headline_only:
        result["copy_ceiling_GBps"] = copy_ceiling(torch, ins, outs)
        result["write_ceiling_GBps"] = write_ceiling(torch, ins)
        halves = fold_halves(torch, ins, outs)
        if halves:
            half = alg_bytes / 2  # N*S read and N*S written
            bound = mix_bound(halves["read_fold_large"], halves["write_fold_large"], half, half)
            best = mix_bound(max(halves["read_fold_large"], halves["read_fold_small"]), max(
                halves["write_fold_large"], halves["write_fold_small"], halves["write_blocks"]), half, half)
            result["read_write_alone_GBps"] = halves
            result["roofline"]["mix_bound_GBps"] = bound
            result["roofline"]["frac_of_mix_bound"] = achieved / bound
            result["roofline"]["mix_bound_best_GBps"] = best
            result["roofline"]["frac_of_mix_bound_best"] = achieved / best
            result["roofline"]["mix_bound"] = (
                "bytes / (read bytes / R + written bytes / W), R and W measured alone in this run (libar_ceiling.so): "
                "mix_bound with the headline kernel's own launch shape and access order, mix_bound_best with the "
                "fastest read and write patterns measured for the same bytes")
        log("compact sweep")
        size_curve = compact_sweep(torch, ar, dev)
        log("overlap row")
        result["overlap"] = overlap_rows(torch, ar, ins, outs, dev)
        result["rows"] = other_rows(torch, ar, inputs, ins, outs, dev, reps=max(5, args.steps // 2), host=host)
        result["rows"]["sweep"] = size_curve
        del ins, outs
        torch.cuda.empty_cache()
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(host)
        result["host"] = host_info(host)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
