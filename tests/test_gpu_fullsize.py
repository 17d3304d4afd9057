"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times, against the oracle.

- headline: 8 ranks x 134,217,728 bf16 (256 MiB each), fp32 ring-order sum, /8, bf16 out: every element of
  every rank, bit for bit; the same inputs through reduce-scatter + all-gather and through the binomial tree, and
  with every rank's input and output at its own odd element offset (the skewed kernel), ring and tree.
- compressed ring: 8 ranks x 67,108,864 bf16 with 0.1% outliers x100, E4M3 blocks of 128: every element; and
  8 ranks x (67,108,864 + 13) fp32 with avg (chunk starts off the 16-byte grid).
- beyond 2^31 elements: 3 ranks x (2^31 + 1001) bf16 in place (ring, tree, rank order, a common offset and
  per-rank offsets), sampled against the oracle.
- largest sweep point: 8 ranks x 268,435,456 fp32 (1 GiB each): ring and ring-stepwise, every element; the
  rank-order and halving-doubling variants (which do not depend on chunk positions) on 2^20 sampled elements,
  for which the oracle is evaluated on exactly those elements.
- buckets: 300 fp32 tensors per rank (log-uniform 1K..16M elements, 604,529,495 elements = 2,418,117,980 B per
  rank), 25 MiB buckets, avg:
  every tensor of every rank, through pack + per-bucket rings + unpack and through the fused tensor path.
- the switch between the two builds of the one-pass kernels at 1 GiB of traffic: ring, rank order and trees on
  both sides of it (fp32, bf16, f16, int32; N = 2, 3, 4, 8, 16; ragged counts), and one shared segment launch of
  small buckets above it: every element.
"""
import concurrent.futures

import numpy as np
import pytest
import torch

import all_reduce_reduction_ring_amd as ar
import oracle
from all_reduce_reduction_ring_amd import inputs
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def _par(fn, items):
    with concurrent.futures.ThreadPoolExecutor(max_workers=16) as ex:
        return list(ex.map(fn, items))


def _up(arrs, tdt):
    return [torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(DEV).view(tdt) for a in arrs]


def _down_bits(t):
    bits = torch.int16 if t.element_size() == 2 else torch.int32
    return t.view(bits).cpu().numpy().view(np.uint16 if t.element_size() == 2 else np.uint32)


def _same_on_all_ranks(outs):
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16 if o.element_size() == 2 else torch.int32),
                           outs[0].view(torch.int16 if o.element_size() == 2 else torch.int32))


@pytest.mark.timeout(600)
def test_headline_eight_ranks_256MiB_bf16_avg():
    n, count = 8, 134_217_728
    host = _par(lambda r: inputs.normal_bf16((2, r), count), range(n))
    ins = _up(host, torch.bfloat16)
    outs = [torch.empty_like(t) for t in ins]
    ar.ar_allreduce(ins, outs, ar.AR_AVG, ar.AR_ALGO_RING)
    torch.cuda.synchronize()
    del ins
    want = oracle.ring_allreduce(host, oracle.BF16, oracle.AVG)
    _same_on_all_ranks(outs)
    for r in range(n):
        np.testing.assert_array_equal(_down_bits(outs[r]), want[r])


@pytest.mark.timeout(600)
def test_headline_size_at_odd_per_rank_offsets():
    """The headline workload with rank r's input r elements and its output 2r + 1 elements past an aligned address:
    the skewed kernel at the size where it walks long strips (32 tiles per wave), in ring order and as the binomial
    tree, every element of every rank against the oracle."""
    n, count = 8, 134_217_728
    host = _par(lambda r: inputs.normal_bf16((2, r), count), range(n))
    ibase = [torch.empty(count + 16, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    obase = [torch.empty(count + 16, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    ins = [b[r:r + count] for r, b in enumerate(ibase)]
    outs = [b[2 * r + 1:2 * r + 1 + count] for r, b in enumerate(obase)]
    for t, h in zip(ins, _up(host, torch.bfloat16)):
        t.copy_(h)
    torch.cuda.synchronize()
    for algo, fn in ((ar.AR_ALGO_RING, oracle.ring_allreduce), (ar.AR_ALGO_TREE, oracle.tree_allreduce)):
        ar.ar_allreduce(ins, outs, ar.AR_AVG, algo)
        torch.cuda.synchronize()
        want = fn(host, oracle.BF16, oracle.AVG)
        for r in range(n):
            np.testing.assert_array_equal(_down_bits(outs[r]), want[r], err_msg=f"algo {algo} rank {r}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n,count", [(3, 134_217_737), (7, 40_000_003)])
def test_odd_per_rank_offsets_three_and_seven_ranks_long_strips(n, count):
    """The skewed kernel's builds for rank counts that are not a power of two, at sizes where it walks long strips
    (32 tiles per wave): rank r's input r elements and its output 3r + 2 elements past an aligned address, ragged
    chunks, ring order, rank order and the binomial tree, every element of every rank against the oracle."""
    host = _par(lambda r: inputs.normal_bf16((7, n, r), count), range(n))
    ibase = [torch.empty(count + 32, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    obase = [torch.empty(count + 32, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    ins = [b[r:r + count] for r, b in enumerate(ibase)]
    outs = [b[3 * r + 2:3 * r + 2 + count] for r, b in enumerate(obase)]
    for t, h in zip(ins, _up(host, torch.bfloat16)):
        t.copy_(h)
    torch.cuda.synchronize()
    for algo, fn in ((ar.AR_ALGO_RING, oracle.ring_allreduce), (ar.AR_ALGO_FUSED, oracle.fused_allreduce),
                     (ar.AR_ALGO_TREE, oracle.tree_allreduce)):
        print(f"case n={n} count={count} algo={algo}", flush=True)
        ar.ar_allreduce(ins, outs, ar.AR_SUM, algo)
        torch.cuda.synchronize()
        want = fn(host, oracle.BF16, oracle.SUM)
        for r in range(n):
            np.testing.assert_array_equal(_down_bits(outs[r]), want[r], err_msg=f"algo {algo} rank {r}")


@pytest.mark.timeout(600)
def test_headline_size_reduce_scatter_all_gather_and_tree():
    """The headline inputs through reduce-scatter then all-gather (must equal the ring all-reduce, every element)
    and through the binomial tree (against its own oracle, every element)."""
    n, count = 8, 134_217_728
    host = _par(lambda r: inputs.normal_bf16((2, r), count), range(n))
    ins = _up(host, torch.bfloat16)
    lo = ar.chunk_bounds(count, n)
    parts = [torch.empty(int(lo[c + 1] - lo[c]), dtype=torch.bfloat16, device=DEV) for c in range(n)]
    outs = [torch.empty_like(t) for t in ins]
    ar.ar_reduce_scatter(ins, parts, ar.AR_AVG)
    ar.ar_all_gather(parts, outs)
    torch.cuda.synchronize()
    want = oracle.ring_allreduce(host, oracle.BF16, oracle.AVG)[0]
    for c in range(n):
        np.testing.assert_array_equal(_down_bits(parts[c]), want[lo[c]:lo[c + 1]])
    _same_on_all_ranks(outs)
    np.testing.assert_array_equal(_down_bits(outs[3]), want)
    del parts, want
    ar.ar_allreduce(ins, outs, ar.AR_AVG, ar.AR_ALGO_TREE)
    torch.cuda.synchronize()
    del ins
    _same_on_all_ranks(outs)
    np.testing.assert_array_equal(_down_bits(outs[6]), oracle.tree_allreduce(host, oracle.BF16, oracle.AVG)[0])


BEYOND_2_31 = [("ring", ar.AR_ALGO_RING, (0, 0, 0)), ("tree", ar.AR_ALGO_TREE, (0, 0, 0)),
               ("fused", ar.AR_ALGO_FUSED, (0, 0, 0)), ("ring_common_offset", ar.AR_ALGO_RING, (3, 3, 3)),
               ("ring_per_rank_offsets", ar.AR_ALGO_RING, (0, 1, 2)),
               ("ring_per_rank_even_offsets", ar.AR_ALGO_RING, (0, 2, 6))]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,algo,offs", BEYOND_2_31, ids=[c[0] for c in BEYOND_2_31])
def test_beyond_two_to_the_31_elements_sampled(name, algo, offs):
    """Maximum size: 3 ranks x (2^31 + 1001) bf16 (4 GiB each), in place, avg, with 64-bit element and byte
    offsets: the one-front ring kernel, the one-pass tree and rank-order kernels, a common offset (head, then
    slots), per-rank odd offsets (element by element) and per-rank even offsets (slots at 4-byte alignment). Sampled positions (random, both ends, around every chunk
    boundary) against the oracle. For the ring each chunk's samples go into the same chunk of a small array, so
    the oracle folds them from the same rank as the ring does at full size; the other orders do not depend on
    the position."""
    n, count = 3, (1 << 31) + 1001
    g = torch.Generator(device=DEV)
    g.manual_seed(2031)
    bufs = []
    for r in range(n):
        t = torch.empty(count + 8, dtype=torch.bfloat16, device=DEV)[offs[r]:offs[r] + count]
        for s0 in range(0, count, 1 << 28):
            m = min(1 << 28, count - s0)
            t[s0:s0 + m] = (torch.randn(m, generator=g, device=DEV) * 1e-3).to(torch.bfloat16)
        bufs.append(t)
    lo = ar.chunk_bounds(count, n)
    rng = np.random.default_rng(31)
    pos = np.unique(np.concatenate([rng.integers(0, count, 1 << 20), np.arange(1000), np.arange(count - 1000, count)]
                                   + [np.arange(b - 40, b + 40) for b in lo[1:-1]]))
    idx = torch.from_numpy(pos).to(DEV)
    samples = [_down_bits(b[idx]) for b in bufs]
    ar.ar_allreduce(bufs, bufs, ar.AR_AVG, algo)
    torch.cuda.synchronize()
    got = [_down_bits(b[idx]) for b in bufs]
    del bufs
    torch.cuda.empty_cache()
    if algo == ar.AR_ALGO_RING:
        chunk_of = np.searchsorted(lo, pos, side="right") - 1
        want = np.empty(len(pos), np.uint16)
        for c in range(n):
            sel = np.nonzero(chunk_of == c)[0]
            k = len(sel)
            small = [np.zeros(n * k, np.uint16) for _ in range(n)]
            for r in range(n):
                small[r][c * k:(c + 1) * k] = samples[r][sel]
            want[sel] = oracle.ring_allreduce(small, oracle.BF16, oracle.AVG)[0][c * k:(c + 1) * k]
    else:
        fn = oracle.tree_allreduce if algo == ar.AR_ALGO_TREE else oracle.fused_allreduce
        want = np.asarray(fn(samples, oracle.BF16, oracle.AVG)[0])
    for r in range(n):
        np.testing.assert_array_equal(got[r], want, err_msg=f"{name} rank {r}")


@pytest.mark.timeout(600)
def test_fp8_ring_eight_ranks_128MiB_bf16():
    n, count = 8, 67_108_864
    host = _par(lambda r: inputs.outlier_bf16((5, r), count), range(n))
    ins = _up(host, torch.bfloat16)
    outs = [torch.empty_like(t) for t in ins]
    ar.ar_allreduce(ins, outs, ar.AR_SUM, ar.AR_ALGO_RING_FP8)
    torch.cuda.synchronize()
    del ins
    want = oracle.fp8_ring_allreduce(host, oracle.BF16, oracle.SUM)
    _same_on_all_ranks(outs)
    np.testing.assert_array_equal(_down_bits(outs[0]), want[0])
    np.testing.assert_array_equal(_down_bits(outs[n - 1]), want[n - 1])
    # reported, not gated: error of the compressed sum against the exact sum, relative to the block scale
    exact = np.zeros(count, np.float64)
    for h in host:
        exact += oracle.bf16_to_f32(h)
    got = oracle.bf16_to_f32(want[0]).astype(np.float64)
    print(f"fp8 ring: max |err| = {np.max(np.abs(got - exact)):.3e}, mean |exact| = {np.mean(np.abs(exact)):.3e}")


@pytest.mark.timeout(600)
def test_fp8_ring_eight_ranks_fp32_avg_ragged():
    """The compressed ring on fp32 inputs with avg, at the same element count plus 13 (chunk starts off the 16-byte
    grid, so the shifted fp32 vector path and its lane-assembled stores run at scale): every element of the first
    and last rank, and all ranks equal."""
    n, count = 8, 67_108_864 + 13
    host = _par(lambda r: inputs.normal_f32((5, r, 32), count, 1e-3), range(n))
    for h in host:
        h[::997] *= np.float32(100)
    ins = _up(host, torch.float32)
    outs = [torch.empty_like(t) for t in ins]
    ar.ar_allreduce(ins, outs, ar.AR_AVG, ar.AR_ALGO_RING_FP8)
    torch.cuda.synchronize()
    del ins
    want = oracle.fp8_ring_allreduce(host, oracle.F32, oracle.AVG)
    _same_on_all_ranks(outs)
    np.testing.assert_array_equal(_down_bits(outs[0]), np.asarray(want[0]).view(np.uint32))
    np.testing.assert_array_equal(_down_bits(outs[n - 1]), np.asarray(want[n - 1]).view(np.uint32))


@pytest.mark.timeout(900)
def test_sweep_largest_point_one_GiB_per_rank():
    n, count = 8, 268_435_456
    host = _par(lambda r: inputs.uniform_pm1((4, r, 30), count), range(n))
    ins = _up(host, torch.float32)
    outs = [torch.empty_like(t) for t in ins]
    want = oracle.ring_allreduce(host, oracle.F32, oracle.SUM)
    for algo in (ar.AR_ALGO_RING, ar.AR_ALGO_RING_STEPWISE):
        for o in outs:
            o.fill_(float("nan"))
        ar.ar_allreduce(ins, outs, ar.AR_SUM, algo)
        torch.cuda.synchronize()
        _same_on_all_ranks(outs)
        np.testing.assert_array_equal(_down_bits(outs[0]), want[0].view(np.uint32))
        np.testing.assert_array_equal(_down_bits(outs[5]), want[5].view(np.uint32))
    del want
    rng = np.random.default_rng(44)
    idx = np.unique(np.concatenate([rng.integers(0, count, 1 << 20), np.arange(1000), np.arange(count - 1000, count)]))
    sub = [h[idx] for h in host]
    for algo, fn in ((ar.AR_ALGO_FUSED, oracle.fused_allreduce), (ar.AR_ALGO_RHD, oracle.rhd_allreduce),
                     (ar.AR_ALGO_RHD_STEPWISE, oracle.rhd_allreduce), (ar.AR_ALGO_TREE, oracle.tree_allreduce),
                     (ar.AR_ALGO_TREE_STEPWISE, oracle.tree_allreduce)):
        ar.ar_allreduce(ins, outs, ar.AR_SUM, algo)
        torch.cuda.synchronize()
        _same_on_all_ranks(outs)
        w = fn(sub, oracle.F32, oracle.SUM)[0].view(np.uint32)
        got = outs[3][torch.from_numpy(idx).to(DEV)]
        np.testing.assert_array_equal(_down_bits(got), w)


@pytest.mark.timeout(900)
def test_buckets_300_tensors_full_size():
    n = 8
    sizes = inputs.bucket_sizes()
    host = _par(lambda r: inputs.bucket_tensors(r, sizes), range(n))
    ins = [[torch.from_numpy(t).to(DEV) for t in host[r]] for r in range(n)]
    outs = [[torch.empty_like(t) for t in ins[r]] for r in range(n)]
    bar = ar.BucketedAllReduce(ins, outs, op=ar.AR_AVG, cap_bytes=25 << 20)
    bo, oo, bc = oracle.bucket_plan(sizes, 4, n, 25 << 20)
    np.testing.assert_array_equal(bar.bucket_of, bo)
    np.testing.assert_array_equal(bar.offset_of, oo)
    np.testing.assert_array_equal(bar.bucket_count, bc)
    bar()
    torch.cuda.synchronize()
    outs_fused = [[torch.empty_like(t) for t in ins[r]] for r in range(n)]
    bar_fused = ar.BucketedAllReduce(ins, outs_fused, op=ar.AR_AVG, cap_bytes=25 << 20)
    bar_fused.fused()
    torch.cuda.synchronize()
    del ins, bar, bar_fused
    want = oracle.bucketed_allreduce(host, oracle.F32, oracle.AVG, cap_bytes=25 << 20)
    for r in range(n):
        for t in range(len(sizes)):
            np.testing.assert_array_equal(_down_bits(outs[r][t]), want[r][t].view(np.uint32))
            np.testing.assert_array_equal(_down_bits(outs_fused[r][t]), want[r][t].view(np.uint32))


@pytest.mark.timeout(900)
def test_fp8_encoder_exhaustive_every_fp32_up_to_448():
    """Every fp32 bit pattern with |v| <= 448 (both signs, subnormals included) goes through ar_fp8_quant in
    blocks of 128 led by 448, so each block's scale is 1 and the encoder sees the raw values; every code must
    equal the oracle's. Together with the scale rule (|v * inv| < 464) this covers every value the compressed
    ring can quantize."""
    lim = int(np.float32(448.0).view(np.uint32))
    slab = 127 << 20
    for start in range(0, lim + 1, slab):
        pats = np.arange(start, min(start + slab, lim + 1), dtype=np.uint32)
        for sign in (0, 0x80000000):
            v = (pats | np.uint32(sign)).view(np.float32)
            nb = -(-v.size // 127)
            body = np.zeros(nb * 127, np.float32)
            body[: v.size] = v
            x = np.empty((nb, 128), np.float32)
            x[:, 0] = 448.0
            x[:, 1:] = body.reshape(nb, 127)
            x = x.reshape(-1)
            assert np.array_equal(x.reshape(nb, 128)[:, 1:].reshape(-1)[: v.size].view(np.uint32), v.view(np.uint32))
            xd = torch.from_numpy(x).to(DEV)
            codes = torch.empty(x.size, dtype=torch.uint8, device=DEV)
            scales = torch.empty(nb, dtype=torch.float32, device=DEV)
            ar.ar_fp8_quant(xd, codes, scales)
            torch.cuda.synchronize()
            wc, ws = oracle.fp8_quant(x, oracle.F32)
            assert np.all(ws == 1.0)
            got = codes.cpu().numpy()
            if not np.array_equal(got, wc):
                bad = np.nonzero(got != wc)[0][:5]
                raise AssertionError(f"codes differ at inputs {x[bad].view(np.uint32)}: got {got[bad]} want {wc[bad]}")
            del xd, codes, scales


# One-pass launches switch builds at 1 GiB of HBM traffic (2 * N * count * element size): non-temporal loads and
# 256-thread workgroups up to it, default-policy loads and 128-thread workgroups above. Both sides of the switch,
# with ragged counts, every element against the oracle.
THRESHOLD_CASES = [
    # (n, dt, count): N=8 fp32 at exactly 1 GiB (small build) and just above it (large build); N=3 bf16 on
    # both sides of 1 GiB with chunk starts inside 16-byte slots
    (8, ar.AR_F32, 1 << 25),
    (8, ar.AR_F32, (1 << 25) + 1003),
    (3, ar.AR_BF16, (1 << 30) // 12 - 5),
    (3, ar.AR_BF16, (1 << 30) // 12 + 7),
    # the large build for the other element types and compile-time rank counts
    (2, ar.AR_I32, (1 << 26) + 5),
    (4, ar.AR_F16, (1 << 26) + 3),
    (16, ar.AR_F16, (1 << 24) + 9),
    # N = 16 on the small build with four tiles or more per workgroup: the one-front ring and the rank-order and
    # tree kernels on a quarter of the workgroups, the latter with every load issued first
    (16, ar.AR_BF16, (1 << 23) + 5),
    (16, ar.AR_F32, (1 << 22) + 3),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n,dt,count", THRESHOLD_CASES, ids=[f"n{c[0]}_dt{c[1]}_{c[2]}" for c in THRESHOLD_CASES])
def test_one_pass_builds_on_both_sides_of_the_switch(n, dt, count):
    from gpu_util import KIND, ORACLE_DT, ORACLE_OP, from_dev
    print(f"case n={n} dt={dt} count={count}", flush=True)
    xs = inputs.rank_inputs(KIND[dt], n, count, cfg=41, extra=(n, count))
    tdt = {ar.AR_F32: torch.float32, ar.AR_BF16: torch.bfloat16, ar.AR_F16: torch.float16, ar.AR_I32: torch.int32}[dt]
    ins = [torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(DEV).view(tdt) for x in xs]
    outs = [torch.empty_like(t) for t in ins]
    algos = [(ar.AR_ALGO_RING, oracle.ring_allreduce), (ar.AR_ALGO_FUSED, oracle.fused_allreduce),
             (ar.AR_ALGO_TREE, oracle.tree_allreduce)] + ([(ar.AR_ALGO_RHD, oracle.rhd_allreduce)]
                                                          if n & (n - 1) == 0 else [])
    for algo, ofn in algos:
        for op in (ar.AR_AVG, ar.AR_MAX):
            ar.ar_allreduce(ins, outs, op, algo)
            torch.cuda.synchronize()
            _same_on_all_ranks(outs)
            want = ofn(xs, ORACLE_DT[dt], ORACLE_OP[op])[0]
            got = from_dev(outs[0], dt)
            assert np.array_equal(got, np.asarray(want).view(got.dtype)), f"algo={algo} op={op}"
    if n == 16:  # in place on the quarter grid (every load of a slot issued before its stores)
        for algo, ofn in ((ar.AR_ALGO_RING, oracle.ring_allreduce), (ar.AR_ALGO_TREE, oracle.tree_allreduce)):
            work = [t.clone() for t in ins]
            ar.ar_allreduce(work, work, ar.AR_AVG, algo)
            torch.cuda.synchronize()
            _same_on_all_ranks(work)
            want = ofn(xs, ORACLE_DT[dt], ORACLE_OP[ar.AR_AVG])[0]
            got = from_dev(work[0], dt)
            assert np.array_equal(got, np.asarray(want).view(got.dtype)), f"in place algo={algo}"
            del work
    del ins, outs
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_shared_segment_launch_above_the_switch():
    """Twelve buckets of just under 16 MiB per rank (8 ranks, fp32) share one segment launch of 1.5 GiB of
    traffic (the large build); every bucket must equal its own ring, every element."""
    from gpu_util import from_dev
    n, dt = 8, ar.AR_F32
    unit = n * 4
    counts = np.array([((16 << 20) // 4 // unit - 1 - 7 * b) * unit for b in range(12)], dtype=np.int64)
    assert counts.max() * 4 < (16 << 20) and 2 * n * 4 * int(counts.sum()) > (1 << 30)
    total = int(counts.sum())
    xs = inputs.rank_inputs("uniform_f32", n, total, cfg=42)
    ins = _up(xs, torch.float32)
    outs = [torch.empty_like(t) for t in ins]
    ar.ar_allreduce_buckets(ins, outs, counts, ar.AR_AVG, ar.AR_ALGO_RING)
    torch.cuda.synchronize()
    _same_on_all_ranks(outs)
    got = from_dev(outs[0], dt)
    starts = np.concatenate([[0], np.cumsum(counts)])
    for b in range(len(counts)):
        seg = [x[starts[b]:starts[b + 1]] for x in xs]
        want = np.asarray(oracle.ring_allreduce(seg, oracle.F32, oracle.AVG)[0]).view(np.uint32)
        assert np.array_equal(got[starts[b]:starts[b + 1]], want), f"bucket {b}"
