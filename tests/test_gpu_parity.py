"""GPU parity: every all-reduce algorithm, dtype, op and rank count through the C ABI, compared element by
element with the CPU oracle on the same seeded inputs. Bit-exact where the association order is fixed (all
algorithms against their own-order oracle); reordered variants are also checked against the ring within the
stated tolerance."""
import os

import numpy as np
import pytest
import torch

import all_reduce_reduction_ring_amd as ar
import oracle
from all_reduce_reduction_ring_amd import inputs
from gpu_util import (DEV, KIND, NP_BITS, ORACLE_DT, ORACLE_OP, assert_bitwise, empty_like_dev, expect, from_dev,
                      run, to_dev)

pytestmark = pytest.mark.gpu

DTYPES = [ar.AR_F32, ar.AR_BF16, ar.AR_F16, ar.AR_I32]
OPS = [ar.AR_SUM, ar.AR_AVG, ar.AR_MIN, ar.AR_MAX]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(dt, n, count, seed):
    return inputs.rank_inputs(KIND[dt], n, count, cfg=seed, extra=(n, count))


# ---------------------------------------------------------------- the pages' worked example


@pytest.mark.parametrize("algo", [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_RING_STEPWISE,
                                  ar.AR_ALGO_RHD_STEPWISE, ar.AR_ALGO_TREE, ar.AR_ALGO_TREE_STEPWISE])
@pytest.mark.parametrize("dt", [ar.AR_I32, ar.AR_F32])
def test_worked_example(algo, dt):
    rows = {}
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                k, _, v = ln.partition(":")
                rows[k.strip()] = [int(t) for t in v.split()]
    npd = np.int32 if dt == ar.AR_I32 else np.float32
    xs = [np.array(rows[f"rank {r}"], dtype=npd) for r in range(4)]
    want = np.array(rows["result"], dtype=npd).view(NP_BITS[dt])
    for o in run(xs, dt, ar.AR_SUM, algo):
        np.testing.assert_array_equal(o, want)


# ---------------------------------------------------------------- ring: every dtype, op and rank count


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 16])
@pytest.mark.parametrize("dt", DTYPES)
def test_ring_all_ops(n, dt):
    count = 4099 + 8 * n  # several vector slots per chunk plus ragged edges
    xs = _inputs(dt, n, count, 10)
    for op in OPS:
        got = run(xs, dt, op, ar.AR_ALGO_RING)
        assert_bitwise(got, expect(xs, dt, op, ar.AR_ALGO_RING), f"ring n={n} dt={dt} op={op}")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 13])
@pytest.mark.parametrize("dt", DTYPES)
def test_fused_all_ops(n, dt):
    xs = _inputs(dt, n, 3001, 11)
    for op in OPS:
        assert_bitwise(run(xs, dt, op, ar.AR_ALGO_FUSED), expect(xs, dt, op, ar.AR_ALGO_FUSED), f"fused n={n}")


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("dt", DTYPES)
def test_rhd_all_ops(n, dt):
    count = 2053 if n <= 16 else 517
    xs = _inputs(dt, n, count, 12)
    for op in OPS:
        assert_bitwise(run(xs, dt, op, ar.AR_ALGO_RHD), expect(xs, dt, op, ar.AR_ALGO_RHD), f"rhd n={n} op={op}")


@pytest.mark.parametrize("n", [2, 3, 4, 8])
@pytest.mark.parametrize("dt", DTYPES)
def test_ring_stepwise(n, dt):
    xs = _inputs(dt, n, 2500 + n, 13)
    for op in OPS:
        got = run(xs, dt, op, ar.AR_ALGO_RING_STEPWISE)
        assert_bitwise(got, expect(xs, dt, op, ar.AR_ALGO_RING), f"ring stepwise n={n} op={op}")


@pytest.mark.parametrize("n", [2, 4, 8, 16])
@pytest.mark.parametrize("dt", DTYPES)
def test_rhd_stepwise(n, dt):
    xs = _inputs(dt, n, 2500 + n, 14)
    for op in OPS:
        got = run(xs, dt, op, ar.AR_ALGO_RHD_STEPWISE)
        assert_bitwise(got, expect(xs, dt, op, ar.AR_ALGO_RHD), f"rhd stepwise n={n} op={op}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 33, 64])
@pytest.mark.parametrize("dt", DTYPES)
def test_tree_all_ops(n, dt):
    """Binomial tree, one pass: compile-time rank counts (2, 4, 8, 16) and the run-time fold (all others)."""
    count = 2053 if n <= 16 else 517
    xs = _inputs(dt, n, count, 18)
    for op in OPS:
        assert_bitwise(run(xs, dt, op, ar.AR_ALGO_TREE), expect(xs, dt, op, ar.AR_ALGO_TREE), f"tree n={n} op={op}")


@pytest.mark.parametrize("n", [2, 3, 5, 6, 8, 13])
@pytest.mark.parametrize("dt", DTYPES)
def test_tree_stepwise(n, dt):
    xs = _inputs(dt, n, 2500 + n, 19)
    for op in OPS:
        got = run(xs, dt, op, ar.AR_ALGO_TREE_STEPWISE)
        assert_bitwise(got, expect(xs, dt, op, ar.AR_ALGO_TREE), f"tree stepwise n={n} op={op}")


@pytest.mark.parametrize("n,count", [(8, 1000), (8, 4_651_199), (8, 4_651_200), (4, 306_000), (3, 5000), (16, 70_001)])
def test_auto_runs_the_algorithm_it_reports(n, count):
    dt = ar.AR_BF16
    xs = inputs.rank_inputs("uniform_bf16", n, count, cfg=20, extra=(n, count))
    picked = ar.ar_auto_algo(n, count, dt)
    got = run(xs, dt, ar.AR_AVG, ar.AR_ALGO_AUTO)
    rec = ar.ar_last_call()
    assert rec["algo"] == picked and rec["status"] == ar.AR_OK
    assert_bitwise(got, expect(xs, dt, ar.AR_AVG, picked), f"auto n={n} count={count} -> {picked}")


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16])
def test_ring_one_front_kernel_ragged(n, dt):
    """Aligned buffers of more than a grid of tiles take the one-front ring kernel: chunk boundaries inside
    tiles and inside 16-byte slots, and a ragged tail, every op, against the literal ring."""
    # at least a grid of tiles for every rank count on 256 CUs (the largest need: 4,194,304 bf16 elements)
    count = 4_500_007 + 3 * n
    xs = _inputs(dt, n, count, 21)
    for op in OPS:
        got = run(xs, dt, op, ar.AR_ALGO_RING)
        assert_bitwise(got, expect(xs, dt, op, ar.AR_ALGO_RING), f"one-front ring n={n} dt={dt} op={op}")


@pytest.mark.parametrize("n,dt,count", [(8, ar.AR_F32, 400_003), (8, ar.AR_BF16, 1_000_005),
                                         (16, ar.AR_F32, 1_500_001), (4, ar.AR_F32, 3_000_017),
                                         (2, ar.AR_BF16, 6_000_011)])
def test_ring_one_front_kernel_one_tile_per_workgroup(n, dt, count):
    """Between one and two grids of tiles (on 256 CUs) the one-front ring gives every tile a workgroup of its own:
    ragged counts, chunk boundaries inside tiles and slots, every op, against the literal ring."""
    xs = _inputs(dt, n, count, 29)
    for op in OPS:
        got = run(xs, dt, op, ar.AR_ALGO_RING)
        assert_bitwise(got, expect(xs, dt, op, ar.AR_ALGO_RING), f"tile per workgroup n={n} dt={dt} op={op}")


def test_ring_one_front_kernel_sixty_four_ranks():
    """The largest rank count on the one-front kernel (rank count known only at run time), ragged count."""
    n, count = 64, 2_200_007  # above a grid of tiles for a run-time rank count (2,097,152 fp32 elements)
    xs = _inputs(ar.AR_F32, n, count, 23)
    for op in (ar.AR_SUM, ar.AR_MAX):
        got = run(xs, ar.AR_F32, op, ar.AR_ALGO_RING)
        assert_bitwise(got, expect(xs, ar.AR_F32, op, ar.AR_ALGO_RING), f"one-front ring n=64 op={op}")


# ---------------------------------------------------------------- edges: tiny, ragged, unaligned, in place


@pytest.mark.parametrize("count", [1, 2, 3, 7, 8, 9, 31, 33, 63, 65, 127, 1023])
@pytest.mark.parametrize("algo", [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_RING_STEPWISE,
                                  ar.AR_ALGO_RHD_STEPWISE, ar.AR_ALGO_TREE, ar.AR_ALGO_TREE_STEPWISE])
def test_small_and_ragged_counts(count, algo):
    for dt in (ar.AR_F32, ar.AR_BF16):
        xs = _inputs(dt, 8, count, 15)
        assert_bitwise(run(xs, dt, ar.AR_SUM, algo), expect(xs, dt, ar.AR_SUM, algo), f"count={count} algo={algo}")


@pytest.mark.parametrize("algo", [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_RING_STEPWISE,
                                  ar.AR_ALGO_RHD_STEPWISE, ar.AR_ALGO_TREE, ar.AR_ALGO_TREE_STEPWISE])
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16, ar.AR_I32])
def test_unaligned_buffers(algo, dt):
    xs = _inputs(dt, 4, 1000, 16)
    want = expect(xs, dt, ar.AR_AVG, algo)
    assert_bitwise(run(xs, dt, ar.AR_AVG, algo, offset=1), want, f"offset 1 algo={algo}")


ONE_PASS = [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_TREE]


@pytest.mark.parametrize("offset", [1, 3, 8, 64, 127])
@pytest.mark.parametrize("algo", ONE_PASS)
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16, ar.AR_I32])
def test_same_offset_in_every_buffer_vector_path_after_a_head(offset, algo, dt):
    """Every buffer the same number of elements past an aligned address: a head of elements one by one, then
    16-byte slots (from a 256-byte boundary on 1 MiB and more). Small (per-chunk grid) and large (one-front
    ring) calls, in place and out of place, against the oracle."""
    for n, count in ((4, 1000), (8, 600_003)):
        xs = _inputs(dt, n, count, 24)
        want = expect(xs, dt, ar.AR_SUM, algo)
        for inplace in (False, True):
            got = run(xs, dt, ar.AR_SUM, algo, offset=offset, inplace=inplace)
            assert_bitwise(got, want, f"offset {offset} n={n} count={count} algo={algo} in place={inplace}")


@pytest.mark.parametrize("algo", ONE_PASS)
@pytest.mark.parametrize("in_off,out_off", [(3, 11), (0, 1), (5, 5 + 128)])
def test_inputs_and_outputs_at_different_offsets(algo, in_off, out_off):
    """Inputs and outputs at different residues: (3, 11) bf16 agree modulo 16 bytes but not 256 (16-byte head),
    (0, 1) share no residue (element path), (5, 133) agree modulo 256 bytes."""
    dt, n, count = ar.AR_BF16, 8, 600_003
    xs = _inputs(dt, n, count, 25)
    ins = [to_dev(x, dt, offset=in_off)[1] for x in xs]
    outs = [empty_like_dev(count, dt, offset=out_off)[1] for _ in xs]
    ar.ar_allreduce(ins, outs, ar.AR_MAX, algo)
    torch.cuda.synchronize()
    assert_bitwise([from_dev(o, dt) for o in outs], expect(xs, dt, ar.AR_MAX, algo), f"{in_off}/{out_off} {algo}")


# Rank counts and one-pass orders for buffers at per-rank offsets: the skewed kernel's builds (2, 4, 8, 16 for every
# order; 3, 5, 6, 7 for the ring and rank order, the trees there going element by element) and halving-doubling
# only where it is defined (a power of two).
SKEW_CASES = [(n, algo) for n in (2, 3, 4, 5, 6, 7, 8, 16)
              for algo in (ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_TREE)
              if not (algo == ar.AR_ALGO_RHD and n & (n - 1))]


@pytest.mark.parametrize("n,algo", SKEW_CASES)
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16, ar.AR_F16, ar.AR_I32])
def test_skewed_rank_buffers_every_residue(n, dt, algo):
    """Every rank's input and output at an element offset of its own (residues modulo 16 bytes all over, inputs
    and outputs different). 2-byte types (odd offsets among them): aligned loads shifted per rank, aligned stores
    assembled across lanes and carried between the tiles of a strip, wave tiles that straddle a chunk boundary
    and the first and last tiles element by element. 4-byte types: 16-byte accesses at 4-byte alignment. Counts
    with ragged chunks, and the smallest count the skewed kernel takes and one below it; out of place and in
    place, sum and min."""
    v = 16 // (2 if dt in (ar.AR_BF16, ar.AR_F16) else 4)
    for count in (64 * v * 37 + 5 * n + 3, 4 * 64 * v, 4 * 64 * v - 1):
        xs = _inputs(dt, n, count, 27)
        in_off = [(3 * r + 1) % v for r in range(n)]
        out_off = [(5 * r + 2) % v for r in range(n)]
        for op in (ar.AR_SUM, ar.AR_MIN):
            want = expect(xs, dt, op, algo)
            ins = [to_dev(x, dt, offset=in_off[r], guard=8)[1] for r, x in enumerate(xs)]
            outs = [empty_like_dev(count, dt, offset=out_off[r], guard=8) for r in range(n)]
            ar.ar_allreduce(ins, [o[1] for o in outs], op, algo)
            torch.cuda.synchronize()
            assert_bitwise([from_dev(o[1], dt) for o in outs], want, f"skewed n={n} dt={dt} count={count} op={op}")
            for r, (base, _) in enumerate(outs):  # nothing written outside the views (poisoned all-ones)
                bits = from_dev(base, dt)
                lo = 8 + out_off[r]
                full = np.iinfo(bits.dtype).max
                assert np.all(bits[:lo] == full) and np.all(bits[lo + count:] == full), f"guard band rank {r}"
            ar.ar_allreduce(ins, ins, op, algo)
            torch.cuda.synchronize()
            assert_bitwise([from_dev(t, dt) for t in ins], want, f"skewed in place n={n} dt={dt} count={count}")


@pytest.mark.parametrize("n,algo", SKEW_CASES)
@pytest.mark.parametrize("dt", [ar.AR_BF16, ar.AR_F16])
def test_skewed_outputs_at_every_line_slot(n, algo, dt):
    """2-byte rank buffers whose views start anywhere in their 128-byte lines (output rank r at 9r + 3 elements
    past a line, input at 5r + 1, both modulo 64): the skewed kernel's stores rotated per output rank onto whole
    lines, with the held-back slots carried between the tiles of a strip and stored at strip ends; every element
    against the oracle, nothing written outside the views, out of place and in place, sum and max."""
    count = 64 * 8 * 53 + 7 * n + 5
    xs = _inputs(dt, n, count, 28)
    in_off = [(5 * r + 1) % 64 for r in range(n)]
    out_off = [(9 * r + 3) % 64 for r in range(n)]
    for op in (ar.AR_SUM, ar.AR_MAX):
        want = expect(xs, dt, op, algo)
        ins = [to_dev(x, dt, offset=in_off[r], guard=64)[1] for r, x in enumerate(xs)]
        outs = [empty_like_dev(count, dt, offset=out_off[r], guard=64) for r in range(n)]
        ar.ar_allreduce(ins, [o[1] for o in outs], op, algo)
        torch.cuda.synchronize()
        assert_bitwise([from_dev(o[1], dt) for o in outs], want, f"line slots n={n} algo={algo} op={op}")
        for r, (base, _) in enumerate(outs):
            bits = from_dev(base, dt)
            lo = 64 + out_off[r]
            full = np.iinfo(bits.dtype).max
            assert np.all(bits[:lo] == full) and np.all(bits[lo + count:] == full), f"guard band rank {r}"
        ar.ar_allreduce(ins, ins, op, algo)
        torch.cuda.synchronize()
        assert_bitwise([from_dev(t, dt) for t in ins], want, f"line slots in place n={n} algo={algo} op={op}")


@pytest.mark.parametrize("algo", ONE_PASS)
@pytest.mark.parametrize("dt,step", [(ar.AR_F32, 1), (ar.AR_BF16, 2), (ar.AR_BF16, 1), (ar.AR_I32, 3)])
@pytest.mark.parametrize("count", [300_001, 5_000_011])
def test_rank_buffers_at_different_offsets(algo, dt, step, count):
    """Rank r at r*step elements past an aligned address: 4-byte types take 16-byte slots at 4-byte alignment,
    bf16 (even offsets among them) the skewed kernel. Small calls and one-front-sized ones, in place."""
    n = 8
    xs = _inputs(dt, n, count, 26)
    ins = [to_dev(x, dt, offset=r * step)[1] for r, x in enumerate(xs)]
    ar.ar_allreduce(ins, ins, ar.AR_AVG, algo)
    torch.cuda.synchronize()
    assert_bitwise([from_dev(t, dt) for t in ins], expect(xs, dt, ar.AR_AVG, algo),
                   f"per-rank offsets x{step} dt={dt} count={count} algo={algo}")


@pytest.mark.parametrize("algo", [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_RING_STEPWISE,
                                  ar.AR_ALGO_RHD_STEPWISE, ar.AR_ALGO_RING_FP8, ar.AR_ALGO_TREE,
                                  ar.AR_ALGO_TREE_STEPWISE])
def test_in_place_equals_out_of_place(algo):
    for dt in (ar.AR_F32, ar.AR_BF16):
        xs = _inputs(dt, 8, 70000, 17)
        a = run(xs, dt, ar.AR_SUM, algo)
        b = run(xs, dt, ar.AR_SUM, algo, inplace=True)
        assert_bitwise(b, a, f"in place algo={algo}")


@pytest.mark.parametrize("algo", [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_RING_STEPWISE,
                                  ar.AR_ALGO_RHD_STEPWISE, ar.AR_ALGO_RING_FP8, ar.AR_ALGO_TREE,
                                  ar.AR_ALGO_TREE_STEPWISE])
def test_guard_bands_untouched_and_every_output_written(algo):
    dt, n, count, guard = ar.AR_BF16, 8, 50001, 64
    xs = _inputs(dt, n, count, 18)
    ins = [to_dev(x, dt, guard=guard) for x in xs]
    outs = [empty_like_dev(count, dt, guard=guard, poison=True) for _ in range(n)]
    need = ar.ar_allreduce_workspace_size(n, count, dt, ar.AR_SUM, algo)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV) if need else None
    ar.ar_allreduce_ws([v for _, v in ins], [v for _, v in outs], ar.AR_SUM, algo, ws)
    torch.cuda.synchronize()
    want = expect(xs, dt, ar.AR_SUM, algo)
    for (base, view), w in zip(outs, want):
        b = from_dev(base, dt)
        assert np.all(b[:guard] == 0xFFFF) and np.all(b[guard + count:] == 0xFFFF)
        np.testing.assert_array_equal(from_dev(view, dt), w)
    for (base, _), x in zip(ins, xs):  # inputs untouched
        b = from_dev(base, dt)
        np.testing.assert_array_equal(b[guard:guard + count], x)
        assert np.all(b[:guard] == 0x5A5A) and np.all(b[guard + count:] == 0x5A5A)


def test_nan_and_signed_zero_rules():
    z = [np.array([0.0, -0.0, 1.0, np.nan, 3.0] * 40, np.float32), np.array([-0.0, 0.0, np.nan, 2.0, 4.0] * 40,
                                                                              np.float32)]
    for algo in (ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_RING_STEPWISE):
        for op in (ar.AR_MIN, ar.AR_MAX):
            assert_bitwise(run(z, ar.AR_F32, op, algo), expect(z, ar.AR_F32, op, algo), f"nan/zero op={op}")
    b = [oracle.f32_to_bf16(v) for v in z]
    for op in (ar.AR_MIN, ar.AR_MAX, ar.AR_SUM):
        got = run(b, ar.AR_BF16, op, ar.AR_ALGO_RING)
        assert_bitwise(got, expect(b, ar.AR_BF16, op, ar.AR_ALGO_RING), f"bf16 nan op={op}")


# ---------------------------------------------------------------- reordered variants within tolerance


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_fused_and_rhd_within_tolerance_of_ring(n):
    """fp32: |y - y_ring| <= 1e-6 * N * sum|x|; bf16: within 1 ulp of the ring result except where cancellation
    makes the fp32 reordering bound exceed half an ulp."""
    count = 100_003
    xs = _inputs(ar.AR_F32, n, count, 19)
    ring = run(xs, ar.AR_F32, ar.AR_SUM, ar.AR_ALGO_RING)[0].view(np.float32).astype(np.float64)
    abss = np.sum(np.abs(np.array(xs, np.float64)), axis=0)
    for algo in (ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_TREE):
        y = run(xs, ar.AR_F32, ar.AR_SUM, algo)[0].view(np.float32).astype(np.float64)
        assert np.all(np.abs(y - ring) <= 1e-6 * n * abss)
    xb = inputs.rank_inputs("normal_bf16", n, count, cfg=19)
    ringb = run(xb, ar.AR_BF16, ar.AR_SUM, ar.AR_ALGO_RING)[0]
    rf = oracle.bf16_to_f32(ringb).astype(np.float64)
    absb = np.sum(np.abs(np.array([oracle.bf16_to_f32(x) for x in xb], np.float64)), axis=0)
    ulp = np.abs(rf) * 2.0 ** -7
    ulp = np.maximum(ulp, 2.0 ** -133)
    reorder = 2 * (n - 1) * 2.0 ** -24 * absb
    for algo in (ar.AR_ALGO_FUSED, ar.AR_ALGO_RHD, ar.AR_ALGO_TREE):
        yb = oracle.bf16_to_f32(run(xb, ar.AR_BF16, ar.AR_SUM, algo)[0]).astype(np.float64)
        d = np.abs(yb - rf)
        tol = np.where(reorder > ulp / 2, ulp + reorder, ulp)
        assert np.all(d <= tol)


# ---------------------------------------------------------------- the small ring workload: N=4, 1M fp32


def test_four_rank_one_million_fp32_ring():
    n, count = 4, 1 << 20
    xs = inputs.rank_inputs("uniform_f32", n, count, cfg=1)
    got = run(xs, ar.AR_F32, ar.AR_SUM, ar.AR_ALGO_RING)
    want = expect(xs, ar.AR_F32, ar.AR_SUM, ar.AR_ALGO_RING)
    assert_bitwise(got, want, "N=4 1M fp32")
    lo = oracle.chunk_bounds(count, n)
    assert list(np.diff(lo)) == [262144] * 4


# ---------------------------------------------------------------- buckets


def test_bucket_pack_unpack_round_trip():
    rng = np.random.default_rng(5)
    sizes = [1, 3, 4, 5, 1000, 4096, 17, 70001, 0, 2]
    for dt, tdt in ((ar.AR_F32, torch.float32), (ar.AR_BF16, torch.bfloat16)):
        src = [torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(tdt).to(DEV) for s in sizes]
        es = src[0].element_size()
        g = 16 // es
        total = sum((s + g - 1) // g * g for s in sizes) + 8 * g
        bucket = torch.full((total,), 7, dtype=tdt, device=DEV)
        back = [torch.full_like(t, 3) for t in src]
        tasks, offs, off = [], [], 0
        for t, s in zip(src, sizes):
            pad = (s + g - 1) // g * g - s
            tasks.append((t.data_ptr(), bucket.data_ptr() + off * es, s, pad))
            offs.append(off)
            off += s + pad
        ar.ar_bucket_pack(ar.make_copy_descs(tasks, DEV), dt)
        ar.ar_bucket_unpack(ar.make_copy_descs([(bucket.data_ptr() + o * es, b.data_ptr(), s, 0)
                                                for o, b, s in zip(offs, back, sizes)], DEV), dt)
        torch.cuda.synchronize()
        for t, b in zip(src, back):
            assert torch.equal(t, b)
        hb = bucket.cpu()
        for t, o, s in zip(src, offs, sizes):
            assert torch.equal(hb[o:o + s], t.cpu())
            pad = (s + g - 1) // g * g - s
            assert torch.all(hb[o + s:o + s + pad] == 0)
        assert torch.all(hb[off:] == 7)  # nothing written past the last pad


@pytest.mark.parametrize("n", [2, 8])
def test_bucketed_allreduce_matches_oracle(n):
    sizes = inputs.bucket_sizes(ntensors=40, lo_log2=4, hi_log2=16, seed_parts=(3, 1000 + n))
    cap = 64 << 10
    host = [inputs.bucket_tensors(r, sizes) for r in range(n)]
    ins = [[torch.from_numpy(t).to(DEV) for t in host[r]] for r in range(n)]
    outs = [[torch.full_like(t, float("nan")) for t in ins[r]] for r in range(n)]
    bar = ar.BucketedAllReduce(ins, outs, op=ar.AR_AVG, cap_bytes=cap)
    assert bar.nbuckets > 3
    bar()
    torch.cuda.synchronize()
    want = oracle.bucketed_allreduce(host, oracle.F32, oracle.AVG, cap_bytes=cap)
    for r in range(n):
        for t in range(len(sizes)):
            np.testing.assert_array_equal(outs[r][t].cpu().numpy().view(np.uint32), want[r][t].view(np.uint32))


# ---------------------------------------------------------------- fp8 codec and compressed ring


def _special_fp32(count, seed):
    x = inputs.normal_f32((seed,), count, 1.0)
    x[::101] *= np.float32(1e4)
    x[::103] = np.float32(0.0)
    x[5:128] = np.float32(0.0)  # a zero block
    x[256:384] = np.float32(3e-39)  # subnormal block
    x[384:512] = np.float32(1e-44)  # block whose inverse scale overflows
    if count > 800:
        x[600] = np.float32(np.nan)  # NaN never counts towards a block's amax and encodes as 0x7F
        x[700] = -np.float32(np.nan)
    return x


def _f32_bits_equal_nan_aware(got_bits, want_bits):
    """fp32 outputs: NaN payloads are unspecified, so NaN matches NaN; everything else bit for bit."""
    g = np.asarray(got_bits).view(np.uint32)
    w = np.asarray(want_bits).view(np.uint32)
    gn = (g & 0x7FFFFFFF) > 0x7F800000
    wn = (w & 0x7FFFFFFF) > 0x7F800000
    np.testing.assert_array_equal(gn, wn)
    np.testing.assert_array_equal(g[~gn], w[~wn])


@pytest.mark.parametrize("count", [1, 100, 128, 129, 1000, 128 * 1000 + 77])
def test_fp8_quant_dequant_match_oracle(count):
    x = _special_fp32(max(count, 512), 21)[:count]
    xd = torch.from_numpy(x).to(DEV)
    nb = (count + 127) // 128
    codes = torch.empty(count, dtype=torch.uint8, device=DEV)
    scales = torch.empty(nb, dtype=torch.float32, device=DEV)
    ar.ar_fp8_quant(xd, codes, scales)
    out = torch.empty(count, dtype=torch.float32, device=DEV)
    ar.ar_fp8_dequant(codes, scales, out)
    outb = torch.empty(count, dtype=torch.bfloat16, device=DEV)
    ar.ar_fp8_dequant(codes, scales, outb)
    torch.cuda.synchronize()
    wc, ws = oracle.fp8_quant(x, oracle.F32)
    np.testing.assert_array_equal(codes.cpu().numpy(), wc)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    _f32_bits_equal_nan_aware(out.cpu().numpy(), oracle.fp8_dequant(wc, ws, oracle.F32))
    np.testing.assert_array_equal(from_dev(outb, ar.AR_BF16), oracle.fp8_dequant(wc, ws, oracle.BF16))
    # bf16 input path
    xb = oracle.f32_to_bf16(x)
    ar.ar_fp8_quant(to_dev(xb, ar.AR_BF16)[1], codes, scales)
    torch.cuda.synchronize()
    wc, ws = oracle.fp8_quant(xb, oracle.BF16)
    np.testing.assert_array_equal(codes.cpu().numpy(), wc)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("x_off,c_off,o_off", [(1, 0, 0), (0, 3, 0), (0, 0, 1), (3, 5, 2)])
def test_fp8_codec_at_unaligned_offsets(x_off, c_off, o_off):
    """Inputs, codes and outputs as views off the 16-byte grid (element offsets for fp32 and bf16, byte offsets for
    codes): the element-by-element paths of both codec kernels, against the oracle."""
    count = 128 * 37 + 51
    x = _special_fp32(count, 23)
    xb_all = torch.empty(count + 8, dtype=torch.float32, device=DEV)
    xd = xb_all[x_off:x_off + count]
    xd.copy_(torch.from_numpy(x))
    cb = torch.empty(count + 16, dtype=torch.uint8, device=DEV)
    codes = cb[c_off:c_off + count]
    scales = torch.empty((count + 127) // 128, dtype=torch.float32, device=DEV)
    ar.ar_fp8_quant(xd, codes, scales)
    ob = torch.empty(count + 8, dtype=torch.float32, device=DEV)
    out = ob[o_off:o_off + count]
    ar.ar_fp8_dequant(codes, scales, out)
    obb = torch.empty(count + 8, dtype=torch.bfloat16, device=DEV)
    outb = obb[o_off:o_off + count]
    ar.ar_fp8_dequant(codes, scales, outb)
    torch.cuda.synchronize()
    wc, ws = oracle.fp8_quant(x, oracle.F32)
    np.testing.assert_array_equal(codes.cpu().numpy(), wc)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    _f32_bits_equal_nan_aware(out.cpu().numpy(), oracle.fp8_dequant(wc, ws, oracle.F32))
    np.testing.assert_array_equal(from_dev(outb, ar.AR_BF16), oracle.fp8_dequant(wc, ws, oracle.BF16))


def test_fp8_encoder_dense_sweep_of_fp32_patterns():
    """Every 997th fp32 bit pattern with |v| <= 448, quantized in blocks whose amax is exactly 448 (scale 1), so
    the E4M3 encoder sees raw values across all binades, ties included."""
    pats = np.arange(0, 1 << 32, 997, dtype=np.uint64).astype(np.uint32)
    v = pats.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    m = v.size // 127 * 127
    blocks = v[:m].reshape(-1, 127)
    x = np.concatenate([np.full((blocks.shape[0], 1), 448.0, np.float32), blocks], axis=1).reshape(-1)
    xd = torch.from_numpy(x).to(DEV)
    codes = torch.empty(x.size, dtype=torch.uint8, device=DEV)
    scales = torch.empty(x.size // 128, dtype=torch.float32, device=DEV)
    ar.ar_fp8_quant(xd, codes, scales)
    torch.cuda.synchronize()
    wc, ws = oracle.fp8_quant(x, oracle.F32)
    assert np.all(ws == 1.0)
    np.testing.assert_array_equal(codes.cpu().numpy(), wc)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("count", [1000, 128 * 8 * 40, 128 * 8 * 40 + 13])
def test_fp8_ring_matches_oracle(n, count):
    for dt in (ar.AR_BF16, ar.AR_F32):
        if dt == ar.AR_BF16:
            xs = inputs.rank_inputs("outlier_bf16", n, count, cfg=5, extra=(n, count))
        else:
            xs = [_special_fp32(count, 30 + r) for r in range(n)]
        for op in (ar.AR_SUM, ar.AR_AVG):
            got = run(xs, dt, op, ar.AR_ALGO_RING_FP8)
            want = expect(xs, dt, op, ar.AR_ALGO_RING_FP8)
            if dt == ar.AR_F32:
                for g, w in zip(got, want):
                    _f32_bits_equal_nan_aware(g, w)
            else:
                assert_bitwise(got, want, f"fp8 ring n={n} count={count} dt={dt}")


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7, 8, 12])
@pytest.mark.parametrize("extra", [1, 3, 5, 7, 26, 4096 * 3 + 5])
@pytest.mark.parametrize("dt", [ar.AR_BF16, ar.AR_F32])
def test_fp8_ring_chunks_off_the_16_byte_grid(n, extra, dt):
    """Counts that are not a multiple of 8 N (bf16) or 4 N (fp32) put chunk starts 1..7 (1..3) elements past the
    16-byte grid (n = 8, extra = 7 gives every bf16 one); chunks of several 512-element wave tasks take shifted
    vector loads and lane-exchanged aligned stores carried along strips of tasks, the chunk ends and the last
    slots of the buffer element by element. Rank counts other than 2, 4, 8 run the build whose rank count is known
    only at run time, which loads and shifts one rank after another. Bitwise against the oracle, out of place and in
    place."""
    count = n * 4096 + extra
    kind = "outlier_bf16" if dt == ar.AR_BF16 else "uniform_f32"
    xs = inputs.rank_inputs(kind, n, count, cfg=6, extra=(n, count))
    for op in (ar.AR_SUM, ar.AR_AVG):
        want = expect(xs, dt, op, ar.AR_ALGO_RING_FP8)
        assert_bitwise(run(xs, dt, op, ar.AR_ALGO_RING_FP8), want, f"fp8 ring n={n} count={count} dt={dt}")
        assert_bitwise(run(xs, dt, op, ar.AR_ALGO_RING_FP8, inplace=True), want,
                       f"fp8 ring in place n={n} count={count} dt={dt}")


@pytest.mark.parametrize("n", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("q", [4096 + 8, 4096 + 24, 4096 + 64 + 56, 4096 + 3, 4096 + 4, 4096 + 13])
@pytest.mark.parametrize("out_offs", ["aligned", "common_16B", "common_80B", "mixed"])
@pytest.mark.parametrize("dt", [ar.AR_BF16, ar.AR_F32])
def test_fp8_ring_chunk_starts_off_the_line_grid(n, q, out_offs, dt):
    """Chunk starts on the 16-byte grid but off the 128-byte line grid (bf16: q = 4104, 4120, 4216 elements per
    chunk; fp32: also 4100), or off both (4099, 4109), with every output buffer at the same place in its line
    (aligned, 16 or 80 bytes in: the rotated aligned stores) or at different places (rank r at 16 (r % 2) bytes:
    unrotated): bitwise against the oracle, every element of every rank."""
    count = n * q
    kind = "outlier_bf16" if dt == ar.AR_BF16 else "uniform_f32"
    xs = inputs.rank_inputs(kind, n, count, cfg=7, extra=(n, q))
    per16 = 8 if dt == ar.AR_BF16 else 4  # elements in 16 bytes
    offs = {"aligned": [0] * n, "common_16B": [per16] * n, "common_80B": [5 * per16] * n,
            "mixed": [per16 * (r % 2) for r in range(n)]}[out_offs]
    ins = [to_dev(x, dt)[1] for x in xs]
    outs = [empty_like_dev(count, dt, offset=o, guard=64)[1] for o in offs]
    for op in (ar.AR_SUM, ar.AR_AVG):
        ar.ar_allreduce(ins, outs, op, ar.AR_ALGO_RING_FP8)
        torch.cuda.synchronize()
        assert_bitwise([from_dev(o, dt) for o in outs], expect(xs, dt, op, ar.AR_ALGO_RING_FP8),
                       f"fp8 ring n={n} q={q} dt={dt} outputs {out_offs}")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16, ar.AR_I32])
def test_allreduce_buckets_equals_one_call_per_bucket(n, dt):
    """One launch over many buckets (more than one launch's worth of segments, some empty) gives exactly the
    bits of one ar_allreduce per bucket, in place and out of place, for every op and one-pass algorithm."""
    unit = n * (16 // (2 if dt == ar.AR_BF16 else 4))
    rng = np.random.default_rng(n * 10 + dt)
    counts = (rng.integers(0, 40, 150) * unit).astype(np.int64)
    counts[[3, 77]] = 0
    counts[5] = unit * 3001
    total = int(counts.sum())
    xs = _inputs(dt, n, total, 20)
    starts = np.concatenate([[0], np.cumsum(counts)])
    algos = [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_TREE] + ([ar.AR_ALGO_RHD] if n & (n - 1) == 0 else [])
    for algo in algos:
        for op in OPS:
            want_flat = [np.empty(total, dtype=NP_BITS[dt]) for _ in range(n)]
            for b in range(len(counts)):
                if counts[b] == 0:
                    continue
                seg = [x.view(NP_BITS[dt])[starts[b]:starts[b + 1]] for x in xs]
                got_b = expect([s.view(xs[0].dtype) for s in seg], dt, op, algo)
                for r in range(n):
                    want_flat[r][starts[b]:starts[b + 1]] = got_b[r]
            ins = [to_dev(x, dt)[1] for x in xs]
            outs = [empty_like_dev(total, dt)[1] for _ in range(n)]
            ar.ar_allreduce_buckets(ins, outs, counts, op, algo)
            torch.cuda.synchronize()
            assert_bitwise([from_dev(o, dt) for o in outs], want_flat, f"buckets n={n} op={op} algo={algo}")
            ar.ar_allreduce_buckets(ins, ins, counts, op, algo)  # in place
            torch.cuda.synchronize()
            assert_bitwise([from_dev(o, dt) for o in ins], want_flat, f"buckets in place n={n} op={op}")


@pytest.mark.parametrize("n,dt", [(3, ar.AR_F32), (4, ar.AR_BF16)])
def test_allreduce_buckets_mixing_own_launch_and_shared_launch_buckets(n, dt):
    """Buckets of 16 MiB or more per rank get a launch of their own and the runs of smaller buckets between them
    share segment launches; the result must still be one ring per bucket, in place and out of place."""
    es = 2 if dt == ar.AR_BF16 else 4
    unit = n * (16 // es)
    big = ((16 << 20) // es + unit - 1) // unit * unit  # exactly 16 MiB per rank, rounded up to the unit
    counts = np.array([unit * 5, big, unit * 7, 0, unit * 3, big + unit * 11, unit], dtype=np.int64)
    total = int(counts.sum())
    xs = _inputs(dt, n, total, 22)
    starts = np.concatenate([[0], np.cumsum(counts)])
    for op in (ar.AR_SUM, ar.AR_AVG):
        want = [np.empty(total, dtype=NP_BITS[dt]) for _ in range(n)]
        for b in range(len(counts)):
            if counts[b]:
                seg = [x.view(NP_BITS[dt])[starts[b]:starts[b + 1]].view(xs[0].dtype) for x in xs]
                for r, w in enumerate(expect(seg, dt, op, ar.AR_ALGO_RING)):
                    want[r][starts[b]:starts[b + 1]] = w
        ins = [to_dev(x, dt)[1] for x in xs]
        outs = [empty_like_dev(total, dt)[1] for _ in range(n)]
        ar.ar_allreduce_buckets(ins, outs, counts, op, ar.AR_ALGO_RING)
        torch.cuda.synchronize()
        assert_bitwise([from_dev(o, dt) for o in outs], want, f"mixed buckets n={n} op={op}")
        ar.ar_allreduce_buckets(ins, ins, counts, op, ar.AR_ALGO_RING)
        torch.cuda.synchronize()
        assert_bitwise([from_dev(o, dt) for o in ins], want, f"mixed buckets in place n={n} op={op}")


@pytest.mark.parametrize("algo", [ar.AR_ALGO_RING, ar.AR_ALGO_RHD, ar.AR_ALGO_RING_STEPWISE, ar.AR_ALGO_RING_FP8,
                                  ar.AR_ALGO_TREE_STEPWISE])
def test_hip_graph_capture_replays_match_eager(algo):
    """Calls captured in a HIP graph replay to the eager result, every replay, with eager work in between."""
    n, count = 8, 50_003
    dt = ar.AR_BF16
    xs = inputs.rank_inputs("normal_bf16", n, count, cfg=31)
    ins = [to_dev(x, dt)[1] for x in xs]
    outs = [empty_like_dev(count, dt)[1] for _ in range(n)]
    need = ar.ar_allreduce_workspace_size(n, count, dt, ar.AR_SUM, algo)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV) if need else None
    call = lambda: ar.ar_allreduce_ws(ins, outs, ar.AR_SUM, algo, ws)
    call()
    torch.cuda.synchronize()
    eager = [from_dev(o, dt) for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for o in outs:
            o.view(torch.int16).fill_(-1)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise([from_dev(o, dt) for o in outs], eager, f"graph replay {rep} algo={algo}")


ORACLE_BUCKET_ALGO = {ar.AR_ALGO_RING: "ring", ar.AR_ALGO_FUSED: "fused", ar.AR_ALGO_RHD: "rhd",
                      ar.AR_ALGO_TREE: "tree"}


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16, ar.AR_I32])
def test_bucketed_paths_match_the_oracle_in_every_order(n, dt):
    """Both bucketed paths, pack + per-bucket all-reduce + unpack (BucketedAllReduce) and the fused path that
    reads and writes the tensors directly (ar_allreduce_tensors), against the oracle's bucketed all-reduce in the
    same order (its plan, zero-padded packing on the host, the literal ring / rank-order / halving / binomial
    oracle per bucket, unpacking), every op. Small caps make buckets whose chunks are shorter than a tile, odd
    sizes leave element tails, and one tensor starting one element into its allocation takes the element path."""
    rng = np.random.default_rng(40 + n + 10 * dt)
    sizes = [int(s) for s in rng.integers(1, 3000, 23)] + [1, 2, 9, 70001, 4096, 40000]
    algos = [ar.AR_ALGO_RING, ar.AR_ALGO_FUSED, ar.AR_ALGO_TREE] + ([ar.AR_ALGO_RHD] if n & (n - 1) == 0 else [])
    for cap in (4096, 200 << 10):
        host = [[inputs.rank_inputs(KIND[dt], 1, s, cfg=41, extra=(r, t, n))[0] for t, s in enumerate(sizes)]
                for r in range(n)]
        ins, bases = [], []
        for r in range(n):
            row = []
            for t, s in enumerate(sizes):
                base, view = to_dev(host[r][t], dt, offset=1 if t == 5 else 0)
                bases.append(base)
                row.append(view)
            ins.append(row)
        for algo in algos:
            for op in OPS:
                want = oracle.bucketed_allreduce(host, ORACLE_DT[dt], ORACLE_OP[op], cap_bytes=cap,
                                                 algo=ORACLE_BUCKET_ALGO[algo])
                packed = [[torch.empty_like(x) for x in ins[r]] for r in range(n)]
                fused = [[torch.empty_like(x) for x in ins[r]] for r in range(n)]
                ar.BucketedAllReduce(ins, packed, op=op, algo=algo, cap_bytes=cap)()
                ar.BucketedAllReduce(ins, fused, op=op, algo=algo, cap_bytes=cap).fused()
                torch.cuda.synchronize()
                for path, got in (("pack+reduce+unpack", packed), ("fused tensors", fused)):
                    for r in range(n):
                        for t in range(len(sizes)):
                            g = from_dev(got[r][t], dt)
                            w = np.asarray(want[r][t]).view(NP_BITS[dt])
                            if not np.array_equal(g, w):
                                bad = np.nonzero(g != w)[0][:5]
                                raise AssertionError(f"{path}: n={n} dt={dt} cap={cap} algo={algo} op={op} rank {r} "
                                                     f"tensor {t} (numel {sizes[t]}): first differences at {bad}")


def _chunks(x_np, lo):
    return [x_np[lo[c]:lo[c + 1]] for c in range(len(lo) - 1)]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("count", [1, 7, 64, 4099, 65536, "many_tiles", "many_tiles_ragged"])
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16, ar.AR_I32])
def test_reduce_scatter_and_all_gather_match_oracle(n, count, dt):
    if count in ("many_tiles", "many_tiles_ragged"):
        # several tiles per block on the one-front grid; slot-aligned chunk starts, or starts inside slots (the
        # shifted vector path, plus each chunk's edge elements)
        count = n * (16 // (2 if dt == ar.AR_BF16 else 4)) * 150_001 + (13 if count == "many_tiles_ragged" else 0)
    xs = _inputs(dt, n, count, 50)
    lo = ar.chunk_bounds(count, n)
    tdt = {ar.AR_F32: torch.float32, ar.AR_BF16: torch.bfloat16, ar.AR_I32: torch.int32}[dt]
    for op in OPS:
        ins = [to_dev(x, dt)[1] for x in xs]
        outs = [torch.empty(lo[c + 1] - lo[c], dtype=tdt, device=DEV) for c in range(n)]
        ar.ar_reduce_scatter(ins, outs, op)
        torch.cuda.synchronize()
        want = oracle.reduce_scatter(xs, ORACLE_DT[dt], ORACLE_OP[op])
        for c in range(n):
            np.testing.assert_array_equal(from_dev(outs[c], dt), np.asarray(want[c]).view(NP_BITS[dt]))
        # all-gather of the reduced chunks reproduces the ring all-reduce bit for bit
        full = [empty_like_dev(count, dt)[1] for _ in range(n)]
        ar.ar_all_gather(outs, full)
        torch.cuda.synchronize()
        ring = expect(xs, dt, op, ar.AR_ALGO_RING)
        assert_bitwise([from_dev(f, dt) for f in full], ring, f"RS then AG n={n} count={count} op={op}")
    # all-gather against the oracle with arbitrary parts
    parts = _chunks(xs[0].view(NP_BITS[dt]), lo)
    pin = [to_dev(p.view(xs[0].dtype), dt)[1] if p.size else None for p in parts]
    full = [empty_like_dev(count, dt)[1] for _ in range(n)]
    ar.ar_all_gather(pin, full)
    torch.cuda.synchronize()
    want = oracle.allgather([p.view(xs[0].dtype) for p in parts], ORACLE_DT[dt])
    assert_bitwise([from_dev(f, dt) for f in full], [np.asarray(w).view(NP_BITS[dt]) for w in want], "all-gather")


@pytest.mark.parametrize("layout", ["full_at_common_offset", "chunks_at_offsets", "both_offset",
                                    "full_at_different_offsets", "full_at_different_even_offsets",
                                    "in_place_full_offset"])
@pytest.mark.parametrize("n,count", [(3, 5003), (8, 1_200_013), (5, 80_003)])
@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_BF16])
def test_reduce_scatter_and_all_gather_at_any_alignment(layout, n, count, dt):
    """Full buffers and chunk buffers at any element offset: a common offset of the full buffers (a head, then
    slots), chunk buffers at assorted offsets (each vector assembled from two aligned slots), in place inside
    offset full buffers (no shift), and full buffers at different residues (slots at 4-byte alignment from
    element 0 where every address is a multiple of 4, else element by element). Every result bit-exact against
    the oracle; RS then AG equals the ring all-reduce."""
    xs = _inputs(dt, n, count, 53)
    lo = ar.chunk_bounds(count, n)
    full_off = {"full_at_common_offset": [3] * n, "chunks_at_offsets": [0] * n, "both_offset": [1] * n,
                "full_at_different_offsets": list(range(n)), "full_at_different_even_offsets": [2 * r for r in range(n)],
                "in_place_full_offset": [5] * n}[layout]
    part_off = [(c * 3 + 1) % 8 for c in range(n)] if layout in ("chunks_at_offsets", "both_offset") else [0] * n
    full = [to_dev(x, dt, offset=full_off[r])[1] for r, x in enumerate(xs)]
    if layout == "in_place_full_offset":
        parts = [full[c][lo[c]:lo[c + 1]] for c in range(n)]
    else:
        parts = [empty_like_dev(lo[c + 1] - lo[c], dt, offset=part_off[c])[1] for c in range(n)]
    ar.ar_reduce_scatter(full, parts, ar.AR_SUM)
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, ORACLE_DT[dt], ORACLE_OP[ar.AR_SUM])
    for c in range(n):
        np.testing.assert_array_equal(from_dev(parts[c], dt), np.asarray(want[c]).view(NP_BITS[dt]),
                                      err_msg=f"reduce-scatter {layout} chunk {c}")
    outs = full if layout == "in_place_full_offset" else [empty_like_dev(count, dt, offset=full_off[r])[1]
                                                          for r in range(n)]
    ar.ar_all_gather(parts, outs)
    torch.cuda.synchronize()
    assert_bitwise([from_dev(o, dt) for o in outs], expect(xs, dt, ar.AR_SUM, ar.AR_ALGO_RING),
                   f"RS then AG {layout} n={n} count={count}")


def test_reduce_scatter_all_gather_page_examples_and_in_place():
    # two-rank reduce-scatter halves and the four-rank all-gather placement (tests/golden fixtures)
    ins = [torch.tensor(v, dtype=torch.int32, device=DEV) for v in ([1, 2, 3, 4], [10, 20, 30, 40])]
    outs = [torch.empty(2, dtype=torch.int32, device=DEV) for _ in range(2)]
    ar.ar_reduce_scatter(ins, outs)
    assert outs[0].tolist() == [11, 22] and outs[1].tolist() == [33, 44]
    parts = [torch.tensor([v], dtype=torch.int32, device=DEV) for v in (65, 66, 67, 68)]
    full = [torch.zeros(4, dtype=torch.int32, device=DEV) for _ in range(4)]
    ar.ar_all_gather(parts, full)
    assert all(f.tolist() == [65, 66, 67, 68] for f in full)
    # in place: each rank's chunk lives at its own position in its full buffer
    n, count = 8, 80_000
    xs = _inputs(ar.AR_F32, n, count, 51)
    lo = ar.chunk_bounds(count, n)
    bufs = [to_dev(x, ar.AR_F32)[1] for x in xs]
    ar.ar_reduce_scatter(bufs, [bufs[c][lo[c]:lo[c + 1]] for c in range(n)], ar.AR_SUM)
    ar.ar_all_gather([bufs[c][lo[c]:lo[c + 1]] for c in range(n)], bufs)
    torch.cuda.synchronize()
    assert_bitwise([from_dev(b, ar.AR_F32) for b in bufs], expect(xs, ar.AR_F32, ar.AR_SUM, ar.AR_ALGO_RING),
                   "in-place RS + AG")
    # in place with chunk starts inside 16-byte slots (the chunk views are then not 16-byte aligned)
    n, count = 5, 80_003
    xs = _inputs(ar.AR_BF16, n, count, 52)
    lo = ar.chunk_bounds(count, n)
    bufs = [to_dev(x, ar.AR_BF16)[1] for x in xs]
    ar.ar_reduce_scatter(bufs, [bufs[c][lo[c]:lo[c + 1]] for c in range(n)], ar.AR_AVG)
    ar.ar_all_gather([bufs[c][lo[c]:lo[c + 1]] for c in range(n)], bufs)
    torch.cuda.synchronize()
    assert_bitwise([from_dev(b, ar.AR_BF16) for b in bufs], expect(xs, ar.AR_BF16, ar.AR_AVG, ar.AR_ALGO_RING),
                   "in-place RS + AG, ragged")


def test_allreduce_on_a_side_stream_beside_other_kernels_is_bit_exact():
    """The all-reduce on its own stream, running concurrently with a copy and a GEMM on another stream."""
    n, count = 8, 3_000_007
    xs = inputs.rank_inputs("normal_bf16", n, count, cfg=60)
    ins = [to_dev(x, ar.AR_BF16)[1] for x in xs]
    outs = [empty_like_dev(count, ar.AR_BF16)[1] for _ in range(n)]
    s_ar, s_p = torch.cuda.Stream(), torch.cuda.Stream()
    a = torch.randn(2048, 2048, device=DEV)
    src = torch.randn(1 << 24, device=DEV)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    with torch.cuda.stream(s_p):
        for _ in range(4):
            torch.mm(a, a)
            dst.copy_(src)
    ar.ar_allreduce(ins, outs, ar.AR_AVG, ar.AR_ALGO_RING, stream=s_ar)
    torch.cuda.synchronize()
    assert_bitwise([from_dev(o, ar.AR_BF16) for o in outs], expect(xs, ar.AR_BF16, ar.AR_AVG, ar.AR_ALGO_RING),
                   "side stream")
    assert torch.equal(dst, src)


def test_concurrent_calls_from_host_threads_on_their_own_streams():
    """The library keeps no shared state across calls (the last-call record is per thread): four host threads,
    each with its own stream, algorithm and inputs, call at once; every result matches the oracle and every
    thread sees its own last call."""
    import threading
    cases = [(ar.AR_ALGO_RING, ar.AR_BF16, 8, 2_000_003), (ar.AR_ALGO_TREE, ar.AR_F32, 5, 700_001),
             (ar.AR_ALGO_FUSED, ar.AR_BF16, 3, 900_007), (ar.AR_ALGO_RHD, ar.AR_I32, 4, 1_000_003)]
    data = []
    for k, (algo, dt, n, count) in enumerate(cases):
        xs = _inputs(dt, n, count, 70 + k)
        ins = [to_dev(x, dt)[1] for x in xs]
        outs = [empty_like_dev(count, dt)[1] for _ in range(n)]
        data.append((xs, ins, outs, torch.cuda.Stream()))
    torch.cuda.synchronize()
    barrier = threading.Barrier(len(cases))
    records, errors = [None] * len(cases), []

    def work(k):
        try:
            algo, dt, n, count = cases[k]
            _, ins, outs, s = data[k]
            barrier.wait()
            for _ in range(3):
                ar.ar_allreduce(ins, outs, ar.AR_SUM, algo, stream=s)
            records[k] = ar.ar_last_call()
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    for k, (algo, dt, n, count) in enumerate(cases):
        xs, _, outs, _ = data[k]
        assert records[k]["algo"] == algo and records[k]["count"] == count and records[k]["nranks"] == n
        assert_bitwise([from_dev(o, dt) for o in outs], expect(xs, dt, ar.AR_SUM, algo), f"thread {k} algo {algo}")
