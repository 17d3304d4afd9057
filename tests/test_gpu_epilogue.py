"""The owner's epilogue through ar_epilogue, against the oracle's.

- every one of the 2^32 fp32 bit patterns through the bf16 rounding and through the f16 rounding (sum: no
  division), and through the fp32 average by 3 (one IEEE division each, subnormals included): bit for bit, NaN
  inputs to the canonical NaN of bf16/f16 and to some NaN in fp32;
- int32 averages (truncating division) at the extremes and on random values;
- every dtype and op at ragged counts, with partials and outputs at element offsets off the 16-byte grid, in place
  for the 4-byte types, and nothing written outside the output.

The kernels apply the same element functions in registers before their stores, so the first group checks the
rounding of every result the library produces, over every value a sum in fp32 can take.
"""
import concurrent.futures

import numpy as np
import pytest
import torch

import all_reduce_reduction_ring_amd as ar
import oracle
from gpu_util import DEV, NP_BITS, ORACLE_DT, ORACLE_OP, TORCH_DT, empty_like_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu

SLAB = 1 << 28  # fp32 patterns per launch
HOST_THREADS = 16


def _oracle_threads(acc, dt, op, n):
    """The oracle over slices of acc on host threads (its C loop runs without the interpreter lock)."""
    parts = np.array_split(acc, HOST_THREADS)
    with concurrent.futures.ThreadPoolExecutor(HOST_THREADS) as ex:
        return np.concatenate(list(ex.map(lambda p: oracle.epilogue(p, ORACLE_DT[dt], ORACLE_OP[op], n), parts)))


EXHAUSTIVE = [(ar.AR_BF16, ar.AR_SUM, 1), (ar.AR_F16, ar.AR_SUM, 1), (ar.AR_F32, ar.AR_AVG, 3)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dt,op,n", EXHAUSTIVE, ids=["bf16_round", "f16_round", "f32_avg3"])
def test_every_fp32_pattern(dt, op, n):
    print(f"case dt={dt} op={op} n={n}", flush=True)
    acc = torch.empty(SLAB, dtype=torch.int32, device=DEV)
    out = torch.empty(SLAB, dtype=TORCH_DT[dt], device=DEV)
    for lo in range(-(1 << 31), 1 << 31, SLAB):
        torch.arange(lo, lo + SLAB, dtype=torch.int32, device=DEV, out=acc)
        ar.ar_epilogue(acc.view(torch.float32), out, op, n)
        got = from_dev(out, dt)
        pats = np.arange(lo, lo + SLAB, dtype=np.int32).view(np.float32)
        want = _oracle_threads(pats, dt, op, n).view(NP_BITS[dt])
        if dt == ar.AR_F32:
            # NaN payloads of fp32 results are not specified: NaN where the oracle has NaN, bits elsewhere
            gn, wn = np.isnan(got.view(np.float32)), np.isnan(want.view(np.float32))
            bad = np.nonzero((gn != wn) | (~wn & (got != want)))[0]
        else:
            bad = np.nonzero(got != want)[0]
        if bad.size:
            b = bad[:5]
            raise AssertionError(f"{bad.size} results differ in slab from {lo}; inputs "
                                 f"{pats[b].view(np.uint32)}: got {got[b]} want {want[b]}")


def test_int32_average_truncates():
    rng = np.random.default_rng(5)
    edges = np.array([0, 1, -1, 2, -2, 3, -3, 63, -63, 64, -64, 65, -65, 2 ** 31 - 1, -2 ** 31, -2 ** 31 + 1],
                     np.int64)
    x = np.concatenate([edges, rng.integers(-2 ** 31, 2 ** 31, 1 << 22)]).astype(np.int32)
    acc = torch.from_numpy(x).to(DEV)
    for n in (1, 2, 3, 7, 64):
        out = torch.empty_like(acc)
        ar.ar_epilogue(acc, out, ar.AR_AVG, n)
        np.testing.assert_array_equal(out.cpu().numpy(), oracle.epilogue(x, oracle.I32, oracle.AVG, n))


def _partials(dt, count, seed):
    rng = np.random.default_rng(seed)
    if dt == ar.AR_I32:
        return rng.integers(-2 ** 31, 2 ** 31, count).astype(np.int32)
    v = (rng.standard_normal(count) * 10.0 ** rng.integers(-6, 6, count)).astype(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.3895314e38, 65520.0, 1e-45], np.float32)
    v[: min(count, special.size)] = special[: min(count, special.size)]
    return v


CASES = [(dt, op) for dt in (ar.AR_F32, ar.AR_BF16, ar.AR_F16, ar.AR_I32)
         for op in (ar.AR_SUM, ar.AR_AVG, ar.AR_MIN, ar.AR_MAX)]


@pytest.mark.parametrize("dt,op", CASES, ids=[f"dt{c[0]}_op{c[1]}" for c in CASES])
def test_ragged_counts_offsets_and_guards(dt, op):
    acc_dt = ar.AR_I32 if dt == ar.AR_I32 else ar.AR_F32
    for count in (1, 7, 8, 9, 2047, 1_000_003):
        for acc_off, out_off in ((0, 0), (1, 0), (0, 1), (3, 5)):
            x = _partials(dt, count, seed=count + 10 * acc_off + out_off)
            _, acc = to_dev(x, acc_dt, offset=acc_off, guard=64)
            obase, out = empty_like_dev(count, dt, offset=out_off, guard=64)
            ar.ar_epilogue(acc, out, op, 5)
            want = oracle.epilogue(x, ORACLE_DT[dt], ORACLE_OP[op], 5).view(NP_BITS[dt])
            got = from_dev(out, dt)
            if dt == ar.AR_F32:
                wn, gn = np.isnan(want.view(np.float32)), np.isnan(got.view(np.float32))
                np.testing.assert_array_equal(gn, wn)
                np.testing.assert_array_equal(got[~wn], want[~wn])
            else:
                np.testing.assert_array_equal(got, want)
            rest, ones = from_dev(obase, dt), np.iinfo(NP_BITS[dt]).max  # the poison outside the output
            assert np.all(rest[:64 + out_off] == ones) and np.all(rest[64 + out_off + count:] == ones)


@pytest.mark.parametrize("dt", [ar.AR_F32, ar.AR_I32])
def test_in_place(dt):
    count = 1_000_003
    x = _partials(dt, count, seed=3)
    _, acc = to_dev(x, dt)
    ar.ar_epilogue(acc, acc, ar.AR_AVG, 7)
    want = oracle.epilogue(x, ORACLE_DT[dt], oracle.AVG, 7).view(NP_BITS[dt])
    got = from_dev(acc, dt)
    if dt == ar.AR_F32:
        wn = np.isnan(want.view(np.float32))
        np.testing.assert_array_equal(np.isnan(got.view(np.float32)), wn)
        np.testing.assert_array_equal(got[~wn], want[~wn])
    else:
        np.testing.assert_array_equal(got, want)
