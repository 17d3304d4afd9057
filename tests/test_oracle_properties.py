"""Property tests of the oracle (hypothesis): random rank counts N <= 8, element counts <= 64, every element
type and op, with values drawn to make association visible (large opposite values, signed zeros, NaN and
infinities among them).

Each property is checked against something written here from the definitions, not against the oracle itself:
  - every rank's output is the same;
  - the standalone reduce-scatter followed by the all-gather equals the ring all-reduce;
  - the ring equals the left fold from chunk c's own rank for the elements of chunk c (the balanced split);
  - the rank-order reduce, the halving tree and the binomial tree equal their own folds;
  - int32 results equal the exact sum modulo 2^32, the truncating avg, the min and the max.
The folds use numpy float32 scalar arithmetic (one IEEE rounding per operation) with the min/max rules (any
NaN gives NaN; -0 orders below +0), the avg as one fp32 division by N, and library conversions (torch for
bf16, numpy for f16) for the narrowing to the output type."""
from __future__ import annotations

import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])

_SPECIAL = [0.0, -0.0, 1.0, -1.0, 0.5, 2.0 ** 24, -(2.0 ** 24), 3.0, 2.0 ** -20, 1e30, -1e30]


def _values(draw, dtype, size):
    if dtype == oracle.I32:
        return np.array(draw(st.lists(st.integers(-(2 ** 31), 2 ** 31 - 1), min_size=size, max_size=size)),
                        dtype=np.int32)
    special = st.sampled_from(_SPECIAL + [float("nan"), float("inf"), float("-inf")])
    finite = st.sampled_from(_SPECIAL) | st.floats(-4.0, 4.0, width=32)
    elem = st.one_of(finite, finite, finite, special)
    f = np.array(draw(st.lists(elem, min_size=size, max_size=size)), dtype=np.float32)
    if dtype == oracle.F32:
        return f
    if dtype == oracle.BF16:
        return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    with np.errstate(over="ignore"):
        return f.astype(np.float16).view(np.uint16)


@st.composite
def cases(draw, ops=(oracle.SUM, oracle.AVG, oracle.MIN, oracle.MAX), pow2=False):
    n = draw(st.sampled_from([1, 2, 4, 8]) if pow2 else st.integers(1, 8))
    count = draw(st.integers(0, 64))
    dtype = draw(st.sampled_from([oracle.F32, oracle.BF16, oracle.F16, oracle.I32]))
    op = draw(st.sampled_from(ops))
    return n, count, dtype, op, [_values(draw, dtype, count) for _ in range(n)]


def _widen(x, dtype):
    if dtype == oracle.F32:
        return x.astype(np.float32)
    if dtype == oracle.BF16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    if dtype == oracle.F16:
        return x.view(np.float16).astype(np.float32)
    return x


def _combine(a, b, op):
    if op in (oracle.SUM, oracle.AVG):
        with np.errstate(over="ignore", invalid="ignore"):
            return np.float32(np.float32(a) + np.float32(b))
    if np.isnan(a) or np.isnan(b):
        return np.float32(np.nan)
    if a == b:  # equal values differ at most in the sign of a zero: -0 is the smaller
        if op == oracle.MIN:
            return np.float32(a if np.signbit(a) else b)
        return np.float32(b if np.signbit(a) else a)
    return np.float32(min(a, b) if op == oracle.MIN else max(a, b))


def _narrow(v, dtype, op, n):
    """The owner's epilogue and the rounding into the output type, for a vector of fp32 results."""
    v = np.asarray(v, np.float32)
    if op == oracle.AVG:
        v = (v / np.float32(n)).astype(np.float32)
    if dtype == oracle.F32:
        return v
    if dtype == oracle.BF16:
        return torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    with np.errstate(over="ignore"):
        return v.astype(np.float16).view(np.uint16)


def _same(got, want, dtype):
    """Bitwise, except that any NaN matches any NaN (NaN payloads are not specified)."""
    got, want = np.asarray(got), np.asarray(want)
    if dtype == oracle.I32:
        return np.array_equal(got, want)
    if dtype == oracle.F32:
        gf, wf = got.view(np.float32), want.view(np.float32)
    elif dtype == oracle.BF16:
        gf = torch.from_numpy(got.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
        wf = torch.from_numpy(want.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    else:
        gf, wf = got.view(np.float16), want.view(np.float16)
    both_nan = np.isnan(gf) & np.isnan(wf)
    gb = got.view(np.uint32 if dtype == oracle.F32 else np.uint16)
    wb = want.view(np.uint32 if dtype == oracle.F32 else np.uint16)
    return bool(np.all(both_nan | (gb == wb)))


def _fold(vals, order, op):
    acc = np.float32(vals[order[0]])
    for r in order[1:]:
        acc = _combine(acc, np.float32(vals[r]), op)
    return acc


def _int_expected(xs, op, n):
    big = np.array([[int(v) for v in x] for x in xs], dtype=object).reshape(n, -1)
    out = []
    for e in range(big.shape[1]):
        col = [int(v) for v in big[:, e]]
        s = (sum(col) + 2 ** 31) % 2 ** 32 - 2 ** 31
        out.append({oracle.SUM: s, oracle.AVG: abs(s) // n * (1 if s >= 0 else -1),
                    oracle.MIN: min(col), oracle.MAX: max(col)}[op])
    return np.array(out, dtype=np.int64).astype(np.int32)


def _closed_form(xs, dtype, op, order_of):
    """Element e folded in the order order_of(e) (a list of ranks), then finished and narrowed."""
    n = len(xs)
    if dtype == oracle.I32:
        return _int_expected(xs, op, n)
    w = [_widen(x, dtype) for x in xs]
    count = xs[0].size
    acc = np.array([_fold([w[r][e] for r in range(n)], order_of(e), op) for e in range(count)], np.float32)
    return _narrow(acc, dtype, op, n)


def _chunk_of(count, n):
    q, r = divmod(count, n)
    lo = [c * q + min(c, r) for c in range(n + 1)]
    return lambda e: next(c for c in range(n) if lo[c] <= e < lo[c + 1])


def _binomial_order(n):
    """Nested order T(lo, m) = T(lo, h) (+) T(lo + h, m - h), h the largest power of two below m, as a tree."""
    def t(lo, m):
        if m == 1:
            return lo
        h = 1
        while h * 2 < m:
            h *= 2
        return (t(lo, h), t(lo + h, m - h))
    return t(0, n)


def _xor_order(n):
    """Pairs N/2 apart first: level lists combine element i with element i + half."""
    level = list(range(n))
    while len(level) > 1:
        h = len(level) // 2
        level = [(level[i], level[i + h]) for i in range(h)]
    return level[0]


def _tree_eval(tree, vals, op):
    if isinstance(tree, int):
        return np.float32(vals[tree])
    return _combine(_tree_eval(tree[0], vals, op), _tree_eval(tree[1], vals, op), op)


def _tree_form(xs, dtype, op, tree):
    n = len(xs)
    if dtype == oracle.I32:
        return _int_expected(xs, op, n)
    w = [_widen(x, dtype) for x in xs]
    acc = np.array([_tree_eval(tree, [w[r][e] for r in range(n)], op) for e in range(xs[0].size)], np.float32)
    return _narrow(acc, dtype, op, n)


def _all_same(outs, dtype):
    return all(_same(o, outs[0], dtype) for o in outs[1:])


@SETTINGS
@given(cases())
def test_ring_is_the_fold_from_each_chunks_rank(case):
    n, count, dtype, op, xs = case
    outs = oracle.ring_allreduce(xs, dtype, op)
    assert _all_same(outs, dtype)
    chunk = _chunk_of(count, n) if count else None
    want = _closed_form(xs, dtype, op, lambda e: [(chunk(e) + k) % n for k in range(n)])
    assert _same(outs[0], want, dtype)


@SETTINGS
@given(cases())
def test_reduce_scatter_then_all_gather_is_the_ring(case):
    n, count, dtype, op, xs = case
    ring = oracle.ring_allreduce(xs, dtype, op)
    parts = oracle.reduce_scatter(xs, dtype, op)
    q, r = divmod(count, n)
    assert [p.size for p in parts] == [q + (1 if c < r else 0) for c in range(n)]
    gathered = oracle.allgather(parts, dtype) if count else [np.empty(0, ring[0].dtype)] * n
    for g, w in zip(gathered, ring):
        assert _same(g, w, dtype)


@SETTINGS
@given(cases())
def test_rank_order_reduce_and_binomial_tree(case):
    n, count, dtype, op, xs = case
    fused = oracle.fused_allreduce(xs, dtype, op)
    assert _all_same(fused, dtype)
    assert _same(fused[0], _closed_form(xs, dtype, op, lambda e: list(range(n))), dtype)
    tree = oracle.tree_allreduce(xs, dtype, op)
    assert _all_same(tree, dtype)
    assert _same(tree[0], _tree_form(xs, dtype, op, _binomial_order(n)), dtype)


@SETTINGS
@given(cases(pow2=True))
def test_halving_doubling_is_the_xor_tree(case):
    n, count, dtype, op, xs = case
    outs = oracle.rhd_allreduce(xs, dtype, op)
    assert _all_same(outs, dtype)
    assert _same(outs[0], _tree_form(xs, dtype, op, _xor_order(n)), dtype)
