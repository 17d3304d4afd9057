"""CPU oracle for the ring all-reduce: ctypes access to ``liboracle.so`` (built from ``oracle.c`` by gcc).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never imports or links it, and it never imports the GPU library.

Arrays are numpy: fp32 -> float32, bf16 and f16 -> uint16 bit patterns, int32 -> int32.
Dtype and op codes are this package's own: F32=0, BF16=1, F16=2, I32=3; SUM=0, AVG=1, MIN=2, MAX=3.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16, F16, I32 = 0, 1, 2, 3
SUM, AVG, MIN, MAX = 0, 1, 2, 3
NP_DTYPE = {F32: np.float32, BF16: np.uint16, F16: np.uint16, I32: np.int32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB names another build of oracle.c to load instead (the tests use it to run the pins against a
# sanitizer build and against builds with planted mistakes); that file is never rebuilt here.
_LIB_PATH = os.environ.get("ORACLE_LIB") or _DEFAULT_LIB
_lib = None

# gcc flags of every build: IEEE fp32 (no contraction, no fast-math), OpenMP over element loops.
CFLAGS = ["-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def compile_library(src: str, out: str, extra=()) -> str:
    """Compile an oracle source file into a shared library at `out` (gcc, CFLAGS plus `extra`)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", *CFLAGS, *extra, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so from oracle.c."""
    if force or not os.path.exists(_DEFAULT_LIB):
        compile_library(_SRC, _DEFAULT_LIB)
    return _DEFAULT_LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            if _LIB_PATH != _DEFAULT_LIB:
                raise RuntimeError(f"ORACLE_LIB={_LIB_PATH} does not exist")
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        pp = ctypes.POINTER(ctypes.c_void_p)
        for name in ("oracle_ring_allreduce", "oracle_fused_allreduce", "oracle_rhd_allreduce",
                     "oracle_tree_allreduce", "oracle_reduce_scatter", "oracle_fp8_ring_allreduce"):
            getattr(L, name).argtypes = [pp, pp, i32, i64, i32, i32]
            getattr(L, name).restype = i32
        L.oracle_ring_rs_state.argtypes = [pp, pp, i32, i64, i32, i32]
        L.oracle_ring_rs_state.restype = i32
        L.oracle_allgather.argtypes = [pp, pp, i32, i64, i32]
        L.oracle_allgather.restype = i32
        L.oracle_chunk_bounds.argtypes = [i64, i32, vp]
        L.oracle_chunk_bounds.restype = None
        for name in ("oracle_f32_to_bf16", "oracle_bf16_to_f32", "oracle_f32_to_f16", "oracle_f16_to_f32",
                     "oracle_f32_to_e4m3", "oracle_e4m3_to_f32"):
            getattr(L, name).argtypes = [vp, vp, i64]
            getattr(L, name).restype = None
        L.oracle_fp8_quant.argtypes = [vp, i32, i64, vp, vp]
        L.oracle_fp8_quant.restype = i32
        L.oracle_fp8_dequant.argtypes = [vp, vp, i64, vp, i32]
        L.oracle_fp8_dequant.restype = i32
        L.oracle_epilogue.argtypes = [vp, vp, i64, i32, i32, i32]
        L.oracle_epilogue.restype = i32
        L.oracle_bucket_plan.argtypes = [vp, i32, i32, i32, i64, vp, vp, vp, ctypes.POINTER(ctypes.c_int)]
        L.oracle_bucket_plan.restype = i32
        L.oracle_bucketed_allreduce.argtypes = [pp, pp, i32, i32, vp, i32, i32, i64]
        L.oracle_bucketed_allreduce.restype = i32
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_set_num_threads.restype = None
        L.oracle_version.restype = i32
        _lib = L
    return _lib


def _ptrs(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _prep(xs, dtype):
    xs = [np.ascontiguousarray(x, dtype=NP_DTYPE[dtype]) for x in xs]
    n = len(xs)
    count = xs[0].size if n else 0
    if any(x.size != count for x in xs):
        raise ValueError("all ranks must hold the same element count")
    return xs, n, count


def _collective(name, xs, dtype, op, out=None):
    xs, n, count = _prep(xs, dtype)
    outs = out if out is not None else [np.empty(count, dtype=NP_DTYPE[dtype]) for _ in range(n)]
    _check(getattr(lib(), name)(_ptrs(xs), _ptrs(outs), n, count, dtype, op), name)
    return outs


def ring_allreduce(xs, dtype=F32, op=SUM):
    """The ring schedule executed literally (reduce-scatter rounds, owner epilogue, all-gather rounds)."""
    return _collective("oracle_ring_allreduce", xs, dtype, op)


def fused_allreduce(xs, dtype=F32, op=SUM):
    """Reduce at one root in rank order 0..N-1, then broadcast."""
    return _collective("oracle_fused_allreduce", xs, dtype, op)


def rhd_allreduce(xs, dtype=F32, op=SUM):
    """Recursive halving then recursive doubling, executed literally (N a power of two)."""
    return _collective("oracle_rhd_allreduce", xs, dtype, op)


def tree_allreduce(xs, dtype=F32, op=SUM):
    """Binomial-tree reduce to rank 0 (rank i takes rank i + 2^j at step j), then binomial broadcast."""
    return _collective("oracle_tree_allreduce", xs, dtype, op)


def fp8_ring_allreduce(xs, dtype=BF16, op=SUM):
    """Ring with every reduce-scatter message carried as E4M3 codes + fp32 per-128-element scales."""
    return _collective("oracle_fp8_ring_allreduce", xs, dtype, op)


def chunk_bounds(count, n):
    lo = np.empty(n + 1, dtype=np.int64)
    lib().oracle_chunk_bounds(count, n, lo.ctypes.data)
    return lo


def ring_rs_state(xs, dtype=F32, op=SUM):
    """Per-rank widened state after the reduce-scatter rounds (uint32: fp32 bits or int32 bits)."""
    xs, n, count = _prep(xs, dtype)
    st = [np.empty(count, dtype=np.uint32) for _ in range(n)]
    _check(lib().oracle_ring_rs_state(_ptrs(xs), _ptrs(st), n, count, dtype, op), "rs_state")
    return st


def reduce_scatter(xs, dtype=F32, op=SUM):
    """Rank c receives chunk c of the reduced vector."""
    xs, n, count = _prep(xs, dtype)
    lo = chunk_bounds(count, n)
    outs = [np.empty(max(int(lo[c + 1] - lo[c]), 1), dtype=NP_DTYPE[dtype]) for c in range(n)]
    _check(lib().oracle_reduce_scatter(_ptrs(xs), _ptrs(outs), n, count, dtype, op), "reduce_scatter")
    return [o[: int(lo[c + 1] - lo[c])] for c, o in enumerate(outs)]


def allgather(parts, dtype=F32):
    """Rank r contributes parts[r] (the balanced chunk r); every rank gets the concatenation."""
    parts = [np.ascontiguousarray(p, dtype=NP_DTYPE[dtype]) for p in parts]
    n = len(parts)
    count = sum(p.size for p in parts)
    lo = chunk_bounds(count, n)
    for c, p in enumerate(parts):
        if p.size != lo[c + 1] - lo[c]:
            raise ValueError("parts must follow the balanced chunk split")
    ins = [p if p.size else np.empty(1, dtype=p.dtype) for p in parts]
    outs = [np.empty(count, dtype=NP_DTYPE[dtype]) for _ in range(n)]
    _check(lib().oracle_allgather(_ptrs(ins), _ptrs(outs), n, count, dtype), "allgather")
    return outs


def _conv(name, x, out_dtype):
    x = np.ascontiguousarray(x)
    y = np.empty(x.size, dtype=out_dtype)
    getattr(lib(), name)(x.ctypes.data, y.ctypes.data, x.size)
    return y


def f32_to_bf16(x):
    return _conv("oracle_f32_to_bf16", np.asarray(x, dtype=np.float32), np.uint16)


def bf16_to_f32(x):
    return _conv("oracle_bf16_to_f32", np.asarray(x, dtype=np.uint16), np.float32)


def f32_to_f16(x):
    return _conv("oracle_f32_to_f16", np.asarray(x, dtype=np.float32), np.uint16)


def f16_to_f32(x):
    return _conv("oracle_f16_to_f32", np.asarray(x, dtype=np.uint16), np.float32)


def f32_to_e4m3(x):
    return _conv("oracle_f32_to_e4m3", np.asarray(x, dtype=np.float32), np.uint8)


def e4m3_to_f32(x):
    return _conv("oracle_e4m3_to_f32", np.asarray(x, dtype=np.uint8), np.float32)


def fp8_quant(x, dtype=F32):
    x = np.ascontiguousarray(x, dtype=NP_DTYPE[dtype])
    codes = np.empty(x.size, dtype=np.uint8)
    scales = np.empty((x.size + 127) // 128, dtype=np.float32)
    _check(lib().oracle_fp8_quant(x.ctypes.data, dtype, x.size, codes.ctypes.data, scales.ctypes.data), "fp8_quant")
    return codes, scales


def fp8_dequant(codes, scales, dtype=F32):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    out = np.empty(codes.size, dtype=NP_DTYPE[dtype])
    _check(lib().oracle_fp8_dequant(codes.ctypes.data, scales.ctypes.data, codes.size, out.ctypes.data, dtype),
           "fp8_dequant")
    return out


def epilogue(acc, dtype=F32, op=SUM, n=1):
    """The owner's finishing step on fp32 partial results (int32 for I32): avg divides by n, then the value is
    rounded into `dtype`."""
    acc = np.ascontiguousarray(acc, dtype=np.int32 if dtype == I32 else np.float32)
    out = np.empty(acc.size, dtype=NP_DTYPE[dtype])
    _check(lib().oracle_epilogue(acc.ctypes.data, out.ctypes.data, acc.size, dtype, op, n), "epilogue")
    return out


def bucket_plan(numels, esize, n, cap_bytes):
    """Returns (bucket_of[int32], offset_of[int64], bucket_count[int64, nbuckets])."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    nt = numels.size
    bucket_of = np.empty(max(nt, 1), dtype=np.int32)
    offset_of = np.empty(max(nt, 1), dtype=np.int64)
    bcount = np.empty(max(nt, 1), dtype=np.int64)
    nb = ctypes.c_int(0)
    _check(lib().oracle_bucket_plan(numels.ctypes.data, nt, esize, n, cap_bytes, bucket_of.ctypes.data,
                                    offset_of.ctypes.data, bcount.ctypes.data, ctypes.byref(nb)), "bucket_plan")
    return bucket_of[:nt], offset_of[:nt], bcount[: nb.value]


_ALGOS = {"ring": ring_allreduce, "fused": fused_allreduce, "rhd": rhd_allreduce, "tree": tree_allreduce}


def bucketed_allreduce(tensors, dtype=F32, op=AVG, cap_bytes=25 << 20, algo="ring"):
    """tensors[r][t] -> outs[r][t]: plan, pack, all-reduce every bucket, unpack.

    algo "ring" runs the C routine (plan, pack, literal ring per bucket, unpack, all in oracle.c). The other
    algorithms ("fused", "rhd", "tree") and "ring_py" pack here: the C plan, each tensor copied to its offset in
    a zero-filled bucket per rank, the named oracle all-reduce on every bucket, and each tensor's first numel
    elements copied back."""
    if algo != "ring":
        return _bucketed_by_packing(tensors, dtype, op, cap_bytes, _ALGOS[algo.replace("_py", "")])
    n = len(tensors)
    nt = len(tensors[0]) if n else 0
    numels = np.array([np.asarray(t).size for t in tensors[0]], dtype=np.int64)
    flat_in = []
    for r in range(n):
        for t in range(nt):
            a = np.ascontiguousarray(tensors[r][t], dtype=NP_DTYPE[dtype])
            flat_in.append(a if a.size else np.empty(1, dtype=a.dtype))
    outs = [np.empty(max(int(numels[t]), 1), dtype=NP_DTYPE[dtype]) for r in range(n) for t in range(nt)]
    _check(lib().oracle_bucketed_allreduce(_ptrs(flat_in), _ptrs(outs), n, nt, numels.ctypes.data, dtype, op,
                                           cap_bytes), "bucketed_allreduce")
    return [[outs[r * nt + t][: int(numels[t])] for t in range(nt)] for r in range(n)]


def _bucketed_by_packing(tensors, dtype, op, cap_bytes, allreduce):
    n = len(tensors)
    nt = len(tensors[0]) if n else 0
    numels = np.array([np.asarray(t).size for t in tensors[0]], dtype=np.int64)
    es = 2 if dtype in (BF16, F16) else 4
    bucket_of, offset_of, bcount = bucket_plan(numels, es, n, cap_bytes)
    start = np.concatenate([[0], np.cumsum(bcount)]).astype(np.int64)
    flat = [np.zeros(int(start[-1]), dtype=NP_DTYPE[dtype]) for _ in range(n)]
    for r in range(n):
        for t in range(nt):
            at = int(start[bucket_of[t]] + offset_of[t])
            flat[r][at:at + int(numels[t])] = np.asarray(tensors[r][t], dtype=NP_DTYPE[dtype])
    for b in range(len(bcount)):
        lo, hi = int(start[b]), int(start[b + 1])
        red = allreduce([f[lo:hi] for f in flat], dtype, op)
        for r in range(n):
            flat[r][lo:hi] = red[r]
    outs = []
    for r in range(n):
        row = []
        for t in range(nt):
            at = int(start[bucket_of[t]] + offset_of[t])
            row.append(flat[r][at:at + int(numels[t])].copy())
        outs.append(row)
    return outs


def num_threads():
    return lib().oracle_num_threads()


def set_num_threads(n):
    """Threads for the following calls (n < 1: the default); results do not depend on it."""
    lib().oracle_set_num_threads(int(n))
