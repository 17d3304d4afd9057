"""Python binding of libar, the MI355X ring all-reduce library (ctypes over the in-tree ``libar.so``).

The binding only marshals arguments: torch tensors become device pointers, the current torch stream becomes
the hipStream_t, and a non-zero ar_status becomes an :class:`ArError`. Every step of the all-reduce runs in
the library's HIP kernels. There is no CPU fallback: if ``libar.so`` is missing or cannot be loaded, every
call raises.

Entry points (same names as ``include/ar.h``): ar_allreduce, ar_allreduce_ws, ar_allreduce_noalloc,
ar_allreduce_workspace_size,
ar_allreduce_buckets, ar_allreduce_tensors, ar_reduce_scatter, ar_all_gather, ar_bucket_plan, ar_bucket_pack,
ar_bucket_unpack, ar_fp8_quant, ar_fp8_dequant, ar_auto_algo, ar_chunk_bounds, ar_status_string, ar_last_call,
ar_version. Helpers: chunk_bounds, make_copy_descs, BucketedAllReduce.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

__all__ = [
    "AR_OK", "AR_ERR_INVALID", "AR_ERR_UNSUPPORTED", "AR_ERR_ALIAS", "AR_ERR_WORKSPACE", "AR_ERR_HIP",
    "AR_F32", "AR_BF16", "AR_F16", "AR_I32", "AR_SUM", "AR_AVG", "AR_MIN", "AR_MAX",
    "AR_ALGO_RING", "AR_ALGO_FUSED", "AR_ALGO_RHD", "AR_ALGO_RING_STEPWISE", "AR_ALGO_RHD_STEPWISE",
    "AR_ALGO_RING_FP8", "AR_ALGO_TREE", "AR_ALGO_TREE_STEPWISE", "AR_ALGO_AUTO", "AR_AUTO_STEP_NS",
    "AR_AUTO_LINK_GBPS", "AR_MAX_RANKS", "AR_FP8_BLOCK", "AR_NOALLOC_WS_BYTES", "ArError", "lib", "lib_path", "ar_auto_algo",
    "ar_allreduce", "ar_allreduce_ws", "ar_allreduce_noalloc", "ar_allreduce_workspace_size", "ar_allreduce_buckets",
    "ar_allreduce_tensors", "ar_reduce_scatter", "ar_all_gather", "ar_chunk_bounds", "chunk_bounds",
    "ar_bucket_plan",
    "ar_bucket_pack",
    "ar_bucket_unpack", "ar_fp8_quant", "ar_fp8_dequant", "ar_status_string", "ar_last_call", "ar_version",
    "make_copy_descs", "BucketedAllReduce", "dtype_code",
]

AR_OK, AR_ERR_INVALID, AR_ERR_UNSUPPORTED, AR_ERR_ALIAS, AR_ERR_WORKSPACE, AR_ERR_HIP = 0, 1, 2, 3, 4, 5
AR_F32, AR_BF16, AR_F16, AR_I32 = 0, 1, 2, 3
AR_SUM, AR_AVG, AR_MIN, AR_MAX = 0, 1, 2, 3
AR_ALGO_RING, AR_ALGO_FUSED, AR_ALGO_RHD, AR_ALGO_RING_STEPWISE, AR_ALGO_RHD_STEPWISE, AR_ALGO_RING_FP8 = range(6)
AR_ALGO_TREE, AR_ALGO_TREE_STEPWISE, AR_ALGO_AUTO = 6, 7, 8
AR_AUTO_STEP_NS, AR_AUTO_LINK_GBPS = 1900, 153
AR_MAX_RANKS = 64
AR_FP8_BLOCK = 128
AR_NOALLOC_WS_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libar.so")
_lib = None


class ArError(RuntimeError):
    def __init__(self, status: int, entry: str):
        self.status = status
        super().__init__(f"{entry}: {ar_status_string(status)}")


class _CallRecord(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_uint64), ("entry", ctypes.c_char_p), ("nranks", ctypes.c_int),
                ("dtype", ctypes.c_int), ("op", ctypes.c_int), ("algo", ctypes.c_int), ("status", ctypes.c_int),
                ("count", ctypes.c_size_t)]


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libar.so (built in-tree by build.py). Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libar.so not found at {_LIB_PATH}; build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.ar_allreduce.argtypes = [vp, vp, i32, sz, i32, i32, i32, vp]
        L.ar_allreduce_ws.argtypes = [vp, vp, i32, sz, i32, i32, i32, vp, sz, vp]
        L.ar_allreduce_noalloc.argtypes = [vp, vp, i32, sz, i32, i32, i32, vp]
        L.ar_allreduce_workspace_size.argtypes = [i32, sz, i32, i32, i32, ctypes.POINTER(sz)]
        L.ar_allreduce_buckets.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, vp]
        L.ar_allreduce_tensors.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.ar_reduce_scatter.argtypes = [vp, vp, i32, sz, i32, i32, vp]
        L.ar_all_gather.argtypes = [vp, vp, i32, sz, i32, vp]
        L.ar_bucket_plan.argtypes = [vp, i32, i32, i32, sz, vp, vp, vp, ctypes.POINTER(i32)]
        L.ar_bucket_pack.argtypes = [vp, i32, i32, vp]
        L.ar_bucket_unpack.argtypes = [vp, i32, i32, vp]
        L.ar_fp8_quant.argtypes = [vp, i32, sz, vp, vp, vp]
        L.ar_fp8_dequant.argtypes = [vp, vp, sz, vp, i32, vp]
        L.ar_auto_algo.argtypes = [i32, sz, i32]
        L.ar_chunk_bounds.argtypes = [i32, sz, vp]
        L.ar_epilogue.argtypes = [vp, vp, sz, i32, i32, i32, vp]
        L.ar_status_string.argtypes = [i32]
        L.ar_status_string.restype = ctypes.c_char_p
        L.ar_last_call.argtypes = [ctypes.POINTER(_CallRecord)]
        for name in ("ar_allreduce", "ar_allreduce_ws", "ar_allreduce_noalloc", "ar_allreduce_workspace_size",
                     "ar_allreduce_buckets",
                     "ar_allreduce_tensors", "ar_reduce_scatter", "ar_all_gather", "ar_bucket_plan", "ar_bucket_pack",
                     "ar_bucket_unpack", "ar_fp8_quant", "ar_fp8_dequant", "ar_last_call", "ar_version",
                     "ar_auto_algo", "ar_chunk_bounds", "ar_epilogue"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


# ------------------------------------------------------------------------------------------ marshalling
_DTYPE_CODES = {}


def dtype_code(t) -> int:
    if not _DTYPE_CODES:
        import torch
        _DTYPE_CODES.update({torch.float32: AR_F32, torch.bfloat16: AR_BF16, torch.float16: AR_F16,
                             torch.int32: AR_I32})
    if t not in _DTYPE_CODES:
        raise TypeError(f"unsupported dtype {t}; expected float32, bfloat16, float16 or int32")
    return _DTYPE_CODES[t]


def _stream(stream, device=None):
    """The HIP stream handle: `stream` (a torch stream or a raw handle), else the current stream of `device`."""
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)  # the handle without a Stream object
        if raw is not None and device is not None and device.index is not None:
            return ctypes.c_void_p(raw(device.index))
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _on(device):
    """Make `device` current for a call (the library launches on the current device); no switch when it already
    is."""
    import torch
    if device.index is not None and device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _gpu_tensor(t, what, dtype=None, device=None, min_numel=0):
    """Every tensor handed to the library: a contiguous GPU tensor (of `dtype`, on `device`, at least
    `min_numel` elements). A host tensor would give the kernels a host address."""
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{what} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, not {t.dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"{what} must hold at least {min_numel} elements")
    return t


def _check(rc: int, entry: str):
    if rc != AR_OK:
        raise ArError(rc, entry)


def _rank_arrays(ins, outs):
    """Check every rank tensor (all before any address is read), then the host arrays of their addresses. The
    checks are the per-tensor ones of _gpu_tensor plus equal dtype, element count and device, written with the
    cheapest accessors: this runs on every call, and for small messages it is most of the call's host time."""
    n = len(ins)
    if n != len(outs) or not n:
        raise ValueError("ins and outs must be non-empty lists of the same length (one tensor per rank)")
    t0 = ins[0]
    dt0, ne0, dev0 = t0.dtype, t0.numel(), t0.get_device()
    for t in (*ins, *outs):
        # every rank must call with the same count and dtype; one call enforces it
        if t.dtype is not dt0 or t.numel() != ne0 or t.get_device() != dev0:
            raise ValueError("all rank tensors must share dtype, element count and device")
        if not t.is_contiguous():
            raise ValueError("rank tensors must be contiguous")
    if dev0 < 0:  # get_device() is -1 for host tensors
        raise ValueError("rank tensors must be GPU tensors")
    arr_in = (ctypes.c_void_p * n)(*[t.data_ptr() for t in ins])
    arr_out = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    return arr_in, arr_out, n, ne0, dtype_code(dt0)


def ar_allreduce(ins, outs, op=AR_SUM, algo=AR_ALGO_RING, stream=None):
    """All-reduce ins[r] -> outs[r] for every rank r (outs[r] may be ins[r])."""
    arr_in, arr_out, n, count, dt = _rank_arrays(ins, outs)
    dev = ins[0].device
    with _on(dev):
        _check(lib().ar_allreduce(arr_in, arr_out, n, count, dt, op, algo, _stream(stream, dev)), "ar_allreduce")


def ar_allreduce_workspace_size(nranks, count, dtype, op, algo) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().ar_allreduce_workspace_size(nranks, count, dtype, op, algo, ctypes.byref(out)),
           "ar_allreduce_workspace_size")
    return out.value


def ar_allreduce_ws(ins, outs, op=AR_SUM, algo=AR_ALGO_RING, workspace=None, stream=None):
    """ar_allreduce with a caller workspace tensor (any dtype, contiguous, on the same GPU)."""
    if workspace is not None and ins:
        _gpu_tensor(workspace, "workspace", device=ins[0].device)
    arr_in, arr_out, n, count, dt = _rank_arrays(ins, outs)
    dev = ins[0].device
    wp = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with _on(dev):
        _check(lib().ar_allreduce_ws(arr_in, arr_out, n, count, dt, op, algo, wp, wb, _stream(stream, dev)),
               "ar_allreduce_ws")


def ar_allreduce_noalloc(ins, outs, op=AR_SUM, algo=AR_ALGO_RING, stream=None):
    """ar_allreduce_ws with the library's fixed per-GPU scratch instead of a caller workspace (allocates nothing;
    calls that overlap on one GPU race on that scratch)."""
    arr_in, arr_out, n, count, dt = _rank_arrays(ins, outs)
    dev = ins[0].device
    with _on(dev):
        _check(lib().ar_allreduce_noalloc(arr_in, arr_out, n, count, dt, op, algo, _stream(stream, dev)),
               "ar_allreduce_noalloc")


def ar_allreduce_buckets(flat_ins, flat_outs, bucket_count, op=AR_SUM, algo=AR_ALGO_RING, stream=None):
    """All-reduce every bucket of the flat per-rank tensors in one launch (bucket_count: the plan's counts)."""
    arr_in, arr_out, n, total, dt = _rank_arrays(flat_ins, flat_outs)
    counts = np.ascontiguousarray(bucket_count, dtype=np.int64)
    if int(counts.sum()) > total:
        raise ValueError("the buckets do not fit in the flat tensors")
    dev = flat_ins[0].device
    with _on(dev):
        _check(lib().ar_allreduce_buckets(arr_in, arr_out, n, counts.ctypes.data, counts.size, dt, op, algo,
                                          _stream(stream, dev)), "ar_allreduce_buckets")


def ar_allreduce_tensors(descs, in_ptrs, out_ptrs, ntensors, nranks, dtype, op=AR_AVG, algo=AR_ALGO_RING,
                         stream=None):
    """descs: device int64 tensor [ntensors, 4] laid out as ar_tensor_desc; in_ptrs/out_ptrs: device int64
    tensors [ntensors * nranks] of device addresses (entry t * nranks + r)."""
    import torch
    dev = descs.device
    _gpu_tensor(descs, "descs", torch.int64, dev, 4 * ntensors)
    _gpu_tensor(in_ptrs, "in_ptrs", torch.int64, dev, ntensors * nranks)
    _gpu_tensor(out_ptrs, "out_ptrs", torch.int64, dev, ntensors * nranks)
    with _on(dev):
        _check(lib().ar_allreduce_tensors(ctypes.c_void_p(descs.data_ptr()), ctypes.c_void_p(in_ptrs.data_ptr()),
                                          ctypes.c_void_p(out_ptrs.data_ptr()), ntensors, nranks, dtype, op, algo,
                                          _stream(stream, dev)), "ar_allreduce_tensors")


def ar_chunk_bounds(nranks, count):
    """The library's balanced split (host only): chunk c = [lo[c], lo[c+1]), a list of nranks + 1 ints."""
    lo = (ctypes.c_int64 * (nranks + 1))() if 1 <= nranks <= AR_MAX_RANKS else None
    _check(lib().ar_chunk_bounds(nranks, count, lo), "ar_chunk_bounds")
    return list(lo)


def chunk_bounds(count, nranks):
    """ar_chunk_bounds with the arguments in (count, nranks) order."""
    return ar_chunk_bounds(nranks, count)


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else 0


def _chunk_tensors(full, parts, what):
    """Check N full tensors and N chunk tensors (None allowed for an empty chunk) of one dtype and device."""
    n = len(full)
    if n == 0 or len(parts) != n:
        raise ValueError("one full tensor and one chunk tensor per rank")
    t0 = full[0]
    for t in full:
        if t.numel() != t0.numel():
            raise ValueError("all full tensors must have the same element count")
        _gpu_tensor(t, "full tensors", t0.dtype, t0.device)
    lo = chunk_bounds(t0.numel(), n)
    for c, p in enumerate(parts):
        want = lo[c + 1] - lo[c]
        if p is None:
            if want:
                raise ValueError(f"{what}[{c}] is None but chunk {c} has {want} elements")
            continue
        if p.numel() != want:
            raise ValueError(f"{what}[{c}] must hold exactly chunk {c} of the balanced split ({want} elements)")
        if want:
            _gpu_tensor(p, f"{what}[{c}]", t0.dtype, t0.device)
    return n, t0.numel(), t0.device


def ar_reduce_scatter(ins, outs, op=AR_SUM, stream=None):
    """ins: N full tensors; outs[c]: a tensor of chunk c's length (the balanced split) receiving chunk c."""
    n, count, dev = _chunk_tensors(ins, outs, "outs")
    arr_in = (ctypes.c_void_p * n)(*[t.data_ptr() for t in ins])
    arr_out = (ctypes.c_void_p * n)(*[_ptr(o) for o in outs])
    with _on(dev):
        _check(lib().ar_reduce_scatter(arr_in, arr_out, n, count, dtype_code(ins[0].dtype), op,
                                       _stream(stream, dev)), "ar_reduce_scatter")


def ar_all_gather(ins, outs, stream=None):
    """ins[r]: rank r's chunk (the balanced split of the outputs' length); outs: N full tensors."""
    n, count, dev = _chunk_tensors(outs, ins, "ins")
    arr_in = (ctypes.c_void_p * n)(*[_ptr(i) for i in ins])
    arr_out = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    with _on(dev):
        _check(lib().ar_all_gather(arr_in, arr_out, n, count, dtype_code(outs[0].dtype), _stream(stream, dev)),
               "ar_all_gather")


def ar_bucket_plan(numels, dtype, nranks, cap_bytes=25 << 20):
    """Host-only plan; returns (bucket_of int32[T], offset_of int64[T], bucket_count int64[nbuckets])."""
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    nt = numels.size
    bucket_of = np.zeros(max(nt, 1), np.int32)
    offset_of = np.zeros(max(nt, 1), np.int64)
    bcount = np.zeros(max(nt, 1), np.int64)
    nb = ctypes.c_int(0)
    _check(lib().ar_bucket_plan(numels.ctypes.data, nt, dtype, nranks, cap_bytes, bucket_of.ctypes.data,
                                offset_of.ctypes.data, bcount.ctypes.data, ctypes.byref(nb)), "ar_bucket_plan")
    return bucket_of[:nt], offset_of[:nt], bcount[: nb.value]


def make_copy_descs(tasks, device):
    """tasks: iterable of (src_ptr, dst_ptr, numel, zero_pad_after) -> device int64 tensor [ndescs, 4]
    laid out as ar_copy_desc (two pointers, two int64)."""
    import torch
    host = np.array(list(tasks), dtype=np.uint64).reshape(-1, 4).view(np.int64)
    return torch.from_numpy(host).to(device)


def _copy_descs(descs):
    import torch
    _gpu_tensor(descs, "descs", torch.int64)
    if descs.dim() != 2 or descs.shape[1] != 4:
        raise ValueError("descs must be an int64 tensor [ndescs, 4] (ar_copy_desc rows)")
    return descs.device


def ar_bucket_pack(descs, dtype, stream=None):
    dev = _copy_descs(descs)
    with _on(dev):
        _check(lib().ar_bucket_pack(ctypes.c_void_p(descs.data_ptr()), descs.shape[0], dtype, _stream(stream, dev)),
               "ar_bucket_pack")


def ar_bucket_unpack(descs, dtype, stream=None):
    dev = _copy_descs(descs)
    with _on(dev):
        _check(lib().ar_bucket_unpack(ctypes.c_void_p(descs.data_ptr()), descs.shape[0], dtype,
                                      _stream(stream, dev)), "ar_bucket_unpack")


def ar_fp8_quant(x, codes, scales, stream=None):
    """x: float32/bfloat16 GPU tensor; codes: uint8[numel]; scales: float32[ceil(numel/128)]."""
    import torch
    dev = _gpu_tensor(x, "x").device
    _gpu_tensor(codes, "codes", torch.uint8, dev, x.numel())
    _gpu_tensor(scales, "scales", torch.float32, dev, (x.numel() + AR_FP8_BLOCK - 1) // AR_FP8_BLOCK)
    with _on(dev):
        _check(lib().ar_fp8_quant(ctypes.c_void_p(x.data_ptr()), dtype_code(x.dtype), x.numel(),
                                  ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                  _stream(stream, dev)), "ar_fp8_quant")


def ar_fp8_dequant(codes, scales, out, stream=None):
    """codes: uint8[numel]; scales: float32[ceil(numel/128)]; out: float32/bfloat16 GPU tensor of numel."""
    import torch
    dev = _gpu_tensor(out, "out").device
    _gpu_tensor(codes, "codes", torch.uint8, dev, out.numel())
    _gpu_tensor(scales, "scales", torch.float32, dev, (out.numel() + AR_FP8_BLOCK - 1) // AR_FP8_BLOCK)
    with _on(dev):
        _check(lib().ar_fp8_dequant(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                    out.numel(), ctypes.c_void_p(out.data_ptr()), dtype_code(out.dtype),
                                    _stream(stream, dev)), "ar_fp8_dequant")


def ar_epilogue(acc, out, op=AR_SUM, nranks=1, stream=None):
    """acc: float32 GPU tensor of partial results (int32 when `out` is int32); out: GPU tensor of as many elements,
    whose dtype is the output type (may be acc itself for float32/int32)."""
    import torch
    dev = _gpu_tensor(acc, "acc").device
    _gpu_tensor(out, "out", None, dev)
    _gpu_tensor(acc, "acc", torch.int32 if out.dtype == torch.int32 else torch.float32)
    if out.numel() != acc.numel():
        raise ValueError("acc and out must hold the same number of elements")
    with _on(dev):
        _check(lib().ar_epilogue(ctypes.c_void_p(acc.data_ptr()), ctypes.c_void_p(out.data_ptr()), acc.numel(),
                                 dtype_code(out.dtype), op, nranks, _stream(stream, dev)), "ar_epilogue")


def ar_auto_algo(nranks, count, dtype) -> int:
    """The algorithm AR_ALGO_AUTO runs for this shape (AR_ALGO_TREE or AR_ALGO_RING)."""
    a = lib().ar_auto_algo(nranks, count, dtype)
    if a < 0:
        raise ArError(-a, "ar_auto_algo")
    return a


def ar_status_string(status: int) -> str:
    return lib().ar_status_string(status).decode()


def ar_last_call():
    rec = _CallRecord()
    if lib().ar_last_call(ctypes.byref(rec)) != AR_OK:
        return None
    return {"seq": rec.seq, "entry": rec.entry.decode() if rec.entry else None, "nranks": rec.nranks,
            "count": rec.count, "dtype": rec.dtype, "op": rec.op, "algo": rec.algo, "status": rec.status}


def ar_version() -> int:
    return lib().ar_version()


# ------------------------------------------------------------------------------------------ bucketing
class BucketedAllReduce:
    """DDP-style bucketed all-reduce of per-rank tensor lists: pack every rank's tensors into its bucket
    buffer (one launch), all-reduce each bucket with the ring kernel, unpack to per-tensor outputs (one
    launch). The plan and descriptor tables are built once; bucket buffers are torch allocations."""

    def __init__(self, ins, outs, op=AR_AVG, algo=AR_ALGO_RING, cap_bytes=25 << 20):
        import torch
        self.n = len(ins)
        self.nt = len(ins[0])
        if any(len(x) != self.nt for x in list(ins) + list(outs)):
            raise ValueError("every rank needs the same number of tensors")
        for t in range(self.nt):
            _rank_arrays([ins[r][t] for r in range(self.n)], [outs[r][t] for r in range(self.n)])
        t00 = ins[0][0]
        self.dtype = dtype_code(t00.dtype)
        self.op, self.algo = op, algo
        numels = [ins[0][t].numel() for t in range(self.nt)]
        self.bucket_of, self.offset_of, self.bucket_count = ar_bucket_plan(numels, self.dtype, self.n, cap_bytes)
        self.bucket_start = np.concatenate([[0], np.cumsum(self.bucket_count)]).astype(np.int64)
        total = int(self.bucket_start[-1])
        self.buffers = [torch.empty(total, dtype=t00.dtype, device=t00.device) for _ in range(self.n)]
        es = t00.element_size()
        g = 16 // es
        pack, unpack = [], []
        for r in range(self.n):
            base = self.buffers[r].data_ptr()
            for t in range(self.nt):
                b = int(self.bucket_of[t])
                off = int(self.bucket_start[b] + self.offset_of[t])
                numel = numels[t]
                # zero pad up to the next tensor's start (or the bucket's end)
                nxt = t + 1
                end = (int(self.bucket_start[b] + self.offset_of[nxt])
                       if nxt < self.nt and int(self.bucket_of[nxt]) == b else int(self.bucket_start[b + 1]))
                pad = end - off - numel
                assert pad >= 0 and pad < max(g * self.n, g) + g * self.n
                pack.append((ins[r][t].data_ptr(), base + off * es, numel, pad))
                unpack.append((base + off * es, outs[r][t].data_ptr(), numel, 0))
        self.pack_descs = make_copy_descs(pack, t00.device)
        self.unpack_descs = make_copy_descs(unpack, t00.device)
        # the fused path: one descriptor per tensor (numel, offset in its bucket, bucket count / N) and the
        # [tensor, rank] pointer tables
        import torch as _t
        tdesc = np.zeros((self.nt, 4), np.int64)
        for t in range(self.nt):
            b = int(self.bucket_of[t])
            tdesc[t] = (numels[t], int(self.offset_of[t]), int(self.bucket_count[b]) // self.n, 0)
        self.tensor_descs = _t.from_numpy(tdesc).to(t00.device)
        iptr = np.array([[ins[r][t].data_ptr() for r in range(self.n)] for t in range(self.nt)], np.uint64)
        optr = np.array([[outs[r][t].data_ptr() for r in range(self.n)] for t in range(self.nt)], np.uint64)
        self.in_ptrs = _t.from_numpy(iptr.reshape(-1).view(np.int64)).to(t00.device)
        self.out_ptrs = _t.from_numpy(optr.reshape(-1).view(np.int64)).to(t00.device)
        self.views = [[self.buffers[r][int(self.bucket_start[b]):int(self.bucket_start[b + 1])]
                       for r in range(self.n)] for b in range(len(self.bucket_count))]

    @property
    def nbuckets(self):
        return len(self.bucket_count)

    def pack(self, stream=None):
        ar_bucket_pack(self.pack_descs, self.dtype, stream)

    def reduce(self, stream=None):
        """Every bucket in one launch (per-bucket rings, bit-identical to one ar_allreduce per bucket)."""
        ar_allreduce_buckets(self.buffers, self.buffers, self.bucket_count, self.op, self.algo, stream)

    def reduce_per_bucket(self, stream=None):
        """One ar_allreduce launch per bucket."""
        for v in self.views:
            ar_allreduce(v, v, self.op, self.algo, stream)

    def unpack(self, stream=None):
        ar_bucket_unpack(self.unpack_descs, self.dtype, stream)

    def fused(self, stream=None):
        """The whole bucketed all-reduce in one launch, reading and writing the tensors in place of the buckets
        (same bits as pack + reduce + unpack)."""
        ar_allreduce_tensors(self.tensor_descs, self.in_ptrs, self.out_ptrs, self.nt, self.n, self.dtype, self.op,
                             self.algo, stream)

    def __call__(self, stream=None):
        self.pack(stream)
        self.reduce(stream)
        self.unpack(stream)
