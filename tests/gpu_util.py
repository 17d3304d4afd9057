"""Helpers for the GPU tests: numpy storage arrays <-> torch device tensors, and one-call wrappers."""
import numpy as np
import torch

import all_reduce_reduction_ring_amd as ar
import oracle

TORCH_DT = {ar.AR_F32: torch.float32, ar.AR_BF16: torch.bfloat16, ar.AR_F16: torch.float16, ar.AR_I32: torch.int32}
BITS_DT = {ar.AR_F32: torch.int32, ar.AR_BF16: torch.int16, ar.AR_F16: torch.int16, ar.AR_I32: torch.int32}
NP_BITS = {ar.AR_F32: np.uint32, ar.AR_BF16: np.uint16, ar.AR_F16: np.uint16, ar.AR_I32: np.uint32}
# the oracle's dtype and op codes are its own; they happen to be numbered the same way
ORACLE_DT = {ar.AR_F32: oracle.F32, ar.AR_BF16: oracle.BF16, ar.AR_F16: oracle.F16, ar.AR_I32: oracle.I32}
ORACLE_OP = {ar.AR_SUM: oracle.SUM, ar.AR_AVG: oracle.AVG, ar.AR_MIN: oracle.MIN, ar.AR_MAX: oracle.MAX}
KIND = {ar.AR_F32: "uniform_f32", ar.AR_BF16: "uniform_bf16", ar.AR_F16: "uniform_f16", ar.AR_I32: "int32"}
DEV = "cuda:0"


def to_dev(x, dt, offset=0, guard=0, fill_bits=None):
    """Storage array -> device tensor view of len(x) elements, placed `offset` elements into an allocation
    with `guard` spare elements on each side (filled with fill_bits, default 0x5A pattern)."""
    bits = np.ascontiguousarray(x).view(NP_BITS[dt]).astype(NP_BITS[dt], copy=False)
    n = bits.size
    total = n + offset + 2 * guard
    base = torch.empty(total, dtype=BITS_DT[dt], device=DEV)
    base.fill_(0x5A5A if BITS_DT[dt] == torch.int16 else 0x5A5A5A5A) if fill_bits is None else base.fill_(fill_bits)
    host = torch.from_numpy(bits.view(np.int16 if BITS_DT[dt] == torch.int16 else np.int32).copy())
    view = base[guard + offset: guard + offset + n]
    view.copy_(host.to(DEV))
    return base, view.view(TORCH_DT[dt])


def from_dev(t, dt):
    return t.detach().view(BITS_DT[dt]).cpu().numpy().view(NP_BITS[dt])


def empty_like_dev(n, dt, offset=0, guard=0, poison=True):
    base = torch.empty(n + offset + 2 * guard, dtype=BITS_DT[dt], device=DEV)
    base.fill_(-1 if poison else 0)  # all-ones: a NaN pattern for floats, -1 for int32
    return base, base[guard + offset: guard + offset + n].view(TORCH_DT[dt])


def run(xs, dt, op, algo, offset=0, inplace=False):
    """Upload rank arrays, all-reduce on the GPU, return the rank outputs as storage arrays."""
    ins = [to_dev(x, dt, offset=offset)[1] for x in xs]
    outs = ins if inplace else [empty_like_dev(len(x), dt, offset=offset)[1] for x in xs]
    need = ar.ar_allreduce_workspace_size(len(xs), len(xs[0]), dt, op, algo)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        ar.ar_allreduce_ws(ins, outs, op, algo, ws)
    else:
        ar.ar_allreduce(ins, outs, op, algo)
    torch.cuda.synchronize()
    return [from_dev(o, dt) for o in outs]


ORACLE_FOR = {
    ar.AR_ALGO_RING: oracle.ring_allreduce,
    ar.AR_ALGO_RING_STEPWISE: oracle.ring_allreduce,
    ar.AR_ALGO_FUSED: oracle.fused_allreduce,
    ar.AR_ALGO_RHD: oracle.rhd_allreduce,
    ar.AR_ALGO_RHD_STEPWISE: oracle.rhd_allreduce,
    ar.AR_ALGO_RING_FP8: oracle.fp8_ring_allreduce,
    ar.AR_ALGO_TREE: oracle.tree_allreduce,
    ar.AR_ALGO_TREE_STEPWISE: oracle.tree_allreduce,
}


def expect(xs, dt, op, algo):
    return [np.asarray(o).view(NP_BITS[dt]) for o in ORACLE_FOR[algo](xs, ORACLE_DT[dt], ORACLE_OP[op])]


def assert_bitwise(got, want, what=""):
    for r, (g, w) in enumerate(zip(got, want)):
        if not np.array_equal(g, w):
            bad = np.nonzero(g != w)[0]
            raise AssertionError(f"{what}: rank {r}: {bad.size} of {g.size} elements differ; first at {bad[:5]}: "
                                 f"got {g[bad[:5]]} want {w[bad[:5]]}")
