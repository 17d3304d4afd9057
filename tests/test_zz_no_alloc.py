"""ar_allreduce_noalloc (the entry point for callers that cannot allocate) against ar_allreduce_ws with a caller
workspace: the same bits on two calls in a row, the second smaller, for every round-per-launch schedule on the 2-byte
types (the calls that use the scratch), plus a call that needs no scratch and a request beyond the scratch's size."""
import numpy as np
import pytest
import torch

import all_reduce_reduction_ring_amd as ar
from all_reduce_reduction_ring_amd import inputs
from gpu_util import DEV, KIND, assert_bitwise, empty_like_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu

STEPWISE = [ar.AR_ALGO_RING_STEPWISE, ar.AR_ALGO_RHD_STEPWISE, ar.AR_ALGO_TREE_STEPWISE]


def _pair(xs, dt, op, algo):
    """(noalloc outputs, workspace outputs) for the same inputs."""
    ins = [to_dev(x, dt)[1] for x in xs]
    got = [empty_like_dev(len(x), dt)[1] for x in xs]
    ref = [empty_like_dev(len(x), dt)[1] for x in xs]
    need = ar.ar_allreduce_workspace_size(len(xs), len(xs[0]), dt, op, algo)
    assert 0 < need <= ar.AR_NOALLOC_WS_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ar.ar_allreduce_ws(ins, ref, op, algo, ws)
    ar.ar_allreduce_noalloc(ins, got, op, algo)
    torch.cuda.synchronize()
    return [from_dev(o, dt) for o in got], [from_dev(o, dt) for o in ref]


@pytest.mark.parametrize("dt", [ar.AR_BF16, ar.AR_F16])
@pytest.mark.parametrize("algo", STEPWISE)
def test_noalloc_equals_caller_workspace_on_two_calls(dt, algo):
    n = 8
    # first call: 1,000,003 elements per rank (a 32 MB fp32 mirror); second: smaller and ragged, so a stale first
    # call's partials in the shared scratch would show
    for count, op in ((1_000_003, ar.AR_AVG), (77_777, ar.AR_SUM)):
        xs = inputs.rank_inputs(KIND[dt], n, count, cfg=120, extra=(algo, count))
        got, ref = _pair(xs, dt, op, algo)
        assert_bitwise(got, ref, f"noalloc vs workspace algo={algo} dt={dt} count={count}")


def test_noalloc_without_scratch_and_beyond_its_size():
    n = 4
    xs = inputs.rank_inputs("uniform_f32", n, 10_001, cfg=121)
    ins = [to_dev(x, ar.AR_F32)[1] for x in xs]
    got = [empty_like_dev(len(x), ar.AR_F32)[1] for x in xs]
    ref = [empty_like_dev(len(x), ar.AR_F32)[1] for x in xs]
    for algo in (ar.AR_ALGO_RING, ar.AR_ALGO_RING_STEPWISE):  # fp32 needs no scratch in either
        ar.ar_allreduce_noalloc(ins, got, ar.AR_SUM, algo)
        ar.ar_allreduce(ins, ref, ar.AR_SUM, algo)
        torch.cuda.synchronize()
        assert_bitwise([from_dev(o, ar.AR_F32) for o in got], [from_dev(o, ar.AR_F32) for o in ref], f"algo={algo}")
    # a bf16 schedule whose fp32 mirror would exceed the scratch: rejected before anything is enqueued
    n, count = 8, (ar.AR_NOALLOC_WS_BYTES // (8 * 4)) + 64
    assert ar.ar_allreduce_workspace_size(n, count, ar.AR_BF16, ar.AR_SUM, ar.AR_ALGO_RING_STEPWISE) > \
        ar.AR_NOALLOC_WS_BYTES
    big = [torch.zeros(count, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    outs = [torch.full((count,), 7.0, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    with pytest.raises(ar.ArError) as ei:
        ar.ar_allreduce_noalloc(big, outs, ar.AR_SUM, ar.AR_ALGO_RING_STEPWISE)
    assert ei.value.status == ar.AR_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert all(bool((o == 7.0).all()) for o in outs)
