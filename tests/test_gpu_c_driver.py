"""One all-reduce driven from a plain C program (tests/c/allreduce_from_c.c, built with gcc by
__graft_entry__.build()): the process that calls the library holds no Python and no PyTorch, only the C ABI
and the HIP runtime's C API, with its own device buffers and stream. Inputs come from the seeded generators
through a file; every output element of every rank is compared with the oracle."""
import os
import subprocess

import numpy as np
import pytest

import all_reduce_reduction_ring_amd as ar
import oracle
from all_reduce_reduction_ring_amd import inputs
from gpu_util import ORACLE_DT, ORACLE_OP

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "build", "allreduce_from_c")
ORACLE_ALGO = {ar.AR_ALGO_RING: oracle.ring_allreduce, ar.AR_ALGO_TREE: oracle.tree_allreduce,
               ar.AR_ALGO_FUSED: oracle.fused_allreduce, ar.AR_ALGO_RING_FP8: oracle.fp8_ring_allreduce}
CASES = [  # (nranks, count, dtype, op, algo, input kind)
    (8, 1_000_003, ar.AR_BF16, ar.AR_AVG, ar.AR_ALGO_RING, "normal_bf16"),
    (4, 262_147, ar.AR_F32, ar.AR_SUM, ar.AR_ALGO_TREE, "uniform_f32"),
    (3, 100_001, ar.AR_I32, ar.AR_MAX, ar.AR_ALGO_FUSED, "int32"),
    (8, 65_543, ar.AR_BF16, ar.AR_SUM, ar.AR_ALGO_RING_FP8, "outlier_bf16"),
]


@pytest.mark.parametrize("n,count,dt,op,algo,kind", CASES, ids=[f"n{c[0]}_dt{c[2]}_algo{c[4]}" for c in CASES])
def test_allreduce_from_c(tmp_path, n, count, dt, op, algo, kind):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: __graft_entry__.build() builds it")
    xs = inputs.rank_inputs(kind, n, count, cfg=61, extra=(n, count))
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    np.concatenate([x.view(np.uint8) for x in xs]).tofile(fin)
    print(f"case n={n} count={count} dtype={dt} op={op} algo={algo}", flush=True)
    r = subprocess.run([EXE, str(fin), str(fout), str(n), str(count), str(dt), str(op), str(algo)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = np.fromfile(fout, dtype=np.uint8).reshape(n, -1)
    want = ORACLE_ALGO[algo](xs, ORACLE_DT[dt], ORACLE_OP[op])
    for rank in range(n):
        np.testing.assert_array_equal(got[rank], want[rank].view(np.uint8))
