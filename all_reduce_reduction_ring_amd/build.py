"""Build libar.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, with IEEE fp32 semantics kept intact
(-ffp-contract=off: no a*b+c contraction anywhere, so sums and the fp8 quantize/dequantize round trips are
single IEEE operations) and packed-fp32 instruction selection disabled. Objects go to _build/, the library
next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libar.so")
# measurement kernels for the benchmark's roofline context (the fold's read and write halves on their own); a
# library of their own, so that nothing in libar exists only to be measured
CEILING_SRC = "ar_ceiling.hip"
CEILING_LIB = os.path.join(HERE, "libar_ceiling.so")
ARCH = "gfx950"

SOURCES = ["ar_api.hip", "ar_collapsed.hip", "ar_stepwise.hip", "ar_bucket.hip", "ar_fp8.hip", "ar_tensors.hip",
           "ar_rsag.hip", "ar_epilogue.hip"]
# ar_collapsed.hip holds several hundred kernel instances; it is compiled once per element type (AR_F32 = 0 ..
# AR_I32 = 3) and per build of its launch shape and load policy (AR_COLLAPSED_LARGE = 0, 1), so the eight parts
# build in parallel.
UNITS = [(src, []) for src in SOURCES if src != "ar_collapsed.hip"] + [
    ("ar_collapsed.hip", [f"-DAR_COLLAPSED_DTYPE={dt}", f"-DAR_COLLAPSED_LARGE={lg}"]) for dt in range(4) for lg in (0, 1)]

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libar")


def _compile(unit) -> str:
    src, defs = unit
    tag = "".join("_" + d.split("=")[-1] for d in defs)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc(), "-c", *CFLAGS, *defs, "-o", obj, os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    # -z defs: an unresolved symbol (say a missing per-type part) fails the link instead of the first call
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None) -> str:
    """Compile every source and link libar.so (and libar_ceiling.so); returns libar's path."""
    os.makedirs(BUILD, exist_ok=True)
    units = UNITS + [(CEILING_SRC, [])]
    jobs = jobs or min(len(units), max(1, (os.cpu_count() or 4)))
    # the slowest units first, so they are not left running alone at the end
    order = sorted(units, key=lambda u: u[0] not in ("ar_collapsed.hip", "ar_tensors.hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip([u[0] + "".join(u[1]) for u in order], ex.map(_compile, order)))
    ceiling = objs.pop(CEILING_SRC)
    _link(list(objs.values()), LIB)
    _link([ceiling], CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
