"""The C ABI from a plain C99 program (tests/c/abi_from_c.c): include/ar.h compiles as C with every warning
enabled, the program links against the built libar.so, and its host-only and validation calls answer as the
header documents. No GPU is needed: nothing in the program reaches a kernel launch."""
import os
import shutil
import subprocess

import pytest

import all_reduce_reduction_ring_amd as ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_header_and_library_from_c(tmp_path):
    lib = ar.lib_path()
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", exe, lib,
           "-Wl,-rpath," + os.path.dirname(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert lines[-1] == "0 failure(s)"
    assert all(ln.startswith("ok ") for ln in lines[:-1]) and len(lines) > 10
