"""The oracle's pins run once more against an AddressSanitizer + UndefinedBehaviorSanitizer build of oracle.c
(gcc, host code only): an out-of-bounds access, a use after free, a signed overflow or an invalid shift anywhere
in the oracle's paths fails this test, even where the values it returns happen to be right."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    oracle.compile_library(SRC, lib, extra=["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                            "-fno-sanitize-recover=all"])
    # reports go to files: pytest's own output capture would swallow them when the process stops
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS=f"detect_leaks=0:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", PINS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(tmp_path / f).read() for f in sorted(os.listdir(tmp_path)) if f.startswith("sanitizer"))
    assert not reports, reports[-4000:]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
