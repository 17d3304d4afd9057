"""Planted mistakes in the oracle, on the CPU: each mutant is oracle.c with one plausible mistake written in (a
wrong chunk index, a wrong rounding rule, a wrong scale, a wrong bucket rule ...), built into a library of its
own and run under the oracle's pins (tests/test_oracle_pins.py, through ORACLE_LIB). Every mutant must make at
least one pin fail, so the pins are shown to constrain each part of the oracle; an unmodified build run the same
way must pass, so a failure is the mutant's and not the harness's.

Two mistakes are left out because they are equivalent (no input tells them apart): which half a
halving-doubling rank keeps (only which rank holds a block changes, never its bits), and the operands of one
fp32 add swapped (IEEE addition is commutative)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# name -> [(text in oracle.c, replacement, number of occurrences replaced)]
MUTANTS = {
    "ring reduce-scatter sends chunk (i+s) mod N": [("int c = imod(i - s, n)", "int c = imod(i + s, n)", 4)],
    "ring all-gather forwards chunk (i+off+s) mod N": [("imod(i + off - s, n)", "imod(i + off + s, n)", 2)],
    "owner finishes chunk i instead of (i+1) mod N": [("int c = (i + 1) % n;", "int c = i;", 2)],
    "standalone reduce-scatter takes chunk c from rank c": [("int owner = imod(c - 1, n);", "int owner = c;", 1)],
    "avg multiplies by 1/N": [("return u_of(f_of(v) / (float)n);", "return u_of(f_of(v) * (1.0f / (float)n));", 1)],
    "int32 avg rounds toward minus infinity": [("if (isint) return (uint32_t)((int32_t)v / n);",
                                                "if (isint) return (uint32_t)(int32_t)floor((double)(int32_t)v / n);",
                                                1)],
    "remainder of the split all in the last chunk": [("lo[c] = (int64_t)c * q + (c < r ? c : r);",
                                                      "lo[c] = (c < n) ? (int64_t)c * q : count;", 1)],
    "rounding ties away from zero": [("double r = nearbyint(q);", "double r = round(q);", 1)],
    "bf16 by truncation": [("double r = round_binary(f, 7, -126);", "double r = f;", 1)],
    "E4M3 encoded with bias 8": [("((ex + 7) << 3)", "((ex + 8) << 3)", 1)],
    "E4M3 decoded one binade low": [("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)", 1)],
    "min takes +0 over -0": [("return signbit(a) ? a : b;", "return signbit(a) ? b : a;", 1)],
    "rank-order reduce folds from the last rank": [
        ("uint32_t acc = widen(ins[0], dt, e);\n        for (int r = 1; r < n; ++r) acc = combine(acc, widen(ins[r], dt, e), isint, op);",
         "uint32_t acc = widen(ins[n - 1], dt, e);\n        for (int r = n - 2; r >= 0; --r) acc = combine(acc, widen(ins[r], dt, e), isint, op);",
         1)],
    "halving pairs distance 1 first": [("int d = n >> (j + 1);", "int d = 1 << j;", 2)],
    "binomial tree takes a wrong partner above level 0": [("int src = i + (1 << j);", "int src = i + (1 << j) - (j > 0);", 1)],
    "binomial broadcast skips level 0": [("for (int j = top - 1; j >= 0; --j)", "for (int j = top - 1; j >= 1; --j)", 1)],
    "fp8 scale as 1/inv": [("scale = amax / 448.0f;", "scale = 1.0f / inv;", 1)],
    "fp8 without the infinite-inverse fallback": [("if (isinf(inv)) { inv = 1.0f; scale = 1.0f; }", "", 1)],
    "fp8 amax counts NaN": [("if (a > amax) amax = a;", "if (!(a <= amax)) amax = a;", 1)],
    "fp8 messages travel unquantized": [("dst[e] = deq(mc[e], ms[e / FP8_BLOCK]) + dst[e];",
                                        "dst[e] = ((const float*)(w[i] + lo[c]))[e] + dst[e];", 1)],
    "fp8 avg applied after decoding": [
        ("for (int64_t e = 0; e < lo[c + 1] - lo[c]; ++e) v[e] = f_of(finalize(u_of(v[e]), 0, op, n));", ";", 1),
        ("narrow_store(outs[r], dt, e, u_of(deq(gc[e], gs[bbase[c] + (e - lo[c]) / FP8_BLOCK])));",
         "narrow_store(outs[r], dt, e, finalize(u_of(deq(gc[e], gs[bbase[c] + (e - lo[c]) / FP8_BLOCK])), 0, op, n));",
         1)],
    "bucket counts left unpadded": [("bucket_count[b] = (fill + g * n - 1) / (g * n) * (g * n);",
                                     "bucket_count[b] = fill;", 2)],
    "bucket closed when it reaches the cap": [("(fill + pad) * es > cap_bytes", "(fill + pad) * es >= cap_bytes", 1)],
    "standalone epilogue skips the average": [("narrow_store(out, dt, e, finalize(acc[e], isint, op, n));",
                                               "narrow_store(out, dt, e, acc[e]);", 1)],
}


def _mutate(text, edits):
    for old, new, count in edits:
        found = text.count(old)
        if found != count:
            raise AssertionError(f"mutation site {old!r} occurs {found} times in oracle.c, expected {count}")
        text = text.replace(old, new)
    return text


def _run_pins(lib_path):
    env = dict(os.environ, ORACLE_LIB=lib_path, OMP_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", PINS]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with open(SRC) as f:
        text = f.read()
    jobs = {"(unmodified)": text}
    for name, edits in MUTANTS.items():
        jobs[name] = _mutate(text, edits)
    libs = {}
    for k, (name, src) in enumerate(jobs.items()):
        c = tmp_path / f"m{k}.c"
        c.write_text(src)
        libs[name] = str(tmp_path / f"libm{k}.so")
        oracle.compile_library(str(c), libs[name], extra=["-w"])
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = dict(zip(libs, ex.map(_run_pins, libs.values())))
    ctrl = results.pop("(unmodified)")
    assert ctrl.returncode == 0, f"the unmodified build failed its pins:\n{ctrl.stdout[-3000:]}"
    survivors = [name for name, r in results.items() if r.returncode != 1]
    assert not survivors, "mutants not caught by any pin (or crashed): " + "; ".join(
        f"{name} (exit {results[name].returncode})" for name in survivors)
