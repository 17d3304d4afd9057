"""Seeded synthetic inputs for the all-reduce workloads.

This module is shared by the GPU tests, the benchmark and the CPU oracle's tests. It draws random numbers and
converts dtypes with library routines only; it holds none of the all-reduce's own arithmetic (no reduction,
no chunking, no rounding rule of the method).

Every generator is a pure function of its seed, so the GPU path and the oracle always see identical bytes.
Storage conventions (numpy has no bfloat16):
  * fp32  -> np.float32
  * bf16  -> np.uint16 holding the bfloat16 bit pattern
  * f16   -> np.uint16 holding the binary16 bit pattern
  * int32 -> np.int32

Workloads (sizes use binary units: 1 MB = 2**20 bytes, 1K = 1024 elements):
  * ``uniform_pm1``: x = 2*U - 1 with U = rng.random(float32); every value is a multiple of 2**-24 in [-1, 1),
    so fp64 sums of a few of them are exact.
  * ``normal_bf16``: bf16(round-to-nearest-even(z * sigma)), z = rng.standard_normal(float32), the gradient-like
    data of a data-parallel step (the pages describe all-reduce as the gradient synchronisation of data-parallel
    training: astro-wiki "AllReduce", section on DDP).
  * ``outlier_bf16``: as ``normal_bf16`` but each element is multiplied by 100 with probability 0.001.
  * ``bucket_tensors``: 300 per-rank fp32 gradient tensors with log-uniform sizes in [1K, 16M] elements.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "uniform_pm1",
    "normal_f32",
    "normal_bf16",
    "outlier_bf16",
    "f32_to_bf16_bits_lib",
    "bucket_sizes",
    "bucket_tensors",
    "rank_inputs",
]


def _rng(seed_parts):
    return np.random.default_rng(list(seed_parts))


def f32_to_bf16_bits_lib(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns using torch's CPU conversion (a library routine, round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def uniform_pm1(seed_parts, count: int) -> np.ndarray:
    """2*U - 1 in float32, U = rng.random(count, float32). Exact: values are multiples of 2**-24."""
    u = _rng(seed_parts).random(count, dtype=np.float32)
    return (np.float32(2.0) * u - np.float32(1.0)).astype(np.float32, copy=False)


def normal_f32(seed_parts, count: int, sigma: float) -> np.ndarray:
    z = _rng(seed_parts).standard_normal(count, dtype=np.float32)
    return (z * np.float32(sigma)).astype(np.float32, copy=False)


def normal_bf16(seed_parts, count: int, sigma: float = 1e-3) -> np.ndarray:
    """bf16 bits of z*sigma, z ~ N(0,1) drawn in float32."""
    return f32_to_bf16_bits_lib(normal_f32(seed_parts, count, sigma))


def outlier_bf16(seed_parts, count: int, sigma: float = 1e-3, p: float = 1e-3, factor: float = 100.0):
    """bf16 bits of z*sigma*(factor if Bernoulli(p) else 1); the mask is drawn after z from the same stream."""
    rng = _rng(seed_parts)
    z = rng.standard_normal(count, dtype=np.float32)
    mask = rng.random(count, dtype=np.float32) < np.float32(p)
    v = z * np.float32(sigma)
    v[mask] *= np.float32(factor)
    return f32_to_bf16_bits_lib(v)


def bucket_sizes(ntensors: int = 300, lo_log2: float = 10.0, hi_log2: float = 24.0,
                 seed_parts=(3, 999)) -> np.ndarray:
    """Per-tensor element counts, log-uniform: clamp(round(2**u), 2**lo, 2**hi), u ~ U[lo, hi)."""
    u = _rng(seed_parts).uniform(lo_log2, hi_log2, ntensors)
    n = np.rint(np.exp2(u)).astype(np.int64)
    return np.clip(n, 1 << int(lo_log2), 1 << int(hi_log2))


def bucket_tensors(rank: int, sizes, sigma: float = 1e-2, cfg: int = 3):
    """The rank's list of fp32 gradient tensors, tensor t drawn from default_rng([cfg, rank, t])."""
    return [normal_f32((cfg, rank, t), int(n), sigma) for t, n in enumerate(sizes)]


def rank_inputs(kind: str, nranks: int, count: int, cfg: int, extra=()):
    """One array per rank for the named workload kind, rank r seeded with (cfg, r, *extra)."""
    out = []
    for r in range(nranks):
        seed = (cfg, r) + tuple(extra)
        if kind == "uniform_f32":
            out.append(uniform_pm1(seed, count))
        elif kind == "normal_bf16":
            out.append(normal_bf16(seed, count))
        elif kind == "outlier_bf16":
            out.append(outlier_bf16(seed, count))
        elif kind == "uniform_bf16":
            out.append(f32_to_bf16_bits_lib(uniform_pm1(seed, count)))
        elif kind == "uniform_f16":
            x = uniform_pm1(seed, count).astype(np.float16)  # numpy's fp32->fp16 conversion (library)
            out.append(x.view(np.uint16).copy())
        elif kind == "int32":
            out.append(_rng(seed).integers(-(1 << 31), (1 << 31) - 1, count, dtype=np.int32, endpoint=True))
        elif kind == "small_int32":
            out.append(_rng(seed).integers(-1000, 1000, count, dtype=np.int32, endpoint=True))
        else:
            raise ValueError(f"unknown input kind {kind!r}")
    return out
