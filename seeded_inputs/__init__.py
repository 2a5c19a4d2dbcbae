"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws numbers and describes workload shapes.  It holds none of
the attention arithmetic, no index map and no merge rule: both the HIP library's
callers and the CPU oracle take their inputs from here, and nothing else is
shared between them.

Values
------
Every tensor is a global ``[B, S, H, D]`` array in global sequence order.  It is
cut into blocks of ``TOKENS_PER_BLOCK`` consecutive tokens of one batch entry;
block ``(b, n)`` is drawn from its own PCG64 stream seeded with
``SeedSequence([BASE_SEED, seed_id, tensor_id, b, n])``.  Any slice of the
sequence (one rank's shard, a sampled row) can therefore be regenerated on its
own and is bit-identical to the same slice of the full tensor.

Draws are standard normal in float32, multiplied by ``scale`` (a power of two in
every workload, so exact), then rounded to bfloat16 with round-to-nearest-even
when the workload is bf16.  bf16 tensors are returned as ``uint16`` bit patterns;
``bf16_bits_to_f32`` widens them exactly.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .workloads import WORKLOADS, Workload, workload  # noqa: F401

BASE_SEED = 20261203
TOKENS_PER_BLOCK = 128
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 0, 1, 2, 3


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Integer bit manipulation: add 0x7FFF plus the lowest kept bit, truncate the
    low 16 bits.  NaNs are kept as a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _block(seed_id: int, tensor_id: int, b: int, n: int, H: int, D: int,
           scale: float) -> np.ndarray:
    ss = np.random.SeedSequence([BASE_SEED, seed_id, tensor_id, b, n])
    rng = np.random.Generator(np.random.PCG64(ss))
    out = rng.standard_normal((TOKENS_PER_BLOCK, H, D), dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def tokens(seed_id: int, tensor_id: int, B: int, S: int, H: int, D: int,
           spans, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Rows of the global tensor at the given global spans, concatenated in order.

    ``spans`` is a list of ``(start, length)`` pairs of global token positions.
    Returns ``[B, sum(length), H, D]``: float32 for ``dtype == "f32"``, uint16
    bf16 bit patterns for ``dtype == "bf16"``.
    """
    spans = [(int(a), int(n)) for a, n in spans]
    for a, n in spans:
        if a < 0 or n < 0 or a + n > S:
            raise ValueError(f"span ({a}, {n}) outside [0, {S})")
    total = sum(n for _, n in spans)
    out = np.empty((B, total, H, D), dtype=np.float32)
    jobs = []
    col = 0
    for a, n in spans:
        t = a
        while t < a + n:
            blk = t // TOKENS_PER_BLOCK
            lo = t - blk * TOKENS_PER_BLOCK
            hi = min(TOKENS_PER_BLOCK, a + n - blk * TOKENS_PER_BLOCK)
            for b in range(B):
                jobs.append((b, blk, lo, hi, col))
            col += hi - lo
            t = blk * TOKENS_PER_BLOCK + hi

    def run(job):
        b, blk, lo, hi, c0 = job
        out[b, c0:c0 + hi - lo] = _block(seed_id, tensor_id, b, blk, H, D, scale)[lo:hi]

    if len(jobs) > 8:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    if dtype == "f32":
        return out
    if dtype == "bf16":
        return f32_to_bf16_bits(out).reshape(out.shape)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a tensor returned by ``tokens``."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)
