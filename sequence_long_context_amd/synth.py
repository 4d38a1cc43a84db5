"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU checker.

This module holds random draws and storage-format rounding only -- none of the
layout or attention arithmetic -- so that the HIP path and the CPU oracle can
be fed the same bits without sharing any of the method's code.

Recipe: numpy ``Generator(PCG64(seed))``, ``standard_normal`` in float32,
stored either as float32 or rounded to bfloat16 (round to nearest, ties to
even).  bfloat16 arrays are carried as their uint16 bit patterns.
Seeds: ``1000 * workload + {q: 1, k: 2, v: 3}``.
"""
from __future__ import annotations

import numpy as np

# "do": the output gradient; "pq", "pk", "pv": inputs in the exchange's piece order
TENSOR_SEED = {"q": 1, "k": 2, "v": 3, "do": 4, "pq": 5, "pk": 6, "pv": 7}
_CHUNK = 1 << 24


def seed_for(workload: int, tensor: str) -> int:
    return 1000 * int(workload) + TENSOR_SEED[tensor]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, shape, dtype: str = "bf16") -> np.ndarray:
    """N(0,1) draws of the given shape: float32, or bfloat16 as uint16 bits."""
    n = int(np.prod(shape))
    g = np.random.Generator(np.random.PCG64(seed))
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        for s in range(0, n, _CHUNK):
            out[s:s + _CHUNK] = g.standard_normal(min(_CHUNK, n - s), dtype=np.float32)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        for s in range(0, n, _CHUNK):
            out[s:s + _CHUNK] = f32_to_bf16_bits(
                g.standard_normal(min(_CHUNK, n - s), dtype=np.float32))
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def uniform_ints(seed: int, shape, dtype=np.int32) -> np.ndarray:
    """Arbitrary bit patterns (for bitwise-copy checks)."""
    g = np.random.Generator(np.random.PCG64(seed))
    info = np.iinfo(dtype)
    return g.integers(info.min, info.max, size=shape, dtype=dtype, endpoint=True)
