"""Chunked, seeded random arrays.

Every array is identified by a key tuple, e.g. (42, workload_code, tensor_id). Element i of the
flat array lives in chunk c = i // CHUNK and is drawn from
numpy.random.Generator(PCG64(SeedSequence(key + (c,)))). Chunks are independent, so large tensors
are generated in parallel threads and any slice can be regenerated on its own.

bf16 values are produced by rounding the fp32 sample to the nearest bf16 with ties to even and
are carried as their raw 16-bit patterns (numpy.uint16).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the bit patterns as uint16.

    Inputs are finite by construction (no NaN handling)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_chunks(n: int, key: tuple, fn, out: np.ndarray) -> None:
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key) + [c])))
        out[lo:hi] = fn(g, hi - lo)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))


def normal(shape, std: float, key: tuple, dtype: str = "f32", mean: float = 0.0) -> np.ndarray:
    """N(mean, std^2) samples. dtype 'f32' -> float32 array, 'bf16' -> uint16 bf16 bit patterns."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    s32 = np.float32(std)
    m32 = np.float32(mean)

    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)

        def fn(g, cnt):
            z = g.standard_normal(cnt, dtype=np.float32)
            z *= s32
            if mean != 0.0:
                z += m32
            return z
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)

        def fn(g, cnt):
            z = g.standard_normal(cnt, dtype=np.float32)
            z *= s32
            if mean != 0.0:
                z += m32
            return f32_to_bf16_bits(z)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    _fill_chunks(n, key, fn, out)
    return out.reshape(shape)


def uniform_open01(shape, key: tuple) -> np.ndarray:
    """float32 samples in the open interval (0, 1)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(n, dtype=np.float32)

    def fn(g, cnt):
        u = g.random(cnt, dtype=np.float32)
        # random() draws from [0, 1); move exact zeros into the open interval
        u[u == 0.0] = np.float32(2.0 ** -24)
        return u

    _fill_chunks(n, key, fn, out)
    return out.reshape(shape)


def randint(shape, low: int, high: int, key: tuple) -> np.ndarray:
    """int32 samples uniform in [low, high)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(n, dtype=np.int32)
    _fill_chunks(n, key, lambda g, cnt: g.integers(low, high, cnt, dtype=np.int32), out)
    return out.reshape(shape)


def permutation(n: int, key: tuple) -> np.ndarray:
    """A seeded permutation of range(n) as int32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))
    return g.permutation(n).astype(np.int32)


def generator(key: tuple) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))
