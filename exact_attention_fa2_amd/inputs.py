"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module holds no attention arithmetic: it draws iid N(0,1) values, rounds
them to a storage dtype and promotes them back exactly.  Both the HIP path and
the oracle consume what it produces; neither is imported here.

Recipe (fixed, independent of thread count):
  * tensor t (0 = Q, 1 = K, 2 = V, 3 and up = extras such as dO) is drawn in
    chunks of ``CHUNK`` elements in row-major order; chunk c is
    ``numpy.random.Generator(PCG64(SeedSequence([seed, t, c]))).standard_normal(n, float32)``;
  * the float32 values are rounded to nearest-even into the storage dtype:
    float16 via numpy's cast, bfloat16 via the bit routine below;
  * promotion to float64 is exact for all three storage dtypes.

bfloat16 values are carried in numpy as their uint16 bit patterns.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

CHUNK = 1 << 22

DTYPES = ("f32", "f16", "bf16")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError("unknown dtype %r" % dtype)


def storage_numpy_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, seed: int, tensor_id: int, dtype: str = "f32") -> np.ndarray:
    """iid N(0,1) of the given shape, rounded into ``dtype`` storage."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    out = np.empty(n, dtype=storage_numpy_dtype(dtype))
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, c])))
        out[lo:hi] = _storage(g.standard_normal(hi - lo, dtype=np.float32), dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with cf.ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact promotion of storage values to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64).reshape(a.shape)
    return np.asarray(a).astype(np.float64)


def qkv(q_shape, kv_shape, seed: int, dtype: str):
    """Q, K, V drawn in that order (tensor ids 0, 1, 2) from one seed."""
    return (normal(q_shape, seed, 0, dtype), normal(kv_shape, seed, 1, dtype),
            normal(kv_shape, seed, 2, dtype))
