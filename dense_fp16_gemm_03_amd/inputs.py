"""Seeded synthetic operands for C = A * B^T (binary16, row-major, K contiguous).

This module only *makes inputs*; it holds none of the product's arithmetic, so
both the GPU path's tests and the CPU reference read the same bytes from it.

Distributions:
  * ``uniform``: i.i.d. uniform on [-1, 1] drawn in binary64 by numpy's
    ``default_rng(seed)`` and rounded to nearest-even binary16.
  * ``integer``: i.i.d. uniform on the integers {lo..hi} (default -2..2), so
    every partial sum of C is an exact small integer in fp32.
  * ``hash_int``: integers in [-3, 3] from one hash of the element index, the
    kind of input "SASS-Level Kernel Generation for Blackwell" times on
    (section "How we measured", "The same inputs on both sides"); the hash is
    our own choice (the page does not give it): splitmix64 of the flat index.

Structured operands (identity, a permutation-like pattern, all-ones and a
k-block-weighted ones pattern) give closed-form products for the pins.

Standard seeds: A = 1, B = 2 for ``uniform``; A = 3, B = 4 for ``integer``.

``device_uniform`` draws multi-gigabyte operands on the GPU with torch's
seeded generator instead (same distribution, binary32 draws rounded to
binary16); the reference then reads back the rows it checks.

bfloat16 operands are numpy ``uint16`` arrays of bfloat16 bit patterns (numpy
has no bfloat16 type): the same draws, rounded binary64 -> binary32 -> bfloat16,
each step to nearest-even (``to_bf16_bits``). Integers up to 256 in magnitude
and the structured patterns below are exact in bfloat16.
"""
from __future__ import annotations

import numpy as np

SEED_A_UNIFORM, SEED_B_UNIFORM = 1, 2
SEED_A_INTEGER, SEED_B_INTEGER = 3, 4

# Shapes (M, N, K) of the five workloads.
WORKLOADS = {
    "256^3": (256, 256, 256),
    "1024^3": (1024, 1024, 1024),
    "2048x2048x16384": (2048, 2048, 16384),
    "1024x1024x65536": (1024, 1024, 65536),
    "8192^3": (8192, 8192, 8192),
}

# The other shapes of the timing table in "SASS-Level Kernel Generation for
# Blackwell" (section "The numbers"): same operation, timed and checked here
# as extra cases.
PAGE_SHAPES = {
    "1536^3": (1536, 1536, 1536),
    "2048^3": (2048, 2048, 2048),
    "3072x1280x2048": (3072, 1280, 2048),
    "4096x4096x1024": (4096, 4096, 1024),
    "4096^3": (4096, 4096, 4096),
    "8192x2048x4096": (8192, 2048, 4096),
    "16384^3": (16384, 16384, 16384),
}

# One GPU's share of each large workload split over 8 GPUs: 8192^3 by rows of
# A (M / 8; no exchange once the inputs are placed), the long-K workloads by
# K (K / 8; each GPU then holds a full fp32 partial C for one reduce-scatter).
SHARD_SHAPES = {
    "8192^3 M/8": (1024, 8192, 8192),
    "2048x2048x16384 K/8": (2048, 2048, 2048),
    "1024x1024x65536 K/8": (1024, 1024, 8192),
}


def uniform(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows x cols binary16, i.i.d. uniform on [-1, 1]."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), dtype=np.float16)
    # draw in row blocks to bound the binary64 temporary at large sizes
    step = max(1, (1 << 24) // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = rng.uniform(-1.0, 1.0, size=(r1 - r0, cols)).astype(np.float16)
    return out


def integer(rows: int, cols: int, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """rows x cols binary16 holding i.i.d. integers uniform on {lo..hi}."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.float16)


def _splitmix64(x: np.ndarray) -> np.ndarray:
    x = (x + np.uint64(0x9E3779B97F4A7C15)).astype(np.uint64)
    x = (x ^ (x >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    x = (x ^ (x >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return x ^ (x >> np.uint64(31))


def hash_int(rows: int, cols: int, salt: int = 0) -> np.ndarray:
    """rows x cols binary16 integers in [-3, 3] from a hash of the flat index."""
    idx = np.arange(rows * cols, dtype=np.uint64) + np.uint64(salt) * np.uint64(1 << 40)
    with np.errstate(over="ignore"):
        h = _splitmix64(idx)
    v = (h % np.uint64(7)).astype(np.int64) - 3
    return v.reshape(rows, cols).astype(np.float16)


def device_uniform(rows: int, cols: int, seed: int, device, ld: int | None = None):
    """rows x cols binary16 torch tensor on `device`, i.i.d. uniform on [-1, 1]:
    binary32 draws on [-1, 1) from torch's seeded generator for that device,
    rounded to binary16.

    For operands too large to draw on the host (gigabytes); whoever checks a
    result copies back the rows it needs. With ld > cols the tensor is a view
    of a rows x ld buffer whose columns past `cols` hold NaN, so a read beyond
    K poisons the result.
    """
    import torch

    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld must be >= cols")
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    if ld == cols:
        buf = torch.empty((rows, ld), dtype=torch.float16, device=device)
    else:
        buf = torch.full((rows, ld), float("nan"), dtype=torch.float16, device=device)
    view = buf[:, :cols]
    view.uniform_(-1.0, 1.0, generator=gen)
    return view


def identity(n: int, cols: int | None = None) -> np.ndarray:
    """n x cols binary16 with ones where row == column."""
    return np.eye(n, cols if cols is not None else n, dtype=np.float16)


def perm_pattern(rows: int, cols: int) -> np.ndarray:
    """P[j][k] = ((37 j + 11 k) mod 2048) - 1024, every value exact in binary16."""
    j = np.arange(rows, dtype=np.int64)[:, None]
    k = np.arange(cols, dtype=np.int64)[None, :]
    return (((37 * j + 11 * k) % 2048) - 1024).astype(np.float16)


def ones(rows: int, cols: int) -> np.ndarray:
    return np.ones((rows, cols), dtype=np.float16)


def kblock_weights(rows: int, cols: int, block: int) -> np.ndarray:
    """W[j][k] = 1 + ((k // block) mod 7): marks which k-blocks a sum covered."""
    k = np.arange(cols, dtype=np.int64)
    w = 1 + ((k // block) % 7)
    return np.broadcast_to(w.astype(np.float16), (rows, cols)).copy()


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of finite values: round to binary32, then
    keep the upper 16 bits rounded to nearest-even on the lower 16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return (b >> np.uint64(16)).astype(np.uint16)


def uniform_bf16(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows x cols bfloat16 bits, i.i.d. uniform on [-1, 1] (the ``uniform`` draw)."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, (1 << 24) // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = to_bf16_bits(rng.uniform(-1.0, 1.0, size=(r1 - r0, cols)))
    return out


def integer_bf16(rows: int, cols: int, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """rows x cols bfloat16 bits holding i.i.d. integers uniform on {lo..hi}."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.integers(lo, hi + 1, size=(rows, cols)))


def perm_pattern_bf16(rows: int, cols: int) -> np.ndarray:
    """P[j][k] = ((37 j + 11 k) mod 256) - 128 as bfloat16 bits (exact)."""
    j = np.arange(rows, dtype=np.int64)[:, None]
    k = np.arange(cols, dtype=np.int64)[None, :]
    return to_bf16_bits(((37 * j + 11 * k) % 256) - 128)


def workload_operands(shape, kind: str = "uniform", dtype: str = "f16"):
    """(A, B) for an (M, N, K) shape with the standard seeds of ``kind``;
    dtype "bf16" gives bfloat16 bit arrays (uint16) of the same draws."""
    M, N, K = shape
    if dtype == "bf16":
        if kind == "uniform":
            return uniform_bf16(M, K, SEED_A_UNIFORM), uniform_bf16(N, K, SEED_B_UNIFORM)
        if kind == "integer":
            return integer_bf16(M, K, SEED_A_INTEGER), integer_bf16(N, K, SEED_B_INTEGER)
        if kind == "hash_int":
            return (to_bf16_bits(hash_int(M, K, 1).astype(np.float32)),
                    to_bf16_bits(hash_int(N, K, 2).astype(np.float32)))
        raise ValueError(f"unknown input kind {kind!r}")
    if dtype != "f16":
        raise ValueError(f"unknown dtype {dtype!r}")
    if kind == "uniform":
        return uniform(M, K, SEED_A_UNIFORM), uniform(N, K, SEED_B_UNIFORM)
    if kind == "integer":
        return integer(M, K, SEED_A_INTEGER), integer(N, K, SEED_B_INTEGER)
    if kind == "hash_int":
        return hash_int(M, K, 1), hash_int(N, K, 2)
    raise ValueError(f"unknown input kind {kind!r}")
