"""Reference for C = A * B^T on binary16 (or bfloat16) inputs, summed in binary64.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product library never does, and nothing here imports the
GPU package. The arithmetic lives in ``oracle.c`` (plain C, built with gcc);
this module only marshals numpy arrays into it.

Definition followed: "SASS-Level Kernel Generation for Blackwell", section
"The numbers" (Setup): fp16 inputs, fp32 accumulation and output, C = A B^T.
The oracle sums in binary64 (the double-accumulated CPU reference of the
handbook page "Asynchronous copies and the Hopper/Blackwell features", section
"Thread-block clusters and distributed shared memory"), in increasing k.

Pins (tests/test_oracle.py): exhaustive binary16 decode against numpy; brute
force in exact rational arithmetic on tiny inputs; identity, permutation and
all-ones closed forms; the transpose invariant; numpy binary64 matmul; the
absolute-sum identity S(A, B) = C(|A|, |B|); planted-mistake variants of the
C source that each pin must reject. The bfloat16 entry points (``*_bf16``)
take uint16 arrays of bfloat16 bit patterns and have pins of their own
(exhaustive decode against numpy's binary32 reading of the same bits, known
values, brute force, closed forms, numpy matmul).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None


def compile_library(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile ``source`` into a shared library with gcc (no fast-math: k order is kept)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", *extra_flags, source, "-o", output, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return output


def _bind(lib):
    i64 = ctypes.c_int64
    p = ctypes.c_void_p
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_gemm_abt.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, ctypes.c_int]
    lib.oracle_gemm_abt.restype = ctypes.c_int
    lib.oracle_gemm_abt_elems.argtypes = [i64, p, p, i64, p, i64, p, i64, p, p, ctypes.c_int]
    lib.oracle_gemm_abt_elems.restype = ctypes.c_int
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_gemm_abt_bf16.argtypes = lib.oracle_gemm_abt.argtypes
    lib.oracle_gemm_abt_bf16.restype = ctypes.c_int
    lib.oracle_gemm_abt_elems_bf16.argtypes = lib.oracle_gemm_abt_elems.argtypes
    lib.oracle_gemm_abt_elems_bf16.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it first if it is absent)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            compile_library()
        _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _as_f16_rows(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float16 array")
    if x.size and x.shape[1] > 1 and x.strides[1] != 2:
        raise ValueError(f"{name} rows must be contiguous")
    return x


def _as_bf16_rows(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 array of bfloat16 bit patterns")
    if x.size and x.shape[1] > 1 and x.strides[1] != 2:
        raise ValueError(f"{name} rows must be contiguous")
    return x


def _ld(x: np.ndarray) -> int:
    """Row stride in elements (any value >= K is fine for one-row or empty arrays)."""
    if x.shape[0] <= 1 or x.size == 0:
        return max(x.shape[1], 1)
    return x.strides[0] // 2


def half_to_double(bits: int, lib=None) -> float:
    """Decode one binary16 bit pattern (0..65535)."""
    return (lib or load()).oracle_half_to_double(bits)


def bf16_to_double(bits: int, lib=None) -> float:
    """Decode one bfloat16 bit pattern (0..65535)."""
    return (lib or load()).oracle_bf16_to_double(bits)


def gemm_abt(A: np.ndarray, B: np.ndarray, threads: int | None = None, lib=None):
    """Return (C, S): C = A B^T and S = sum_k |a_ik b_jk|, both float64 M x N."""
    lib = lib or load()
    A = _as_f16_rows(A, "A")
    B = _as_f16_rows(B, "B")
    return _full(lib.oracle_gemm_abt, A, B, threads)


def gemm_abt_bf16(A: np.ndarray, B: np.ndarray, threads: int | None = None, lib=None):
    """gemm_abt for bfloat16 operands given as uint16 bit-pattern arrays."""
    lib = lib or load()
    A = _as_bf16_rows(A, "A")
    B = _as_bf16_rows(B, "B")
    return _full(lib.oracle_gemm_abt_bf16, A, B, threads)


def _full(fn, A, B, threads):
    M, K = A.shape
    N, Kb = B.shape
    if Kb != K:
        raise ValueError("A and B must have the same number of columns K")
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    r = fn(M, N, K, A.ctypes.data, _ld(A), B.ctypes.data, _ld(B), C.ctypes.data, N,
           S.ctypes.data, N, threads or default_threads())
    if r < 0:
        raise ValueError("oracle rejected the arguments")
    return C, S


def gemm_abt_elems(A: np.ndarray, B: np.ndarray, rows, cols, threads: int | None = None,
                   lib=None):
    """Return (C, S) at the listed (rows[e], cols[e]) positions only."""
    lib = lib or load()
    A = _as_f16_rows(A, "A")
    B = _as_f16_rows(B, "B")
    return _elems(lib.oracle_gemm_abt_elems, A, B, rows, cols, threads)


def gemm_abt_elems_bf16(A: np.ndarray, B: np.ndarray, rows, cols, threads: int | None = None,
                        lib=None):
    """gemm_abt_elems for bfloat16 operands given as uint16 bit-pattern arrays."""
    lib = lib or load()
    A = _as_bf16_rows(A, "A")
    B = _as_bf16_rows(B, "B")
    return _elems(lib.oracle_gemm_abt_elems_bf16, A, B, rows, cols, threads)


def _elems(fn, A, B, rows, cols, threads):
    K = A.shape[1]
    if B.shape[1] != K:
        raise ValueError("A and B must have the same number of columns K")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and equally long")
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or cols.min() < 0
                      or cols.max() >= B.shape[0]):
        raise IndexError("element index out of range")
    C = np.empty(rows.size, dtype=np.float64)
    S = np.empty(rows.size, dtype=np.float64)
    r = fn(rows.size, rows.ctypes.data, cols.ctypes.data, K, A.ctypes.data, _ld(A),
           B.ctypes.data, _ld(B), C.ctypes.data, S.ctypes.data, threads or default_threads())
    if r < 0:
        raise ValueError("oracle rejected the arguments")
    return C, S


def within_tolerance(C_test: np.ndarray, C_ref: np.ndarray, S_ref: np.ndarray,
                     rel: float = 1e-5) -> np.ndarray:
    """Elementwise acceptance: |C_test - C_ref| <= rel * S (exact equality where S == 0)."""
    err = np.abs(C_test.astype(np.float64) - C_ref)
    ok = err <= rel * S_ref
    return ok & np.isfinite(C_test)
