"""Pins for the CPU reference: checks against facts fixed outside the reference itself.

Each pin takes a loaded reference library (the real one, or a planted-mistake
variant) and returns a list of failure strings (empty = pass). Kept separate
from the test functions so the planted-mistake test can run every pin against
every mutated build.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

import oracle
from dense_fp16_gemm_03_amd import inputs


def _exact(h: np.ndarray) -> list:
    return [[Fraction(float(v)) for v in row] for row in h]


def pin_half_exhaustive(lib) -> list:
    """All 65536 binary16 patterns decode as numpy's independent float16 -> float64."""
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([lib.oracle_half_to_double(int(b)) for b in bits])
    bad = []
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    if not np.array_equal(nan_ref, nan_got):
        bad.append(f"NaN classification differs at {np.flatnonzero(nan_ref != nan_got)[:5]}")
    fin = ~nan_ref & ~nan_got
    diff = fin & ((got != ref) | (np.signbit(got) != np.signbit(ref)))
    if diff.any():
        i = np.flatnonzero(diff)[:5]
        bad.append(f"decode differs at {[hex(int(b)) for b in i]}: {got[i]} vs {ref[i]}")
    return bad


# IEEE 754 binary16 values fixed by the format's definition.
HALF_KNOWN = {
    0x0000: 0.0, 0x8000: -0.0, 0x3C00: 1.0, 0xBC00: -1.0, 0x4000: 2.0, 0xC000: -2.0,
    0x3800: 0.5, 0x3555: 0.333251953125, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14,
    0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x8001: -(2.0 ** -24),
    0x7C00: float("inf"), 0xFC00: float("-inf"),
}


def pin_half_known(lib) -> list:
    bad = []
    for h, v in HALF_KNOWN.items():
        g = lib.oracle_half_to_double(h)
        if g != v or np.signbit(g) != np.signbit(v):
            bad.append(f"{h:#06x} -> {g}, expected {v}")
    for h in (0x7C01, 0x7E00, 0xFFFF):
        if not np.isnan(lib.oracle_half_to_double(h)):
            bad.append(f"{h:#06x} should be NaN")
    return bad


def pin_brute_integer(lib) -> list:
    """Tiny shapes, integer entries: the reference equals exact Python-integer sums."""
    bad = []
    sizes = (1, 2, 3, 5, 8, 17, 33)
    rng = np.random.default_rng(11)
    for M, N, K in itertools.product(sizes, repeat=3):
        if M * N * K > 20000:
            continue
        A = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
        B = rng.integers(-2, 3, size=(N, K)).astype(np.float16)
        C, S = oracle.gemm_abt(A, B, threads=2, lib=lib)
        Ai, Bi = A.astype(np.int64), B.astype(np.int64)
        for i in range(M):
            for j in range(N):
                c = sum(int(Ai[i, k]) * int(Bi[j, k]) for k in range(K))
                s = sum(abs(int(Ai[i, k]) * int(Bi[j, k])) for k in range(K))
                if C[i, j] != c or S[i, j] != s:
                    bad.append(f"{M}x{N}x{K} at ({i},{j}): C {C[i, j]} vs {c}, S {S[i, j]} vs {s}")
                    return bad
    return bad


def pin_brute_rational(lib) -> list:
    """Tiny shapes, uniform fp16: within the binary64 summation bound of the exact sum."""
    bad = []
    for M, N, K in ((3, 4, 5), (2, 2, 40), (5, 3, 17), (1, 1, 257)):
        A = inputs.uniform(M, K, 21)
        B = inputs.uniform(N, K, 22)
        C, S = oracle.gemm_abt(A, B, threads=1, lib=lib)
        EA, EB = _exact(A), _exact(B)
        for i in range(M):
            for j in range(N):
                prods = [EA[i][k] * EB[j][k] for k in range(K)]
                exact_c = sum(prods, Fraction(0))
                exact_s = sum((abs(p) for p in prods), Fraction(0))
                bound = (K * 2.0 ** -52) * float(exact_s)
                if abs(Fraction(C[i, j]) - exact_c) > Fraction(bound):
                    bad.append(f"{M}x{N}x{K} ({i},{j}): C {C[i, j]!r} exact {float(exact_c)!r}")
                    return bad
                if abs(Fraction(S[i, j]) - exact_s) > Fraction(bound):
                    bad.append(f"{M}x{N}x{K} ({i},{j}): S {S[i, j]!r} exact {float(exact_s)!r}")
                    return bad
    return bad


def pin_identity(lib) -> list:
    """A = I gives C = B^T; B = I gives C = A (exact)."""
    bad = []
    K = 48
    X = inputs.uniform(40, K, 31)
    C, _ = oracle.gemm_abt(inputs.identity(K), X, lib=lib)
    if not np.array_equal(C, X.astype(np.float64).T):
        bad.append("A = I: C != B^T")
    C, _ = oracle.gemm_abt(X, inputs.identity(K), lib=lib)
    if not np.array_equal(C, X.astype(np.float64)):
        bad.append("B = I: C != A")
    return bad


def pin_perm(lib) -> list:
    """A = I, B = ((37 j + 11 k) mod 2048) - 1024: C[i][j] = B[j][i] (non-symmetric)."""
    K = 64
    P = inputs.perm_pattern(50, K)
    C, _ = oracle.gemm_abt(inputs.identity(K), P, lib=lib)
    if not np.array_equal(C, P.astype(np.float64).T):
        return ["perm pattern: C != B^T"]
    return []


def pin_ones(lib) -> list:
    """All-ones gives C = K; k-block weights give a sum that names missing k-blocks."""
    bad = []
    for K in (1, 7, 64, 129):
        C, S = oracle.gemm_abt(inputs.ones(3, K), inputs.ones(4, K), lib=lib)
        if not (np.all(C == K) and np.all(S == K)):
            bad.append(f"ones K={K}: C {C.ravel()[:3]}")
    K, blk = 1000, 64
    C, _ = oracle.gemm_abt(inputs.ones(2, K), inputs.kblock_weights(3, K, blk), lib=lib)
    expect = sum((1 + (b % 7)) * min(blk, K - b * blk) for b in range((K + blk - 1) // blk))
    if not np.all(C == expect):
        bad.append(f"k-block weights: {C.ravel()[:3]} vs {expect}")
    return bad


def pin_transpose(lib) -> list:
    """(A B^T)^T = B A^T with identical products in identical order: bitwise."""
    A = inputs.uniform(37, 70, 41)
    B = inputs.uniform(29, 70, 42)
    C1, S1 = oracle.gemm_abt(A, B, lib=lib)
    C2, S2 = oracle.gemm_abt(B, A, lib=lib)
    if not (np.array_equal(C1, C2.T) and np.array_equal(S1, S2.T)):
        return ["transpose invariant broken"]
    return []


def pin_abs_identity(lib) -> list:
    """S(A, B) = C(|A|, |B|) bitwise (|a b| = |a| |b|, same order)."""
    A = inputs.uniform(20, 90, 51)
    B = inputs.uniform(24, 90, 52)
    _, S = oracle.gemm_abt(A, B, lib=lib)
    C, _ = oracle.gemm_abt(np.abs(A), np.abs(B), lib=lib)
    return [] if np.array_equal(S, C) else ["S != C(|A|,|B|)"]


def pin_numpy(lib, M=256, N=256, K=256) -> list:
    """Against numpy's binary64 matmul (a library routine, different summation order)."""
    bad = []
    A, B = inputs.workload_operands((M, N, K), "integer")
    C, _ = oracle.gemm_abt(A, B, lib=lib)
    if not np.array_equal(C, A.astype(np.float64) @ B.astype(np.float64).T):
        bad.append("integer: oracle != numpy")
    A, B = inputs.workload_operands((M, N, K), "uniform")
    C, S = oracle.gemm_abt(A, B, lib=lib)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    if not np.all(np.abs(C - ref) <= 2 * K * 2.0 ** -52 * S):
        bad.append(f"uniform: max |oracle-numpy|/S = {np.max(np.abs(C - ref) / S):.3g}")
    return bad


def pin_strided(lib) -> list:
    """Row strides larger than K read the same logical matrices."""
    A = inputs.uniform(33, 80, 61)
    B = inputs.uniform(35, 72, 62)
    a, b = A[:, 5:69], B[:, 3:67]  # views with lda = 80, ldb = 72
    C1, S1 = oracle.gemm_abt(a, b, lib=lib)
    C2, S2 = oracle.gemm_abt(np.ascontiguousarray(a), np.ascontiguousarray(b), lib=lib)
    return [] if (np.array_equal(C1, C2) and np.array_equal(S1, S2)) else ["strided != contiguous"]


def pin_elems(lib) -> list:
    """The element-list entry agrees with the full one, bitwise."""
    A = inputs.uniform(40, 100, 71)
    B = inputs.uniform(45, 100, 72)
    C, S = oracle.gemm_abt(A, B, lib=lib)
    rows = np.array([0, 39, 7, 12, 39, 0])
    cols = np.array([0, 44, 3, 40, 0, 44])
    c, s = oracle.gemm_abt_elems(A, B, rows, cols, lib=lib)
    ok = np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])
    return [] if ok else ["elems != full"]


# --- bfloat16 entry points ---------------------------------------------------

def _bf16_values(bits: np.ndarray) -> np.ndarray:
    """numpy's own binary32 reading of bfloat16 bits (the upper half of a binary32)."""
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def pin_bf16_exhaustive(lib) -> list:
    """All 65536 bfloat16 patterns decode as numpy reads the same bits as binary32."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _bf16_values(bits)
    got = np.array([lib.oracle_bf16_to_double(int(b)) for b in bits])
    bad = []
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    if not np.array_equal(nan_ref, nan_got):
        bad.append(f"NaN classification differs at {np.flatnonzero(nan_ref != nan_got)[:5]}")
    fin = ~nan_ref & ~nan_got
    diff = fin & ((got != ref) | (np.signbit(got) != np.signbit(ref)))
    if diff.any():
        i = np.flatnonzero(diff)[:5]
        bad.append(f"bf16 decode differs at {[hex(int(b)) for b in i]}: {got[i]} vs {ref[i]}")
    return bad


# bfloat16 values fixed by the format (1 sign, 8 exponent bits with bias 127, 7 fraction bits).
BF16_KNOWN = {
    0x0000: 0.0, 0x8000: -0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F00: 0.5,
    0x3EAB: 0.333984375, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x0080: 2.0 ** -126,
    0x0001: 2.0 ** -133, 0x007F: 127 * 2.0 ** -133, 0x4300: 128.0, 0x4380: 256.0,
    0x7F80: float("inf"), 0xFF80: float("-inf"),
}


def pin_bf16_known(lib) -> list:
    bad = []
    for h, v in BF16_KNOWN.items():
        g = lib.oracle_bf16_to_double(h)
        if g != v or np.signbit(g) != np.signbit(v):
            bad.append(f"bf16 {h:#06x} -> {g}, expected {v}")
    for h in (0x7F81, 0x7FC0, 0xFFFF):
        if not np.isnan(lib.oracle_bf16_to_double(h)):
            bad.append(f"bf16 {h:#06x} should be NaN")
    return bad


def pin_bf16_brute_integer(lib) -> list:
    """Tiny shapes, integer bfloat16 entries: exact Python-integer sums."""
    rng = np.random.default_rng(13)
    for M, N, K in ((1, 1, 1), (2, 3, 5), (5, 2, 17), (3, 3, 33), (8, 5, 9)):
        ai = rng.integers(-3, 4, size=(M, K))
        bi = rng.integers(-3, 4, size=(N, K))
        C, S = oracle.gemm_abt_bf16(inputs.to_bf16_bits(ai), inputs.to_bf16_bits(bi),
                                    threads=2, lib=lib)
        for i in range(M):
            for j in range(N):
                c = sum(int(ai[i, k]) * int(bi[j, k]) for k in range(K))
                s = sum(abs(int(ai[i, k]) * int(bi[j, k])) for k in range(K))
                if C[i, j] != c or S[i, j] != s:
                    return [f"bf16 {M}x{N}x{K} at ({i},{j}): C {C[i, j]} vs {c}, S {S[i, j]} vs {s}"]
    return []


def pin_bf16_closed_forms(lib) -> list:
    """Identity, a non-symmetric bfloat16-exact pattern, all-ones and k-block weights."""
    bad = []
    K = 48
    I = inputs.to_bf16_bits(np.eye(K))
    X = inputs.uniform_bf16(40, K, 33)
    C, _ = oracle.gemm_abt_bf16(I, X, lib=lib)
    if not np.array_equal(C, _bf16_values(X).T):
        bad.append("bf16 A = I: C != B^T")
    C, _ = oracle.gemm_abt_bf16(X, I, lib=lib)
    if not np.array_equal(C, _bf16_values(X)):
        bad.append("bf16 B = I: C != A")
    P = inputs.perm_pattern_bf16(50, 64)
    C, _ = oracle.gemm_abt_bf16(inputs.to_bf16_bits(np.eye(64)), P, lib=lib)
    if not np.array_equal(C, _bf16_values(P).T):
        bad.append("bf16 perm pattern: C != B^T")
    for K in (1, 7, 129):
        one = inputs.to_bf16_bits(np.ones((3, K)))
        C, S = oracle.gemm_abt_bf16(one, one[:2], lib=lib)
        if not (np.all(C == K) and np.all(S == K)):
            bad.append(f"bf16 ones K={K}: {C.ravel()[:3]}")
    K, blk = 1000, 64
    w = inputs.to_bf16_bits(1 + ((np.arange(K) // blk) % 7))[None, :].repeat(3, axis=0)
    C, _ = oracle.gemm_abt_bf16(inputs.to_bf16_bits(np.ones((2, K))), w, lib=lib)
    expect = sum((1 + (b % 7)) * min(blk, K - b * blk) for b in range((K + blk - 1) // blk))
    if not np.all(C == expect):
        bad.append(f"bf16 k-block weights: {C.ravel()[:3]} vs {expect}")
    return bad


def pin_bf16_numpy_and_transpose(lib) -> list:
    """numpy binary64 matmul of numpy-decoded operands; transpose invariant; elements."""
    bad = []
    M = N = K = 128
    A, B = inputs.workload_operands((M, N, K), "integer", "bf16")
    C, _ = oracle.gemm_abt_bf16(A, B, lib=lib)
    if not np.array_equal(C, _bf16_values(A) @ _bf16_values(B).T):
        bad.append("bf16 integer: oracle != numpy")
    A, B = inputs.workload_operands((M, N, K), "uniform", "bf16")
    C, S = oracle.gemm_abt_bf16(A, B, lib=lib)
    ref = _bf16_values(A) @ _bf16_values(B).T
    if not np.all(np.abs(C - ref) <= 2 * K * 2.0 ** -52 * S):
        bad.append("bf16 uniform: oracle != numpy within the binary64 bound")
    C2, S2 = oracle.gemm_abt_bf16(B, A, lib=lib)
    if not (np.array_equal(C, C2.T) and np.array_equal(S, S2.T)):
        bad.append("bf16 transpose invariant broken")
    rows, cols = np.array([0, 127, 5, 64]), np.array([127, 0, 9, 64])
    c, s = oracle.gemm_abt_elems_bf16(A, B, rows, cols, lib=lib)
    if not (np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])):
        bad.append("bf16 elems != full")
    return bad


ALL_PINS = [pin_half_exhaustive, pin_half_known, pin_brute_integer, pin_brute_rational,
            pin_identity, pin_perm, pin_ones, pin_transpose, pin_abs_identity, pin_numpy,
            pin_strided, pin_elems, pin_bf16_exhaustive, pin_bf16_known,
            pin_bf16_brute_integer, pin_bf16_closed_forms, pin_bf16_numpy_and_transpose]
