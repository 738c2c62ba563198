"""The CPU reference against facts fixed outside it (CPU only).

A planted mistake in the reference's C source (compiled into a scratch
library) must be caught by at least one pin; that shows the pins constrain
each part of the reference: the binary16 and bfloat16 decodes, the k range,
operand indexing, the output index, the absolute sum and the format each
entry point decodes.
"""
import os

import numpy as np
import pytest

import oracle
from dense_fp16_gemm_03_amd import inputs
import oracle_pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    assert pin(oracle_lib) == []


def _read_worked(path):
    rows = {"A": [], "B": [], "C": [], "S": []}
    dims = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key in dims or key in ("M", "N", "K"):
                dims[key] = int(vals[0])
            else:
                rows[key].append([float(v) for v in vals])
    return dims, {k: np.array(v) for k, v in rows.items()}


def test_worked_example(oracle_lib):
    dims, m = _read_worked(os.path.join(GOLDEN, "worked_2x3x4.txt"))
    A = m["A"].astype(np.float16)
    B = m["B"].astype(np.float16)
    assert A.shape == (dims["M"], dims["K"]) and B.shape == (dims["N"], dims["K"])
    C, S = oracle.gemm_abt(A, B, lib=oracle_lib)
    assert np.array_equal(C, m["C"])
    assert np.array_equal(S, m["S"])


def test_degenerate_shapes(oracle_lib):
    A = np.zeros((3, 0), np.float16)
    B = np.zeros((4, 0), np.float16)
    C, S = oracle.gemm_abt(A, B, lib=oracle_lib)
    assert C.shape == (3, 4) and np.all(C == 0) and np.all(S == 0)
    C, S = oracle.gemm_abt(np.zeros((0, 5), np.float16), np.ones((2, 5), np.float16),
                           lib=oracle_lib)
    assert C.shape == (0, 2)


def test_thread_count_invariance(oracle_lib):
    A = inputs.uniform(97, 300, 81)
    B = inputs.uniform(61, 300, 82)
    C1, S1 = oracle.gemm_abt(A, B, threads=1, lib=oracle_lib)
    C7, S7 = oracle.gemm_abt(A, B, threads=7, lib=oracle_lib)
    assert np.array_equal(C1, C7) and np.array_equal(S1, S7)


def test_tolerance_helper():
    ref = np.array([1.0, 2.0, 0.0])
    S = np.array([10.0, 1.0, 0.0])
    assert oracle.within_tolerance(np.array([1.00005, 2.0, 0.0], np.float32), ref, S).all()
    assert not oracle.within_tolerance(np.array([1.0002, 2.0, 0.0], np.float32), ref, S)[0]
    assert not oracle.within_tolerance(np.array([1.0, 2.0, 1e-30], np.float32), ref, S)[2]
    assert not oracle.within_tolerance(np.array([np.nan, 2.0, 0.0], np.float32), ref, S)[0]


# Planted mistakes: (description, text in oracle.c, replacement).
MUTATIONS = [
    ("dropped last k term", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k < K - 1; ++k)"),
    ("skipped first k term", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 1; k < K; ++k)"),
    ("A used for both operands", "dec[a_row[k]] * dec[b_row[k]]", "dec[a_row[k]] * dec[a_row[k]]"),
    ("B row stride ignored", "j->B + c * j->ldb, j->K", "j->B + c * j->K, j->K"),
    ("output transposed", "&j->C[i * j->ldc + c]", "&j->C[c * j->ldc + i]"),
    ("S without absolute value", "s += fabs(p);", "s += p;"),
    ("sign bit ignored", "return sign ? -mag : mag;", "return mag;"),
    ("exponent bias off by one", "expo - 25", "expo - 24"),
    ("subnormal scale wrong", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("implicit bit missing", "(double)(1024 + frac)", "(double)(frac)"),
    ("Inf read as NaN", "frac == 0 ? INFINITY : NAN", "NAN"),
    ("k loop reads element k+1", "dec[a_row[k]] * dec[b_row[k]]", "dec[a_row[k]] * dec[b_row[k + (k + 1 < K)]]"),
    ("bf16 exponent bias off by one", "expo - 134", "expo - 133"),
    ("bf16 subnormal scale wrong", "ldexp((double)frac, -133)", "ldexp((double)frac, -132)"),
    ("bf16 implicit bit missing", "(double)(128 + frac)", "(double)(frac)"),
    ("bf16 exponent field misplaced", "(h >> 7) & 0xff", "(h >> 8) & 0xff"),
    ("bf16 fraction field narrowed", "h & 0x7f;", "h & 0x3f;"),
    ("bf16 operands decoded as binary16", "return fmt == 1 ? g_bf16_table : g_half_table;",
     "return g_half_table;"),
    ("binary16 operands decoded as bf16", "return fmt == 1 ? g_bf16_table : g_half_table;",
     "return g_bf16_table;"),
    ("bf16 entry point passes the binary16 format", "return gemm_full(1, M, N, K",
     "return gemm_full(0, M, N, K"),
    ("bf16 element entry passes the binary16 format", "return gemm_elems(1, n",
     "return gemm_elems(0, n"),
]


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(desc, old, new, tmp_path):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.load(oracle.compile_library(str(mutated), str(tmp_path / "libmutant.so")))
    failures = []
    for pin in oracle_pins.ALL_PINS:
        if pin in (oracle_pins.pin_half_exhaustive, oracle_pins.pin_bf16_exhaustive) \
                and ("dec[" in old or "gemm_full" in old or "gemm_elems" in old):
            continue  # decode untouched: skip the slow exhaustive pins
        failures += pin(lib)
        if failures:
            break
    assert failures, f"no pin caught: {desc}"
