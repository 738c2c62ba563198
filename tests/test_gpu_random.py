"""Seeded random cases (needs an MI355X).

Each case draws, from one fixed seed, a shape (M, N up to 700, K up to 2200),
row strides and pointer offsets for A, B and C, the operand type (binary16 or
bfloat16) and a forced plan (kernel id, data-parallel / split-K / stream-K /
data-parallel rounds then stream-K, grid). Inputs are integers in {-2..2}, where every partial sum is exact in
fp32, so C must equal the CPU reference bit for bit whatever the summation
order. C sits inside a NaN-filled buffer with padding columns on both sides:
after the call the padding must still be NaN (no store outside C).

About a quarter of the cases use unaligned pointers or strides (or K not a
multiple of 8): the plan rule packs those operands into aligned copies when
the product is large enough, else runs the general kernel; about one case in
ten forces the general kernel.

Two more families run on the default plan with the same strides, offsets and
operand types: 60 shapes up to 1200 x 1200 (checked in full) and 16 large
ones, M and N up to 6000 (checked on sampled rows, columns and points, after
checking that every element of C was written).
"""
import numpy as np
import pytest

import oracle
from dense_fp16_gemm_03_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from dense_fp16_gemm_03_amd import gemm  # noqa: E402

DEV = torch.device("cuda:0")
SEED = 20261202
N_CASES = 200
KIDS_F16 = (16, 18, 27, 28, 35, 36, 37, 38)
KIDS_BF16 = (16, 18, 27, 37, 38)


def draw(i):
    rng = np.random.default_rng([SEED, i])
    M, N, K = int(rng.integers(1, 701)), int(rng.integers(1, 701)), int(rng.integers(1, 2201))
    aligned = rng.random() < 0.75
    if aligned:
        K = max(8, K // 8 * 8)
        pad_a, pad_b = (int(rng.choice([0, 8, 40, 128])) for _ in range(2))
        off_a = off_b = 0
    else:
        pad_a, pad_b = int(rng.integers(0, 9)), int(rng.integers(0, 9))
        off_a, off_b = int(rng.integers(0, 8)), int(rng.integers(0, 8))
    pad_c = int(rng.choice([0, 1, 3, 4, 12]))
    off_c = int(rng.choice([0, 1, 2, 4]))
    dtype = "bf16" if rng.random() < 0.4 else "f16"
    kid = int(rng.choice(KIDS_BF16 if dtype == "bf16" else KIDS_F16))
    plan = f"kid={kid}"
    mode = int(rng.integers(0, 4))
    if mode == 1:
        plan += f",mode=1,splits={int(rng.integers(2, 9))}"
    elif mode in (2, 3):  # stream-K, or whole data-parallel rounds then stream-K
        plan += f",mode={mode}"
    if rng.random() < 0.5:
        plan += f",grid={int(rng.integers(1, 300))}"
    if rng.random() < 0.1:
        plan = "general=1"
    return dict(M=M, N=N, K=K, pad_a=pad_a, pad_b=pad_b, off_a=off_a, off_b=off_b,
                pad_c=pad_c, off_c=off_c, dtype=dtype, plan=plan)


N_DEFAULT_CASES = 60


def draw_default(i):
    """A random shape on the default plan: up to 1200 x 1200 with K up to 8200
    (products of at most 4e9 multiply-adds), so the cases reach every branch
    of the plan rule below a round of 256x256 tiles (direct kernel, 32x32
    tiles, the predicted-time choice among 64x64, 128x128 and 256x256 tiles,
    split or not, packed operands)."""
    rng = np.random.default_rng([SEED, 7, i])
    M, N = int(rng.integers(1, 1201)), int(rng.integers(1, 1201))
    K = int(rng.integers(1, 8201))
    K = max(1, min(K, int(4e9 // (M * N))))
    c = draw(i)
    c.update(M=M, N=N, plan="")
    if c["off_a"] == 0 and c["off_b"] == 0:
        K = max(8, K // 8 * 8)
    c["K"] = K
    return c


N_LARGE_CASES = 16


def draw_large(i):
    """A random large shape on the default plan: M, N in 1100..6000 and K up
    to 8192 (products of at most 1.2e11 multiply-adds), which reaches whole
    rounds of 256x256 tiles, the stream-K share of a last partial round, the
    32- and 64-wide rings and, with unaligned operands, the packed path."""
    rng = np.random.default_rng([SEED, 11, i])
    M, N = int(rng.integers(1100, 6001)), int(rng.integers(1100, 6001))
    K = int(rng.integers(8, 8193))
    K = max(8, min(K, int(1.2e11 // (M * N))))
    c = draw(2000 + i)
    c.update(M=M, N=N, plan="")
    if c["off_a"] == 0 and c["off_b"] == 0:
        K = max(8, K // 8 * 8)
    c["K"] = K
    return c


def operand(bits_or_half, off, pad, dtype):
    """Device view of the operand inside a larger buffer (offset `off`
    elements into each row, `pad` spare elements after it)."""
    rows, cols = bits_or_half.shape
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(bits_or_half).view(np.int16)).view(torch.bfloat16)
        tdt = torch.bfloat16
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits_or_half))
        tdt = torch.float16
    buf = torch.zeros((rows, off + cols + pad), dtype=tdt, device=DEV)
    buf[:, off:off + cols] = t.to(DEV)
    return buf[:, off:off + cols]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i, monkeypatch):
    check_case(i, draw(i))


@pytest.mark.parametrize("i", range(N_DEFAULT_CASES))
def test_random_default_plan(i):
    """Random shapes, strides, offsets and operand types on the default plan."""
    check_case(1000 + i, draw_default(i))


@pytest.mark.parametrize("i", range(N_LARGE_CASES))
def test_random_large_default_plan(i):
    """Random large shapes, strides, offsets and operand types on the default
    plan, checked on sampled rows, columns and points (every element written,
    none outside C)."""
    check_case(3000 + i, draw_large(i), sampled=True)


def sample(M, N, seed):
    rng = np.random.default_rng(seed)
    rows = [0, M - 1, M // 2, int(rng.integers(0, M))]
    cols = [0, N - 1, N // 2, int(rng.integers(0, N))]
    r = [np.full(N, x) for x in rows] + [np.arange(M) for _ in cols] + [rng.integers(0, M, 2000)]
    c = [np.arange(N) for _ in rows] + [np.full(M, x) for x in cols] + [rng.integers(0, N, 2000)]
    return np.concatenate(r), np.concatenate(c)


def check_case(i, c, sampled=False):
    print(f"[gpu test] random case {i}: {c}", flush=True)
    print(f"  plan: {gemm.gemm_f16_f32_abt_describe(c['M'], c['N'], c['K'])}", flush=True)
    gemm.gemm_f16_set_plan_override(c["plan"])
    M, N, K = c["M"], c["N"], c["K"]
    bf16 = c["dtype"] == "bf16"
    if bf16:
        A, B = inputs.integer_bf16(M, K, 1000 + i), inputs.integer_bf16(N, K, 2000 + i)
    else:
        A, B = inputs.integer(M, K, 1000 + i), inputs.integer(N, K, 2000 + i)
    if sampled:
        rows, cols = sample(M, N, i)
        elems = oracle.gemm_abt_elems_bf16 if bf16 else oracle.gemm_abt_elems
        ref, _ = elems(A, B, rows, cols)
    else:
        ref, _ = (oracle.gemm_abt_bf16 if bf16 else oracle.gemm_abt)(A, B)
    Av = operand(A, c["off_a"], c["pad_a"], c["dtype"])
    Bv = operand(B, c["off_b"], c["pad_b"], c["dtype"])
    off_c, pad_c = c["off_c"], c["pad_c"]
    Cbuf = torch.full((M, off_c + N + pad_c), float("nan"), dtype=torch.float32, device=DEV)
    gemm.gemm_abt(Av, Bv, Cbuf[:, off_c:off_c + N])
    torch.cuda.synchronize()
    out = Cbuf.cpu().numpy()
    got = out[:, off_c:off_c + N].astype(np.float64)
    if sampled:
        assert np.isfinite(got).all(), f"case {i}: C not fully written"
        got = got[rows, cols]
    bad = got != ref
    assert not bad.any(), f"case {i}: {bad.sum()} mismatches, first at {np.argwhere(bad)[:3].tolist()}"
    assert np.isnan(out[:, :off_c]).all() and np.isnan(out[:, off_c + N:]).all(), \
        f"case {i}: a store landed outside C"
