"""bfloat16 inputs on the GPU against the CPU reference (needs an MI355X).

The same bars as the binary16 path: bit-exact on integer-valued inputs (every
partial sum exact in fp32), |C_gpu - C_ref| <= 1e-5 * sum_k |a_ik b_jk| on
uniform [-1, 1] inputs. Operands are bfloat16 bit patterns from
dense_fp16_gemm_03_amd.inputs (uint16 arrays), read by the reference's
bfloat16 entry points and, as torch.bfloat16 tensors, by gemm_bf16_f32_abt
through the C ABI.
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
WORKLOADS = inputs.WORKLOADS


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _name(request, monkeypatch):
    gemm.gemm_f16_set_plan_override("")
    log(f"[gpu test] {request.node.name}")
    yield


def values(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def run(A, B, fill=np.nan, **kw):
    At = A if isinstance(A, torch.Tensor) else to_dev(A)
    Bt = B if isinstance(B, torch.Tensor) else to_dev(B)
    C = torch.full((At.shape[0], Bt.shape[0]), fill, dtype=torch.float32, device=DEV)
    gemm.gemm_abt(At, Bt, C, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def sample_points(M, N, n_rand=2000, seed=0):
    rng = np.random.default_rng(seed)
    rows = [0, M - 1, M // 2, 257 % M]
    cols = [0, N - 1, N // 2, 259 % N]
    # whole rows `rows`, whole columns `cols`, then random points
    r = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols)),
                        rng.integers(0, M, n_rand)])
    c = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M),
                        rng.integers(0, N, n_rand)])
    return r, c


def assert_exact(got, ref, what):
    bad = got.astype(np.float64) != ref
    if bad.any():
        raise AssertionError(f"{what}: {bad.sum()} mismatches, first at "
                             f"{np.argwhere(bad)[:5].tolist()}")


def assert_tol(got, ref, S, what):
    ok = oracle.within_tolerance(got, ref, S)
    err = np.abs(got.astype(np.float64) - ref) / np.where(S > 0, S, 1)
    log(f"  {what}: max |err|/S = {err.max():.3e}")
    if not ok.all():
        raise AssertionError(f"{what}: {(~ok).sum()} elements outside 1e-5*S")


def check(A, B, got, kind, what, sampled=False):
    if sampled:
        rows, cols = sample_points(A.shape[0], B.shape[0])
        ref, S = oracle.gemm_abt_elems_bf16(A, B, rows, cols)
        got = got[rows, cols]
    else:
        ref, S = oracle.gemm_abt_bf16(A, B)
    if kind == "integer":
        assert_exact(got, ref, what)
    else:
        assert_tol(got, ref, S, what)


@pytest.mark.parametrize("n", [64, 256])
def test_identity_left_and_right(n):
    X = inputs.uniform_bf16(n, n, 31)
    I = inputs.to_bf16_bits(np.eye(n))
    assert_exact(run(I, X), values(X).T, "A = I -> B^T")
    assert_exact(run(X, I), values(X), "B = I -> A")


def test_perm_pattern():
    n = 512
    P = inputs.perm_pattern_bf16(n, n)
    assert_exact(run(inputs.to_bf16_bits(np.eye(n)), P), values(P).T, "A = I, B = perm")


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("kind", ["integer", "uniform"])
def test_workload_parity(name, kind):
    M, N, K = WORKLOADS[name]
    A, B = inputs.workload_operands((M, N, K), kind, "bf16")
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    got = run(A, B)
    assert np.isfinite(got).all(), "non-finite output (C not fully written?)"
    check(A, B, got, kind, f"{name} bf16 {kind}", sampled=M * N * K > 1024 ** 3)


@pytest.mark.parametrize("name", ["2048x2048x16384", "1024x1024x65536"])
def test_kblock_weighted_ones(name):
    """Split-K coverage: a missing or doubled k-range changes every element."""
    M, N, K = WORKLOADS[name]
    w = 1 + (np.arange(K) // 64) % 7
    B = np.broadcast_to(inputs.to_bf16_bits(w), (N, K)).copy()
    got = run(inputs.to_bf16_bits(np.ones((M, K))), B)
    assert np.all(got == float(w.sum()))


@pytest.mark.parametrize("M,N,K", [(4352, 4352, 4096), (4100, 4150, 4104)])
def test_default_rounds_then_stream_k(M, N, K):
    """bfloat16 on the default plans that share the tiles left after whole
    data-parallel rounds (64-wide stages; the second shape ragged in M, N
    and K): integers bit-exact, uniform within tolerance, on sampled points."""
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    log(f"  plan: {text}")
    assert "mode=dp_stream_k" in text and "kid=37" in text
    A, B = inputs.integer_bf16(M, K, 191), inputs.integer_bf16(N, K, 192)
    check(A, B, run(A, B), "integer", f"{M}x{N}x{K} bf16 integer", sampled=True)
    A, B = inputs.uniform_bf16(M, K, 193), inputs.uniform_bf16(N, K, 194)
    check(A, B, run(A, B), "uniform", f"{M}x{N}x{K} bf16 uniform", sampled=True)


@pytest.mark.parametrize("M,N,K", [(600, 520, 1352), (1, 1, 8), (129, 77, 200),
                                   (300, 264, 24), (1000, 1000, 1000)])
def test_ragged_shapes(M, N, K):
    A, B = inputs.integer_bf16(M, K, 161), inputs.integer_bf16(N, K, 162)
    check(A, B, run(A, B), "integer", f"{M}x{N}x{K} integer")
    A, B = inputs.uniform_bf16(M, K, 163), inputs.uniform_bf16(N, K, 164)
    check(A, B, run(A, B), "uniform", f"{M}x{N}x{K} uniform")


def test_general_kernel_odd_k_and_unaligned_views():
    A, B = inputs.integer_bf16(130, 37, 171), inputs.integer_bf16(70, 37, 172)
    check(A, B, run(A, B), "integer", "odd K")
    big_a, big_b = inputs.uniform_bf16(90, 301, 173), inputs.uniform_bf16(50, 301, 174)
    At, Bt = to_dev(big_a)[:, 1:261], to_dev(big_b)[:, 3:263]  # misaligned, strided
    check(np.ascontiguousarray(big_a[:, 1:261]), np.ascontiguousarray(big_b[:, 3:263]),
          run(At, Bt), "uniform", "unaligned strided views")


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1001), (600, 520, 1355)])
def test_packed_operands(M, N, K):
    """K % 8 != 0 on a product large enough to pack both operands into
    aligned, zero-padded copies before the tiled kernel."""
    assert "pack=AB" in gemm.gemm_f16_f32_abt_describe(M, N, K)
    A, B = inputs.integer_bf16(M, K, 175), inputs.integer_bf16(N, K, 176)
    check(A, B, run(A, B), "integer", f"packed {M}x{N}x{K} integer")
    A, B = inputs.uniform_bf16(M, K, 177), inputs.uniform_bf16(N, K, 178)
    check(A, B, run(A, B), "uniform", f"packed {M}x{N}x{K} uniform")
    # K % 8 == 0 with A one element off a 16-byte boundary: A alone is packed
    big_a = inputs.integer_bf16(M, 1025, 179)
    B = inputs.integer_bf16(N, 1024, 180)
    check(np.ascontiguousarray(big_a[:, 1:]), B, run(to_dev(big_a)[:, 1:], to_dev(B)),
          "integer", "packed misaligned A")


def test_k_zero_writes_zeros():
    A = torch.empty((40, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((30, 0), dtype=torch.bfloat16, device=DEV)
    assert np.all(run(A, B) == 0)


PLANS = ["kid=16", "kid=18", "kid=27", "kid=27,grid=3", "kid=27,grid=2",
         "kid=27,mode=1,splits=3", "kid=27,mode=2,grid=37", "kid=16,mode=1,splits=2",
         "kid=18,mode=2,grid=29", "kid=37", "kid=37,grid=3", "kid=37,mode=1,splits=3",
         "kid=37,mode=3,grid=4", "kid=37,grid=1", "kid=38", "kid=38,mode=2,grid=29",
         # kernel ids not built for bfloat16 (the comparison kernels, and an
         # id no kernel has): the plan keeps the shape rule's kernel
         "kid=35", "kid=36", "kid=0"]


@pytest.mark.parametrize("plan", PLANS)
def test_forced_plans(plan, monkeypatch):
    gemm.gemm_f16_set_plan_override(plan)
    M, N, K = 600, 520, 1352
    A, B = inputs.integer_bf16(M, K, 181), inputs.integer_bf16(N, K, 182)
    check(A, B, run(A, B), "integer", f"{plan} integer")
    A, B = inputs.uniform_bf16(M, K, 183), inputs.uniform_bf16(N, K, 184)
    check(A, B, run(A, B), "uniform", f"{plan} uniform")


def test_caller_workspace_and_repeat():
    M, N, K = WORKLOADS["2048x2048x16384"]
    A, B = inputs.workload_operands((M, N, K), "uniform", "bf16")
    At, Bt = to_dev(A), to_dev(B)
    first = run(At, Bt)
    nbytes = gemm.gemm_bf16_f32_abt_workspace_size(M, N, K)
    assert nbytes == gemm.gemm_f16_f32_abt_workspace_size(M, N, K) > 0
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    assert np.array_equal(first, run(At, Bt, workspace=ws))
    assert np.array_equal(first, run(At, Bt, fill=-7.0))
