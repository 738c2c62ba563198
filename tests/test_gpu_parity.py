"""GPU results against the CPU reference and closed forms (needs an MI355X).

Every call goes through the C ABI (libgemm_f16.so) via the ctypes binding;
torch only allocates device memory and provides streams.

Bars:
  * integer-valued inputs (|C| < 2^24, all partial sums exact in fp32):
    bit-exact against the reference;
  * uniform [-1, 1] inputs: |C_gpu - C_ref| <= 1e-5 * sum_k |a_ik b_jk| per
    element (exact equality where that sum is 0).
Full-size workloads are checked at sampled elements (whole rows and columns
plus random points) against the reference, and in full against closed forms
(A = I gives B^T, all-ones and k-block weights give known sums).
"""
import os

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
_cache = {}


def log(msg):
    print(msg, flush=True)


def operands(shape, kind):
    key = (shape, kind)
    if key not in _cache:
        if len(_cache) > 6:
            _cache.clear()
        _cache[key] = inputs.workload_operands(shape, kind)
    return _cache[key]


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def run(A, B, fill=np.nan, **kw):
    """gemm on the GPU; C pre-filled with `fill` (NaN by default: C must be overwritten)."""
    At = A if isinstance(A, torch.Tensor) else to_dev(A)
    Bt = B if isinstance(B, torch.Tensor) else to_dev(B)
    C = torch.full((At.shape[0], Bt.shape[0]), fill, dtype=torch.float32, device=DEV)
    gemm.gemm_abt(At, Bt, C, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def sample_points(M, N, n_rand=3000, seed=0):
    rng = np.random.default_rng(seed)
    rows = [0, M - 1, M // 2, 257 % M]
    cols = [0, N - 1, N // 2, 129 % N]
    r = [np.full(N, i) for i in rows] + [np.arange(M) for _ in cols]
    c = [np.arange(N) for _ in rows] + [np.full(M, j) for j in cols]
    r.append(rng.integers(0, M, n_rand))
    c.append(rng.integers(0, N, n_rand))
    return np.concatenate(r), np.concatenate(c)


def assert_exact(got, ref, what):
    bad = got.astype(np.float64) != ref
    if bad.any():
        idx = np.argwhere(bad)[:5] if got.ndim == 2 else np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} mismatches, first at {idx.tolist()}")


def assert_tol(got, ref, S, what):
    ok = oracle.within_tolerance(got, ref, S)
    err = np.abs(got.astype(np.float64) - ref) / np.where(S > 0, S, 1)
    log(f"  {what}: max |err|/S = {err.max():.3e}")
    if not ok.all():
        idx = np.argwhere(~ok)[:5] if got.ndim == 2 else np.flatnonzero(~ok)[:5]
        raise AssertionError(f"{what}: {(~ok).sum()} elements outside 1e-5*S, first {idx.tolist()}")


@pytest.fixture(autouse=True)
def _name(request, monkeypatch):
    gemm.gemm_f16_set_plan_override("")
    log(f"[gpu test] {request.node.name}")
    yield


# --- operand lane maps and the epilogue: closed forms -----------------------

@pytest.mark.parametrize("n", [64, 256, 1024])
def test_identity_left_and_right(n):
    X = inputs.uniform(n, n, 31)
    I = inputs.identity(n)
    assert_exact(run(I, X), X.astype(np.float64).T, "A = I -> B^T")
    assert_exact(run(X, I), X.astype(np.float64), "B = I -> A")


def test_perm_pattern():
    n = 512
    P = inputs.perm_pattern(n, n)
    assert_exact(run(inputs.identity(n), P), P.astype(np.float64).T, "A = I, B = perm")


@pytest.mark.parametrize("name", ["8192^3"])
def test_identity_full_size(name):
    M, N, K = WORKLOADS[name]
    B = operands((M, N, K), "uniform")[1]
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    assert_exact(run(inputs.identity(M, K), B), B.astype(np.float64).T, "A = I at 8192^3")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_kblock_weighted_ones(name):
    """A = 1, B[j][k] = 1 + (k//64 mod 7): C = sum of the weights. A missing or
    doubled k-range (a split or stream-K share) changes every element."""
    M, N, K = WORKLOADS[name]
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    w = 1 + (np.arange(K) // 64) % 7
    expect = float(w.sum())
    got = run(inputs.ones(M, K), inputs.kblock_weights(N, K, 64))
    assert np.all(got == expect), f"k-block sum: expected {expect}, got {np.unique(got)[:5]}"


# --- the five workloads against the reference -------------------------------

@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("kind", ["integer", "uniform"])
def test_workload_parity(name, kind):
    M, N, K = WORKLOADS[name]
    A, B = operands((M, N, K), kind)
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    got = run(A, B)
    assert np.isfinite(got).all(), "non-finite output (C not fully written?)"
    if M * N * K <= 1024 ** 3:
        ref, S = oracle.gemm_abt(A, B)
        g = got
    else:
        rows, cols = sample_points(M, N)
        ref, S = oracle.gemm_abt_elems(A, B, rows, cols)
        g = got[rows, cols]
    if kind == "integer":
        assert_exact(g, ref, f"{name} integer")
    else:
        assert_tol(g, ref, S, f"{name} uniform")


@pytest.mark.parametrize("name", list(inputs.PAGE_SHAPES))
def test_page_shape_parity(name):
    """The other shapes of the pages' timing table, integer inputs, bit-exact
    (sampled rows, columns and points where the full reference is too slow)."""
    M, N, K = inputs.PAGE_SHAPES[name]
    A, B = operands((M, N, K), "integer")
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    got = run(A, B)
    if M * N * K <= 2048 ** 3:
        ref, _ = oracle.gemm_abt(A, B)
        assert_exact(got, ref, f"{name} integer")
    else:
        rows, cols = sample_points(M, N, n_rand=2000)
        ref, _ = oracle.gemm_abt_elems(A, B, rows, cols)
        assert_exact(got[rows, cols], ref, f"{name} integer")


@pytest.mark.parametrize("name", list(inputs.SHARD_SHAPES))
def test_shard_shape_parity(name):
    """One GPU's share of each large workload split over 8 GPUs (M/8 of
    8192^3, K/8 of the long-K shapes): integer inputs, bit-exact (sampled
    rows, columns and points above 2048^3)."""
    M, N, K = inputs.SHARD_SHAPES[name]
    A, B = operands((M, N, K), "integer")
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    got = run(A, B)
    if M * N * K <= 2048 ** 3:
        ref, _ = oracle.gemm_abt(A, B)
        assert_exact(got, ref, f"{name} integer")
    else:
        rows, cols = sample_points(M, N, n_rand=2000)
        ref, _ = oracle.gemm_abt_elems(A, B, rows, cols)
        assert_exact(got[rows, cols], ref, f"{name} integer")


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 4096), (512, 512, 8192), (2048, 1024, 8192),
                                   (2048, 2048, 4096), (3072, 3072, 2048), (1000, 1100, 8200)])
def test_default_fewer_tiles_than_cus(M, N, K):
    """Default plans below a full round of 256x256 tiles (chosen by predicted
    time: 64x64, 128x128 or 256x256 tiles, split or not): integers bit-exact
    (sampled above 2048^3 products), uniform within tolerance."""
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    Ai, Bi = inputs.integer(M, K, 171), inputs.integer(N, K, 172)
    got = run(Ai, Bi)
    if M * N * K <= 2048 ** 3:
        ref, _ = oracle.gemm_abt(Ai, Bi)
        assert_exact(got, ref, f"{M}x{N}x{K} integer")
    else:
        rows, cols = sample_points(M, N, n_rand=2000)
        ref, _ = oracle.gemm_abt_elems(Ai, Bi, rows, cols)
        assert_exact(got[rows, cols], ref, f"{M}x{N}x{K} integer")
    A, B = inputs.uniform(M, K, 173), inputs.uniform(N, K, 174)
    rows, cols = sample_points(M, N, n_rand=2000)
    ref, S = oracle.gemm_abt_elems(A, B, rows, cols)
    assert_tol(run(A, B)[rows, cols], ref, S, f"{M}x{N}x{K} uniform")


@pytest.mark.parametrize("M,N,K", [(4608, 4608, 8192), (4352, 4352, 4096)])
def test_default_rounds_then_stream_k(M, N, K):
    """Shapes whose last round of 256x256 tiles is at most half full, with long
    K, run whole data-parallel rounds and then stream-K over the tiles left:
    integer inputs bit-exact on sampled points (rows and columns through
    the shared tiles), and k-block weights, where a missing or doubled
    share changes every element."""
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    log(f"  plan: {text}")
    assert "mode=dp_stream_k" in text
    A, B = operands((M, N, K), "integer")
    got = run(A, B)
    rows, cols = sample_points(M, N, n_rand=2000)
    ref, _ = oracle.gemm_abt_elems(A, B, rows, cols)
    assert_exact(got[rows, cols], ref, f"{M}x{N}x{K} integer")
    w = 1 + (np.arange(K) // 64) % 7
    got = run(inputs.ones(M, K), inputs.kblock_weights(N, K, 64))
    assert np.all(got == float(w.sum())), f"k-block sum: got {np.unique(got)[:5]}"


@pytest.mark.parametrize("M,N,K", [(4100, 4150, 4104), (8200, 8000, 8200), (4100, 4150, 2056),
                                   (6144, 6144, 2048)])
def test_default_large_ragged(M, N, K):
    """Large shapes with ragged M, N and K on the default plan (64-wide stages
    from K = 2048, the tiles past whole rounds shared by stream-K, a partial
    last k-stage): integers bit-exact on sampled rows, columns and points,
    including the last row and column."""
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    log(f"  plan: {text}")
    assert "kid=37" in text
    A, B = inputs.integer(M, K, 171), inputs.integer(N, K, 172)
    got = run(A, B)
    assert np.isfinite(got).all(), "C not fully written"
    rows, cols = sample_points(M, N, n_rand=2000)
    ref, _ = oracle.gemm_abt_elems(A, B, rows, cols)
    assert_exact(got[rows, cols], ref, f"{M}x{N}x{K} integer")


@pytest.mark.parametrize("name", ["2048x2048x16384", "1024x1024x65536"])
def test_long_k_five_slot_ring(name):
    """The long-K workloads on the five-slot ring (kid 37) with the default
    split: integers bit-exact at sampled points, k-block weights everywhere."""
    M, N, K = WORKLOADS[name]
    gemm.gemm_f16_set_plan_override("kid=37")
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    A, B = operands((M, N, K), "integer")
    got = run(A, B)
    rows, cols = sample_points(M, N, n_rand=2000)
    ref, _ = oracle.gemm_abt_elems(A, B, rows, cols)
    assert_exact(got[rows, cols], ref, f"{name} integer, kid 37")
    w = 1 + (np.arange(K) // 64) % 7
    got = run(inputs.ones(M, K), inputs.kblock_weights(N, K, 64))
    assert np.all(got == float(w.sum())), f"k-block sum: got {np.unique(got)[:5]}"


def test_hash_int_inputs():
    """Integers in [-3, 3] from a hash of the index: exact."""
    M, N, K = 1024, 1024, 4096
    A, B = inputs.workload_operands((M, N, K), "hash_int")
    ref, _ = oracle.gemm_abt(A, B)
    assert_exact(run(A, B), ref, "hash_int")


# --- ragged shapes, strides, alignment, degenerate cases --------------------

RAGGED = [
    (1000, 1300, 776),    # several tiles, ragged M, N and K tail (776 % 64 = 8)
    (333, 517, 1096),
    (1, 1, 8),
    (1, 700, 64),
    (700, 1, 64),
    (65, 129, 8),
    (257, 255, 4104),
]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_shapes(M, N, K):
    A = inputs.uniform(M, K, 101)
    B = inputs.uniform(N, K, 102)
    ref, S = oracle.gemm_abt(A, B)
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    assert_tol(run(A, B), ref, S, f"{M}x{N}x{K}")
    Ai = inputs.integer(M, K, 103)
    Bi = inputs.integer(N, K, 104)
    ref, _ = oracle.gemm_abt(Ai, Bi)
    assert_exact(run(Ai, Bi), ref, f"{M}x{N}x{K} integer")


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 200, 136), (1, 1, 8), (17, 33, 1000),
                                   (129, 250, 4104), (512, 512, 2048), (1000, 1300, 1001)])
def test_direct_kernel(M, N, K):
    """The direct kernel (16x16 tiles, no LDS) forced on ragged shapes, odd k
    tails (K % 32 != 0) and, with K % 8 != 0, packed operands: integers
    bit-exact, uniform within tolerance."""
    gemm.gemm_f16_set_plan_override("direct=1")
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    Ai, Bi = inputs.integer(M, K, 161), inputs.integer(N, K, 162)
    ref, _ = oracle.gemm_abt(Ai, Bi)
    assert_exact(run(Ai, Bi), ref, f"direct {M}x{N}x{K} integer")
    A, B = inputs.uniform(M, K, 163), inputs.uniform(N, K, 164)
    ref, S = oracle.gemm_abt(A, B)
    assert_tol(run(A, B), ref, S, f"direct {M}x{N}x{K} uniform")


@pytest.mark.parametrize("M,N,K,force", [(100, 90, 13, False), (64, 64, 7, False),
                                         (5, 3, 1, False), (300, 200, 1001, True)])
def test_general_kernel_odd_k(M, N, K, force, monkeypatch):
    """The general kernel: small products with K % 8 != 0 take it by the plan
    rule; a larger one is forced onto it (it would otherwise be packed)."""
    if force:
        gemm.gemm_f16_set_plan_override("general=1")
    assert "general" in gemm.gemm_f16_f32_abt_describe(M, N, K)
    A = inputs.uniform(M, K, 111)
    B = inputs.uniform(N, K, 112)
    ref, S = oracle.gemm_abt(A, B)
    assert_tol(run(A, B), ref, S, f"general {M}x{N}x{K}")


@pytest.mark.parametrize("plan", ["", "general=1"])
def test_strided_and_unaligned_views(plan, monkeypatch):
    """Views with row strides past K and pointers off 16 bytes: (1, 3) is
    packed into aligned copies by default and run on the general kernel when
    forced."""
    if plan:
        gemm.gemm_f16_set_plan_override(plan)
    M, N, K = 300, 200, 256
    Abig = to_dev(inputs.integer(M, K + 24, 121))
    Bbig = to_dev(inputs.integer(N, K + 40, 122))
    for a0, b0 in ((0, 0), (8, 16), (1, 3)):
        a = Abig[:, a0:a0 + K]
        b = Bbig[:, b0:b0 + K]
        ref, _ = oracle.gemm_abt(a.cpu().numpy(), b.cpu().numpy())
        assert_exact(run(a, b), ref, f"views offset {a0},{b0} {plan}")
    # C with a row stride larger than N
    Cbig = torch.full((M, N + 12), np.nan, dtype=torch.float32, device=DEV)
    c = Cbig[:, 4:4 + N]
    gemm.gemm_abt(Abig[:, :K], Bbig[:, :K], c)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_abt(Abig[:, :K].cpu().numpy(), Bbig[:, :K].cpu().numpy())
    out = Cbig.cpu().numpy()
    assert_exact(out[:, 4:4 + N], ref, "strided C")
    assert np.isnan(out[:, :4]).all() and np.isnan(out[:, 4 + N:]).all(), "wrote outside C"


# Operands the tiled kernels cannot load directly, large enough to be packed
# into aligned, zero-padded copies first: K % 8 != 0 (both operands), and a
# pointer one element past a 16-byte boundary with K % 8 == 0 (that operand).
PACKED = [(300, 200, 1001, 0), (1024, 1024, 1001, 0), (777, 555, 4095, 0),
          (2048, 2048, 4095, 0), (1024, 768, 1024, 1)]


@pytest.mark.parametrize("M,N,K,a_off", PACKED)
def test_packed_operands(M, N, K, a_off):
    if K % 8:
        assert "pack=AB" in gemm.gemm_f16_f32_abt_describe(M, N, K)
    Ai = inputs.integer(M, K + a_off, 141)
    Bi = inputs.integer(N, K, 142)
    a = to_dev(Ai)[:, a_off:a_off + K]
    A = np.ascontiguousarray(Ai[:, a_off:])
    ref, _ = oracle.gemm_abt(A, Bi)
    assert_exact(run(a, to_dev(Bi)), ref, f"packed {M}x{N}x{K} integer")
    Au = inputs.uniform(M, K + a_off, 143)
    Bu = inputs.uniform(N, K, 144)
    A = np.ascontiguousarray(Au[:, a_off:])
    rows, cols = sample_points(M, N, n_rand=2000, seed=5)
    ref, S = oracle.gemm_abt_elems(A, Bu, rows, cols)
    got = run(to_dev(Au)[:, a_off:a_off + K], to_dev(Bu))[rows, cols]
    assert_tol(got, ref, S, f"packed {M}x{N}x{K} uniform (sampled)")


def test_packed_caller_workspace():
    """With K % 8 != 0 the caller workspace size includes the packed copies and
    the _ws call packs; with no workspace it runs the general kernel instead.
    Integer inputs: both paths equal the reference bit for bit."""
    M, N, K = 1024, 1024, 1001
    Ai, Bi = inputs.integer(M, K, 145), inputs.integer(N, K, 146)
    ref, _ = oracle.gemm_abt(Ai, Bi)
    need = gemm.gemm_f16_f32_abt_workspace_size(M, N, K)
    assert need >= 2 * (M + N) * 1008 // 2  # both packed copies (kp = 1008)
    At, Bt = to_dev(Ai), to_dev(Bi)
    ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
    assert_exact(run(At, Bt, workspace=ws), ref, "packed into the caller workspace")
    small = torch.empty((256,), dtype=torch.uint8, device=DEV)
    assert_exact(run(At, Bt, workspace=small), ref, "general kernel (workspace too small)")


def test_k_zero_writes_zeros():
    A = torch.empty((37, 0), dtype=torch.float16, device=DEV)
    B = torch.empty((41, 0), dtype=torch.float16, device=DEV)
    got = run(A, B)
    assert got.shape == (37, 41) and np.all(got == 0)


def test_empty_m_or_n_is_noop():
    for M, N in ((0, 5), (5, 0)):
        C = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
        gemm.gemm_abt(torch.zeros((M, 16), dtype=torch.float16, device=DEV),
                      torch.zeros((N, 16), dtype=torch.float16, device=DEV), C)
    torch.cuda.synchronize()


def test_subnormal_inputs():
    """fp16 subnormals in A (B = 1): IEEE gives the exact sum; a flush to zero
    would still be inside the tolerance. Records which one the MFMA does."""
    M, N, K = 64, 64, 256
    sub = np.arange(1, 1024, dtype=np.uint16)
    A = np.resize(sub, M * K).reshape(M, K).view(np.float16)
    B = inputs.ones(N, K)
    ref, S = oracle.gemm_abt(A, B)
    got = run(A, B)
    exact = np.array_equal(got.astype(np.float64), ref)
    log(f"  subnormal inputs: {'kept (IEEE)' if exact else 'NOT exact'}")
    assert_tol(got, ref, S, "subnormals")


# --- every kernel variant and schedule mode ---------------------------------

# The kernels built: 16 (128x128x64), 18 (64x64x64) and 38 (32x32x64) run
# the symmetric tiled loop; 27 (32-wide three-stage ring) and 28 (its 32x32x16 form, five
# stages) the ping-pong loop; 35 and 36 (its 32x32x16 form) the ping-pong loop
# over two 64-wide stages; 37 the ping-pong loop over 64-wide stages kept as
# separate A and B halves in five slots. Every one under every schedule mode.
KIDS = [16, 18, 27, 28, 35, 36, 37, 38]
PLANS = [f"kid={k}" for k in KIDS] + [
    "kid=16,mode=1,splits=3", "kid=16,mode=2", "kid=16,mode=2,grid=37",
    "kid=16,mode=1,splits=3,grid=40", "kid=18,mode=1,splits=5", "kid=18,mode=2,grid=130",
    "kid=38,mode=1,splits=3", "kid=38,mode=2,grid=37", "kid=38,mode=3,grid=9", "kid=38,grid=5",
    "kid=27,mode=1,splits=4", "kid=27,mode=2", "kid=27,mode=2,grid=29",
    "kid=28,mode=1,splits=2,grid=40", "kid=28,mode=2,grid=37",
    "kid=36,mode=1,splits=3", "kid=36,mode=2,grid=29",
    # Several units per workgroup: the ping-pong kernels start the next unit's
    # loads before the previous unit's stores, mixing full tiles (vector
    # stores left in flight) with ragged ones (element stores).
    "kid=27,grid=3", "kid=27,grid=1", "kid=27,mode=1,splits=2,grid=7", "kid=28,grid=4",
    "kid=35,grid=1", "kid=35,grid=3", "kid=35,mode=1,splits=2,grid=7", "kid=35,mode=1,splits=3",
    "kid=35,mode=2", "kid=35,mode=2,grid=37", "kid=36,grid=1", "kid=36,grid=3",
    "kid=36,mode=1,splits=2,grid=7", "kid=37,grid=1", "kid=37,grid=3", "kid=37,mode=1,splits=3",
    "kid=37,mode=1,splits=2,grid=7", "kid=37,mode=2", "kid=37,mode=2,grid=37",
    # Whole data-parallel rounds, then stream-K over the tiles left (the
    # forced grids make whole rounds at this size).
    "kid=27,mode=3,grid=4", "kid=16,mode=3,grid=7", "kid=18,mode=3,grid=50",
    "kid=28,mode=3,grid=5", "kid=35,mode=3,grid=4", "kid=36,mode=3,grid=4",
    "kid=37,mode=3,grid=4",
]


@pytest.mark.parametrize("plan", PLANS)
def test_forced_plans(plan, monkeypatch):
    gemm.gemm_f16_set_plan_override(plan)
    M, N, K = 600, 520, 1352
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    Ai = inputs.integer(M, K, 131)
    Bi = inputs.integer(N, K, 132)
    ref, _ = oracle.gemm_abt(Ai, Bi)
    assert_exact(run(Ai, Bi), ref, f"{plan} integer")
    A = inputs.uniform(M, K, 133)
    B = inputs.uniform(N, K, 134)
    ref, S = oracle.gemm_abt(A, B)
    assert_tol(run(A, B), ref, S, f"{plan} uniform")


@pytest.mark.parametrize("kid", KIDS)
@pytest.mark.parametrize("K", [24, 72, 200])
def test_forced_plans_short_k(kid, K, monkeypatch):
    """K of one to a few k-tiles, odd and even counts (one k-step per stage
    runs its stages in pairs plus a tail)."""
    gemm.gemm_f16_set_plan_override(f"kid={kid}")
    M, N = 300, 264
    Ai, Bi = inputs.integer(M, K, 151), inputs.integer(N, K, 152)
    ref, _ = oracle.gemm_abt(Ai, Bi)
    assert_exact(run(Ai, Bi), ref, f"kid={kid} K={K} integer")
    A, B = inputs.uniform(M, K, 153), inputs.uniform(N, K, 154)
    ref, S = oracle.gemm_abt(A, B)
    assert_tol(run(A, B), ref, S, f"kid={kid} K={K} uniform")


@pytest.mark.parametrize("plan", ["kid=28,grid=1", "kid=28,grid=2", "kid=27,grid=1",
                                  "kid=27,mode=1,splits=2,grid=3", "kid=35,grid=1",
                                  "kid=35,grid=2", "kid=35,mode=1,splits=2,grid=3",
                                  "kid=36,grid=2", "kid=37,grid=1",
                                  "kid=37,mode=1,splits=2,grid=3"])
@pytest.mark.parametrize("K", [24, 72, 200])
def test_forced_plans_short_units(plan, K, monkeypatch):
    """Many short units per workgroup: units of one to a few k-tiles follow
    each other while the previous unit's stores may still be in flight."""
    gemm.gemm_f16_set_plan_override(plan)
    M, N = 776, 520
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    Ai, Bi = inputs.integer(M, K, 155), inputs.integer(N, K, 156)
    ref, _ = oracle.gemm_abt(Ai, Bi)
    assert_exact(run(Ai, Bi), ref, f"{plan} K={K} integer")
    A, B = inputs.uniform(M, K, 157), inputs.uniform(N, K, 158)
    ref, S = oracle.gemm_abt(A, B)
    assert_tol(run(A, B), ref, S, f"{plan} K={K} uniform")


# --- invariants -------------------------------------------------------------

def test_transpose_invariant():
    M, N, K = 768, 512, 2048
    Ai, Bi = inputs.integer(M, K, 141), inputs.integer(N, K, 142)
    assert_exact(run(Bi, Ai), run(Ai, Bi).T.astype(np.float64), "integer transpose")
    A, B = inputs.uniform(M, K, 143), inputs.uniform(N, K, 144)
    ref, S = oracle.gemm_abt(A, B)
    assert_tol(run(B, A).T, ref, S, "uniform transpose")


@pytest.mark.parametrize("name", ["2048x2048x16384", "1024x1024x65536", "4352x4352x4096"])
def test_repeat_and_caller_workspace(name):
    """Split-K / stream-K results are bitwise repeatable (partials are summed in
    k order), also on uniform inputs, and a caller workspace holding garbage
    gives the same C. 4352^2 x 4096 runs whole data-parallel rounds and then
    stream-K over the 33 tiles left, whose partials alone use the workspace."""
    M, N, K = WORKLOADS[name] if name in WORKLOADS else tuple(map(int, name.split("x")))
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    A, B = operands((M, N, K), "uniform")
    At, Bt = to_dev(A), to_dev(B)
    first = run(At, Bt)
    rows, cols = sample_points(M, N, n_rand=2000)
    ref, S = oracle.gemm_abt_elems(A, B, rows, cols)
    assert_tol(first[rows, cols], ref, S, f"{name} uniform")
    second = run(At, Bt, fill=-7.0)
    assert np.array_equal(first, second)
    nbytes = gemm.gemm_f16_f32_abt_workspace_size(M, N, K)
    assert nbytes > 0
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    for _ in range(2):
        assert np.array_equal(first, run(At, Bt, workspace=ws))


def test_repeat_full_size_default_plan():
    """8192^3 on its default plan (several units per workgroup, each unit's C
    stores left in flight while the next unit's loads start): two calls on
    uniform inputs and two on hash-integer inputs give the same C bit for bit
    over all 67 million elements, and each input kind matches the reference
    at sampled rows, columns and points (exactly on the integers)."""
    M, N, K = WORKLOADS["8192^3"]
    log(f"  plan: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    rows, cols = sample_points(M, N, n_rand=2000, seed=11)
    for kind in ("uniform", "hash_int"):
        A, B = operands((M, N, K), kind)
        At, Bt = to_dev(A), to_dev(B)
        first = run(At, Bt)
        second = run(At, Bt, fill=-7.0)
        same = first == second
        assert same.all(), f"{kind}: {(~same).sum()} elements differ between two calls"
        ref, S = oracle.gemm_abt_elems(A, B, rows, cols)
        if kind == "hash_int":
            assert_exact(first[rows, cols], ref, "8192^3 hash_int")
        else:
            assert_tol(first[rows, cols], ref, S, "8192^3 uniform")
        del At, Bt, first, second
        torch.cuda.empty_cache()


def test_capture_needs_a_caller_workspace():
    """A split plan called while its stream is being captured, without a
    caller workspace, is refused (GEMM_ERR_WORKSPACE) before anything is
    enqueued: the graph would otherwise keep the address of a library-owned
    workspace a later call may free. A data-parallel plan captures as is."""
    M, N, K = 512, 512, 8192  # split-K plan
    assert "mode=split" in gemm.gemm_f16_f32_abt_describe(M, N, K)
    A, B = operands((M, N, K), "integer")
    At, Bt = to_dev(A), to_dev(B)
    C = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(gemm.GemmError) as e:
        with torch.cuda.graph(g, stream=s):
            gemm.gemm_abt(At, Bt, C)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert torch.isnan(C).all()  # nothing ran
    ref, _ = oracle.gemm_abt(A, B)
    assert_exact(run(At, Bt), ref, "split plan after the refused capture")


@pytest.mark.parametrize("name", ["8192^3", "1024x1024x65536", "1024^3"])
def test_clock_probe(name):
    """The clock probe: with it on, C is bitwise the same; the counters hold
    shader cycles and 100 MHz ticks whose ratio is a plausible clock, and
    whose ticks agree with the event-timed duration of the probed kernels;
    with it off, the counters no longer move."""
    M, N, K = WORKLOADS[name]
    A, B = operands((M, N, K), "integer")
    At, Bt = to_dev(A), to_dev(B)
    plain = run(At, Bt)
    ctr = torch.zeros(2, dtype=torch.int64, device=DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    calls = 5
    torch.cuda.synchronize()
    gemm.gemm_f16_set_clock_probe(ctr.data_ptr())
    try:
        s.record()
        for _ in range(calls):
            gemm.gemm_abt(At, Bt, C)
        e.record()
        torch.cuda.synchronize()
    finally:
        gemm.gemm_f16_set_clock_probe(0)
    assert np.array_equal(C.cpu().numpy(), plain)
    cycles, ticks = (int(v) for v in ctr.tolist())
    mhz = 100.0 * cycles / max(ticks, 1)
    probed_us = ticks / 100.0
    event_us = s.elapsed_time(e) * 1e3
    log(f"  {name}: {mhz:.0f} MHz; probed {probed_us:.1f} us vs {event_us:.1f} us between events")
    assert ticks > 0 and 200 <= mhz <= 2600
    # workgroup 0 spans its main kernel; the events also hold the reduce pass
    # and the gaps between calls (most of the time for the small shape)
    assert 0.25 * event_us <= probed_us <= 1.05 * event_us
    gemm.gemm_abt(At, Bt, C)
    torch.cuda.synchronize()
    assert [int(v) for v in ctr.tolist()] == [cycles, ticks]


def test_non_default_stream():
    M, N, K = WORKLOADS["1024x1024x65536"]
    A, B = operands((M, N, K), "integer")
    At, Bt = to_dev(A), to_dev(B)
    ref = run(At, Bt)
    s = torch.cuda.Stream()
    C = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        gemm.gemm_abt(At, Bt, C)
    s.synchronize()
    assert np.array_equal(C.cpu().numpy(), ref)


def test_workspace_must_be_on_the_gpu():
    M, N, K = WORKLOADS["2048x2048x16384"]
    A = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    B = torch.zeros((N, K), dtype=torch.float16, device=DEV)
    C = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
    need = gemm.gemm_f16_f32_abt_workspace_size(M, N, K)
    for ws in (torch.empty(need, dtype=torch.uint8),  # host memory
               torch.empty(2 * need, dtype=torch.uint8, device=DEV)[::2]):  # strided
        with pytest.raises(ValueError, match="workspace"):
            gemm.gemm_abt(A, B, C, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(C).all()  # rejected before any launch


def test_threads_share_a_stream():
    """Two host threads call the library at once on the same (null) stream,
    each with a split plan of a different workspace size, starting from no
    workspace: one grows the stream's workspace while the other uses it.
    Every result equals the single-threaded one bit for bit."""
    import threading

    shapes = [(512, 512, 8192), (256, 256, 65536)]  # splits 4 and 32
    ops, refs = [], []
    for i, (M, N, K) in enumerate(shapes):
        A, B = inputs.uniform(M, K, 61 + i), inputs.uniform(N, K, 71 + i)
        ref, S = oracle.gemm_abt(A, B)
        At, Bt = to_dev(A), to_dev(B)
        single = run(At, Bt)
        assert_tol(single, ref, S, f"{M}x{N}x{K} single-threaded")
        ops.append((At, Bt))
        refs.append(single)
    torch.cuda.synchronize()
    gemm.gemm_f16_release_workspaces()
    outs = [[torch.full((M, N), np.nan, dtype=torch.float32, device=DEV) for _ in range(8)]
            for (M, N, K) in shapes]
    errors = []

    def worker(i):
        try:
            for C in outs[i]:
                gemm.gemm_abt(*ops[i], C)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, Cs in enumerate(outs):
        for C in Cs:
            assert np.array_equal(C.cpu().numpy(), refs[i]), f"shape {shapes[i]}"


def test_threads_on_separate_streams():
    """Two host threads, each on its own stream, run split plans at the same
    time (the library then keeps one workspace per stream, and the two
    streams' kernels may share the GPU). Every result equals the
    single-stream one bit for bit."""
    import threading

    shapes = [(1024, 1024, 16384), (512, 768, 8192)]
    ops, refs = [], []
    for i, (M, N, K) in enumerate(shapes):
        text = gemm.gemm_f16_f32_abt_describe(M, N, K)
        log(f"  plan: {text}")
        assert "mode=split" in text
        A, B = inputs.uniform(M, K, 81 + i), inputs.uniform(N, K, 91 + i)
        At, Bt = to_dev(A), to_dev(B)
        ops.append((At, Bt))
        refs.append(run(At, Bt))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in shapes]
    outs = [[torch.full((M, N), np.nan, dtype=torch.float32, device=DEV) for _ in range(8)]
            for (M, N, K) in shapes]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for C in outs[i]:
                    gemm.gemm_abt(*ops[i], C)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, Cs in enumerate(outs):
        for C in Cs:
            assert np.array_equal(C.cpu().numpy(), refs[i]), f"shape {shapes[i]}"


@pytest.mark.parametrize("name", ["1024^3", "4096x4096x1024", "2048x2048x16384",
                                  "1024x1024x1001"])
def test_graph_replay(name):
    """A call captured in a HIP graph (torch.cuda.CUDAGraph) replays to the eager
    result, bitwise, on every replay, with eager work between replays. Split
    plans and packed operands (K % 8 != 0) use a caller workspace, allocated
    before capture."""
    M, N, K = (WORKLOADS.get(name) or inputs.PAGE_SHAPES.get(name)
               or tuple(int(v) for v in name.split("x")))
    A, B = operands((M, N, K), "uniform")
    At, Bt = to_dev(A), to_dev(B)
    eager = run(At, Bt)
    nbytes = gemm.gemm_f16_f32_abt_workspace_size(M, N, K)
    ws = (torch.empty((max(nbytes, 256) // 4,), dtype=torch.float32, device=DEV)
          if nbytes else None)
    C = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gemm.gemm_abt(At, Bt, C, workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        gemm.gemm_abt(At, Bt, C, workspace=ws)
    for r in range(3):
        C.fill_(float("nan"))
        if ws is not None:
            ws.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), eager), f"replay {r} differs"
        run(At, Bt)  # eager work between replays
