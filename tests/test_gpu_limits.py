"""The largest sizes (needs an MI355X).

* C and A beyond 2 GiB and 4 GiB (64-bit row offsets in every kernel's
  loads and stores), on the default plan, two forced tiled kernels, a
  misaligned B packed into aligned rows, and the general kernel;
* 65792 output tiles, 257 per workgroup of the persistent grid, with a 17 GB C;
* K = 2^20 on one tile: 256 k-shares, the most the split rule makes;
* row strides on both sides of the 2^31-byte buffer-offset limit of the
  tiled kernels (padding columns hold NaN, so a read past K shows);
* M at the library's 32-bit index limit (2^31 - 1025), on the tiled path
  (B direct or packed) and on the general kernel, whose grid then walks 33.5
  million tiles by stride.

Operands of gigabytes are drawn on the GPU (inputs.device_uniform) and the
rows a check needs are copied back for the CPU reference. Every C starts as
NaN; each test checks that all of it was written, and compares sampled rows
(and columns) with the reference within 1e-5 * sum |a b|.
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
MAX_DIM = (1 << 31) - 1025


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _each(request, monkeypatch):
    gemm.gemm_f16_set_plan_override("")
    log(f"[gpu test] {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def plan_text(M, N, K, path):
    if path == "general":
        return "general kernel (forced; B not 16-byte aligned)"
    if path == "packed":  # describe() sees no pointers: B is packed, then this plan
        return "B packed into aligned rows, then " + gemm.gemm_f16_f32_abt_describe(M, N, K)
    return gemm.gemm_f16_f32_abt_describe(M, N, K)


def misaligned(B_host):
    """B on the GPU one element past a 16-byte boundary (row stride K + 8)."""
    N, K = B_host.shape
    buf = torch.zeros((N, K + 8), dtype=torch.float16, device=DEV)
    buf[:, 1:K + 1] = torch.from_numpy(B_host).to(DEV)
    return buf[:, 1:K + 1]


def nan_c(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)


def assert_all_written(C, what):
    step = max(1, (1 << 28) // max(C.shape[1], 1))
    for r0 in range(0, C.shape[0], step):
        if torch.isnan(C[r0:r0 + step]).any().item():
            bad = torch.isnan(C[r0:r0 + step]).nonzero()[0].tolist()
            raise AssertionError(f"{what}: C not written at row {r0 + bad[0]}, col {bad[1]}")


def assert_rows(C, A, B_host, rows, what):
    """C[rows, :] against the reference; A may live on the device."""
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=A.device)
    A_rows = A.index_select(0, idx).cpu().numpy()
    got = C.index_select(0, idx.to(C.device)).cpu().numpy()
    ref, S = oracle.gemm_abt(A_rows, B_host)
    ok = oracle.within_tolerance(got, ref, S)
    err = (np.abs(got.astype(np.float64) - ref) / np.where(S > 0, S, 1)).max()
    log(f"  {what}: {len(rows)} rows, max |err|/S = {err:.3e}")
    if not ok.all():
        r, c = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {(~ok).sum()} elements outside 1e-5*S, "
                             f"first at row {rows[r]}, col {c}")


def boundary_rows(M, row_bytes):
    """Rows on either side of every 2^31 * 2^j byte offset inside M rows."""
    out = set()
    b = 1 << 31
    while b // row_bytes < M:
        r = b // row_bytes
        out.update(x for x in (r - 1, r, r + 1) if 0 <= x < M)
        b <<= 1
    return out


def sample_rows(M, extra, n_rand, seed):
    rng = np.random.default_rng(seed)
    rows = {0, 1, M // 2, M - 2, M - 1} | set(extra)
    rows |= set(rng.integers(0, M, n_rand).tolist())
    return sorted(r for r in rows if 0 <= r < M)


@pytest.mark.parametrize("plan", ["default", "kid=16", "kid=18", "packed", "general"])
def test_tall_c_beyond_2gib(plan, monkeypatch):
    M, N, K = (1 << 21) + 37, 264, 1032  # A 4.3 GB, C 2.2 GB; N and M ragged
    A = inputs.device_uniform(M, K, 501, DEV)
    B_host = inputs.uniform(N, K, 502)
    if plan in ("packed", "general"):
        B = misaligned(B_host)  # packed into aligned rows, or the general kernel
        if plan == "general":
            gemm.gemm_f16_set_plan_override("general=1")
    else:
        B = torch.from_numpy(B_host).to(DEV)
        if plan != "default":
            gemm.gemm_f16_set_plan_override(plan)
    log(f"  plan: {plan_text(M, N, K, plan)} ({plan})")
    C = nan_c(M, N)
    gemm.gemm_abt(A, B, C)
    torch.cuda.synchronize()
    assert_all_written(C, plan)
    extra = boundary_rows(M, K * 2) | boundary_rows(M, N * 4)
    assert_rows(C, A, B_host, sample_rows(M, extra, 40, 503), plan)


def test_most_tiles_per_workgroup():
    M, N, K = 65536 + 17, 65536 - 5, 40  # 257 x 256 tiles of 256 x 256, C 17.2 GB
    plan = gemm.gemm_f16_f32_abt_describe(M, N, K)
    log(f"  plan: {plan}")
    assert "tiles=65792" in plan and "grid=256" in plan
    A_host = inputs.uniform(M, K, 511)
    B_host = inputs.uniform(N, K, 512)
    A = torch.from_numpy(A_host).to(DEV)
    C = nan_c(M, N)
    gemm.gemm_abt(A, torch.from_numpy(B_host).to(DEV), C)
    torch.cuda.synchronize()
    assert_all_written(C, "65792 tiles")
    assert_rows(C, A, B_host, sample_rows(M, {255, 256, 32768}, 4, 513), "rows")
    cols = [0, 255, 256, N // 2, N - 1]
    got = C[:, cols].cpu().numpy()
    ref, S = oracle.gemm_abt(A_host, np.ascontiguousarray(B_host[cols]))
    assert oracle.within_tolerance(got, ref, S).all(), "sampled columns"


def test_most_k_shares():
    M, N, K = 256, 256, 1 << 20
    plan = gemm.gemm_f16_f32_abt_describe(M, N, K)
    log(f"  plan: {plan}")
    assert "mode=split splits=256" in plan
    A = inputs.device_uniform(M, K, 521, DEV)
    B = inputs.device_uniform(N, K, 522, DEV)
    C = nan_c(M, N)
    gemm.gemm_abt(A, B, C)
    torch.cuda.synchronize()
    assert_all_written(C, "K = 2^20")
    A_host, B_host = A.cpu().numpy(), B.cpu().numpy()
    rng = np.random.default_rng(523)
    # rows 0, 128 and 255 whole, columns 0 and N - 1 whole, 256 random elements
    rows = np.concatenate([np.repeat([0, 128, 255], N), np.arange(M), np.arange(M),
                           rng.integers(0, M, 256)])
    cols = np.concatenate([np.tile(np.arange(N), 3), np.zeros(M, np.int64),
                           np.full(M, N - 1), rng.integers(0, N, 256)])
    ref, S = oracle.gemm_abt_elems(A_host, B_host, rows, cols)
    got = C.cpu().numpy()[rows, cols]
    ok = oracle.within_tolerance(got, ref, S)
    err = (np.abs(got.astype(np.float64) - ref) / np.where(S > 0, S, 1)).max()
    log(f"  {len(rows)} elements, max |err|/S = {err:.3e}")
    assert ok.all(), f"{(~ok).sum()} elements outside 1e-5*S"


def test_row_stride_at_offset_limit(monkeypatch):
    # The tiled kernels address a 256-row operand tile with 32-bit byte
    # offsets: (256 - 1) * ld * 2 + (K + 32) * 2 must stay below 2^31. One
    # stride step further the operands are packed into rows of K elements
    # (or, forced, run on the general kernel).
    M, N, K = 256, 256, 4096
    ld_in = ((2**31 - 1 - (K + 32) * 2) // (255 * 2)) // 8 * 8
    for ld, expect in ((ld_in, "tiled"), (ld_in + 8, "packed"), (ld_in + 8, "general")):
        if expect == "general":
            gemm.gemm_f16_set_plan_override("general=1")
        A = inputs.device_uniform(M, K, 531, DEV, ld=ld)
        B = inputs.device_uniform(N, K, 532, DEV, ld=ld)
        log(f"  ld={ld} ({expect}; A and B {2 * M * ld / 2**30:.2f} GiB each)")
        C = nan_c(M, N)
        gemm.gemm_abt(A, B, C)
        torch.cuda.synchronize()
        assert_all_written(C, f"ld={ld}")
        A_host = A.contiguous().cpu().numpy()
        B_host = B.contiguous().cpu().numpy()
        ref, S = oracle.gemm_abt(A_host, B_host)
        ok = oracle.within_tolerance(C.cpu().numpy(), ref, S)
        assert ok.all(), f"ld={ld}: {(~ok).sum()} elements outside 1e-5*S"
        del A, B, C
        torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["tiled", "packed", "general"])
def test_m_at_index_limit(path, monkeypatch):
    M, N, K = MAX_DIM, 1, 8  # A 34.4 GB, C 8.6 GB
    A = inputs.device_uniform(M, K, 541, DEV)
    B_host = inputs.uniform(N, K, 542)
    if path in ("packed", "general"):
        B = misaligned(B_host)
        if path == "general":
            gemm.gemm_f16_set_plan_override("general=1")
    else:
        B = torch.from_numpy(B_host).to(DEV)
    log(f"  plan: {plan_text(M, N, K, path)} ({path})")
    C = nan_c(M, N)
    gemm.gemm_abt(A, B, C)
    torch.cuda.synchronize()
    assert_all_written(C, path)
    extra = boundary_rows(M, K * 2) | boundary_rows(M, N * 4)
    assert_rows(C, A, B_host, sample_rows(M, extra, 200, 543), path)
