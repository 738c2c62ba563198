"""gemm_f16_f32_abt_noalloc, the entry point that allocates nothing, against
the allocating entry point it mirrors (needs an MI355X).

Two calls in a row through the C ABI, the second with a smaller input, each
compared bit for bit with gemm_f16_f32_abt on the same operands (both use the
same kernels and the same summation order, so any difference is a workspace
fault), on integer inputs (also exact against the CPU reference at sampled
points) and on uniform inputs; then a plan whose partial tiles exceed the
static scratch is refused with GEMM_ERR_SCRATCH before anything runs.
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


def noalloc(A, B, C):
    M, K = A.shape
    N = B.shape[0]
    stream = torch.cuda.current_stream().cuda_stream
    return gemm.gemm_f16_f32_abt_noalloc(M, N, K, A.data_ptr(), A.stride(0), B.data_ptr(),
                                         B.stride(0), C.data_ptr(), C.stride(0), stream)


def sampled(M, N, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.full(N, M - 1), np.arange(M), rng.integers(0, M, 2000)])
    cols = np.concatenate([np.arange(N), np.full(M, N - 1), rng.integers(0, N, 2000)])
    return rows, cols


@pytest.mark.parametrize("kind", ["integer", "uniform"])
def test_noalloc_matches_the_allocating_entry(kind):
    # 1024x1024x65536 fills the 64 MiB scratch with the partial tiles of 16
    # shares of 16 tiles; 512x512x8192 then reuses its first 4 MiB.
    for i, (M, N, K) in enumerate([(1024, 1024, 65536), (512, 512, 8192)]):
        print(f"[gpu test] noalloc {kind} {M}x{N}x{K}: "
              f"{gemm.gemm_f16_f32_abt_describe(M, N, K)}", flush=True)
        A, B = ((inputs.integer(M, K, 301 + i), inputs.integer(N, K, 401 + i))
                if kind == "integer" else
                (inputs.uniform(M, K, 501 + i), inputs.uniform(N, K, 601 + i)))
        At, Bt = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
        want = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        gemm.gemm_abt(At, Bt, want)
        got = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        assert noalloc(At, Bt, got) == 0
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g, w), f"{M}x{N}x{K}: {(g != w).sum()} elements differ"
        rows, cols = sampled(M, N, 7 + i)
        ref, S = oracle.gemm_abt_elems(A, B, rows, cols)
        if kind == "integer":
            assert np.array_equal(g[rows, cols].astype(np.float64), ref)
        else:
            assert oracle.within_tolerance(g[rows, cols], ref, S).all()


def test_noalloc_refuses_plans_beyond_the_scratch():
    """4352^2 x 4096 runs whole data-parallel rounds and shares the 33 tiles
    left by stream-K: 74.25 MiB of partial tiles, more than the 64 MiB array."""
    M, N, K = 4352, 4352, 4096
    assert gemm.gemm_f16_f32_abt_workspace_size(M, N, K) > 64 << 20
    A = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    B = torch.zeros((N, K), dtype=torch.float16, device=DEV)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    assert noalloc(A, B, C) == 6  # GEMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(C).all()
