"""The hipBLASLt context arm checked against the CPU reference (needs an MI355X).

The pages compare their kernels with the vendor library at its best: every
algorithm its heuristic returns is run and the fastest one whose result
matches exactly is kept ("SASS-Level Kernel Generation for Blackwell",
sections "The numbers" and "How we measured"). bench.py --vendor keeps the
algorithms whose C equals this library's C bit for bit on integer-valued
inputs (bench.vendor_screen). Here every algorithm is also compared with the
CPU reference directly, and the set the bench keeps must be exactly the set
that is bit-exact against the reference.
"""
import os
import sys

import numpy as np
import pytest

import oracle
from dense_fp16_gemm_03_amd import build, inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dense_fp16_gemm_03_amd import gemm  # noqa: E402

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (384, 640, 2056)])
def test_vendor_screen_keeps_exactly_the_exact_algorithms(shape):
    if not os.path.exists(build.VENDOR_LIBRARY):
        pytest.fail(f"{build.VENDOR_LIBRARY} is not built (__graft_entry__.build() builds it)")
    M, N, K = shape
    print(f"[gpu test] vendor screen {M}x{N}x{K}", flush=True)
    A, B = inputs.workload_operands((M, N, K), "hash_int")
    ref, _ = oracle.gemm_abt(A, B)
    At, Bt = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    ours = gemm.gemm_abt(At, Bt)
    torch.cuda.synchronize()
    assert np.array_equal(ours.cpu().numpy().astype(np.float64), ref), "our C is not exact"

    lib = bench.load_vendor()
    count, ws, kept = bench.vendor_screen(torch, lib, At, Bt, ours)
    assert count > 0, f"hipBLASLt heuristic returned {count}"

    stream = torch.cuda.current_stream().cuda_stream
    Cv = torch.empty((M, N), dtype=torch.float32, device=DEV)
    against_oracle = []
    for i in range(count):
        Cv.fill_(float("nan"))
        st = lib.vendor_hipblaslt_run(i, At.data_ptr(), Bt.data_ptr(), Cv.data_ptr(),
                                      ws.data_ptr(), ws.numel(), stream)
        torch.cuda.synchronize()
        if st == 0 and np.array_equal(Cv.cpu().numpy().astype(np.float64), ref):
            against_oracle.append(i)
    print(f"  {count} algorithms, {len(kept)} kept by the bench screen, "
          f"{len(against_oracle)} exact against the reference", flush=True)
    assert kept == against_oracle
    assert kept, "no hipBLASLt algorithm is exact"
