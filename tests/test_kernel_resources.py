"""Register, spill and LDS figures of every shipped kernel, read from the gfx950
assembly of the library's own source (no GPU needed).

The assembly is written by ``python -m dense_fp16_gemm_03_amd.build --asm``
(``__graft_entry__.build()`` does it); when it is missing or older than the
sources, this module writes it again (device pass only, a few seconds).

Bars, for every kernel in the code object:
  * no VGPR spills and no private (scratch) segment: such a spill is a round
    trip to memory inside the main loop. (SGPR spills are not memory traffic:
    the compiler parks those scalars in lanes of a VGPR; they are printed,
    not failed.)
  * the registers fit the occupancy the kernel is launched for: two waves
    per SIMD (8-wave workgroups) get 256 registers a lane, one wave per SIMD
    512, VGPRs and AGPRs together;
  * LDS within gfx950's 160 KiB;
  * exactly the tiled configurations the library dispatches to are built.
"""
import os
import re

import pytest
import yaml

from dense_fp16_gemm_03_amd import build

ASM = os.path.join(build.ASM_DIR, f"gemm_kernels-{build.ARCH}.s")


def _asm_is_fresh():
    if not os.path.exists(ASM):
        return False
    t = os.path.getmtime(ASM)
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)]
    return all(os.path.getmtime(f) <= t for f in srcs)


@pytest.fixture(scope="module")
def kernels():
    if not _asm_is_fresh():
        build.emit_asm()
    text = open(ASM).read()
    m = re.search(r"\.amdgpu_metadata\n(.*?)\n\.\.\.\n", text, re.S)
    assert m, "no metadata block in the assembly"
    meta = yaml.safe_load(m.group(1))
    return meta["amdhsa.kernels"]


def _threads(k):
    return int(k[".max_flat_workgroup_size"])


def test_no_spills_and_no_scratch(kernels):
    assert len(kernels) >= 10
    bad = [(k[".name"], k[".vgpr_spill_count"], k[".private_segment_fixed_size"])
           for k in kernels if k[".vgpr_spill_count"] or k[".private_segment_fixed_size"]]
    assert not bad, f"kernels that spill VGPRs or use scratch: {bad}"
    for k in kernels:
        if k[".sgpr_spill_count"]:
            print(f"{k['.name']}: {k['.sgpr_spill_count']} SGPRs kept in VGPR lanes")


def test_registers_fit_the_launch_occupancy(kernels):
    for k in kernels:
        regs = int(k[".vgpr_count"]) + int(k.get(".agpr_count", 0))
        waves = _threads(k) // 64
        # workgroups of 8 waves run two waves per SIMD, of 4 waves one
        limit = 256 if waves >= 8 else 512
        assert regs <= limit, f"{k['.name']}: {regs} registers for {waves} waves"


def test_lds_within_gfx950_limit(kernels):
    for k in kernels:
        assert int(k[".group_segment_fixed_size"]) <= 160 * 1024, k[".name"]


def test_shipped_tiled_configurations(kernels):
    """One main kernel per built configuration: the eight fp16 ids (16, 18,
    27, 28, 35, 36, 37, 38) and the five bf16 ones (16, 18, 27, 37, 38)."""
    main = [k[".name"] for k in kernels
            if re.search(r"gemm_(tiled|pingpong|pingpong64|pingpong_ring)_kernel", k[".name"])]
    assert len(main) == 13, main
