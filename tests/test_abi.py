"""The C ABI without a GPU: exports, argument checks, plans and the schedule model.

No call here launches work: argument errors return before any HIP call, and
describe / schedule_dump are host-only.
"""
import os
import re

import numpy as np
import pytest

from dense_fp16_gemm_03_amd import gemm, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f16.h")


@pytest.fixture(scope="module")
def lib():
    return gemm.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 7
    for name in names:
        assert hasattr(lib, name), f"{name} declared in gemm_f16.h but not exported"
    assert sorted(gemm.EXPORTS) == names


def test_status_strings(lib):
    for code, name in gemm.STATUS_NAMES.items():
        assert gemm.gemm_status_string(code).startswith(name)
    assert "unknown" in gemm.gemm_status_string(99)


# Fake device addresses: validation never dereferences them.
A_PTR, B_PTR, C_PTR = 0x10000000, 0x20000000, 0x30000000
MAX_DIM = (1 << 31) - 1025  # largest M, N or K the library takes


@pytest.mark.parametrize("args,expect", [
    ((-1, 4, 4, A_PTR, 4, B_PTR, 4, C_PTR, 4), 1),          # negative M
    ((4, 4, -2, A_PTR, 4, B_PTR, 4, C_PTR, 4), 1),          # negative K
    ((4, 4, 8, A_PTR, 7, B_PTR, 8, C_PTR, 4), 1),           # lda < K
    ((4, 4, 8, A_PTR, 8, B_PTR, 7, C_PTR, 4), 1),           # ldb < K
    ((4, 5, 8, A_PTR, 8, B_PTR, 8, C_PTR, 4), 1),           # ldc < N
    ((4, 4, 8, A_PTR, 8, B_PTR, 8, 0, 4), 1),               # C NULL with work
    ((4, 4, 8, 0, 8, B_PTR, 8, C_PTR, 4), 1),               # A NULL with K > 0
    ((4, 4, 8, A_PTR, 8, B_PTR, 8, A_PTR + 16, 4), 1),      # C overlaps A
    ((4, 4, 8, A_PTR, 8, B_PTR, 8, B_PTR, 4), 1),           # C overlaps B
    ((4, 4, 8, A_PTR + 1, 8, B_PTR, 8, C_PTR, 4), 2),       # A not 2-byte aligned
    ((4, 4, 8, A_PTR, 8, B_PTR, 8, C_PTR + 2, 4), 2),       # C not 4-byte aligned
    ((1 << 31, 4, 8, A_PTR, 8, B_PTR, 8, 1 << 44, 4), 2),   # M too large
    ((MAX_DIM + 1, 4, 8, A_PTR, 8, B_PTR, 8, 1 << 44, 4), 2),  # M one past the limit
    ((4, MAX_DIM + 1, 8, A_PTR, 8, B_PTR, 8, 1 << 44, MAX_DIM + 1), 2),  # N past it
    ((4, 4, MAX_DIM + 1, A_PTR, MAX_DIM + 1, 1 << 40, MAX_DIM + 1, 1 << 44, 4), 2),  # K
    ((4, 4, 8, A_PTR, 1 << 62, B_PTR, 8, 1 << 44, 4), 2),   # lda: span past 2^60 bytes
    ((4, 4, 8, A_PTR, 8, B_PTR, 8, 1 << 44, 1 << 61), 2),   # ldc: span past 2^60 bytes
    ((0, 4, 8, A_PTR, 8, B_PTR, 8, C_PTR, 4), 0),           # M = 0: nothing to do
    ((4, 0, 8, 0, 8, 0, 8, 0, 0), 0),                       # N = 0: nothing to do
])
def test_argument_checks(lib, args, expect):
    assert gemm.gemm_f16_f32_abt(*args, 0) == expect
    assert gemm.gemm_bf16_f32_abt(*args, 0) == expect  # same contract for bfloat16


def test_bf16_workspace_and_dtype_checks(lib):
    import torch

    for shape in ((2048, 2048, 16384), (1024, 1024, 65536), (8192, 8192, 8192), (7, 9, 13)):
        assert (gemm.gemm_bf16_f32_abt_workspace_size(*shape)
                == gemm.gemm_f16_f32_abt_workspace_size(*shape))
    M, N, K = inputs.WORKLOADS["1024x1024x65536"]
    assert gemm.gemm_bf16_f32_abt_ws(M, N, K, A_PTR, K, B_PTR, K, C_PTR, N, 0, 0, 0) == 5
    with pytest.raises(TypeError):  # mixed operand types, rejected before any device call
        gemm.gemm_abt(torch.zeros(2, 2, dtype=torch.float16),
                      torch.zeros(2, 2, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        gemm.gemm_abt(torch.zeros(2, 2), torch.zeros(2, 2))


def test_noalloc_checks_without_a_device(lib):
    """The no-allocation entry point reports argument errors and plans beyond
    its 64 MiB scratch before it needs a device."""
    assert gemm.gemm_f16_f32_abt_noalloc(-1, 4, 4, A_PTR, 4, B_PTR, 4, C_PTR, 4, 0) == 1
    assert gemm.gemm_f16_f32_abt_noalloc(4, 4, 8, A_PTR, 8, B_PTR, 8, A_PTR + 16, 4, 0) == 1
    assert gemm.gemm_f16_f32_abt_noalloc(0, 4, 8, A_PTR, 8, B_PTR, 8, C_PTR, 4, 0) == 0
    M, N, K = 4352, 4352, 4096  # 74.25 MiB of partial tiles
    assert gemm.gemm_f16_f32_abt_noalloc(M, N, K, A_PTR, K, 1 << 40, K, 1 << 44, N, 0) == 6


def test_caller_workspace_checked_first(lib):
    M, N, K = inputs.WORKLOADS["1024x1024x65536"]
    need = gemm.gemm_f16_f32_abt_workspace_size(M, N, K)
    assert need > 0
    # too small / misaligned / NULL workspace: rejected before any HIP call
    assert gemm.gemm_f16_f32_abt_ws(M, N, K, A_PTR, K, B_PTR, K, C_PTR, N, 0, 0, 0) == 5
    assert gemm.gemm_f16_f32_abt_ws(M, N, K, A_PTR, K, B_PTR, K, C_PTR, N, 0x40000000,
                                    need - 1, 0) == 5
    assert gemm.gemm_f16_f32_abt_ws(M, N, K, A_PTR, K, B_PTR, K, C_PTR, N, 0x40000010,
                                    need, 0) == 5


def test_workspace_sizes(lib):
    assert gemm.gemm_f16_f32_abt_workspace_size(8192, 8192, 8192) == 0
    assert gemm.gemm_f16_f32_abt_workspace_size(0, 8, 8) == 0
    ws = gemm.gemm_f16_f32_abt_workspace_size(2048, 2048, 16384)
    assert ws > 0 and ws % 256 == 0


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_describe_workloads(lib, name):
    M, N, K = inputs.WORKLOADS[name]
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    assert f"M={M} N={N} K={K}" in text and "kernel=" in text


def test_describe_size_limit(lib):
    for M, N, K in ((MAX_DIM, 1, 8), (1, MAX_DIM, 8), (1, 1, MAX_DIM)):
        assert f"M={M} N={N} K={K}" in gemm.gemm_f16_f32_abt_describe(M, N, K)
    for M, N, K in ((MAX_DIM + 1, 1, 8), (1, MAX_DIM + 1, 8), (1, 1, MAX_DIM + 1)):
        with pytest.raises(gemm.GemmError, match="NOT_SUPPORTED"):
            gemm.gemm_f16_f32_abt_describe(M, N, K)


def test_packed_plans(lib, monkeypatch):
    """K % 8 != 0 on a large enough product: both operands are packed into
    rows of K rounded up to 8, and the workspace size counts the copies."""
    M, N, K = 1024, 1024, 1001
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    assert "pack=AB kp=1008" in text and "kernel=64x64x64" in text
    assert gemm.gemm_f16_f32_abt_workspace_size(M, N, K) == 2 * (M * 1008 * 2)
    M, N, K = 1024, 1024, 8191  # packed, and a split plan: partial tiles first
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    assert "pack=AB kp=8192" in text and "mode=split splits=4" in text and "kid=16" in text
    parts = 64 * 4 * 128 * 128 * 4
    assert gemm.gemm_f16_f32_abt_workspace_size(M, N, K) == parts + 2 * (M * 8192 * 2)
    assert "pack" not in gemm.gemm_f16_f32_abt_describe(2048, 2048, 4096)
    gemm.gemm_f16_set_plan_override("general=1")
    assert "general" in gemm.gemm_f16_f32_abt_describe(1024, 1024, 1001)
    assert gemm.gemm_f16_f32_abt_workspace_size(1024, 1024, 1001) == 0


def test_describe_general_and_empty(lib):
    assert "general" in gemm.gemm_f16_f32_abt_describe(100, 100, 13)  # K % 8 != 0
    assert "nothing" in gemm.gemm_f16_f32_abt_describe(0, 100, 13)


# --- schedule model ----------------------------------------------------------

def check_schedule(rows, k_iters, tiles):
    """Every (tile, k-iteration) covered exactly once. A tile covered by one
    segment has role 0; a tile split among s segments has them all role 1,
    numbered 0..s-1 in increasing k, each reporting shares == s."""
    errors = []
    cover = np.zeros((tiles, k_iters), dtype=np.int64)
    per_tile = {}
    for w, t, kb, ke, role, shares, index in rows:
        if not (0 <= t < tiles and 0 <= kb < ke <= k_iters):
            errors.append(f"bad segment {(w, t, kb, ke)}")
            continue
        cover[t, kb:ke] += 1
        per_tile.setdefault(t, []).append((kb, ke, role, shares, index))
    if not np.all(cover == 1):
        bad = np.argwhere(cover != 1)[:3]
        errors.append(f"coverage != 1 at (tile, k) {bad.tolist()}")
    for t, segs in per_tile.items():
        n = len(segs)
        if any(sh != n for _, _, _, sh, _ in segs):
            errors.append(f"tile {t}: shares field != {n}")
        if n == 1:
            if segs[0][2] != 0:
                errors.append(f"tile {t}: single segment with role {segs[0][2]}")
            continue
        if any(r != 1 for _, _, r, _, _ in segs):
            errors.append(f"tile {t}: shared tile with a role other than 1")
        by_k = sorted(segs)
        if [ix for *_, ix in by_k] != list(range(n)):
            errors.append(f"tile {t}: share indices {[ix for *_, ix in by_k]} not 0..{n - 1} in k order")
    if len(per_tile) != tiles:
        errors.append(f"{tiles - len(per_tile)} tiles never scheduled")
    return errors


SCHED_CASES = [
    (8192, 8192, 8192, None),
    (2048, 2048, 16384, None),
    (1024, 1024, 65536, None),
    (1024, 1024, 1024, None),
    (256, 256, 512, None),
    (2048, 2048, 16384, "mode=2"),          # stream-K, even
    (1000, 1500, 4104, "mode=2"),           # stream-K, ranges cross tile ends
    (1000, 1500, 4104, "mode=2,grid=200"),
    (777, 333, 1000, "mode=2,kid=16,grid=77"),
    (5000, 300, 2048, "mode=1,splits=3"),
    (5000, 300, 2048, "mode=1,splits=3,grid=50"),   # split-K over several rounds
    (3000, 2900, 1024, None),
    (4608, 4608, 2048, "mode=3"),           # one data-parallel round, stream-K tail
    (4608, 4608, 2048, "mode=3,grid=100"),  # three whole rounds of 100, 24 tiles shared
    (5000, 300, 2048, "mode=3,grid=7"),     # ranges of the tail cross tile ends
    (3072, 3072, 4096, "mode=3"),           # no whole round: plain stream-K
    (4096, 4096, 4096, "mode=3"),           # no remainder: plain data-parallel
    (630, 621, 80, "mode=3,kid=18,grid=92"),  # 16 stream-K iterations for 92 workgroups
]


@pytest.mark.parametrize("M,N,K,plan", SCHED_CASES)
def test_schedule_covers_once(lib, monkeypatch, M, N, K, plan):
    if plan:
        gemm.gemm_f16_set_plan_override(plan)
    rows, k_iters, tiles = gemm.gemm_f16_schedule_dump(M, N, K)
    assert check_schedule(rows.tolist(), k_iters, tiles) == []
    if plan and "mode=2" in plan:
        assert "stream_k" in gemm.gemm_f16_f32_abt_describe(M, N, K)
    if plan and "mode=3" in plan:
        text = gemm.gemm_f16_f32_abt_describe(M, N, K)
        grid = int(plan.split("grid=")[1]) if "grid" in plan else 256
        whole_rounds = tiles // grid
        if tiles % grid == 0:
            assert "mode=data_parallel" in text
        elif whole_rounds == 0:
            assert "mode=stream_k" in text
        else:
            assert "mode=dp_stream_k" in text and f"grid={grid}" in text
            # whole tiles of the data-parallel rounds are never shared
            base = whole_rounds * grid
            assert all(r[1] >= base or r[5] == 1 for r in rows.tolist())
            assert any(r[1] >= base and r[5] > 1 for r in rows.tolist())


@pytest.mark.parametrize("M,N,K,plan", SCHED_CASES[:3] + SCHED_CASES[6:7] + SCHED_CASES[12:15])
def test_schedule_model_detects_dropped_unit(lib, monkeypatch, M, N, K, plan):
    """Dropping any one segment, or duplicating one, must fail the model."""
    if plan:
        gemm.gemm_f16_set_plan_override(plan)
    rows, k_iters, tiles = gemm.gemm_f16_schedule_dump(M, N, K)
    rows = rows.tolist()
    rng = np.random.default_rng(5)
    for i in rng.choice(len(rows), size=min(5, len(rows)), replace=False):
        assert check_schedule(rows[:i] + rows[i + 1:], k_iters, tiles) != []
        assert check_schedule(rows + [rows[i]], k_iters, tiles) != []


@pytest.mark.parametrize("grid", [1, 3, 7, 8, 9, 15, 100, 200, 243, 245, 250, 252, 256])
def test_xcd_renumbering(lib, grid):
    """Workgroup w runs on XCD w mod 8; the schedule renumbers workgroups so
    that each XCD holds one contiguous block of units, for any grid: the
    first tile of each workgroup (data-parallel, so unit v + n * grid) is a
    permutation of 0 .. grid-1, contiguous and increasing within each XCD,
    the XCDs' blocks in order, block sizes grid / 8 or one more."""
    gemm.gemm_f16_set_plan_override("kid=18,mode=0")
    rows, _, _ = gemm.gemm_f16_schedule_dump(4096, 4096, 256, grid)
    first = {}
    for w, tile in rows[:, :2].tolist():
        first[w] = min(first.get(w, tile), tile)
    assert sorted(first) == list(range(grid))
    assert sorted(first.values()) == list(range(grid))
    blocks = [[first[w] for w in range(x, grid, 8)] for x in range(min(grid, 8))]
    for b in blocks:
        assert b == list(range(b[0], b[0] + len(b)))
        assert len(b) in (grid // 8, grid // 8 + 1)
    for a, b in zip(blocks, blocks[1:]):
        assert a[-1] + 1 == b[0]
    if grid % 8 == 0:
        assert all(first[w] == (w % 8) * (grid // 8) + w // 8 for w in range(grid))


def test_planted_index_error_detected(lib, monkeypatch):
    """Swapping two shares' indices must fail the model (k order matters)."""
    rows, k_iters, tiles = gemm.gemm_f16_schedule_dump(1024, 1024, 65536)
    rows = rows.tolist()
    a = next(i for i, r in enumerate(rows) if r[4] == 1 and r[6] == 0)
    b = next(i for i, r in enumerate(rows) if r[1] == rows[a][1] and r[6] == 1)
    rows[a][6], rows[b][6] = rows[b][6], rows[a][6]
    assert check_schedule(rows, k_iters, tiles) != []


def test_default_plans(lib):
    """The five workloads take the tiled kernels with at most 256 workgroups,
    except 256^3, which takes the direct kernel (no persistent schedule: the
    host model refuses it)."""
    for M, N, K in inputs.WORKLOADS.values():
        if "direct" in gemm.gemm_f16_f32_abt_describe(M, N, K):
            assert (M, N, K) == (256, 256, 256)
            with pytest.raises(gemm.GemmError):
                gemm.gemm_f16_schedule_dump(M, N, K)
            continue
        rows, _, _ = gemm.gemm_f16_schedule_dump(M, N, K)
        assert rows[:, 0].max() < 256


@pytest.mark.parametrize("M,N,K,mode", [
    (4608, 4608, 8192, "dp_stream_k"),   # 324 tiles: 68 left; 188 idle CUs x 256 k-iters
    (4352, 4352, 4096, "dp_stream_k"),   # 289 tiles: 33 left
    (4608, 4608, 2048, "dp_stream_k"),   # 188 idle x 64 k-iters: 47 per CU
    (5120, 5120, 4096, "dp_stream_k"),   # 400 tiles: 112 idle x 128
    (6400, 6400, 2048, "data_parallel"),  # 625 tiles: 143 idle x 64 = 36 per CU
    (8192, 8192, 8192, "data_parallel"),  # whole rounds only
    (4096, 4096, 4096, "data_parallel"),  # exactly one round
    (2048, 2048, 16384, "split"),         # fewer tiles than CUs
])
def test_default_tail_rule(lib, M, N, K, mode):
    """With more tiles than CUs, the tiles left after whole data-parallel
    rounds are shared by stream-K when the last round's idle CUs times the
    k-iterations is at least 44 per CU; the default plan still covers every
    (tile, k-iteration) once."""
    assert f"mode={mode} " in gemm.gemm_f16_f32_abt_describe(M, N, K) + " "
    rows, k_iters, tiles = gemm.gemm_f16_schedule_dump(M, N, K)
    assert check_schedule(rows.tolist(), k_iters, tiles) == []


@pytest.mark.parametrize("M,N,K,kid,mode", [
    (8192, 8192, 8192, 37, "data_parallel"),   # 4 tiles per CU: 64-wide stages
    (16384, 16384, 16384, 37, "data_parallel"),
    (8192, 8192, 4096, 37, "data_parallel"),
    (4096, 4096, 4096, 37, "data_parallel"),   # one round exactly
    (4608, 4608, 8192, 37, "dp_stream_k"),     # tiles left shared by stream-K
    (4096, 4096, 1024, 27, "data_parallel"),   # K below 2048: 32-wide ring
    (4096, 4096, 2048, 37, "data_parallel"),
    (10240, 10240, 2048, 37, "dp_stream_k"),
    (10240, 10240, 1024, 27, "data_parallel"),
    (2048, 2048, 16384, 37, "split"),          # fewer tiles than CUs: split-K
    (1024, 1024, 65536, 37, "split"),
])
def test_default_main_loop(lib, M, N, K, kid, mode):
    """At least a round of 256x256 tiles with K >= 2048, and split plans,
    take the main loop over 64-wide stages in five half-stage slots (whether
    or not the tiles left are shared); shorter K keeps the 32-wide ring."""
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    assert f"kid={kid} " in text and f"mode={mode} " in text
    rows, k_iters, tiles = gemm.gemm_f16_schedule_dump(M, N, K)
    assert check_schedule(rows.tolist(), k_iters, tiles) == []


@pytest.mark.parametrize("M,N,K,kid,mode,splits", [
    (1024, 1024, 4096, 18, "data_parallel", 1),
    (1024, 1024, 8192, 16, "split", 4),
    (512, 512, 8192, 18, "split", 4),
    (2048, 2048, 4096, 16, "data_parallel", 1),
    (2048, 1024, 8192, 16, "split", 2),
    (3072, 3072, 2048, 37, "data_parallel", 1),
    (2048, 2048, 16384, 37, "split", 4),      # the rule's plan, kept
    (1024, 1024, 65536, 37, "split", 16),
    (256, 256, 1 << 20, 37, "split", 256),
])
def test_default_fewer_tiles_than_cus(lib, M, N, K, kid, mode, splits):
    """Below a full round of 256x256 tiles the plan of least predicted time
    is taken (64-wide kernels with 256x256, 128x128 or 64x64 tiles, any split
    that keeps one round), unless the rule's own plan is predicted within
    10% of it. A forced kernel or mode bypasses the prediction."""
    text = gemm.gemm_f16_f32_abt_describe(M, N, K)
    assert f"kid={kid} " in text and f"mode={mode} splits={splits} " in text, text
    gemm.gemm_f16_set_plan_override("kid=37")
    assert "kid=37 " in gemm.gemm_f16_f32_abt_describe(M, N, K)


def test_plan_override_seen_on_many_threads(lib, monkeypatch):
    """Plans are cached and the override is shared state; ctypes releases the
    GIL, so these calls run concurrently and every one must see the same
    plan."""
    import threading

    gemm.gemm_f16_set_plan_override("kid=16,mode=1,splits=3,grid=40,group=2")
    want = gemm.gemm_f16_f32_abt_describe(600, 520, 1352)
    assert "kid=16" in want and "splits=3" in want and "grid=40" in want
    bad = []

    def worker():
        for _ in range(2000):
            got = gemm.gemm_f16_f32_abt_describe(600, 520, 1352)
            if got != want:
                bad.append(got)
                return

    threads = [threading.Thread(target=worker) for _ in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:2]


def test_schedule_model_random_stream_k_plans(lib, monkeypatch):
    """Seeded random shapes, kernels and grids under stream-K and under whole
    data-parallel rounds then stream-K: the host model of every plan covers
    each (tile, k-iteration) once and numbers each tile's shares 0..s-1 in k
    order (a grid larger than the stream-K iterations once broke that)."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        M, N = int(rng.integers(1, 3000)), int(rng.integers(1, 3000))
        K = int(rng.integers(1, 375)) * 8
        kid = int(rng.choice([16, 18, 27, 28, 35, 36, 37, 38]))
        plan = f"kid={kid},mode={int(rng.choice([2, 3]))},grid={int(rng.integers(1, 300))}"
        gemm.gemm_f16_set_plan_override(plan)
        rows, k_iters, tiles = gemm.gemm_f16_schedule_dump(M, N, K)
        assert check_schedule(rows.tolist(), k_iters, tiles) == [], (M, N, K, plan)


@pytest.mark.parametrize("M,N,K,kid", [
    (256, 256, 256, 101),     # 256 tiles of 16x16, K <= 256: the direct kernel
    (256, 256, 512, 38),      # 64 tiles of 32x32: one per CU or fewer
    (384, 384, 256, 38),      # 576 tiles of 16x16
    (512, 512, 512, 38),      # 256 tiles of 32x32
    (512, 512, 2048, 38),
    (640, 640, 1024, 18),     # 400 tiles of 32x32: 64x64 tiles instead
    (1024, 1024, 1024, 18),
    (2048, 2048, 2048, 16),   # enough 128x128 tiles for every CU twice
])
def test_default_small_tiles(lib, M, N, K, kid):
    """Below a round of 256x256 tiles with short K the tile shrinks with the
    problem: 128x128, then 64x64, then 32x32 while those fit the CUs, then
    the direct kernel's 16x16 for K <= 256."""
    assert f"kid={kid} " in gemm.gemm_f16_f32_abt_describe(M, N, K)
