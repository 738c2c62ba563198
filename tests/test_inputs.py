"""Seeded synthetic operands: determinism and value sets (CPU only)."""
import numpy as np
import pytest

from dense_fp16_gemm_03_amd import inputs


def test_uniform_deterministic_and_in_range():
    a = inputs.uniform(300, 70, 1)
    b = inputs.uniform(300, 70, 1)
    c = inputs.uniform(300, 70, 2)
    assert a.dtype == np.float16 and a.shape == (300, 70)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert not np.array_equal(a, c)
    assert a.min() >= -1 and a.max() <= 1
    # binary64 draw rounded to binary16, in row blocks: same as one draw
    ref = np.random.default_rng(1).uniform(-1.0, 1.0, size=(300, 70)).astype(np.float16)
    assert np.array_equal(a.view(np.uint16), ref.view(np.uint16))


def test_uniform_block_draw_matches_single_draw():
    rows, cols = 5000, 4000  # > 2^24 elements: exercises the row-block loop
    a = inputs.uniform(rows, cols, 7)
    ref = np.random.default_rng(7).uniform(-1.0, 1.0, size=(rows, cols)).astype(np.float16)
    assert np.array_equal(a.view(np.uint16), ref.view(np.uint16))


def test_integer_values():
    a = inputs.integer(200, 64, 3)
    assert set(np.unique(a.astype(np.float32)).tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}
    assert np.array_equal(a, inputs.integer(200, 64, 3))


def test_hash_int_values():
    h = inputs.hash_int(64, 64, 1)
    assert set(np.unique(h.astype(np.float32)).tolist()) <= set(range(-3, 4))
    assert len(np.unique(h.astype(np.float32))) == 7
    assert np.array_equal(h, inputs.hash_int(64, 64, 1))


def test_perm_pattern_exact():
    p = inputs.perm_pattern(100, 300)
    j, k = np.meshgrid(np.arange(100), np.arange(300), indexing="ij")
    assert np.array_equal(p.astype(np.int64), ((37 * j + 11 * k) % 2048) - 1024)


def test_kblock_weights():
    w = inputs.kblock_weights(2, 200, 64)
    assert w[0, 0] == 1 and w[0, 64] == 2 and w[1, 199] == 4


def test_workloads_table():
    assert inputs.WORKLOADS["8192^3"] == (8192, 8192, 8192)
    assert inputs.WORKLOADS["1024x1024x65536"] == (1024, 1024, 65536)


def _bf16_values(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def test_to_bf16_bits_matches_torch_rounding():
    """Round-to-nearest-even binary32 -> bfloat16, checked against torch's own
    conversion (an independent implementation), halfway cases included."""
    import torch

    rng = np.random.default_rng(5)
    x = rng.uniform(-4, 4, size=20000).astype(np.float32)
    base = (np.arange(1, 2001, dtype=np.uint32) << np.uint32(16))
    halfway = np.concatenate([(base | np.uint32(0x8000)).view(np.float32),   # ties
                              (base | np.uint32(0x7FFF)).view(np.float32),
                              (base | np.uint32(0x8001)).view(np.float32)])
    for v in (x, halfway, -halfway):
        ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(inputs.to_bf16_bits(v), ref)


def test_bf16_generators():
    a = inputs.uniform_bf16(300, 70, 1)
    assert a.dtype == np.uint16 and a.shape == (300, 70)
    assert np.array_equal(a, inputs.uniform_bf16(300, 70, 1))
    va = _bf16_values(a)
    assert va.min() >= -1 and va.max() <= 1
    ref = np.random.default_rng(1).uniform(-1.0, 1.0, size=(300, 70))
    assert np.array_equal(a, inputs.to_bf16_bits(ref))
    i = inputs.integer_bf16(200, 64, 3)
    assert set(np.unique(_bf16_values(i)).tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}
    p = inputs.perm_pattern_bf16(100, 300)
    j, k = np.meshgrid(np.arange(100), np.arange(300), indexing="ij")
    assert np.array_equal(_bf16_values(p).astype(np.int64), ((37 * j + 11 * k) % 256) - 128)
    A, B = inputs.workload_operands((64, 32, 16), "hash_int", "bf16")
    assert np.array_equal(_bf16_values(A), inputs.hash_int(64, 16, 1).astype(np.float32))


def test_device_uniform_on_the_cpu_generator():
    """The device-side generator, run on torch's CPU device: seeded, in
    [-1, 1], padding columns NaN, rows contiguous with stride ld."""
    import torch

    a = inputs.device_uniform(50, 40, 7, "cpu")
    assert a.dtype == torch.float16 and tuple(a.shape) == (50, 40) and a.is_contiguous()
    assert torch.equal(a, inputs.device_uniform(50, 40, 7, "cpu"))
    assert not torch.equal(a, inputs.device_uniform(50, 40, 8, "cpu"))
    v = a.float()
    assert v.min().item() >= -1 and v.max().item() <= 1 and v.std().item() > 0.5
    p = inputs.device_uniform(50, 40, 7, "cpu", ld=56)
    assert p.stride() == (56, 1)
    full = p.as_strided((50, 56), (56, 1))
    assert torch.isnan(full[:, 40:]).all() and not torch.isnan(p).any()
    with pytest.raises(ValueError):
        inputs.device_uniform(4, 8, 1, "cpu", ld=7)


def test_generators_match_the_recorded_first_values():
    """The first 16 bit patterns of every seeded generator, recorded in
    tests/golden/inputs_first16.txt (written by make_inputs_golden.py)."""
    import importlib.util
    import os

    here = os.path.join(os.path.dirname(__file__), "golden")
    spec = importlib.util.spec_from_file_location(
        "make_inputs_golden", os.path.join(here, "make_inputs_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    recorded = {}
    for line in open(os.path.join(here, "inputs_first16.txt")):
        if line.strip() and not line.startswith("#"):
            name, *vals = line.split()
            recorded[name] = [int(v, 16) for v in vals]
    now = {name: [int(x) for x in v] for name, v in mod.entries()}
    assert now == recorded
