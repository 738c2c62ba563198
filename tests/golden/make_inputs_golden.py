"""Writes inputs_first16.txt: the first 16 bit patterns (row 0) of each seeded
input generator, so that a change to an input recipe, or to the stream of
numpy's generator, shows in the tests. Calls only dense_fp16_gemm_03_amd.inputs.

    python tests/golden/make_inputs_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from dense_fp16_gemm_03_amd import inputs  # noqa: E402


def entries():
    bits = lambda a: a.view(np.uint16)[0, :16]  # noqa: E731
    yield "uniform_seed1", bits(inputs.uniform(1, 16, 1))
    yield "uniform_seed2", bits(inputs.uniform(1, 16, 2))
    yield "integer_seed3", bits(inputs.integer(1, 16, 3))
    yield "integer_seed4", bits(inputs.integer(1, 16, 4))
    yield "hash_int_salt1", bits(inputs.hash_int(1, 16, 1))
    yield "hash_int_salt2", bits(inputs.hash_int(1, 16, 2))
    yield "uniform_bf16_seed1", inputs.uniform_bf16(1, 16, 1)[0, :16]
    yield "integer_bf16_seed3", inputs.integer_bf16(1, 16, 3)[0, :16]


def main():
    lines = ["# First 16 bit patterns (hex) of row 0 of each seeded generator;",
             "# written by make_inputs_golden.py from dense_fp16_gemm_03_amd.inputs."]
    for name, v in entries():
        lines.append(name + " " + " ".join(f"{int(x):04x}" for x in v))
    with open(os.path.join(HERE, "inputs_first16.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
