"""MI355X (gfx950) fp16 x fp16 -> fp32 GEMM, C = A * B^T, behind a C ABI.

The compiled library ``libgemm_f16.so`` (HIP, built for gfx950) does all the
arithmetic; ``gemm`` is a ctypes binding with the same entry-point names. The
binding is imported lazily so that ``inputs`` can be used without a GPU stack.
"""
from __future__ import annotations

__all__ = ["gemm", "inputs"]


def __getattr__(name):
    if name in ("gemm", "inputs", "build"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
