"""ctypes binding of libgemm_f16.so (see include/gemm_f16.h for the contract).

The functions named like the C entry points take raw integers (device
addresses, sizes, a hipStream_t as an int) and only marshal arguments.
``gemm_abt`` is a convenience wrapper for torch tensors: torch supplies device
memory and the current stream, the library does all the arithmetic. There is
no fallback: if the library is missing or fails to load, calls raise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libgemm_f16.so")

GEMM_OK = 0
STATUS_NAMES = {
    0: "GEMM_OK", 1: "GEMM_ERR_INVALID_VALUE", 2: "GEMM_ERR_NOT_SUPPORTED",
    3: "GEMM_ERR_HIP", 4: "GEMM_ERR_ALLOC", 5: "GEMM_ERR_WORKSPACE", 6: "GEMM_ERR_SCRATCH",
}

# Every symbol include/gemm_f16.h declares.
EXPORTS = (
    "gemm_f16_f32_abt", "gemm_f16_f32_abt_workspace_size", "gemm_f16_f32_abt_ws",
    "gemm_status_string", "gemm_f16_f32_abt_describe", "gemm_f16_release_workspaces",
    "gemm_f16_schedule_dump", "gemm_f16_lds_chunk", "gemm_bf16_f32_abt",
    "gemm_bf16_f32_abt_workspace_size",
    "gemm_bf16_f32_abt_ws", "gemm_f16_set_plan_override", "gemm_f16_set_clock_probe",
    "gemm_f16_f32_abt_noalloc",
)

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load(path: str = LIBRARY):
    """Load and bind the library (raises if it is missing)."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() or "
                           "python -m dense_fp16_gemm_03_amd.build")
    lib = ctypes.CDLL(path)
    i64, p, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    st = ctypes.c_int
    lib.gemm_f16_f32_abt.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    lib.gemm_f16_f32_abt.restype = st
    lib.gemm_f16_f32_abt_workspace_size.argtypes = [i64, i64, i64]
    lib.gemm_f16_f32_abt_workspace_size.restype = sz
    lib.gemm_f16_f32_abt_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, sz, p]
    lib.gemm_f16_f32_abt_ws.restype = st
    lib.gemm_f16_f32_abt_noalloc.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    lib.gemm_f16_f32_abt_noalloc.restype = st
    lib.gemm_bf16_f32_abt.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    lib.gemm_bf16_f32_abt.restype = st
    lib.gemm_bf16_f32_abt_workspace_size.argtypes = [i64, i64, i64]
    lib.gemm_bf16_f32_abt_workspace_size.restype = sz
    lib.gemm_bf16_f32_abt_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, sz, p]
    lib.gemm_bf16_f32_abt_ws.restype = st
    lib.gemm_status_string.argtypes = [st]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_f16_f32_abt_describe.argtypes = [i64, i64, i64, ctypes.c_char_p, sz]
    lib.gemm_f16_f32_abt_describe.restype = st
    lib.gemm_f16_release_workspaces.argtypes = []
    lib.gemm_f16_release_workspaces.restype = None
    lib.gemm_f16_schedule_dump.argtypes = [i64, i64, i64, i64, p, i64, p, p]
    lib.gemm_f16_schedule_dump.restype = i64
    lib.gemm_f16_lds_chunk.argtypes = [ctypes.c_int32] * 4
    lib.gemm_f16_lds_chunk.restype = ctypes.c_int32
    lib.gemm_f16_set_plan_override.argtypes = [ctypes.c_char_p]
    lib.gemm_f16_set_plan_override.restype = None
    lib.gemm_f16_set_clock_probe.argtypes = [p]
    lib.gemm_f16_set_clock_probe.restype = None
    if path == LIBRARY:
        _lib = lib
    return lib


def _check(status: int):
    if status != GEMM_OK:
        msg = load().gemm_status_string(status).decode()
        raise GemmError(status, msg)


# --- entry points with the C names (raw integers in, status checked) -------

def gemm_f16_f32_abt(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """Raw call; returns the status code (does not raise)."""
    return load().gemm_f16_f32_abt(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f16_f32_abt_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                        stream=0) -> int:
    return load().gemm_f16_f32_abt_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace,
                                      workspace_bytes, stream)


def gemm_f16_f32_abt_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """Raw call with the workspace in the library's static scratch array;
    returns the status code (does not raise)."""
    return load().gemm_f16_f32_abt_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f16_f32_abt_workspace_size(M, N, K) -> int:
    return load().gemm_f16_f32_abt_workspace_size(M, N, K)


def gemm_bf16_f32_abt(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """Raw call with bfloat16 operands; returns the status code (does not raise)."""
    return load().gemm_bf16_f32_abt(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_f32_abt_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                         stream=0) -> int:
    return load().gemm_bf16_f32_abt_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace,
                                       workspace_bytes, stream)


def gemm_bf16_f32_abt_workspace_size(M, N, K) -> int:
    return load().gemm_bf16_f32_abt_workspace_size(M, N, K)


def gemm_status_string(status: int) -> str:
    return load().gemm_status_string(status).decode()


def gemm_f16_f32_abt_describe(M, N, K) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(load().gemm_f16_f32_abt_describe(M, N, K, buf, len(buf)))
    return buf.value.decode()


def gemm_f16_release_workspaces() -> None:
    load().gemm_f16_release_workspaces()


def gemm_f16_set_plan_override(text: str = "") -> None:
    """Plan override for tests and experiments ("" restores the default rule)."""
    load().gemm_f16_set_plan_override(text.encode() if text else None)


def gemm_f16_set_clock_probe(counters: int = 0) -> None:
    """Clock probe: device address of two uint64 counters (0 turns it off)."""
    load().gemm_f16_set_clock_probe(counters or None)


def gemm_f16_lds_chunk(chunks_per_row, block_dim, row, chunk) -> int:
    """LDS position of logical chunk `chunk` of tile row `row` (-1: bad arguments)."""
    return load().gemm_f16_lds_chunk(chunks_per_row, block_dim, row, chunk)


def gemm_f16_schedule_dump(M, N, K, grid=0):
    """(rows, k_iters, tiles): rows is an int64 array of
    (workgroup, tile, k_begin, k_end, role, shares, index)."""
    import numpy as np

    lib = load()
    ki, nt = ctypes.c_int64(0), ctypes.c_int64(0)
    n = lib.gemm_f16_schedule_dump(M, N, K, grid, None, 0, ctypes.byref(ki), ctypes.byref(nt))
    if n < 0:
        raise GemmError(1, "schedule_dump rejected the arguments")
    out = np.zeros((max(n, 1), 7), dtype=np.int64)
    n2 = lib.gemm_f16_schedule_dump(M, N, K, grid, out.ctypes.data, n, None, None)
    assert n2 == n
    return out[:n], ki.value, nt.value


# --- torch convenience -----------------------------------------------------

def gemm_abt(A, B, C=None, stream=None, workspace=None):
    """C = A @ B^T for torch tensors: A (M, K) and B (N, K) both float16 or
    both bfloat16, C (M, N) float32, all on one GPU with unit stride along the
    last dimension. Returns C. Enqueued on ``stream`` (default: torch's
    current stream). ``workspace``, if given, is a contiguous tensor on the
    same GPU of at least ``gemm_f16_f32_abt_workspace_size(M, N, K)`` bytes,
    256-byte aligned (the ``_ws`` entry points); otherwise the library uses
    its own per-stream workspace."""
    import torch

    global _DTYPES
    if _DTYPES is None:
        _DTYPES = (torch.float16, torch.bfloat16)
    dt = A.dtype
    if dt != B.dtype or dt not in _DTYPES:
        raise TypeError("A and B must be both float16 or both bfloat16")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("A must be (M, K) and B (N, K)")
    M, K = A.shape
    N = B.shape[0]
    dev = A.device
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
    elif C.dtype != torch.float32 or C.shape != (M, N):
        raise ValueError("C must be float32 (M, N)")
    for t, name in ((A, "A"), (B, "B"), (C, "C")):
        if t.device != dev or not t.is_cuda:
            raise ValueError(f"{name} must be on A's GPU")
        if t.shape[1] > 1 and t.stride(1) != 1 and t.numel() > 0:
            raise ValueError(f"{name} must have unit stride along its last dimension")
    if workspace is not None and (not workspace.is_cuda or workspace.device != dev
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on A's GPU")
    lda = A.stride(0) if M > 1 else max(K, 1)
    ldb = B.stride(0) if N > 1 else max(K, 1)
    ldc = C.stride(0) if M > 1 else max(N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lib = _lib if _lib is not None else load()
    bf16 = dt == torch.bfloat16
    if workspace is None:
        fn = lib.gemm_bf16_f32_abt if bf16 else lib.gemm_f16_f32_abt
        args = (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, s)
    else:
        fn = lib.gemm_bf16_f32_abt_ws if bf16 else lib.gemm_f16_f32_abt_ws
        args = (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                workspace.data_ptr(), workspace.numel() * workspace.element_size(), s)
    # the library works on the current HIP device: make it A's for the call
    if dev.index == torch.cuda.current_device():
        st = fn(*args)
    else:
        with torch.cuda.device(dev):
            st = fn(*args)
    _check(st)
    return C


_DTYPES = None  # (torch.float16, torch.bfloat16), set at the first call
