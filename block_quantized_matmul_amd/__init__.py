"""Python binding of liblqmm, block-quantized matmul for MI355X (gfx950).

The functions mirror the C entry points of ``include/lqmm.h`` one to one and
only marshal arguments: they check devices, dtypes, shapes and contiguity,
pass raw device pointers and the current HIP stream to the library, and
return the output tensor. Every arithmetic step runs in the library's HIP
kernels; PyTorch provides device memory and streams only.

Weight tensors are flat ``torch.uint8`` device tensors (or 2-D, rows of
packed blocks) holding the llama.cpp block bytes described in ``lqmm.h``.

The shared library is loaded on first use; if it has not been built
(``python -m block_quantized_matmul_amd.build``) every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LqmmError", "library_path", "load",
    "lqmm_sgemm", "lqmm_gemv_q4_0", "lqmm_gemv_q4_0_noalloc", "lqmm_gemm_q8_0_f16",
    "lqmm_gemv_q4_k", "lqmm_gemv_q8_0", "lqmm_gemv_q6_k", "lqmm_gemv_q2_k", "lqmm_gemv_q1_0",
    "lqmm_gemv_i4g32",
    "lqmm_gemm_q4_0_f16", "lqmm_gemm_q4_k_f16",
    "lqmm_gemv_workspace_bytes", "lqmm_status_string", "lqmm_version",
    "Q4_0_BLOCK_BYTES", "Q8_0_BLOCK_BYTES", "Q4_K_BLOCK_BYTES", "Q6_K_BLOCK_BYTES",
    "Q2_K_BLOCK_BYTES", "Q1_0_BLOCK_BYTES",
]

Q4_0_BLOCK_BYTES = 18   # 32 weights
Q8_0_BLOCK_BYTES = 34   # 32 weights
Q4_K_BLOCK_BYTES = 144  # 256 weights
Q6_K_BLOCK_BYTES = 210  # 256 weights
Q2_K_BLOCK_BYTES = 84   # 256 weights
Q1_0_BLOCK_BYTES = 6    # 32 weights

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblqmm.so")
_lib = None

# Entry points exported by liblqmm.so (the declarations of include/lqmm.h).
EXPORTS = ("lqmm_sgemm", "lqmm_gemv_q4_0", "lqmm_gemv_q4_0_noalloc", "lqmm_gemm_q8_0_f16",
           "lqmm_gemv_q4_k", "lqmm_gemv_q8_0", "lqmm_gemv_q6_k", "lqmm_gemv_q2_k",
           "lqmm_gemv_q1_0", "lqmm_gemv_i4g32", "lqmm_gemm_q4_0_f16", "lqmm_gemm_q4_k_f16",
           "lqmm_gemv_workspace_bytes", "lqmm_status_string", "lqmm_version")


class LqmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load liblqmm.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"liblqmm.so not found at {_LIB_PATH}; build it with "
            "`python -m block_quantized_matmul_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    lib.lqmm_sgemm.argtypes = [p, p, p, i64, i64, i64, p]
    lib.lqmm_sgemm.restype = st
    for name in ("lqmm_gemv_q4_0", "lqmm_gemv_q4_k", "lqmm_gemv_q8_0", "lqmm_gemv_q6_k",
                 "lqmm_gemv_q2_k", "lqmm_gemv_q1_0"):
        f = getattr(lib, name)
        f.argtypes = [p, p, p, i64, i64, i64, p, sz, p]
        f.restype = st
    lib.lqmm_gemv_i4g32.argtypes = [p, p, p, p, p, i64, i64, i64, p, sz, p]
    lib.lqmm_gemv_i4g32.restype = st
    for name in ("lqmm_gemm_q4_0_f16", "lqmm_gemm_q4_k_f16"):
        f = getattr(lib, name)
        f.argtypes = [p, p, p, i64, i64, i64, p]
        f.restype = st
    lib.lqmm_gemv_q4_0_noalloc.argtypes = [p, p, p, i64, i64, i64, p]
    lib.lqmm_gemv_q4_0_noalloc.restype = st
    lib.lqmm_gemm_q8_0_f16.argtypes = [p, p, p, i64, i64, i64, p]
    lib.lqmm_gemm_q8_0_f16.restype = st
    lib.lqmm_gemv_workspace_bytes.argtypes = [i64, i64, i64]
    lib.lqmm_gemv_workspace_bytes.restype = sz
    lib.lqmm_status_string.argtypes = [ctypes.c_int]
    lib.lqmm_status_string.restype = ctypes.c_char_p
    lib.lqmm_version.argtypes = []
    lib.lqmm_version.restype = ctypes.c_int
    _lib = lib
    return lib


def lqmm_status_string(status: int) -> str:
    return load().lqmm_status_string(int(status)).decode()


def lqmm_version() -> int:
    return load().lqmm_version()


def lqmm_gemv_workspace_bytes(N: int, K: int, batch: int) -> int:
    return load().lqmm_gemv_workspace_bytes(int(N), int(K), int(batch))


def _check(status: int):
    if status != 0:
        raise LqmmError(status, lqmm_status_string(status))


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_tensor(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_device(*ts):
    d = ts[0].device
    for t in ts[1:]:
        if t.device != d:
            raise ValueError("all tensors must be on the same device")
    return d


def lqmm_sgemm(A, B, out=None, stream=None):
    """C = A @ B, fp32, row-major: A (M, K), B (K, N) -> C (M, N)."""
    torch = _torch()
    _dev_tensor(A, torch.float32, "A")
    _dev_tensor(B, torch.float32, "B")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)} B {tuple(B.shape)}")
    M, K = A.shape
    N = B.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _dev_tensor(out, torch.float32, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(A, B, out)
    with torch.cuda.device(A.device):
        _check(load().lqmm_sgemm(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
                                 _stream(stream)))
    return out


# Split-K workspaces the binding provides when the caller passes none: one
# zero-filled buffer per (device, stream), grown on demand. Every completed
# library call leaves the bytes it used zero again, so a buffer stays
# reusable; calls on different streams never share one.
_workspaces = {}


def _default_workspace(device, stream_handle, nbytes):
    torch = _torch()
    key = (device.index, int(stream_handle or 0))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
        # The fill runs on the current stream; make it complete before any
        # other stream uses the buffer (under graph capture the fill is part
        # of the graph, on the capturing stream, and nothing may synchronize).
        if not torch.cuda.is_current_stream_capturing():
            torch.cuda.synchronize(device)
        _workspaces[key] = ws
    return ws


def _gemv(fn, blk, blk_bytes, W, x, N, out, workspace, stream):
    torch = _torch()
    _dev_tensor(W, torch.uint8, "W")
    _dev_tensor(x, torch.float32, "x")
    squeeze = x.dim() == 1
    x2 = x.view(1, -1) if squeeze else x
    if x2.dim() != 2:
        raise ValueError("x must be (K,) or (batch, K)")
    batch, K = x2.shape
    N = int(N)
    if W.numel() != N * (K // blk) * blk_bytes or K % blk:
        raise ValueError(f"W holds {W.numel()} bytes, expected N*K/{blk}*{blk_bytes} "
                         f"for N={N}, K={K}")
    if out is None:
        out = torch.empty((batch, N), dtype=torch.float32, device=x.device)
    _dev_tensor(out, torch.float32, "out")
    if out.numel() != batch * N:
        raise ValueError("out has the wrong size")
    _same_device(W, x, out)
    ws_ptr, ws_bytes = None, 0
    with torch.cuda.device(x.device):
        st = _stream(stream)
        if workspace is None:
            need = load().lqmm_gemv_workspace_bytes(N, K, batch)
            if need:
                workspace = _default_workspace(x.device, st, need)
        elif workspace is False:  # explicitly none: plans that need one are not used
            workspace = None
        if workspace is not None:
            _dev_tensor(workspace, torch.uint8, "workspace")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
        _check(fn(W.data_ptr(), x2.data_ptr(), out.data_ptr(), N, K, batch, ws_ptr, ws_bytes, st))
    return out.view(-1) if squeeze and out.dim() == 2 and out.shape[0] == 1 else out


def lqmm_gemv_q4_0(W, x, N, out=None, workspace=None, stream=None):
    """y = x @ W^T with W an N x K matrix of Q4_0 blocks; x (batch, K) or (K,)
    fp32 -> y (batch, N) (or (N,)) fp32. workspace: a uint8 device tensor
    (zero-filled before first use) for split-K plans; None lets the binding
    provide one per device and stream; False passes none."""
    return _gemv(load().lqmm_gemv_q4_0, 32, Q4_0_BLOCK_BYTES, W, x, N, out, workspace, stream)


def lqmm_gemv_q4_0_noalloc(W, x, N, out=None, stream=None):
    """lqmm_gemv_q4_0 through the allocation-free entry point (split-K plans
    use the library's static per-GPU scratch; calls on one GPU must not
    overlap). ``out`` must be given to avoid the binding's own allocation."""
    torch = _torch()
    _dev_tensor(W, torch.uint8, "W")
    _dev_tensor(x, torch.float32, "x")
    squeeze = x.dim() == 1
    x2 = x.view(1, -1) if squeeze else x
    if x2.dim() != 2:
        raise ValueError("x must be (K,) or (batch, K)")
    batch, K = x2.shape
    N = int(N)
    if K % 32 or W.numel() != N * (K // 32) * Q4_0_BLOCK_BYTES:
        raise ValueError(f"W holds {W.numel()} bytes, expected N*K/32*18 for N={N}, K={K}")
    if out is None:
        out = torch.empty((batch, N), dtype=torch.float32, device=x.device)
    _dev_tensor(out, torch.float32, "out")
    if out.numel() != batch * N:
        raise ValueError("out has the wrong size")
    _same_device(W, x, out)
    with torch.cuda.device(x.device):
        _check(load().lqmm_gemv_q4_0_noalloc(W.data_ptr(), x2.data_ptr(), out.data_ptr(), N, K,
                                             batch, _stream(stream)))
    return out.view(-1) if squeeze and out.dim() == 2 and out.shape[0] == 1 else out


def lqmm_gemv_q4_k(W, x, N, out=None, workspace=None, stream=None):
    """y = x @ W^T with W an N x K matrix of Q4_K super-blocks."""
    return _gemv(load().lqmm_gemv_q4_k, 256, Q4_K_BLOCK_BYTES, W, x, N, out, workspace, stream)


def _gemm(fn, blk, blk_bytes, W, X, N, out, stream):
    torch = _torch()
    _dev_tensor(W, torch.uint8, "W")
    _dev_tensor(X, torch.float16, "X")
    if X.dim() != 2:
        raise ValueError("X must be (M, K)")
    M, K = X.shape
    N = int(N)
    if K % blk or W.numel() != N * (K // blk) * blk_bytes:
        raise ValueError(f"W holds {W.numel()} bytes, expected N*K/{blk}*{blk_bytes} "
                         f"for N={N}, K={K}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _dev_tensor(out, torch.float16, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _same_device(W, X, out)
    with torch.cuda.device(X.device):
        _check(fn(W.data_ptr(), X.data_ptr(), out.data_ptr(), M, N, K, _stream(stream)))
    return out


def lqmm_gemm_q8_0_f16(W, X, N, out=None, stream=None):
    """Y = X @ W^T: X (M, K) fp16, W an N x K matrix of Q8_0 blocks ->
    Y (M, N) fp16 (fp32 accumulation)."""
    return _gemm(load().lqmm_gemm_q8_0_f16, 32, Q8_0_BLOCK_BYTES, W, X, N, out, stream)


def lqmm_gemm_q4_0_f16(W, X, N, out=None, stream=None):
    """Y = X @ W^T with W an N x K matrix of Q4_0 blocks (prefill)."""
    return _gemm(load().lqmm_gemm_q4_0_f16, 32, Q4_0_BLOCK_BYTES, W, X, N, out, stream)


def lqmm_gemm_q4_k_f16(W, X, N, out=None, stream=None):
    """Y = X @ W^T with W an N x K matrix of Q4_K super-blocks (prefill)."""
    return _gemm(load().lqmm_gemm_q4_k_f16, 256, Q4_K_BLOCK_BYTES, W, X, N, out, stream)


def lqmm_gemv_q8_0(W, x, N, out=None, workspace=None, stream=None):
    """y = x @ W^T with W an N x K matrix of Q8_0 blocks (decode)."""
    return _gemv(load().lqmm_gemv_q8_0, 32, Q8_0_BLOCK_BYTES, W, x, N, out, workspace, stream)


def lqmm_gemv_q6_k(W, x, N, out=None, workspace=None, stream=None):
    """y = x @ W^T with W an N x K matrix of Q6_K super-blocks (decode)."""
    return _gemv(load().lqmm_gemv_q6_k, 256, Q6_K_BLOCK_BYTES, W, x, N, out, workspace, stream)


def lqmm_gemv_q2_k(W, x, N, out=None, workspace=None, stream=None):
    """y = x @ W^T with W an N x K matrix of Q2_K super-blocks (decode)."""
    return _gemv(load().lqmm_gemv_q2_k, 256, Q2_K_BLOCK_BYTES, W, x, N, out, workspace, stream)


def lqmm_gemv_q1_0(W, x, N, out=None, workspace=None, stream=None):
    """y = x @ W^T with W an N x K matrix of 1-bit q1_0 blocks (decode)."""
    return _gemv(load().lqmm_gemv_q1_0, 32, Q1_0_BLOCK_BYTES, W, x, N, out, workspace, stream)


def lqmm_gemv_i4g32(Wq, scales, zeros, x, N, out=None, workspace=None, stream=None):
    """y = x @ W^T for the int4 group-32 layout: Wq int32/uint32-packed codes
    (N*K/8 words, as a torch.int32 tensor), scales and zeros float32
    (N, K/32)."""
    torch = _torch()
    _dev_tensor(Wq, torch.int32, "Wq")
    _dev_tensor(scales, torch.float32, "scales")
    _dev_tensor(zeros, torch.float32, "zeros")
    _dev_tensor(x, torch.float32, "x")
    squeeze = x.dim() == 1
    x2 = x.view(1, -1) if squeeze else x
    if x2.dim() != 2:
        raise ValueError("x must be (K,) or (batch, K)")
    batch, K = x2.shape
    N = int(N)
    if K % 32 or Wq.numel() != N * K // 8 or scales.numel() != N * K // 32 \
            or zeros.numel() != N * K // 32:
        raise ValueError(f"int4 arrays do not match N={N}, K={K}")
    if out is None:
        out = torch.empty((batch, N), dtype=torch.float32, device=x.device)
    _dev_tensor(out, torch.float32, "out")
    if out.numel() != batch * N:
        raise ValueError("out has the wrong size")
    _same_device(Wq, scales, zeros, x, out)
    ws_ptr, ws_bytes = None, 0
    with torch.cuda.device(x.device):
        st = _stream(stream)
        if workspace is None:
            need = load().lqmm_gemv_workspace_bytes(N, K, batch)
            if need:
                workspace = _default_workspace(x.device, st, need)
        elif workspace is False:
            workspace = None
        if workspace is not None:
            _dev_tensor(workspace, torch.uint8, "workspace")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
        _check(load().lqmm_gemv_i4g32(Wq.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                      x2.data_ptr(), out.data_ptr(), N, K, batch, ws_ptr,
                                      ws_bytes, st))
    return out.view(-1) if squeeze and out.dim() == 2 and out.shape[0] == 1 else out
