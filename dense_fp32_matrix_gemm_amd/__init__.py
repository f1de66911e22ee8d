"""FP32 dense GEMM for AMD Instinct MI355X (gfx950).

The product runs in hand-written HIP kernels behind a C ABI
(``include/gemm_f32.h``, library ``libgemm_f32.so``).  This package is the
thin Python side: the raw ABI calls (``gemm_f32``, ``gemm_f32_naive``,
``gemm_f32_ex``, ``gemm_f32_strerror``, ``gemm_f32_version``) and ``matmul``,
which takes PyTorch device tensors, reads their pointers, strides and the
current stream, and calls the library.  PyTorch owns memory and streams.
"""

from __future__ import annotations

from ._lib import (ALGOS, LibraryNotBuilt, gemm_f32, gemm_f32_ex, gemm_f32_naive,
                   gemm_f32_strerror, gemm_f32_version, library_path, load)

__all__ = ["ALGOS", "GemmError", "LibraryNotBuilt", "gemm_f32", "gemm_f32_ex",
           "gemm_f32_naive", "gemm_f32_strerror", "gemm_f32_version", "library_path",
           "load", "matmul", "operand_layout"]


class GemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"gemm_f32 status {status}: {gemm_f32_strerror(status)}")


def operand_layout(t) -> tuple:
    """(trans, ld) describing a 2-D tensor view for the row-major ABI.

    A row-major view (stride(1) == 1) is passed as is with ld = stride(0); a
    transposed view of a row-major array (stride(0) == 1) is passed as the
    stored array with the transpose flag, so no copy is made.
    """
    if t.dim() != 2:
        raise ValueError("matmul operands are 2-D")
    rows, cols = t.shape
    s0, s1 = t.stride()
    if s1 == 1 or cols <= 1:
        return 0, max(s0, cols, 1) if rows > 1 else max(cols, 1)
    if s0 == 1 or rows <= 1:
        return 1, max(s1, rows, 1) if cols > 1 else max(rows, 1)
    raise ValueError("operand must have unit stride in one dimension")


def matmul(a, b, out=None, algo: str = "auto", stream=None):
    """out = a @ b for float32 CUDA(HIP) tensors, computed by the HIP library.

    ``a`` is M x K and ``b`` is K x N, each row-major or a transposed view;
    ``out`` (allocated if None) is M x N with unit column stride.  Runs on
    ``stream`` (default: the current PyTorch stream) and does not synchronise.
    """
    import torch

    if a.dtype != torch.float32 or b.dtype != torch.float32:
        raise TypeError("matmul takes float32 tensors")
    if not (a.is_cuda and b.is_cuda):
        raise ValueError("matmul takes device tensors")
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    if out.shape != (M, N) or out.dtype != torch.float32 or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be an M x N float32 tensor with unit column stride")
    ta, lda = operand_layout(a)
    tb, ldb = operand_layout(b)
    ldc = max(out.stride(0), N, 1) if M > 1 else max(N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    st = gemm_f32_ex(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc,
                     ta, tb, stream, ALGOS[algo])
    if st != 0:
        raise GemmError(st)
    return out
