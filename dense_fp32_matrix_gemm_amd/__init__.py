"""FP32 dense GEMM for AMD Instinct MI355X (gfx950).

The product runs in hand-written HIP kernels behind a C ABI
(``include/gemm_f32.h`` and ``include/rows_f32.h``, library
``libgemm_f32.so``).  This package is the thin Python side: the raw ABI
calls under their C names, and tensor-level helpers (``matmul``, ``bmm``,
``linear``, ``matmul_splitk``, ``matmul_bf16``, ``pack_bf16``,
``matmul_bf16_packed``, ``softmax``, ``softmax_backward``, ``normalize``,
``normalize_backward``) that take PyTorch device tensors,
read their pointers, strides and the current stream, and call the library.
PyTorch owns memory and streams; every step of the computation runs in the
library's kernels.
"""

from __future__ import annotations

from ._lib import (ACT_GELU, ACT_NONE, ALGOS, PLANS, LibraryNotBuilt, gemm_f32, gemm_f32_bf16,
                   gemm_f32_bf16_packed, gemm_f32_bias_act, gemm_f32_pack_bf16,
                   gemm_f32_ex, gemm_f32_naive, gemm_f32_plan, gemm_f32_splitk,
                   gemm_f32_splitk_noalloc,
                   gemm_f32_splitk_workspace_size,
                   gemm_f32_strerror, gemm_f32_strided_batched, gemm_f32_version, library_path,
                   load, rows_normalize_backward_f32, rows_normalize_f32,
                   rows_softmax_backward_f32, rows_softmax_f32)

__all__ = ["ACT_GELU", "ACT_NONE", "ALGOS", "PLANS", "GemmError", "LibraryNotBuilt", "bmm", "gemm_f32",
           "gemm_f32_bf16", "gemm_f32_bf16_packed", "gemm_f32_bias_act", "gemm_f32_ex",
           "gemm_f32_pack_bf16", "linear", "matmul_bf16", "matmul_bf16_packed", "pack_bf16",
           "gemm_f32_naive", "gemm_f32_plan", "gemm_f32_splitk", "gemm_f32_splitk_noalloc",
           "gemm_f32_splitk_workspace_size",
           "gemm_f32_strerror", "gemm_f32_strided_batched",
           "gemm_f32_version", "library_path", "load", "matmul", "matmul_splitk",
           "normalize", "normalize_backward", "operand_layout", "rows_normalize_backward_f32",
           "rows_normalize_f32", "rows_softmax_backward_f32", "rows_softmax_f32", "softmax",
           "softmax_backward"]


class GemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"gemm_f32 status {status}: {gemm_f32_strerror(status)}")


def _check_tensor(t, name, device=None, dims=2, dtype=None):
    """A float32 (or ``dtype``) tensor on the GPU (and on ``device`` if
    given): the library dereferences its pointer on the device, so anything
    else is refused here."""
    import torch
    dtype = torch.float32 if dtype is None else dtype
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError(f"{name} must be a {str(dtype).replace('torch.', '')} tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands on {device}")
    if t.dim() != dims:
        raise ValueError(f"{name} must be {dims}-D")


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

    _check_tensor(a, "a")
    _check_tensor(b, "b", a.device)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _check_tensor(out, "out", a.device)
    if out.shape != (M, N) or (N > 1 and out.stride(1) != 1):
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


def bmm(a, b, out=None, stream=None):
    """out[i] = a[i] @ b[i] for 3-D float32 device tensors, one strided-batched call.

    ``a`` is (batch, M, K) and ``b`` is (batch, K, N); each may be a view with
    its last two dimensions transposed (e.g. ``k.transpose(1, 2)``), mapped to
    the transpose flag without a copy, and a batch stride of 0 (an expanded
    operand) shares one matrix across the batch.
    """
    import torch

    _check_tensor(a, "a", dims=3)
    _check_tensor(b, "b", a.device, dims=3)
    batch, M, K = a.shape
    if b.shape[0] != batch or b.shape[1] != K:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not chain")
    N = b.shape[2]
    if out is None:
        out = torch.empty((batch, M, N), dtype=torch.float32, device=a.device)
    _check_tensor(out, "out", a.device, dims=3)
    if out.shape != (batch, M, N) or (N > 1 and out.stride(2) != 1):
        raise ValueError("out must be (batch, M, N) with unit column stride")
    ta, lda = operand_layout(a[0]) if batch else (0, max(K, 1))
    tb, ldb = operand_layout(b[0]) if batch else (0, max(N, 1))
    ldc = max(out.stride(1), N, 1) if M > 1 else max(N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    st = gemm_f32_strided_batched(M, N, K, a.data_ptr(), lda, a.stride(0), b.data_ptr(), ldb,
                                  b.stride(0), out.data_ptr(), ldc, out.stride(0), batch,
                                  ta, tb, stream)
    if st != 0:
        raise GemmError(st)
    return out


def linear(x, w, bias=None, activation=None, out=None, stream=None):
    """act(x @ w + bias) in one fused call (``activation``: None or "gelu").

    ``x`` is M x K and ``w`` is K x N (either may be a transposed view);
    ``bias`` is None or a length-N float32 device tensor.
    """
    import torch

    _check_tensor(x, "x")
    _check_tensor(w, "w", x.device)
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(x.shape)} @ {tuple(w.shape)}")
    act = {None: ACT_NONE, "gelu": ACT_GELU}[activation]
    if bias is not None:
        _check_tensor(bias, "bias", x.device, dims=1)
        if bias.shape != (N,) or (N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous float32 vector of N entries")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_tensor(out, "out", x.device)
    if out.shape != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be an M x N float32 tensor with unit column stride")
    ta, lda = operand_layout(x)
    tb, ldb = operand_layout(w)
    ldc = max(out.stride(0), N, 1) if M > 1 else max(N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = gemm_f32_bias_act(M, N, K, x.data_ptr(), lda, w.data_ptr(), ldb, out.data_ptr(), ldc,
                           ta, tb, None if bias is None else bias.data_ptr(), act, stream)
    if st != 0:
        raise GemmError(st)
    return out


def matmul_splitk(a, b, splits: int, out=None, workspace=None, stream=None):
    """out = a @ b as ``splits`` partial products over runs of k and their sum
    (gemm_f32_splitk).  ``workspace`` is a float32 device tensor of at least
    gemm_f32_splitk_workspace_size bytes; if None one is allocated here."""
    import torch

    _check_tensor(a, "a")
    _check_tensor(b, "b", a.device)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _check_tensor(out, "out", a.device)
    if out.shape != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be an M x N float32 tensor with unit column stride")
    need = gemm_f32_splitk_workspace_size(M, N, K, splits)
    if need < 0:
        raise GemmError(int(need))
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=a.device)
    if workspace is not None:
        _check_tensor(workspace, "workspace", a.device, dims=workspace.dim())
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ta, lda = operand_layout(a)
    tb, ldb = operand_layout(b)
    ldc = max(out.stride(0), N, 1) if M > 1 else max(N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    st = gemm_f32_splitk(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc,
                         ta, tb, splits, ws_ptr, ws_bytes, stream)
    if st != 0:
        raise GemmError(st)
    return out


# ------------------------------------------------------------ mixed precision ---

def _gemm_out(out, M, N, device):
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=device)
    _check_tensor(out, "out", device)
    if out.shape != (M, N) or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be an M x N float32 tensor with unit column stride")
    return out, (max(out.stride(0), N, 1) if M > 1 else max(N, 1))


def matmul_bf16(a, b, out=None, stream=None):
    """out = a @ b with each operand element rounded to bf16 on the way in
    and FP32 sums (gemm_f32_bf16); a, b and out are float32 tensors as for
    ``matmul``."""
    _check_tensor(a, "a")
    _check_tensor(b, "b", a.device)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(a.shape)} @ {tuple(b.shape)}")
    out, ldc = _gemm_out(out, M, N, a.device)
    ta, lda = operand_layout(a)
    tb, ldb = operand_layout(b)
    st = gemm_f32_bf16(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc,
                       ta, tb, _stream(a, stream))
    if st != 0:
        raise GemmError(st)
    return out


def pack_bf16(x, out=None, stream=None):
    """A bf16 copy of the float32 matrix ``x`` (row-major or a transposed
    view), rounded to nearest with ties to even (gemm_f32_pack_bf16).

    The result is a row-major bf16 view whose rows are padded to a multiple
    of 8 elements, the layout ``matmul_bf16_packed`` copies fastest.  To use
    a @ b on packed operands: ``matmul_bf16_packed(pack_bf16(a),
    pack_bf16(b.t()))``.  ``out`` (optional) is a bf16 tensor of x's shape
    with unit column stride.
    """
    import torch

    _check_tensor(x, "x")
    rows, cols = x.shape
    trans, lds = operand_layout(x)
    if out is None:
        ld = max(8, (cols + 7) // 8 * 8)
        out = torch.empty((rows, ld), dtype=torch.bfloat16, device=x.device)[:, :cols]
    _check_tensor(out, "out", x.device, dtype=torch.bfloat16)
    if out.shape != x.shape or (cols > 1 and out.stride(1) != 1):
        raise ValueError("out must be a bf16 tensor of x's shape with unit column stride")
    ldd = max(out.stride(0), cols, 1) if rows > 1 else max(cols, 1)
    st = gemm_f32_pack_bf16(rows, cols, x.data_ptr(), lds, trans, out.data_ptr(), ldd,
                            _stream(x, stream))
    if st != 0:
        raise GemmError(st)
    return out


def matmul_bf16_packed(a, b, out=None, stream=None):
    """out = a @ b.T for packed bf16 operands (gemm_f32_bf16_packed): ``a`` is
    M x K and ``b`` N x K, both bf16 with unit column stride (as
    ``pack_bf16`` makes them); the products are summed in FP32 into the
    float32 M x N ``out``."""
    import torch

    _check_tensor(a, "a", dtype=torch.bfloat16)
    _check_tensor(b, "b", a.device, dtype=torch.bfloat16)
    M, K = a.shape
    N, K2 = b.shape
    if K2 != K:
        raise ValueError(f"a and b must have the same number of columns: {tuple(a.shape)}, {tuple(b.shape)}")
    for t, name in ((a, "a"), (b, "b")):
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit column stride")
    lda = max(a.stride(0), K, 1) if M > 1 else max(K, 1)
    ldb = max(b.stride(0), K, 1) if N > 1 else max(K, 1)
    out, ldc = _gemm_out(out, M, N, a.device)
    st = gemm_f32_bf16_packed(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc,
                              _stream(a, stream))
    if st != 0:
        raise GemmError(st)
    return out


# ------------------------------------------------------------ row operations ---

def _row_major(t, name, like=None):
    """Leading dimension of a 2-D row-major device tensor; ``like``: a tensor
    it must match in shape and device."""
    _check_tensor(t, name, None if like is None else like.device)
    if like is not None and t.shape != like.shape:
        raise ValueError(f"{name} must have shape {tuple(like.shape)}, not {tuple(t.shape)}")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return max(t.stride(0), cols, 1) if rows > 1 else max(cols, 1)


def _out_like(x, out):
    import torch
    return torch.empty_like(x, memory_format=torch.contiguous_format) if out is None else out


def _stream(x, stream):
    import torch
    return torch.cuda.current_stream(x.device).cuda_stream if stream is None else stream


def softmax(x, scale: float = 1.0, queries=None, causal: bool = True, out=None, stream=None):
    """Softmax of scale * x along rows; causal: rows are groups of ``queries``
    query rows (default: the row length) masking the future (rows_softmax_f32)."""
    rows, width = x.shape
    out = _out_like(x, out)
    q = width if queries is None else queries
    st = rows_softmax_f32(rows, width, q, int(causal), scale, x.data_ptr(), _row_major(x, "x"),
                          out.data_ptr(), _row_major(out, "out", x), _stream(x, stream))
    if st != 0:
        raise GemmError(st)
    return out


def softmax_backward(y, dy, scale: float = 1.0, out=None, stream=None):
    rows, width = y.shape
    out = _out_like(y, out)
    st = rows_softmax_backward_f32(rows, width, scale, y.data_ptr(), _row_major(y, "y"),
                                   dy.data_ptr(), _row_major(dy, "dy", y), out.data_ptr(),
                                   _row_major(out, "out", y), _stream(y, stream))
    if st != 0:
        raise GemmError(st)
    return out


def normalize(x, eps: float = 1e-5, out=None, stream=None):
    rows, n = x.shape
    out = _out_like(x, out)
    st = rows_normalize_f32(rows, n, eps, x.data_ptr(), _row_major(x, "x"), out.data_ptr(),
                            _row_major(out, "out", x), _stream(x, stream))
    if st != 0:
        raise GemmError(st)
    return out


def normalize_backward(x, dy, eps: float = 1e-5, out=None, stream=None):
    rows, n = x.shape
    out = _out_like(x, out)
    st = rows_normalize_backward_f32(rows, n, eps, x.data_ptr(), _row_major(x, "x"),
                                     dy.data_ptr(), _row_major(dy, "dy", x), out.data_ptr(),
                                     _row_major(out, "out", x), _stream(x, stream))
    if st != 0:
        raise GemmError(st)
    return out
