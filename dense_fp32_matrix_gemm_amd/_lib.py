"""ctypes binding of ``libgemm_f32.so`` (declarations: include/gemm_f32.h and
include/rows_f32.h).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  Loading fails loudly if the library has not been built; there
is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

ALGO_AUTO, ALGO_MFMA, ALGO_FMA, ALGO_TILED, ALGO_NAIVE = 0, 1, 2, 3, 4
ALGO_MFMA_TILE128, ALGO_MFMA_TILE64, ALGO_MFMA_TILE256, ALGO_MFMA_WIDE = 5, 6, 7, 8
ALGOS = {"auto": ALGO_AUTO, "mfma": ALGO_MFMA, "fma": ALGO_FMA, "tiled": ALGO_TILED,
         "naive": ALGO_NAIVE, "mfma128": ALGO_MFMA_TILE128, "mfma64": ALGO_MFMA_TILE64,
         "mfma256": ALGO_MFMA_TILE256, "mfmawide": ALGO_MFMA_WIDE}
# gemm_f32_plan codes (enum gemm_f32_plan_code)
PLANS = {0: "nothing", 1: "zero-fill", 2: "mfma-256x256", 3: "mfma-256x128", 4: "mfma-128x128",
         5: "mfma-128x128-one-round", 6: "mfma-128x128-kk", 7: "mfma-128x64", 8: "mfma-64x64",
         9: "mfma-64x64-pair"}

# Every symbol include/gemm_f32.h declares, with (restype, argtypes).
_i64, _ptr, _int, _flt = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_GEMM_ARGS = [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int, _ptr]
SIGNATURES = {
    "gemm_f32": (_int, _GEMM_ARGS),
    "gemm_f32_naive": (_int, _GEMM_ARGS),
    "gemm_f32_ex": (_int, _GEMM_ARGS + [_int]),
    "gemm_f32_strided_batched": (_int, [_i64, _i64, _i64, _ptr, _i64, _i64, _ptr, _i64, _i64,
                                        _ptr, _i64, _i64, _i64, _int, _int, _ptr]),
    "gemm_f32_bias_act": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int,
                                 _ptr, _int, _ptr]),
    "gemm_f32_bf16": (_int, _GEMM_ARGS),
    "gemm_f32_pack_bf16": (_int, [_i64, _i64, _ptr, _i64, _int, _ptr, _i64, _ptr]),
    "gemm_f32_bf16_packed": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr]),
    "gemm_f32_splitk": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _int,
                               _i64, _ptr, _i64, _ptr]),
    "gemm_f32_splitk_noalloc": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64, _int,
                                       _int, _i64, _ptr]),
    "gemm_f32_splitk_workspace_size": (_i64, [_i64, _i64, _i64, _i64]),
    "gemm_f32_strerror": (ctypes.c_char_p, [_int]),
    "rows_softmax_f32": (_int, [_i64, _i64, _i64, _int, _flt, _ptr, _i64, _ptr, _i64, _ptr]),
    "rows_softmax_backward_f32": (_int, [_i64, _i64, _flt, _ptr, _i64, _ptr, _i64, _ptr, _i64, _ptr]),
    "rows_normalize_f32": (_int, [_i64, _i64, _flt, _ptr, _i64, _ptr, _i64, _ptr]),
    "rows_normalize_backward_f32": (_int, [_i64, _i64, _flt, _ptr, _i64, _ptr, _i64, _ptr, _i64,
                                           _ptr]),
    "gemm_f32_plan": (_int, [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _i64, _int, _int, _i64, _i64, _i64]),
    "gemm_f32_version": (_int, []),
}

_lock = threading.Lock()
_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


def library_path() -> str:
    return os.environ.get("GEMM_F32_LIBRARY", _build.LIBRARY)


def load() -> ctypes.CDLL:
    """The loaded library (loaded once per process)."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise LibraryNotBuilt(
                    f"{path} is missing: build it with `python -m dense_fp32_matrix_gemm_amd.build` "
                    "(or __graft_entry__.build()); there is no non-HIP fallback")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def _call(name, *args) -> int:
    return int(getattr(load(), name)(*args))


def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream) -> int:
    """C = op(A) . op(B); pointers are device addresses (ints), stream a hipStream_t (int or None)."""
    return _call("gemm_f32", M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream)


def gemm_f32_naive(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream) -> int:
    return _call("gemm_f32_naive", M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream)


def gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream, algo) -> int:
    return _call("gemm_f32_ex", M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream, algo)


def gemm_f32_strided_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                             batch, transA, transB, stream) -> int:
    return _call("gemm_f32_strided_batched", M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc,
                 strideC, batch, transA, transB, stream)


ACT_NONE, ACT_GELU = 0, 1


def gemm_f32_bias_act(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, bias, act, stream) -> int:
    return _call("gemm_f32_bias_act", M, N, K, A, lda, B, ldb, C, ldc, transA, transB, bias, act,
                 stream)


def gemm_f32_bf16(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream) -> int:
    """C = op(A) . op(B) with operands rounded to bf16, FP32 sums and output."""
    return _call("gemm_f32_bf16", M, N, K, A, lda, B, ldb, C, ldc, transA, transB, stream)


def gemm_f32_pack_bf16(rows, cols, src, lds, trans, dst, ldd, stream) -> int:
    """dst = bf16 bit patterns of op(src) (rows x cols, leading dimension ldd)."""
    return _call("gemm_f32_pack_bf16", rows, cols, src, lds, trans, dst, ldd, stream)


def gemm_f32_bf16_packed(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    """C = A . B^T on packed bf16 operands (A M x K, B N x K), FP32 sums and C."""
    return _call("gemm_f32_bf16_packed", M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, splits, workspace,
                    workspace_bytes, stream) -> int:
    """C = op(A) . op(B) as ``splits`` partial products over runs of k plus
    their fixed-order sum; ``workspace`` is a device address of at least
    ``gemm_f32_splitk_workspace_size`` bytes (0/None when that is 0)."""
    return _call("gemm_f32_splitk", M, N, K, A, lda, B, ldb, C, ldc, transA, transB, splits,
                 workspace, workspace_bytes, stream)


# GEMM_F32_SPLITK_SCRATCH_BYTES: the partial products gemm_f32_splitk_noalloc holds
SPLITK_SCRATCH_BYTES = 64 << 20


def gemm_f32_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, transA, transB, splits,
                            stream) -> int:
    """gemm_f32_splitk with the partials in the library's own per-GPU scratch
    (at most SPLITK_SCRATCH_BYTES); allocates nothing."""
    return _call("gemm_f32_splitk_noalloc", M, N, K, A, lda, B, ldb, C, ldc, transA, transB,
                 splits, stream)


def gemm_f32_splitk_workspace_size(M, N, K, splits) -> int:
    return int(load().gemm_f32_splitk_workspace_size(M, N, K, splits))


def rows_softmax_f32(rows, width, queries, causal, scale, x, ldx, y, ldy, stream) -> int:
    """Causal (or plain) softmax of scale * x along each row (include/rows_f32.h)."""
    return _call("rows_softmax_f32", rows, width, queries, causal, scale, x, ldx, y, ldy, stream)


def rows_softmax_backward_f32(rows, width, scale, y, ldy, dy, lddy, dx, lddx, stream) -> int:
    return _call("rows_softmax_backward_f32", rows, width, scale, y, ldy, dy, lddy, dx, lddx,
                 stream)


def rows_normalize_f32(rows, n, eps, x, ldx, y, ldy, stream) -> int:
    return _call("rows_normalize_f32", rows, n, eps, x, ldx, y, ldy, stream)


def rows_normalize_backward_f32(rows, n, eps, x, ldx, dy, lddy, dx, lddx, stream) -> int:
    return _call("rows_normalize_backward_f32", rows, n, eps, x, ldx, dy, lddy, dx, lddx, stream)


def gemm_f32_strerror(status: int) -> str:
    return load().gemm_f32_strerror(int(status)).decode()


def gemm_f32_version() -> int:
    return _call("gemm_f32_version")


def gemm_f32_plan(M, N, K, A, lda, B, ldb, ldc, transA, transB, strideA=0, strideB=0, batch=1) -> int:
    return _call("gemm_f32_plan", M, N, K, A, lda, B, ldb, ldc, transA, transB, strideA, strideB, batch)
