"""CPU oracle for the FP32 GEMM C = op(A) . op(B).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The HIP library neither imports nor links anything here, and this
package imports nothing from the HIP library.

``gemm_ref`` returns the plain definition of the product (a k-ordered double
precision sum per output element, see ``gemm_ref.c``) as a float64 array.
``schedule`` emulates the memory-access schedules the pages count, to pin
the operation and traffic figures the benchmark divides by.

Parity status of each function is recorded in its docstring; every function
here is pinned by ``tests/test_oracle_pins.py`` or ``tests/test_counts.py``.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import numpy as np

from . import build as _build

_lock = threading.Lock()
_libs = {}

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def load(path: Optional[str] = None) -> "Oracle":
    """Load (building first if absent) the oracle library at ``path``."""
    path = path or _build.LIBRARY
    with _lock:
        if path not in _libs:
            if not os.path.exists(path):
                if path != _build.LIBRARY:
                    raise FileNotFoundError(path)
                _build.build()
            _libs[path] = Oracle(path)
        return _libs[path]


def _as_stored(x: np.ndarray) -> np.ndarray:
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("operands are 2-D float32 arrays of shape (rows, ld)")
    return np.ascontiguousarray(x)


class Oracle:
    """ctypes view of one built oracle library."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.gemm_ref_f64.restype = ctypes.c_int
        lib.gemm_ref_f64.argtypes = [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64,
                                     _ptr, _i64, ctypes.c_int, ctypes.c_int, _ptr]
        lib.gemm_ref_f64_entries.restype = ctypes.c_int
        lib.gemm_ref_f64_entries.argtypes = [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64,
                                             ctypes.c_int, ctypes.c_int, _i64,
                                             _ptr, _ptr, _ptr]
        lib.gemm_ref_epilogue.restype = ctypes.c_int
        lib.gemm_ref_epilogue.argtypes = [_i64, _i64, _ptr, _i64, _ptr, ctypes.c_int]
        lib.gemm_ref_f64_bf16.restype = ctypes.c_int
        lib.gemm_ref_f64_bf16.argtypes = [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64,
                                          _ptr, _i64, ctypes.c_int, ctypes.c_int]
        lib.gemm_ref_f64_bf16_entries.restype = ctypes.c_int
        lib.gemm_ref_f64_bf16_entries.argtypes = lib.gemm_ref_f64_entries.argtypes
        lib.gemm_ref_round_bf16.restype = None
        lib.gemm_ref_round_bf16.argtypes = [_i64, _ptr, _ptr]
        lib.gemm_ref_threads.restype = ctypes.c_int
        lib.gemm_ref_threads.argtypes = []
        self._lib = lib

    def threads(self) -> int:
        return int(self._lib.gemm_ref_threads())

    def gemm(self, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
             transA: int = 0, transB: int = 0,
             with_stats: bool = False):
        """C = op(A) . op(B) in float64, shape (M, N).

        ``A`` and ``B`` are stored matrices of shape (rows, ld) as produced by
        ``gemm_inputs`` (the leading dimension is the array's second extent).
        With ``with_stats`` also returns (multiply-adds, operand reads).
        Pinned: identity, all-ones, rank-1, brute force against exact
        rationals, numpy float64 matmul.
        """
        A = _as_stored(A)
        B = _as_stored(B)
        C = np.zeros((M, max(N, 1)), dtype=np.float64)
        stats = np.zeros(2, dtype=np.int64)
        rc = self._lib.gemm_ref_f64(M, N, K, A.ctypes.data, A.shape[1],
                                    B.ctypes.data, B.shape[1], C.ctypes.data,
                                    C.shape[1], int(transA), int(transB),
                                    stats.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (status {rc})")
        C = C[:, :N]
        if with_stats:
            return C, (int(stats[0]), int(stats[1]))
        return C

    def round_bf16(self, x: np.ndarray) -> np.ndarray:
        """Each float32 element rounded to the nearest bf16 (ties to even),
        returned as float32.  Pinned: hand-worked ties and carries, an exact
        rational rounding, torch's CPU bfloat16 conversion."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty_like(x)
        self._lib.gemm_ref_round_bf16(x.size, x.ctypes.data, out.ctypes.data)
        return out

    def gemm_bf16(self, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
                  transA: int = 0, transB: int = 0) -> np.ndarray:
        """Mixed precision: sum_k bf16(opA(i,k)) * bf16(opB(k,j)) in float64, (M, N).

        Pinned: small-integer exactness, identity, brute force against exact
        rationals of independently rounded operands, numpy float64 matmul of
        torch-rounded operands.
        """
        A = _as_stored(A)
        B = _as_stored(B)
        C = np.zeros((M, max(N, 1)), dtype=np.float64)
        rc = self._lib.gemm_ref_f64_bf16(M, N, K, A.ctypes.data, A.shape[1], B.ctypes.data,
                                         B.shape[1], C.ctypes.data, C.shape[1], int(transA),
                                         int(transB))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (status {rc})")
        return C[:, :N]

    def entries_bf16(self, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
                     transA: int, transB: int, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
        """Selected entries of ``gemm_bf16``.  Pinned against ``gemm_bf16``."""
        A = _as_stored(A)
        B = _as_stored(B)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows and cols differ in length")
        out = np.empty(rows.shape, dtype=np.float64)
        rc = self._lib.gemm_ref_f64_bf16_entries(M, N, K, A.ctypes.data, A.shape[1],
                                                 B.ctypes.data, B.shape[1], int(transA),
                                                 int(transB), rows.size, rows.ctypes.data,
                                                 cols.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (status {rc})")
        return out

    def epilogue(self, C: np.ndarray, bias: Optional[np.ndarray] = None, act: int = 0) -> np.ndarray:
        """act(C + bias) in float64 (a new array); C is (M, N) float64, bias N float32.

        act 0: identity; act 1: GELU, x * Phi(x).  Pinned: normal-distribution
        values, gelu(x) - gelu(-x) = x, limits, scipy's erf.
        """
        out = np.ascontiguousarray(C, dtype=np.float64).copy()
        M, N = out.shape
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        if b is not None and b.shape != (N,):
            raise ValueError("bias has N entries")
        rc = self._lib.gemm_ref_epilogue(M, N, out.ctypes.data, max(N, 1),
                                         None if b is None else b.ctypes.data, int(act))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (status {rc})")
        return out

    def entries(self, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
                transA: int, transB: int, rows: np.ndarray,
                cols: np.ndarray) -> np.ndarray:
        """C[rows[t], cols[t]] for each t, in float64.  Same definition as ``gemm``.

        Pinned against ``gemm`` entry by entry and by the same closed forms.
        """
        A = _as_stored(A)
        B = _as_stored(B)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows and cols differ in length")
        out = np.empty(rows.shape, dtype=np.float64)
        rc = self._lib.gemm_ref_f64_entries(M, N, K, A.ctypes.data, A.shape[1],
                                            B.ctypes.data, B.shape[1], int(transA),
                                            int(transB), rows.size, rows.ctypes.data,
                                            cols.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (status {rc})")
        return out


def gemm_ref_batched(A: np.ndarray, B: np.ndarray, M: int, N: int, K: int, transA: int,
                     transB: int, lda: int, stride_a: int, ldb: int, stride_b: int,
                     batch: int) -> np.ndarray:
    """The strided-batched product, by definition: for each b, the plain
    product of the stored matrices starting b*stride floats into the flat
    buffers A and B.  Returns float64 (batch, M, N).

    Pinned against a single product of block-diagonal matrices
    (tests/test_oracle_pins.py).
    """
    orc = load()
    A = np.ascontiguousarray(A, dtype=np.float32).reshape(-1)
    B = np.ascontiguousarray(B, dtype=np.float32).reshape(-1)
    a_rows = K if transA else M
    b_rows = N if transB else K
    out = np.zeros((batch, M, N), dtype=np.float64)
    for b in range(batch):
        a = A[b * stride_a: b * stride_a + a_rows * lda].reshape(a_rows, lda) if a_rows else \
            np.zeros((0, lda), np.float32)
        bb = B[b * stride_b: b * stride_b + b_rows * ldb].reshape(b_rows, ldb) if b_rows else \
            np.zeros((0, ldb), np.float32)
        out[b] = orc.gemm(a, bb, M, N, K, transA, transB)
    return out


def gemm_ref(A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
             transA: int = 0, transB: int = 0) -> np.ndarray:
    """Module-level shorthand for ``load().gemm(...)``."""
    return load().gemm(A, B, M, N, K, transA, transB)


def gemm_ref_entries(A, B, M, N, K, transA, transB, rows, cols) -> np.ndarray:
    """Module-level shorthand for ``load().entries(...)``."""
    return load().entries(A, B, M, N, K, transA, transB, rows, cols)


def tolerance(C_ref: np.ndarray, K: int) -> Tuple[np.ndarray, float]:
    """The acceptance bounds for an FP32 result against the float64 oracle.

    Elementwise: |C_gpu - C_ref| <= 1e-6*K + 1e-5*|C_ref|.
    Whole matrix: ||C_gpu - C_ref||_F / ||C_ref||_F <= 1e-6.
    """
    return 1e-6 * K + 1e-5 * np.abs(C_ref), 1e-6
