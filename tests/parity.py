"""Helpers for the GPU parity tests: run the library through the C ABI on
seeded inputs and compare with the oracle.

The acceptance bar for floating-point inputs:
    elementwise  |C_gpu - C_ref| <= 1e-6 * K + 1e-5 * |C_ref|
    whole matrix ||C_gpu - C_ref||_F / ||C_ref||_F <= 1e-6
and for integer-valued inputs in [-8, 8] (every partial sum exact in FP32,
whatever the order) bit-for-bit equality.  In every case the padding
columns of C must still hold the sentinel the buffer was filled with.
"""

from __future__ import annotations

import sys
from typing import Optional

import numpy as np

import gemm_inputs as gi

ALGO_IDS = {"auto": 0, "mfma": 1, "fma": 2, "tiled": 3, "naive": 4, "mfma128": 5, "mfma64": 6, "mfma256": 7,
            "mfmawide": 8}
ELEM_ABS, ELEM_REL, FROB_REL = 1e-6, 1e-5, 1e-6


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash log says which."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_device(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def run_gemm(algo: str, A: np.ndarray, B: np.ndarray, C: np.ndarray, M: int, N: int,
             K: int, transA: int, transB: int, stream=None, label: str = "") -> np.ndarray:
    """Copy A, B, C to the device, call gemm_f32_ex, return C from the device."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    dA, dB, dC = to_device(A), to_device(B), to_device(C)
    note(f"{label} algo={algo} M={M} N={N} K={K} tA={transA} tB={transB} "
         f"lda={A.shape[1]} ldb={B.shape[1]} ldc={C.shape[1]}")
    s = stream if stream is not None else torch.cuda.current_stream()
    st = g.gemm_f32_ex(M, N, K, dA.data_ptr(), A.shape[1], dB.data_ptr(), B.shape[1],
                       dC.data_ptr(), C.shape[1], transA, transB, s.cuda_stream,
                       ALGO_IDS[algo])
    assert st == 0, g.gemm_f32_strerror(st)
    s.synchronize()
    return dC.cpu().numpy()


def check_padding(C_out: np.ndarray, N: int, fill: float = gi.OUTPUT_PAD) -> None:
    pad = C_out[:, N:]
    assert np.all(pad == np.float32(fill)), "the library wrote into C's padding"


def check_close(got: np.ndarray, ref: np.ndarray, K: int, what: str = "") -> float:
    """Elementwise and relative-Frobenius bounds; returns the Frobenius error."""
    got = got.astype(np.float64)
    assert got.shape == ref.shape
    assert not np.any(np.isnan(got)), f"{what}: NaN in result"
    err = np.abs(got - ref)
    bound = ELEM_ABS * K + ELEM_REL * np.abs(ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(err <= bound), f"{what}: elementwise bound exceeded (worst ratio {worst:.3g})"
    nref = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err))
    assert frob <= FROB_REL, f"{what}: relative Frobenius error {frob:.3g} > {FROB_REL}"
    return frob


def check_exact(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    got = got.astype(np.float64)
    assert got.shape == ref.shape
    bad = np.argwhere(got != ref)
    assert bad.size == 0, (f"{what}: {len(bad)} entries differ, first at {tuple(bad[0])}: "
                           f"gpu {got[tuple(bad[0])]} vs oracle {ref[tuple(bad[0])]}")


def ragged_operand(rows: int, cols: int, ld: int, seed: int, dist: str,
                   offset: int = 0) -> np.ndarray:
    """A stored matrix preceded by ``offset`` floats of NaN in one flat buffer,
    returned as the flat buffer (so the device pointer can be offset)."""
    m = gi.stored_matrix(seed, rows, cols, ld, dist)
    flat = np.full(offset + m.size, np.nan, dtype=np.float32)
    flat[offset:] = m.reshape(-1)
    return flat
