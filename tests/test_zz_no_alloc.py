"""gemm_f32_splitk_noalloc (partials in the library's own per-GPU scratch)
against gemm_f32_splitk (partials in a workspace the caller allocates).

Marked ``gpu``.  Both run the same kernels in the same order, so their
results must agree bit for bit; each is also held to the oracle (exact on
integer inputs, the FP32 bar of tests/parity.py otherwise).  Two calls in a
row, the second smaller, so the second runs over what the first left in
the scratch.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import parity as P
from dense_fp32_matrix_gemm_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


def _both(w, splits):
    """C from the no-allocation entry point, then from the workspace one."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    s = torch.cuda.current_stream().cuda_stream
    A, B = w.make_a(), w.make_b()
    dA, dB = P.to_device(A), P.to_device(B)
    c_scratch, c_work = P.to_device(w.make_c()), P.to_device(w.make_c())
    need = g.gemm_f32_splitk_workspace_size(w.M, w.N, w.K, splits)
    assert 0 < need <= _lib.SPLITK_SCRATCH_BYTES
    P.note(f"splitk noalloc {w.name} splits={splits} need={need}")
    st = g.gemm_f32_splitk_noalloc(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                                   c_scratch.data_ptr(), w.ldc_, w.transA, w.transB, splits, s)
    assert st == 0, g.gemm_f32_strerror(st)
    ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    P.note(f"splitk workspace {w.name} splits={splits}")
    st = g.gemm_f32_splitk(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                           c_work.data_ptr(), w.ldc_, w.transA, w.transB, splits, ws.data_ptr(),
                           need, s)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    return A, B, c_scratch.cpu().numpy(), c_work.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point(oracle):
    cases = [  # M, N, K, transA, transB, ld padding, inputs, splits: larger, then smaller
        (1024, 2048, 4096, 0, 1, 0, "int8", 4),   # 32 MiB of partials
        (300, 500, 1000, 1, 0, 3, "u11", 3),
    ]
    for (M, N, K, ta, tb, extra, dist, splits) in cases:
        w = gi.make_case(M, N, K, ta, tb, extra, dist, seed=M + N + K)
        A, B, got, want = _both(w, splits)
        P.check_padding(got, N)
        assert np.array_equal(got, want), f"{w.name}: differs from gemm_f32_splitk"
        ref = oracle.gemm(A, B, M, N, K, ta, tb)
        if dist == "int8":
            P.check_exact(got[:, :N], ref, w.name)
        else:
            P.check_close(got[:, :N], ref, K, w.name)


def test_noalloc_refuses_more_partials_than_its_scratch():
    """4096^3 in two runs needs 128 MiB of partials: refused on the host,
    nothing launched, C untouched (the buffers are full size all the same)."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    M = N = K = 4096
    assert g.gemm_f32_splitk_workspace_size(M, N, K, 2) > _lib.SPLITK_SCRATCH_BYTES
    a = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    b = torch.zeros((K, N), dtype=torch.float32, device="cuda")
    c = torch.full((M, N), gi.OUTPUT_PAD, dtype=torch.float32, device="cuda")
    P.note("splitk noalloc oversize (rejected on the host)")
    st = g.gemm_f32_splitk_noalloc(M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N,
                                   0, 0, 2, torch.cuda.current_stream().cuda_stream)
    assert st == -12
    torch.cuda.synchronize()
    assert bool(torch.all(c == gi.OUTPUT_PAD))
