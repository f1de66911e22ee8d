"""GPU parity of the 128 x 64 MFMA tile that the automatic choice takes for
outputs at most 64 columns wide with at least 256 such tiles (one per CU).

Marked ``gpu``.  The shapes below are chosen so that the rule picks this
tile (N <= 64 and ceil(M / 128) * batch >= 256); expected values come only
from the oracle.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle as oracle_pkg
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


def run_batched(w):
    import torch
    import dense_fp32_matrix_gemm_amd as g
    A, B = w.make_a(), w.make_b()
    dA, dB, dC = P.to_device(A), P.to_device(B), P.to_device(w.make_c())
    P.note(f"narrow batched {w.name} batch={w.batch} t{w.transA}{w.transB}")
    st = g.gemm_f32_strided_batched(w.M, w.N, w.K, dA.data_ptr(), w.lda_, w.stride_a, dB.data_ptr(), w.ldb_,
                                    w.stride_b, dC.data_ptr(), w.ldc_, w.stride_c, w.batch, w.transA,
                                    w.transB, torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    flat = dC.cpu().numpy().reshape(w.batch, w.stride_c)
    body = flat[:, :w.M * w.ldc_].reshape(w.batch, w.M, w.ldc_)
    pad = np.concatenate([body[:, :, w.N:].reshape(-1), flat[:, w.M * w.ldc_:].reshape(-1)])
    assert np.all(pad == np.float32(gi.OUTPUT_PAD)), "the library wrote outside the products"
    ref = oracle_pkg.gemm_ref_batched(A, B, w.M, w.N, w.K, w.transA, w.transB, w.lda_, w.stride_a, w.ldb_,
                                      w.stride_b, w.batch)
    return body[:, :, :w.N], ref


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("shape", [(512, 64, 512), (500, 50, 300), (449, 64, 65)],
                         ids=lambda s: "x".join(map(str, s)))
def test_integer_exact(shape, ta, tb):
    """64 products, integers in [-8, 8]: bit-for-bit equality, including
    ragged row and column tails, a partial last k stage and padded leading
    dimensions."""
    M, N, K = shape
    w = gi.Workload(f"narrow{M}x{N}x{K}", M, N, K, 40 + M, 41 + N, "int8", "int8", ta, tb,
                    lda=(M if ta else K) + 3, ldb=(K if tb else N) + 1, ldc=N + 2, batch=64, gap=5)
    got, ref = run_batched(w)
    for b in range(w.batch):
        P.check_exact(got[b], ref[b], f"{w.name}[{b}] t{ta}{tb}")


def test_float_batched():
    """The attention-value shape with U(-1, 1) and N(0, 1) data: within the
    1e-6 bounds."""
    w = gi.Workload("narrow-pv", 512, 64, 512, 3002, 3003, "u11", "n01", batch=64)
    got, ref = run_batched(w)
    for b in range(w.batch):
        P.check_close(got[b], ref[b], w.K, f"narrow-pv[{b}]")


def test_single_long_product(oracle):
    """One 32768 x 64 x 4096 product (256 tiles, 16 accumulation chunks of
    256 k), sampled entries against the oracle."""
    M, N, K = 32768, 64, 4096
    w = gi.make_case(M, N, K, 0, 0, 0, "u11", seed=71)
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm("auto", A, B, w.make_c(), M, N, K, 0, 0, label=w.name)
    rows, cols = gi.sample_entries(M, N, 3000, seed=31)
    frob = P.check_close(out[rows, cols], oracle.entries(A, B, M, N, K, 0, 0, rows, cols), K, "narrow long")
    print(f"narrow 32768x64x4096 sampled relFrob={frob:.3g}")
