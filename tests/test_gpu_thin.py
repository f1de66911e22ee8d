"""GPU parity of the rows left below the last whole row of 64 x 64 tiles.

When the MFMA path runs 64 x 64 tiles and M = 64 q + r with 1 <= r <= 4, the
tiles cover rows 0 .. 64 q - 1 and extra workgroups at the front of the grid
compute the last r rows as a matrix-vector style product (k split over the
waves, the slices added in a fixed order).  Marked ``gpu``.  Expected values
come only from the oracle: integers in [-8, 8] make every partial sum exact,
so those rows must match bit for bit in every layout; floating-point data
must meet the 1e-6 bounds.  Shapes with r = 0 and r = 5 run the tiles alone
and are here for contrast.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]
# one extra row on one tile row; two on a ragged N and K; one over a long k
# (several slices per wave); four rows; r = 5 and r = 0 (tiles only)
SHAPES = [(65, 64, 64), (66, 200, 100), (131, 257, 769), (196, 3071, 33), (1027, 96, 4096),
          (133, 130, 70), (128, 100, 50)]


@pytest.mark.parametrize("algo", ["mfma64", "auto"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_thin_rows_integer_exact(oracle, shape, ta, tb, algo):
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, 4, "int8", seed=7 * M + 3 * N + K + 2 * ta + tb)
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm(algo, A, B, w.make_c(), M, N, K, ta, tb, label=f"{w.name} {algo}")
    P.check_padding(out, N)
    P.check_exact(out[:, :N], oracle.gemm(A, B, M, N, K, ta, tb), f"{w.name} {algo}")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(131, 257, 769), (2049, 3071, 769)], ids=lambda s: "x".join(map(str, s)))
def test_thin_rows_float_tolerance(oracle, shape, ta, tb):
    """U(-1, 1) data within the bounds; for the full ragged workload the last
    row (the one the extra workgroups compute) is checked on its own too."""
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, 3, "u11", seed=M + 5 * K + 2 * ta + tb)
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm("auto", A, B, w.make_c(), M, N, K, ta, tb, label=w.name)
    P.check_padding(out, N)
    if M * N <= 300 * 300:
        P.check_close(out[:, :N], oracle.gemm(A, B, M, N, K, ta, tb), K, w.name)
        return
    rows = np.array([M - 1] * N + list(range(0, M, 97)))
    cols = np.array(list(range(N)) + [(13 * i) % N for i in range(len(range(0, M, 97)))])
    ref = oracle.entries(A, B, M, N, K, ta, tb, rows, cols)
    P.check_close(out[rows, cols], ref, K, f"{w.name} last row and samples")


def test_thin_rows_with_bias_exact(oracle):
    """bias (no activation) on integers: the extra workgroups add it too."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    M, N, K = 1026, 500, 300
    w = gi.make_case(M, N, K, 0, 0, 0, "int8", seed=1234)
    A, B = w.make_a(), w.make_b()
    bias = gi.stored_matrix(99, 1, N, dist="int8")[0]
    dA, dB, dC, db = P.to_device(A), P.to_device(B), P.to_device(w.make_c()), P.to_device(bias)
    P.note(f"thin bias {w.name}")
    st = g.gemm_f32_bias_act(M, N, K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_, dC.data_ptr(),
                             w.ldc_, 0, 0, db.data_ptr(), 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    P.check_exact(dC.cpu().numpy(), oracle.epilogue(oracle.gemm(A, B, M, N, K), bias, 0), "thin bias")
