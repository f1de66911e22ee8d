"""GPU parity of the partial last k stage (K not a multiple of the stage
depth) on the MFMA tiles whose copies go straight into LDS.

There the partial stage is copied like a full one, a stage ahead, and its
copy reads on past k = K: into a row's padding (NaN in these inputs), into
the next stored row, or past the end of the storage (zeros from the range
check).  The compute replaces every value past K by zero, so none of that
may reach C.  Marked ``gpu``.  Expected values come only from the oracle;
integers in [-8, 8] make every partial sum exact, so results match bit for
bit.  The infinity cases put +inf at k = 0 of some rows of op(A) and some
columns of op(B): with unpadded k-contiguous storage those are the values
the neighbouring row's partial-stage copy reads past K, and a missing zero
would turn that row's outputs into NaN.  Non-finite outputs must match the
oracle's exactly (the same infinities, NaN where it has NaN).
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
# (shape, algo): the 64 x 64 tile's 32-k ring (1024 tiles, 3 full stages +
# 4 k), the same tile's 128-k stages on a few tiles (2 full + 4), and the
# 128 x 64 tile (N = 64, 256 row tiles; 64-k stages, 1 full + 36)
CASES = [((2048, 2048, 100), "mfma64"), ((256, 320, 260), "mfma64"), ((32768, 64, 100), "auto"),
         ((2048, 2048, 132), "mfma64")]


@pytest.mark.parametrize("extra", [0, 4])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[0])) + "-" + c[1])
def test_partial_stage_integer_exact(oracle, case, ta, tb, extra):
    (M, N, K), algo = case
    w = gi.make_case(M, N, K, ta, tb, extra, "int8", seed=M + 7 * N + 3 * K + 2 * ta + tb + extra)
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm(algo, A, B, w.make_c(), M, N, K, ta, tb, label=f"{w.name} {algo}")
    P.check_padding(out, N)
    P.check_exact(out[:, :N], oracle.gemm(A, B, M, N, K, ta, tb), f"{w.name} {algo}")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: "x".join(map(str, c[0])) + "-" + c[1])
def test_partial_stage_with_infinities(oracle, case, ta, tb):
    (M, N, K), algo = case
    w = gi.make_case(M, N, K, ta, tb, 0, "int8", seed=11 * M + N + K + 2 * ta + tb)
    A, B = w.make_a(), w.make_b()
    rows = np.arange(1, M, 37)
    cols = np.arange(2, N, 29)
    # op(A)[m, 0] and op(B)[0, n]
    if ta:
        A[0, rows] = np.inf
    else:
        A[rows, 0] = np.inf
    if tb:
        B[cols, 0] = np.inf
    else:
        B[0, cols] = np.inf
    out = P.run_gemm(algo, A, B, w.make_c(), M, N, K, ta, tb, label=f"{w.name} {algo} inf")
    P.check_padding(out, N)
    got = out[:, :N].astype(np.float64)
    ref = oracle.gemm(A, B, M, N, K, ta, tb)
    fin = np.isfinite(ref)
    assert fin.sum() > M * N // 2, "most outputs are finite"
    assert np.array_equal(np.isfinite(got), fin), "non-finite outputs where the oracle has none (or the reverse)"
    P.check_exact(got[fin], ref[fin], f"{w.name} finite outputs")
    assert np.array_equal(got[~fin], ref[~fin], equal_nan=True), f"{w.name}: infinities or NaN differ"
