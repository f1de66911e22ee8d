"""The CPU oracle against closed forms, exact rationals and numpy float64.

CPU only.  See ``tests/oracle_pins.py`` for what each pin fixes.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle_pins as pins


@pytest.fixture(scope="module")
def gemm(oracle):
    return oracle.gemm


def test_identity(gemm):
    pins.pin_identity(gemm)


def test_all_ones(gemm):
    pins.pin_all_ones(gemm)


def test_rank_one(gemm):
    pins.pin_rank_one(gemm)


def test_brute_force_exact_rationals(gemm):
    pins.pin_brute_force(gemm)


def test_integer_exact(gemm):
    pins.pin_integer_exact(gemm)


def test_counts(oracle):
    pins.pin_counts(lambda A, B, M, N, K: oracle.gemm(A, B, M, N, K, 0, 0, with_stats=True))


@pytest.mark.parametrize("name", ["S64", "S1k", "R"])
def test_numpy_f64_full(gemm, name):
    pins.pin_numpy_f64(gemm, gi.WORKLOADS[name])


@pytest.mark.parametrize("name", ["S4k", "T-fwd", "T-dX", "T-dW"])
def test_numpy_f64_sampled(oracle, name):
    """Full-size workloads, checked on sampled entries against numpy float64 dots."""
    w = gi.WORKLOADS[name]
    A, B = w.make_a(), w.make_b()
    rows, cols = gi.sample_entries(w.M, w.N, 300)
    got = oracle.entries(A, B, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
    a = pins._logical(A, w.a_dims, w.transA)
    b = pins._logical(B, w.b_dims, w.transB)
    ref = np.einsum("tk,kt->t", a[rows, :], b[:, cols])
    scale = np.einsum("tk,kt->t", np.abs(a[rows, :]), np.abs(b[:, cols]))
    assert np.all(np.abs(got - ref) <= 2 * w.K * 2.0 ** -53 * scale)


def test_entries_match_full_product(oracle):
    """The one-at-a-time entry point returns exactly the full product's entries."""
    for name in ("S64", "R"):
        w = gi.WORKLOADS[name]
        A, B = w.make_a(), w.make_b()
        full = oracle.gemm(A, B, w.M, w.N, w.K, w.transA, w.transB)
        rows, cols = gi.sample_entries(w.M, w.N, 500)
        got = oracle.entries(A, B, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
        assert np.array_equal(got, full[rows, cols])


def test_empty_and_degenerate(oracle):
    """M or N = 0 gives an empty result; K = 0 gives the empty sum, zero."""
    A = np.zeros((0, 1), np.float32)
    B = np.ones((1, 5), np.float32)
    assert oracle.gemm(A, B, 0, 5, 1).shape == (0, 5)
    A = np.ones((3, 1), np.float32)
    B = np.zeros((0, 1), np.float32)
    assert oracle.gemm(A, B, 3, 0, 1, 0, 1).shape == (3, 0)
    A = np.full((4, 1), np.nan, np.float32)     # K = 0: no element of A is read
    B = np.full((0, 6), np.nan, np.float32)
    C = oracle.gemm(A, B, 4, 6, 0)
    assert C.shape == (4, 6) and np.all(C == 0.0)


def test_rejects_bad_storage(oracle):
    A = np.ones((4, 3), np.float32)
    B = np.ones((3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.gemm(A, B, 4, 4, 5)          # lda = 3 < K = 5
    with pytest.raises(ValueError):
        oracle.entries(A, B, 4, 4, 3, 0, 0, np.array([4]), np.array([0]))


def test_nan_propagates(oracle):
    """A NaN inside the used region reaches exactly the outputs that use it."""
    A = np.ones((3, 4), np.float32)
    B = np.ones((4, 5), np.float32)
    A[1, 2] = np.nan
    C = oracle.gemm(A, B, 3, 5, 4)
    assert np.all(np.isnan(C[1])) and not np.any(np.isnan(C[[0, 2]]))


@pytest.mark.parametrize("ta,tb,gap,shared", [(0, 0, 0, False), (1, 0, 3, False),
                                              (0, 1, 5, True), (1, 1, 1, False)])
def test_batched_equals_block_diagonal_product(oracle, ta, tb, gap, shared):
    """A batch of products equals the diagonal blocks of one product of
    block-diagonal matrices (whose off-diagonal blocks are exactly zero)."""
    import oracle as oracle_pkg
    batch, M, N, K = 5, 7, 6, 9
    w = gi.Workload("bd", M, N, K, 41, 42, transA=ta, transB=tb, batch=batch, gap=gap,
                    shared_b=shared, lda=(M if ta else K) + 2, ldb=(K if tb else N) + 1)
    A, B = w.make_a(), w.make_b()
    got = oracle_pkg.gemm_ref_batched(A, B, M, N, K, ta, tb, w.lda_, w.stride_a, w.ldb_,
                                      w.stride_b, batch)
    # logical operands of each product
    ar, ac = w.a_dims
    br, bc = w.b_dims
    a_flat, b_flat = A.reshape(-1), B.reshape(-1)
    big_a = np.zeros((batch * M, batch * K), np.float32)
    big_b = np.zeros((batch * K, batch * N), np.float32)
    for b in range(batch):
        sa = a_flat[b * w.stride_a: b * w.stride_a + ar * w.lda_].reshape(ar, w.lda_)[:, :ac]
        sb = b_flat[b * w.stride_b: b * w.stride_b + br * w.ldb_].reshape(br, w.ldb_)[:, :bc]
        big_a[b * M:(b + 1) * M, b * K:(b + 1) * K] = sa.T if ta else sa
        big_b[b * K:(b + 1) * K, b * N:(b + 1) * N] = sb.T if tb else sb
    full = oracle.gemm(big_a, big_b, batch * M, batch * N, batch * K)
    for b in range(batch):
        assert np.array_equal(got[b], full[b * M:(b + 1) * M, b * N:(b + 1) * N]), b
        for c in range(batch):
            if c != b:
                assert not np.any(full[b * M:(b + 1) * M, c * N:(c + 1) * N])


def test_epilogue(oracle):
    pins.pin_epilogue(oracle.epilogue)


def test_bf16_rounding(oracle):
    pins.pin_bf16_rounding(oracle.round_bf16)


def test_bf16_product(oracle):
    pins.pin_bf16_gemm(oracle.gemm_bf16)


def test_bf16_entries_match_full_product(oracle):
    w = gi.WORKLOADS["R"]
    A, B = w.make_a(), w.make_b()
    rows, cols = gi.sample_entries(w.M, w.N, 400)
    full = oracle.gemm_bf16(A, B, w.M, w.N, w.K, w.transA, w.transB)
    got = oracle.entries_bf16(A, B, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
    assert np.array_equal(got, full[rows, cols])


def test_bf16_differs_from_f32_by_operand_rounding(oracle):
    """Uniform(-1, 1) operands: the mixed-precision product moves off the
    FP32 product by about the operands' relative rounding (at most 2^-9
    each), far more than the FP32 tolerance, so parity tests against the
    wrong reference would fail."""
    w = gi.WORKLOADS["S64"]
    A, B = w.make_a(), w.make_b()
    exact = oracle.gemm(A, B, w.M, w.N, w.K)
    mixed = oracle.gemm_bf16(A, B, w.M, w.N, w.K)
    rel = np.linalg.norm(mixed - exact) / np.linalg.norm(exact)
    assert 1e-4 < rel < 2 * 2.0 ** -9
