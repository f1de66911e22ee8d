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
