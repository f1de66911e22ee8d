"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` function takes a ``gemm(A, B, M, N, K, transA, transB)``
callable returning a float64 (M, N) array and raises ``AssertionError`` if
the callable disagrees with what mathematics or a library routine fixes.
``tests/test_oracle_pins.py`` runs them on the real oracle and
``tests/test_oracle_mutants.py`` runs them on deliberately broken copies of
it, to show each plausible mistake is caught by at least one pin.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Callable

import numpy as np

import gemm_inputs as gi

Gemm = Callable[..., np.ndarray]

LAYOUTS = [(ta, tb) for ta in (0, 1) for tb in (0, 1)]


def _store(logical: np.ndarray, trans: int, extra_ld: int) -> np.ndarray:
    """Place a logical (rows x cols) matrix into stored form with NaN padding.

    ``trans`` = 1 stores the transpose (so op() of the stored array gives back
    ``logical``).
    """
    mat = logical.T if trans else logical
    r, c = mat.shape
    out = np.full((r, max(1, c) + extra_ld), np.nan, dtype=np.float32)
    out[:, :c] = mat
    return out


def _rand(rng, shape, dist="u11"):
    if dist == "u11":
        return rng.uniform(-1, 1, size=shape).astype(np.float32)
    return rng.integers(-8, 9, size=shape).astype(np.float32)


def pin_identity(gemm: Gemm) -> None:
    """A.I = A and I.B = B exactly, for every transpose and with padded rows."""
    rng = np.random.default_rng(101)
    for (M, K) in [(5, 7), (16, 16), (33, 9)]:
        a = _rand(rng, (M, K))
        eye = np.eye(K, dtype=np.float32)
        for ta, tb in LAYOUTS:
            for extra in (0, 2):
                C = gemm(_store(a, ta, extra), _store(eye, tb, extra), M, K, K, ta, tb)
                assert np.array_equal(C, a.astype(np.float64)), ("A.I", M, K, ta, tb, extra)
                eye_m = np.eye(M, dtype=np.float32)
                C = gemm(_store(eye_m, ta, extra), _store(a, tb, extra), M, K, M, ta, tb)
                assert np.array_equal(C, a.astype(np.float64)), ("I.B", M, K, ta, tb, extra)


def pin_all_ones(gemm: Gemm) -> None:
    """ones(MxK).ones(KxN) = K in every entry, exactly."""
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 4, 129), (8, 8, 1000)]:
        for ta, tb in LAYOUTS:
            a = np.ones((M, K), dtype=np.float32)
            b = np.ones((K, N), dtype=np.float32)
            C = gemm(_store(a, ta, 1), _store(b, tb, 3), M, N, K, ta, tb)
            assert C.shape == (M, N)
            assert np.all(C == float(K)), ("ones", M, N, K, ta, tb)


def pin_rank_one(gemm: Gemm) -> None:
    """K = 1 gives the outer product u v^T exactly; A = u 1^T, B = 1 v^T gives K u_i v_j."""
    rng = np.random.default_rng(102)
    for (M, N) in [(7, 5), (32, 3)]:
        u = _rand(rng, (M, 1))
        v = _rand(rng, (1, N))
        for ta, tb in LAYOUTS:
            C = gemm(_store(u, ta, 2), _store(v, tb, 2), M, N, 1, ta, tb)
            outer = u.astype(np.float64) * v.astype(np.float64)
            assert np.array_equal(C, outer), ("k=1", M, N, ta, tb)
            for K in (4, 32):
                a = np.repeat(u, K, axis=1)
                b = np.repeat(v, K, axis=0)
                C = gemm(_store(a, ta, 1), _store(b, tb, 1), M, N, K, ta, tb)
                # K copies of one product sum exactly in double for K <= 32
                assert np.array_equal(C, K * outer), ("rank1", M, N, K, ta, tb)


def pin_brute_force(gemm: Gemm, sizes=range(1, 5)) -> None:
    """Every M, N, K in 1..4, every transpose, packed and padded: against exact rationals.

    Each product of two float32 is exact in double and the sums of at most
    four terms round at most K - 1 times, so the oracle's double result must
    sit within (K-1) * 2^-53 * sum|terms| of the exact rational value.
    """
    rng = np.random.default_rng(103)
    u = 2.0 ** -53
    for M in sizes:
        for N in sizes:
            for K in sizes:
                a = _rand(rng, (M, K))
                b = _rand(rng, (K, N))
                for ta, tb in LAYOUTS:
                    for extra in (0, 1):
                        C = gemm(_store(a, ta, extra), _store(b, tb, extra), M, N, K, ta, tb)
                        assert C.shape == (M, N)
                        for i in range(M):
                            for j in range(N):
                                terms = [Fraction(float(a[i, k])) * Fraction(float(b[k, j]))
                                         for k in range(K)]
                                exact = sum(terms, Fraction(0))
                                bound = (K - 1) * u * float(sum(abs(t) for t in terms))
                                err = abs(Fraction(float(C[i, j])) - exact)
                                assert err <= Fraction(bound), (M, N, K, ta, tb, extra, i, j)


def pin_integer_exact(gemm: Gemm) -> None:
    """Integer inputs in [-8, 8]: the result equals numpy's exact int64 product."""
    rng = np.random.default_rng(104)
    for (M, N, K) in [(9, 13, 31), (64, 48, 200)]:
        a = rng.integers(-8, 9, size=(M, K))
        b = rng.integers(-8, 9, size=(K, N))
        exact = (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64)
        for ta, tb in LAYOUTS:
            C = gemm(_store(a.astype(np.float32), ta, 3), _store(b.astype(np.float32), tb, 0),
                     M, N, K, ta, tb)
            assert np.array_equal(C, exact), ("int", M, N, K, ta, tb)


def pin_numpy_f64(gemm: Gemm, workload: gi.Workload) -> None:
    """The whole product against numpy's float64 matmul (an independent BLAS dgemm).

    Both sides are double-precision sums of the same exact products in
    different orders; each is within K * 2^-53 * (|A| . |B|) of the exact
    value, so they differ by at most twice that.
    """
    rtol = 2 * max(1, workload.K) * 2.0 ** -53
    A, B = workload.make_a(), workload.make_b()
    M, N, K = workload.M, workload.N, workload.K
    C = gemm(A, B, M, N, K, workload.transA, workload.transB)
    a = _logical(A, workload.a_dims, workload.transA)
    b = _logical(B, workload.b_dims, workload.transB)
    ref = a @ b
    scale = np.abs(a) @ np.abs(b)
    assert C.shape == ref.shape
    assert np.all(np.abs(C - ref) <= rtol * scale + 1e-300), workload.name


def _logical(stored: np.ndarray, dims, trans: int) -> np.ndarray:
    r, c = dims
    m = stored[:r, :c].astype(np.float64)
    return m.T if trans else m


def pin_counts(gemm_with_stats: Callable) -> None:
    """The instrumented oracle performs M*N*K multiply-adds and reads 2*M*N*K operands."""
    rng = np.random.default_rng(105)
    for (M, N, K) in [(1, 1, 1), (3, 4, 5), (64, 64, 64), (7, 1, 300)]:
        a = _rand(rng, (M, K))
        b = _rand(rng, (K, N))
        _, (macs, reads) = gemm_with_stats(_store(a, 0, 0), _store(b, 0, 0), M, N, K)
        assert macs == M * N * K, ("macs", M, N, K, macs)
        assert reads == 2 * M * N * K, ("reads", M, N, K, reads)


ALL_FAST_PINS = (pin_identity, pin_all_ones, pin_rank_one, pin_integer_exact)


# Standard normal distribution function Phi at a few points (statistics-table
# values); GELU(x) = x * Phi(x).
PHI_TABLE = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -1.5: 0.06680720126885807,
             0.5: 0.6914624612740131, -3.0: 0.0013498980316301035}


def pin_epilogue(epilogue) -> None:
    """The fused-epilogue reference against closed forms and a library erf.

    ``epilogue(C, bias, act)`` returns act(C + bias) in float64.
    """
    import math
    from scipy.special import erf
    x = np.array([list(PHI_TABLE)], dtype=np.float64)
    got = epilogue(x, None, 1)[0]
    for k, (xv, phi) in enumerate(PHI_TABLE.items()):
        assert abs(got[k] - xv * phi) <= 1e-15 * max(1.0, abs(xv)), (xv, got[k])
    rng = np.random.default_rng(106)
    v = rng.normal(0, 3, size=(40, 50))
    g_pos, g_neg = epilogue(v, None, 1), epilogue(-v, None, 1)
    assert np.all(np.abs((g_pos - g_neg) - v) <= 1e-14 * np.maximum(1, np.abs(v)))  # x Phi(x) + x Phi(-x) = x
    ref = 0.5 * v * (1 + erf(v / math.sqrt(2)))
    assert np.all(np.abs(g_pos - ref) <= 1e-15 * np.maximum(1, np.abs(v)))
    big = np.array([[10.0, -10.0, 0.0]])
    gb = epilogue(big, None, 1)[0]
    assert abs(gb[0] - 10.0) < 1e-15 and abs(gb[1]) < 1e-20 and gb[2] == 0.0
    bias = rng.uniform(-1, 1, size=50).astype(np.float32)
    assert np.array_equal(epilogue(v, bias, 0), v + bias.astype(np.float64)[None, :])
    assert np.array_equal(epilogue(v, None, 0), v)
    both = epilogue(v, bias, 1)
    vb = v + bias.astype(np.float64)[None, :]
    assert np.all(np.abs(both - 0.5 * vb * (1 + erf(vb / math.sqrt(2)))) <=
                  1e-15 * np.maximum(1, np.abs(vb)))
