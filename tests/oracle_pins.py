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


# ---------------------------------------------------------------------------
# Mixed precision (the Smallem page, "Rendre le GPU rapide", section "Les
# Tensor Cores"): operands rounded to bf16, to nearest with ties to even.

def bf16_nearest(x: float) -> float:
    """The bf16 nearest to ``x`` (ties to even), by exact rational arithmetic.

    Written from the format, not from bit patterns: bf16 keeps 8 significant
    bits and the exponent range of float32, so in the binade [2^(e-1), 2^e)
    its values are the multiples of 2^(e-8), and below 2^-126 the multiples
    of 2^-133 (its subnormals).  A value that rounds to 2^128 overflows to
    infinity.  Zeros keep their sign.
    """
    import math
    if x == 0 or math.isinf(x) or math.isnan(x):
        return x
    _, e = math.frexp(abs(x))                  # |x| in [2^(e-1), 2^e)
    quantum = Fraction(2) ** max(e - 8, -133)
    t = Fraction(abs(x)) / quantum
    n = math.floor(t)
    rest = t - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Fraction(2) ** 128:
        return math.copysign(math.inf, x)
    return math.copysign(float(v), x)


def _f32_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _finite_patterns(rng, n: int) -> np.ndarray:
    x = _f32_from_bits(rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32))
    return x[np.isfinite(x)]


# (input, nearest bf16) worked by hand from the format: 1 + 2^-8 lies halfway
# between 1 and 1 + 2^-7; 2^-134 halfway between 0 and the least subnormal
# 2^-133; 255 * 2^120 is the largest finite bf16 and 2^128 - 2^119 the tie
# above it; 257 and 259 are ties between multiples of 2 (quantum in [256, 512));
# float32(0.1) = 0x3DCCCCCD, whose upper half rounds up to 0x3DCD.
BF16_CASES = [
    (1.0, 1.0), (1 + 2.0 ** -7, 1 + 2.0 ** -7), (1 + 2.0 ** -8, 1.0),
    (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6), (1 + 2.0 ** -8 + 2.0 ** -23, 1 + 2.0 ** -7),
    (1 + 2.0 ** -9, 1.0), (-(1 + 2.0 ** -8), -1.0), (-(1 + 3 * 2.0 ** -8), -(1 + 2.0 ** -6)),
    (2 - 2.0 ** -9, 2.0), (257.0, 256.0), (259.0, 260.0), (float(np.float32(0.1)), 0.10009765625),
    (255 * 2.0 ** 120, 255 * 2.0 ** 120), (2.0 ** 128 - 2.0 ** 119, float("inf")),
    (2.0 ** 128 - 2.0 ** 120 + 2.0 ** 118, 255 * 2.0 ** 120),
    (float(np.finfo(np.float32).max), float("inf")),
    (2.0 ** -133, 2.0 ** -133), (2.0 ** -134, 0.0), (3 * 2.0 ** -135, 2.0 ** -133),
    (2.0 ** -149, 0.0), (2.0 ** -126, 2.0 ** -126), (float("inf"), float("inf")),
    (float("-inf"), float("-inf")),
] + [(float(v), float(v)) for v in range(-8, 9)]


def pin_bf16_rounding(round_bf16) -> None:
    """``round_bf16(float32 array) -> float32 array`` against hand-worked
    cases, the exact rational rounding above, and torch's CPU conversion."""
    import math

    import torch
    x = np.array([c[0] for c in BF16_CASES], dtype=np.float32)
    want = np.array([c[1] for c in BF16_CASES], dtype=np.float32)
    assert np.array_equal(x.astype(np.float64), [c[0] for c in BF16_CASES]), "cases are float32"
    got = round_bf16(x)
    for xi, g, w in zip(x, got, want):
        assert g == w, (float(xi), float(g), float(w))
    z = round_bf16(np.array([0.0, -0.0, np.nan], dtype=np.float32))
    assert z[0] == 0 and not math.copysign(1, z[0]) < 0
    assert z[1] == 0 and math.copysign(1, z[1]) < 0
    assert np.isnan(z[2])

    rng = np.random.default_rng(107)
    sample = _finite_patterns(rng, 6000)
    ties = _f32_from_bits((rng.integers(0, 2 ** 16, size=3000).astype(np.uint32) << 16) | 0x8000)
    ties = ties[np.isfinite(ties)]
    for v in np.concatenate([sample, ties]):
        g = float(round_bf16(np.array([v], dtype=np.float32))[0])
        w = bf16_nearest(float(v))
        assert g == w or (math.isnan(g) and math.isnan(w)), (float(v), g, w)
        assert math.copysign(1, g) == math.copysign(1, w), float(v)

    many = np.concatenate([_finite_patterns(rng, 400000), ties,
                           rng.normal(0, 1, 200000).astype(np.float32)])
    ref = torch.from_numpy(many).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(many).view(np.uint32), ref.view(np.uint32))


def _bf16_logical(stored: np.ndarray, dims, trans: int) -> np.ndarray:
    """Logical operand with each element rounded by torch's CPU bfloat16
    conversion (a library rounding, independent of the oracle), float64."""
    import torch
    m = _logical(stored, dims, trans).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(m)).to(torch.bfloat16).to(torch.float64).numpy()


def pin_bf16_gemm(gemm_bf16) -> None:
    """The mixed-precision product ``gemm_bf16(A, B, M, N, K, transA, transB)``.

    * Integers in [-8, 8] are bf16 values and their products' sums are
      exact: the result is the exact integer product (the page's own test
      for the matrix-core kernel).
    * Times the identity it returns the rounded operand itself.
    * On tiny shapes, the exact rational sum of the products of the
      independently rounded operands, within the double sum's rounding.
    * On a 64 x 64 x 64 workload, numpy's float64 matmul of the torch-rounded
      operands, within twice the double sums' error bound.
    """
    rng = np.random.default_rng(108)
    for (M, N, K) in [(9, 13, 31), (64, 48, 200)]:
        a = rng.integers(-8, 9, size=(M, K))
        b = rng.integers(-8, 9, size=(K, N))
        exact = (a @ b).astype(np.float64)
        for ta, tb in LAYOUTS:
            C = gemm_bf16(_store(a.astype(np.float32), ta, 2), _store(b.astype(np.float32), tb, 1),
                          M, N, K, ta, tb)
            assert np.array_equal(C, exact), ("int", M, N, K, ta, tb)

    nearest = np.vectorize(bf16_nearest, otypes=[np.float64])
    for (M, K) in [(5, 7), (33, 9)]:
        a = _rand(rng, (M, K))
        for ta, tb in LAYOUTS:
            C = gemm_bf16(_store(a, ta, 1), _store(np.eye(K, dtype=np.float32), tb, 0),
                          M, K, K, ta, tb)
            assert np.array_equal(C, nearest(a.astype(np.float64))), ("A.I", M, K, ta, tb)
            C = gemm_bf16(_store(np.eye(M, dtype=np.float32), ta, 0), _store(a, tb, 2),
                          M, K, M, ta, tb)
            assert np.array_equal(C, nearest(a.astype(np.float64))), ("I.B", M, K, ta, tb)

    u = 2.0 ** -53
    for M in range(1, 4):
        for N in range(1, 4):
            for K in range(1, 5):
                a = _rand(rng, (M, K))
                b = _rand(rng, (K, N))
                ra = [[Fraction(bf16_nearest(float(a[i, k]))) for k in range(K)] for i in range(M)]
                rb = [[Fraction(bf16_nearest(float(b[k, j]))) for j in range(N)] for k in range(K)]
                for ta, tb in LAYOUTS:
                    C = gemm_bf16(_store(a, ta, 1), _store(b, tb, 0), M, N, K, ta, tb)
                    for i in range(M):
                        for j in range(N):
                            terms = [ra[i][k] * rb[k][j] for k in range(K)]
                            exact = sum(terms, Fraction(0))
                            bound = (K - 1) * u * float(sum(abs(t) for t in terms))
                            assert abs(Fraction(float(C[i, j])) - exact) <= Fraction(bound), \
                                (M, N, K, ta, tb, i, j)

    w = gi.WORKLOADS["S64"]
    for ta, tb in LAYOUTS:
        wl = gi.make_case(w.M, w.N, w.K, ta, tb, 1, "u11", seed=109 + 2 * ta + tb)
        A, B = wl.make_a(), wl.make_b()
        C = gemm_bf16(A, B, wl.M, wl.N, wl.K, ta, tb)
        a = _bf16_logical(A, wl.a_dims, ta)
        b = _bf16_logical(B, wl.b_dims, tb)
        bound = 2 * wl.K * u * (np.abs(a) @ np.abs(b))
        assert np.all(np.abs(C - a @ b) <= bound), ("numpy", ta, tb)
