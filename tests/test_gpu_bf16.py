"""GPU parity of the mixed-precision product (operands rounded to bf16,
FP32 sums) against the oracle's ``gemm_bf16``.

Marked ``gpu``.  Expected values come only from the oracle: the exact
double sum of the products of the bf16-rounded operands.

Acceptance bar: integer inputs in [-8, 8] (bf16 values, exact sums) give
the oracle's result bit for bit -- the test the Smallem page ("Rendre le GPU
rapide", section "Les Tensor Cores") relies on to catch fragment-layout
mistakes.  Times the identity, the result is the rounded operand itself, so
the hardware's rounding is compared with the page's bit for bit.  Other
inputs: the FP32 bar, |C_gpu - C_ref| <= 1e-6*K + 1e-5*|C_ref| elementwise
and relative Frobenius error <= 1e-6, with C_ref the mixed-precision oracle
(the products of rounded operands are exact in FP32, so only the FP32 sums
round).
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


def run_bf16(M, N, K, A, B, C, ta, tb, label="", offsets=(0, 0, 0)):
    """Call gemm_f32_bf16 on device copies; ``offsets`` shifts each pointer
    by that many floats into its (flat) buffer, for misaligned operands."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    lda, ldb, ldc = A.shape[1], B.shape[1], C.shape[1]
    bufs = []
    for x, off in zip((A, B, C), offsets):
        flat = np.concatenate([np.zeros(off, np.float32), np.ascontiguousarray(x).reshape(-1)])
        bufs.append(P.to_device(flat))
    dA, dB, dC = bufs
    P.note(f"bf16 {label} M={M} N={N} K={K} t{ta}{tb} ld {lda} {ldb} {ldc} off {offsets}")
    st = g.gemm_f32_bf16(M, N, K, dA.data_ptr() + 4 * offsets[0], lda,
                         dB.data_ptr() + 4 * offsets[1], ldb, dC.data_ptr() + 4 * offsets[2], ldc,
                         ta, tb, torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    return dC.cpu().numpy()[offsets[2]:].reshape(C.shape)


# The last shape has enough 256 x 256 tiles (12 x 12) to take the large
# tile, with partial tiles in every dimension and a partial last stage.
SHAPES = [(1, 1, 1), (37, 45, 29), (128, 128, 32), (129, 257, 95), (300, 200, 512),
          (1000, 1000, 1000), (2049, 700, 77), (3001, 2817, 100)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_small_integers_exact(oracle, shape, ta, tb):
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, 3, "int8", seed=7 * M + 3 * N + K)
    A, B = w.make_a(), w.make_b()
    out = run_bf16(M, N, K, A, B, w.make_c(), ta, tb, "int")
    P.check_padding(out, N)
    P.check_exact(out[:, :N], oracle.gemm_bf16(A, B, M, N, K, ta, tb), f"int {shape} t{ta}{tb}")


@pytest.mark.parametrize("shape", SHAPES[1:], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("dist", ["u11", "n01"])
def test_tolerance(oracle, shape, ta, tb, dist):
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, 1, dist, seed=11 * M + N + 5 * K)
    A, B = w.make_a(), w.make_b()
    out = run_bf16(M, N, K, A, B, w.make_c(), ta, tb, dist)
    P.check_padding(out, N)
    P.check_close(out[:, :N], oracle.gemm_bf16(A, B, M, N, K, ta, tb), K, f"{dist} {shape}")


@pytest.mark.parametrize("name", ["S64", "S1k", "R"])
def test_named_workloads(oracle, name):
    w = gi.WORKLOADS[name]
    A, B = w.make_a(), w.make_b()
    out = run_bf16(w.M, w.N, w.K, A, B, w.make_c(), w.transA, w.transB, name)
    P.check_padding(out, w.N)
    P.check_close(out[:, :w.N], oracle.gemm_bf16(A, B, w.M, w.N, w.K, w.transA, w.transB),
                  w.K, name)


@pytest.mark.parametrize("name", ["S4k", "T-fwd", "T-dX", "T-dW"])
def test_full_size_sampled(oracle, name):
    """Full-size products in the benchmark's launch configuration, checked
    on sampled entries of the oracle (one dot product each)."""
    w = gi.WORKLOADS[name]
    A, B = w.make_a(), w.make_b()
    out = run_bf16(w.M, w.N, w.K, A, B, w.make_c(), w.transA, w.transB, name)[:, :w.N]
    rows, cols = gi.sample_entries(w.M, w.N, 2000, seed=23)
    ref = oracle.entries_bf16(A, B, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
    got = out[rows, cols].astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= P.ELEM_ABS * w.K + P.ELEM_REL * np.abs(ref)), name
    assert np.linalg.norm(err) <= P.FROB_REL * np.linalg.norm(ref), name
    assert not np.any(np.isnan(out))


def _bit_patterns(rng, n, lo_exp=-100, hi_exp=100):
    """Float32 values of random sign, exponent in [lo_exp, hi_exp] and random
    significand bits; a third of them exact bf16 ties (low 16 bits 0x8000)."""
    sign = rng.integers(0, 2, n).astype(np.uint32) << 31
    exp = (rng.integers(lo_exp, hi_exp + 1, n) + 127).astype(np.uint32) << 23
    frac = rng.integers(0, 1 << 23, n).astype(np.uint32)
    tie = rng.random(n) < 1 / 3
    frac[tie] = (frac[tie] & 0x7F0000) | 0x8000
    return (sign | exp | frac).view(np.float32)


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)])
def test_rounding_matches_the_page_bit_for_bit(oracle, ta, tb):
    """op(A) . I = bf16(op(A)): every output is one product by 1 plus exact
    zeros, so the result is the rounded operand and nothing else."""
    rng = np.random.default_rng(29)
    M, K = 200, 96
    a = _bit_patterns(rng, M * K).reshape(M, K)
    A = np.ascontiguousarray(a.T if ta else a)
    B = np.eye(K, dtype=np.float32)
    out = run_bf16(M, K, K, A, B, np.zeros((M, K), np.float32), ta, tb, "round")
    want = oracle.round_bf16(a)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))
    # and the same through B: I . op(B) = bf16(op(B))
    b = _bit_patterns(rng, K * M).reshape(K, M)
    Bs = np.ascontiguousarray(b.T if tb else b)
    out = run_bf16(K, M, K, np.eye(K, dtype=np.float32), Bs, np.zeros((K, M), np.float32),
                   ta, tb, "roundB")
    assert np.array_equal(out.view(np.uint32), oracle.round_bf16(b).view(np.uint32))


def test_misaligned_operands_take_the_scalar_path(oracle):
    """Pointers off 16-byte alignment and odd leading dimensions."""
    for (M, N, K, ta, tb) in [(131, 67, 45, 0, 0), (64, 129, 200, 1, 1), (257, 128, 33, 0, 1),
                              (70, 300, 61, 1, 0)]:
        w = gi.make_case(M, N, K, ta, tb, 1, "int8", seed=M + N)
        A, B = w.make_a(), w.make_b()
        out = run_bf16(M, N, K, A, B, w.make_c(), ta, tb, "misaligned", offsets=(1, 3, 1))
        P.check_padding(out, N)
        P.check_exact(out[:, :N], oracle.gemm_bf16(A, B, M, N, K, ta, tb), "misaligned")


def test_k_zero_and_empty(oracle):
    M, N = 20, 37
    A = np.full((M, 1), np.nan, np.float32)
    B = np.full((1, N), np.nan, np.float32)
    out = run_bf16(M, N, 0, A, B, gi.output_matrix(M, N, N + 2), 0, 0, "k0")
    assert np.all(out[:, :N] == 0.0)
    P.check_padding(out, N)
    C = gi.output_matrix(4, N, N)
    out = run_bf16(0, N, 5, np.zeros((1, 5), np.float32), np.zeros((5, N), np.float32), C, 0, 0,
                   "m0")
    assert np.array_equal(out, C)


def test_repeatable(oracle):
    """Two calls on the same inputs give identical bits (no atomics)."""
    w = gi.WORKLOADS["R"]
    A, B = w.make_a(), w.make_b()
    one = run_bf16(w.M, w.N, w.K, A, B, w.make_c(), w.transA, w.transB, "rep1")
    two = run_bf16(w.M, w.N, w.K, A, B, w.make_c(), w.transA, w.transB, "rep2")
    assert np.array_equal(one.view(np.uint32), two.view(np.uint32))
