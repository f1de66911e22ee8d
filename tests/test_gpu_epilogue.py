"""GPU parity of the fused epilogue C = act(op(A) . op(B) + bias).

Marked ``gpu``.  Expected values: the oracle's double product followed by
the oracle's double epilogue (``Oracle.epilogue``).

Tolerance.  With y the exact product, b the bias and E = 1e-6*K + 1e-5*|y|
the product's bound (as for the plain GEMM), the FP32 bias add adds at most
half an ulp of |y + b|, GELU's slope lies in [-0.17, 1.13], and the FP32
evaluation of x * Phi(x) (erff included) adds a few ulp of |y + b|.  Hence
    |C_gpu - act(y + b)| <= 1.2 * E + 5e-7 * |y + b|
elementwise, and the same bound on Frobenius norms.  With no activation and
integer data the result must be exact.
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


def run_fused(w: gi.Workload, A, B, C, bias, act):
    import torch
    import dense_fp32_matrix_gemm_amd as g
    dA, dB, dC = P.to_device(A), P.to_device(B), P.to_device(C)
    dbias = None if bias is None else P.to_device(bias)
    P.note(f"fused {w.name} act={act} bias={bias is not None}")
    st = g.gemm_f32_bias_act(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                             dC.data_ptr(), w.ldc_, w.transA, w.transB,
                             None if dbias is None else dbias.data_ptr(), act,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def check_fused(got, pre, ref, K, what):
    """pre = exact y + b (float64), ref = act(pre) (float64)."""
    got = got.astype(np.float64)
    assert not np.any(np.isnan(got)), what
    err = np.abs(got - ref)
    bound = 1.2 * (1e-6 * K + 1e-5 * np.abs(pre)) + 5e-7 * np.abs(pre)
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(err <= bound), f"{what}: elementwise bound exceeded (worst {worst:.3g})"
    frob_bound = 1.2 * (1e-6 * K * np.sqrt(err.size) + 1e-5 * np.linalg.norm(pre)) + \
        5e-7 * np.linalg.norm(pre)
    assert np.linalg.norm(err) <= frob_bound, what


# small tiles (with the extra-row workgroups at M = 129), the 64 x 64 tile
# two workgroups per CU (1100 x 1000: 288 tiles; 1089 rows: plus one extra
# row), and the 128 x 128 tile
CASES = [(37, 45, 29), (129, 257, 95), (300, 200, 512), (1100, 1000, 300), (1089, 1000, 301),
         (2300, 4100, 200)]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("act,with_bias", [(1, True), (1, False), (0, True)])
def test_fused_epilogue(oracle, shape, ta, tb, act, with_bias):
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, 3, "n01", seed=M + 3 * N + 5 * K)
    A, B = w.make_a(), w.make_b()
    bias = gi.stored_matrix(17 + N, 1, N, dist="n01")[0] if with_bias else None
    y = oracle.gemm(A, B, M, N, K, ta, tb)
    pre = oracle.epilogue(y, bias, 0)
    ref = oracle.epilogue(y, bias, act)
    out = run_fused(w, A, B, w.make_c(), bias, act)
    P.check_padding(out, N)
    check_fused(out[:, :N], pre, ref, K, f"{w.name} act={act} bias={with_bias}")


@pytest.mark.parametrize("shape", [(70, 33, 40), (2300, 4100, 64)], ids=lambda s: "x".join(map(str, s)))
def test_bias_exact_on_integers(oracle, shape):
    M, N, K = shape
    w = gi.make_case(M, N, K, 0, 0, 1, "int8", seed=M + N + K)
    A, B = w.make_a(), w.make_b()
    bias = gi.stored_matrix(5, 1, N, dist="int8")[0]
    ref = oracle.epilogue(oracle.gemm(A, B, M, N, K), bias, 0)
    out = run_fused(w, A, B, w.make_c(), bias, 0)
    P.check_padding(out, N)
    P.check_exact(out[:, :N], ref, "integer bias")


def test_mlp_forward_full_size(oracle):
    """GELU(X . W + b) on the 8192 x 1024 x 4096 forward product, sampled."""
    w = gi.WORKLOADS["T-fwd"]
    A, B = w.make_a(), w.make_b()
    bias = gi.stored_matrix(2003, 1, w.N, dist="n002")[0]
    out = run_fused(w, A, B, w.make_c(), bias, 1)[:, :w.N]
    rows, cols = gi.sample_entries(w.M, w.N, 3000, seed=19)
    y = oracle.entries(A, B, w.M, w.N, w.K, 0, 0, rows, cols)
    pre = y + bias[cols].astype(np.float64)
    ref = oracle.epilogue(pre[None, :], None, 1)[0]
    check_fused(out[rows, cols], pre, ref, w.K, "T-fwd gelu sampled")
    assert not np.any(np.isnan(out))


def test_k_zero_gives_act_of_bias(oracle):
    M, N = 20, 37
    w = gi.Workload("kz", M, N, 0, 1, 2, lda=1, ldb=N)
    A = np.full((M, 1), np.nan, np.float32)
    B = np.full((1, N), np.nan, np.float32)
    bias = gi.stored_matrix(9, 1, N, dist="n01")[0]
    out = run_fused(w, A, B, w.make_c(), bias, 1)
    ref = oracle.epilogue(np.zeros((M, N)), bias, 1)
    check_fused(out[:, :N], np.broadcast_to(bias.astype(np.float64), (M, N)), ref, 0, "K=0")


def test_linear_helper(oracle):
    import torch
    import dense_fp32_matrix_gemm_amd as g
    X = gi.stored_matrix(31, 256, 300, dist="n01")
    W = gi.stored_matrix(32, 300, 200, dist="n002")
    b = gi.stored_matrix(33, 1, 200, dist="n002")[0]
    out = g.linear(P.to_device(X), P.to_device(W), P.to_device(b), "gelu").cpu().numpy()
    y = oracle.gemm(X, W, 256, 200, 300)
    check_fused(out, oracle.epilogue(y, b, 0), oracle.epilogue(y, b, 1), 300, "linear")
