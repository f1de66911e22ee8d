"""GPU parity: every kernel family against the CPU oracle, through the C ABI.

Marked ``gpu``: needs an MI355X and the built library.  Inputs are seeded
(gemm_inputs); expected values come only from the oracle.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import parity as P

pytestmark = pytest.mark.gpu

ALGOS = ["mfma", "mfma256", "mfma128", "mfma64", "fma", "tiled", "naive"]
FAST_ALGOS = ["mfma256", "mfma128", "mfma64", "fma"]

_ref_cache = {}


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    lib = g.load()
    P.note(f"library {g.library_path()} version {g.gemm_f32_version()}")
    return lib


def workload_ref(oracle, w: gi.Workload):
    if w.name not in _ref_cache:
        A, B = w.make_a(), w.make_b()
        _ref_cache[w.name] = (A, B, oracle.gemm(A, B, w.M, w.N, w.K, w.transA, w.transB))
    return _ref_cache[w.name]


# ---------------------------------------------------------------- configs ---

@pytest.mark.parametrize("name", ["S64", "S1k", "R"])
@pytest.mark.parametrize("algo", ALGOS)
def test_config_full(oracle, algo, name):
    """Whole-matrix comparison on the workloads the oracle finishes in seconds."""
    w = gi.WORKLOADS[name]
    A, B, ref = workload_ref(oracle, w)
    out = P.run_gemm(algo, A, B, w.make_c(), w.M, w.N, w.K, w.transA, w.transB, label=name)
    P.check_padding(out, w.N)
    frob = P.check_close(out[:, :w.N], ref, w.K, f"{algo}/{name}")
    print(f"{algo} {name} relFrob={frob:.3g}")


@pytest.mark.parametrize("name", ["S4k", "T-fwd", "T-dX", "T-dW"])
@pytest.mark.parametrize("algo", ALGOS)
def test_config_sampled(oracle, algo, name):
    """Full-size workloads: sampled entries against the oracle one by one,
    and properties of the whole result (no NaN, padding untouched)."""
    w = gi.WORKLOADS[name]
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm(algo, A, B, w.make_c(), w.M, w.N, w.K, w.transA, w.transB, label=name)
    P.check_padding(out, w.N)
    region = out[:, :w.N]
    assert not np.any(np.isnan(region))
    rows, cols = gi.sample_entries(w.M, w.N, 3000, seed=17)
    ref = oracle.entries(A, B, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
    frob = P.check_close(region[rows, cols], ref, w.K, f"{algo}/{name} sampled")
    print(f"{algo} {name} sampled relFrob={frob:.3g}")


# ----------------------------------------------------------- exact layouts ---

EXACT_SHAPES = [(1, 1, 1), (37, 45, 29), (128, 128, 32), (129, 129, 33),
                (255, 257, 95), (2049, 3071, 769)]


def exact_case(oracle, M, N, K, ta, tb, extra):
    key = ("exact", M, N, K, ta, tb, extra)
    if key not in _ref_cache:
        w = gi.make_case(M, N, K, ta, tb, extra, "int8", seed=M * 7 + N * 13 + K)
        A, B = w.make_a(), w.make_b()
        _ref_cache[key] = (w, A, B, oracle.gemm(A, B, M, N, K, ta, tb))
    return _ref_cache[key]


@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ta,tb,extra", list(gi.iter_layouts()))
@pytest.mark.parametrize("algo", ALGOS)
def test_integer_exact_layouts(oracle, algo, ta, tb, extra, shape):
    """Integers in [-8, 8]: bit-for-bit equality for every transpose and ld
    padding, which pins fragment layouts, indexing and edge masks."""
    M, N, K = shape
    w, A, B, ref = exact_case(oracle, M, N, K, ta, tb, extra)
    out = P.run_gemm(algo, A, B, w.make_c(), M, N, K, ta, tb, label=w.name)
    P.check_padding(out, N)
    P.check_exact(out[:, :N], ref, f"{algo}/{w.name}")


@pytest.mark.parametrize("algo", ALGOS)
def test_shape_sweep_exact(oracle, algo):
    """Tiny sizes 1..70 in every dimension and tile sizes +-1, random layouts."""
    rng = np.random.default_rng(5)
    shapes = gi.shape_sweep()
    for (M, N, K) in shapes:
        ta, tb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        extra = int(rng.choice([0, 1, 3, 4]))
        w = gi.make_case(M, N, K, ta, tb, extra, "int8", seed=M + 1000 * N + 7 * K)
        A, B = w.make_a(), w.make_b()
        ref = oracle.gemm(A, B, M, N, K, ta, tb)
        out = P.run_gemm(algo, A, B, w.make_c(), M, N, K, ta, tb, label=w.name)
        P.check_padding(out, N)
        P.check_exact(out[:, :N], ref, f"{algo}/{w.name}")


# ------------------------------------------------------- degenerate cases ---

@pytest.mark.parametrize("algo", ALGOS)
def test_k_zero_writes_zeros(algo):
    M, N = 70, 33
    A = np.full((M, 1), np.nan, np.float32)
    B = np.full((1, N), np.nan, np.float32)         # K = 0: no row of B exists
    C = gi.output_matrix(M, N, N + 2)
    out = P.run_gemm(algo, A, B, C, M, N, 0, 0, 0, label="K=0")
    P.check_padding(out, N)
    assert np.all(out[:, :N] == 0.0)


@pytest.mark.parametrize("algo", ALGOS)
def test_empty_output_is_untouched(algo):
    A = np.ones((4, 4), np.float32)
    B = np.ones((4, 4), np.float32)
    C = gi.output_matrix(4, 4)
    for (M, N) in [(0, 4), (4, 0), (0, 0)]:
        out = P.run_gemm(algo, A, B, C, M, N, 4, 0, 0, label="empty")
        assert np.all(out == np.float32(gi.OUTPUT_PAD))


@pytest.mark.parametrize("algo", ALGOS)
def test_unaligned_and_odd_ld(oracle, algo):
    """Operands not 16-byte aligned and leading dimensions not multiples of 4
    take the element-wise load path and must give the same exact result."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    for (M, N, K, ta, tb) in [(131, 67, 45, 0, 0), (64, 129, 200, 1, 1), (257, 128, 33, 0, 1)]:
        a_rows, a_cols = (K, M) if ta else (M, K)
        b_rows, b_cols = (N, K) if tb else (K, N)
        lda, ldb, ldc = a_cols + 1, b_cols + 3, N + 1
        fa = P.ragged_operand(a_rows, a_cols, lda, 61, "int8", offset=1)
        fb = P.ragged_operand(b_rows, b_cols, ldb, 62, "int8", offset=3)
        A = fa[1:].reshape(a_rows, lda)
        B = fb[3:].reshape(b_rows, ldb)
        ref = oracle.gemm(A, B, M, N, K, ta, tb)
        dA, dB = P.to_device(fa), P.to_device(fb)
        dC = P.to_device(np.concatenate([np.zeros(1, np.float32),
                                         gi.output_matrix(M, N, ldc).reshape(-1)]))
        P.note(f"unaligned algo={algo} {M}x{N}x{K} t{ta}{tb}")
        st = g.gemm_f32_ex(M, N, K, dA.data_ptr() + 4, lda, dB.data_ptr() + 12, ldb,
                           dC.data_ptr() + 4, ldc, ta, tb,
                           torch.cuda.current_stream().cuda_stream, P.ALGO_IDS[algo])
        assert st == 0
        torch.cuda.synchronize()
        out = dC.cpu().numpy()[1:].reshape(M, ldc)
        P.check_padding(out, N)
        P.check_exact(out[:, :N], ref, f"unaligned {algo}")


@pytest.mark.parametrize("algo", ALGOS)
def test_long_k_and_thin_shapes(oracle, algo):
    """Very long K with tiny M x N, and many tiles along one dimension."""
    for (M, N, K) in [(1, 1, 1 << 18), (3, 2, 100003), (70001, 3, 5), (2, 40009, 7)]:
        w = gi.make_case(M, N, K, 0, 0, 0, "int8", seed=M + N + K)
        A, B = w.make_a(), w.make_b()
        ref = oracle.gemm(A, B, M, N, K, 0, 0)
        out = P.run_gemm(algo, A, B, w.make_c(), M, N, K, 0, 0, label=w.name)
        P.check_exact(out[:, :N], ref, f"{algo}/{w.name}")


# ------------------------------------------------ streams and repeatability ---

@pytest.mark.parametrize("algo", FAST_ALGOS)
def test_repeated_runs_bitwise_identical(algo):
    """20 runs give identical bits: no run-to-run race in the LDS pipeline."""
    import torch
    w = gi.WORKLOADS["R"]
    A, B = w.make_a(), w.make_b()
    first = P.run_gemm(algo, A, B, w.make_c(), w.M, w.N, w.K, 0, 0, label="R repeat")
    dA, dB, dC = P.to_device(A), P.to_device(B), P.to_device(w.make_c())
    import dense_fp32_matrix_gemm_amd as g
    for r in range(20):
        dC.fill_(-1.0)
        st = g.gemm_f32_ex(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                           dC.data_ptr(), w.ldc_, 0, 0, torch.cuda.current_stream().cuda_stream,
                           P.ALGO_IDS[algo])
        assert st == 0
        torch.cuda.synchronize()
        got = dC.cpu().numpy()
        assert np.array_equal(got[:, :w.N], first[:, :w.N]), f"run {r} differs"


def test_non_default_stream(oracle):
    import torch
    w = gi.WORKLOADS["S1k"]
    A, B, ref = workload_ref(oracle, w)
    s = torch.cuda.Stream()
    out = P.run_gemm("auto", A, B, w.make_c(), w.M, w.N, w.K, 0, 0, stream=s, label="stream")
    P.check_close(out, ref, w.K, "side stream")


def test_torch_matmul_views(oracle):
    """matmul() maps transposed views to the transpose flags without copies."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    X = gi.stored_matrix(3, 300, 200, dist="n01")
    W = gi.stored_matrix(4, 200, 500, dist="n002")
    dX, dW = P.to_device(X), P.to_device(W)
    for algo in ALGOS:
        ref = oracle.gemm(X, W, 300, 500, 200, 0, 0)
        P.check_close(g.matmul(dX, dW, algo=algo).cpu().numpy(), ref, 200, f"{algo} X.W")
        # (W^T)^T . X^T = (X W)^T, passing transposed views of W and X
        out = g.matmul(dW.t(), dX.t(), algo=algo)
        P.check_close(out.cpu().numpy(), ref.T, 200, f"{algo} W^T.X^T")
