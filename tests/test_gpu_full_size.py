"""Whole-matrix parity at the full-size workloads, on the automatic path and
on the entry points that run at those sizes.

Marked ``gpu``.  Expected values come only from the oracle, over every
element of C (no sampling):
  * integer inputs in [-8, 8] at the exact full shape: every partial sum is
    an integer of magnitude at most 64 * 8192 < 2^24, hence exact in FP32 in
    any order, so C must equal the oracle bit for bit.  Integers of this
    size are also exact in bf16, so the same oracle result pins the
    mixed-precision entry points;
  * the seeded float inputs of each workload: elementwise
    |C - C_ref| <= 1e-6 K + 1e-5 |C_ref| and relative Frobenius <= 1e-6 over
    the whole M x N matrix.
Each oracle product takes 10-25 s on 16 host cores; results are cached per
module so that each is computed once.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import parity as P

pytestmark = pytest.mark.gpu

FULL = ["S4k", "T-fwd", "T-dX", "T-dW"]
_cache = {}


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


def case(oracle, name, dist):
    """(workload, A, B, oracle C) for a full-size workload with its own
    inputs (dist None) or integer inputs in [-8, 8] of the same shapes."""
    key = (name, dist)
    if key not in _cache:
        w = gi.WORKLOADS[name]
        if dist is not None:
            w = w.with_dist(dist)
        A, B = w.make_a(), w.make_b()
        P.note(f"oracle {w.name} {w.M}x{w.N}x{w.K}")
        _cache[key] = (w, A, B, oracle.gemm(A, B, w.M, w.N, w.K, w.transA, w.transB))
    return _cache[key]


@pytest.mark.parametrize("name", FULL + ["S1k", "R"])
def test_integer_exact_whole_matrix(oracle, name):
    w, A, B, ref = case(oracle, name, "int8")
    assert np.max(np.abs(ref)) < 2 ** 24
    out = P.run_gemm("auto", A, B, w.make_c(), w.M, w.N, w.K, w.transA, w.transB, label=w.name)
    P.check_padding(out, w.N)
    P.check_exact(out[:, :w.N], ref, f"auto/{w.name}")


@pytest.mark.parametrize("name", FULL)
def test_float_whole_matrix(oracle, name):
    w, A, B, ref = case(oracle, name, None)
    out = P.run_gemm("auto", A, B, w.make_c(), w.M, w.N, w.K, w.transA, w.transB, label=w.name)
    P.check_padding(out, w.N)
    frob = P.check_close(out[:, :w.N], ref, w.K, f"auto/{w.name} whole matrix")
    print(f"auto {name} whole-matrix relFrob={frob:.3g}")


def test_forward_takes_the_wide_tile():
    """The 8192 x 4096 x 1024 forward product runs on the 256 x 256 kernel,
    so the two tests above pin that kernel at full size."""
    import dense_fp32_matrix_gemm_amd as g
    w = gi.WORKLOADS["T-fwd"]
    plan = g.gemm_f32_plan(w.M, w.N, w.K, 4096, w.lda_, 4096, w.ldb_, w.ldc_, w.transA, w.transB)
    assert g.PLANS[plan] == "mfma-256x256"


def _splitk(w, A, B, splits):
    import torch
    import dense_fp32_matrix_gemm_amd as g
    need = g.gemm_f32_splitk_workspace_size(w.M, w.N, w.K, splits)
    dA, dB, dC = P.to_device(A), P.to_device(B), P.to_device(w.make_c())
    ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    P.note(f"splitk whole matrix {w.name} splits={splits}")
    st = g.gemm_f32_splitk(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                           dC.data_ptr(), w.ldc_, w.transA, w.transB, splits, ws.data_ptr(), need,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


@pytest.mark.parametrize("splits", [2, 4])
@pytest.mark.parametrize("dist", ["int8", None], ids=["int", "float"])
def test_splitk_weight_gradient_whole_matrix(oracle, dist, splits):
    """X^T . dY (1024 x 4096 x 8192) as per-run partial products plus their sum."""
    w, A, B, ref = case(oracle, "T-dW", dist)
    out = _splitk(w, A, B, splits)
    P.check_padding(out, w.N)
    if dist == "int8":
        P.check_exact(out[:, :w.N], ref, f"splitk {splits} {w.name}")
    else:
        frob = P.check_close(out[:, :w.N], ref, w.K, f"splitk {splits} {w.name}")
        print(f"splitk {splits} T-dW whole-matrix relFrob={frob:.3g}")


def test_fused_gelu_forward_whole_matrix(oracle):
    """GELU(X . W + b) at 8192 x 4096 x 1024, every element, to the fused
    epilogue's bound (the product's bound carried through GELU's slope,
    which lies in [-0.17, 1.13], plus a few ulp for the bias add and the
    activation)."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    w, A, B, y = case(oracle, "T-fwd", None)
    bias = gi.stored_matrix(2003, 1, w.N, dist="n002")[0]
    pre = oracle.epilogue(y, bias, 0)
    ref = oracle.epilogue(y, bias, 1)
    dA, dB, dC, db = P.to_device(A), P.to_device(B), P.to_device(w.make_c()), P.to_device(bias)
    P.note("fused gelu whole matrix T-fwd")
    st = g.gemm_f32_bias_act(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                             dC.data_ptr(), w.ldc_, w.transA, w.transB, db.data_ptr(), g.ACT_GELU,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    P.check_padding(out, w.N)
    got = out[:, :w.N].astype(np.float64)
    err = np.abs(got - ref)
    bound = 1.2 * (1e-6 * w.K + 1e-5 * np.abs(pre)) + 5e-7 * np.abs(pre)
    assert np.all(err <= bound), f"worst {np.max(err / bound):.3g}"


@pytest.mark.parametrize("name", ["S4k", "T-dX"])
def test_bf16_integer_exact_whole_matrix(oracle, name):
    """Integers in [-8, 8] are exact in bf16, so both mixed-precision paths
    (rounding on every read, and packed operands) must equal the FP32
    oracle's integer product bit for bit over the whole matrix."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    w, A, B, ref = case(oracle, name, "int8")
    dA, dB = P.to_device(A), P.to_device(B)
    op_a = dA[:, :w.a_dims[1]]
    op_b = dB[:, :w.b_dims[1]]
    op_a = op_a.t() if w.transA else op_a
    op_b = op_b.t() if w.transB else op_b
    P.note(f"bf16 one step whole matrix {w.name}")
    one = g.matmul_bf16(op_a, op_b)
    P.note(f"bf16 packed whole matrix {w.name}")
    packed = g.matmul_bf16_packed(g.pack_bf16(op_a), g.pack_bf16(op_b.t()))
    torch.cuda.synchronize()
    P.check_exact(one.cpu().numpy(), ref, f"bf16/{w.name}")
    P.check_exact(packed.cpu().numpy(), ref, f"bf16 packed/{w.name}")
