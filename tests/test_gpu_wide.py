"""GPU parity of the 256 x 256 MFMA kernel (one running FP32 sum per output,
for aligned products with K <= 1024, any transposes).

Marked ``gpu``.  The kernel is called directly (GEMM_F32_ALGO_MFMA_WIDE) on
problems in its domain, and through the automatic choice, the batched entry
point and the fused epilogue on problems large enough to select it (at least
256 tiles of 256 x 256).  Expected values come only from the oracle; that a
path selected this kernel is shown by bit-for-bit agreement with the direct
call on floating-point data, where any other kernel sums in another order.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import oracle as oracle_pkg
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


# single stage; two and three stages; many tiles, ragged tile grid
# (3 x 1); the longest k it takes
EXACT_SHAPES = [(256, 256, 32), (256, 512, 64), (512, 768, 96), (768, 256, 1024)]


LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.mark.parametrize("extra", [0, 4])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_integer_exact(oracle, shape, ta, tb, extra):
    """Integers in [-8, 8] (every partial sum exact): bit-for-bit equality in
    every layout, which pins the copy swizzles, the fragment maps and the
    store map; padded leading dimensions (multiples of 4) and C's padding
    untouched."""
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, extra, "int8", seed=M + 5 * N + 11 * K + extra + 2 * ta + tb)
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm("mfmawide", A, B, w.make_c(), M, N, K, ta, tb, label=w.name)
    P.check_padding(out, N)
    P.check_exact(out[:, :N], oracle.gemm(A, B, M, N, K, ta, tb), w.name)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("dist", ["u11", "n01"])
@pytest.mark.parametrize("shape", [(512, 512, 1024), (1024, 768, 512)], ids=lambda s: "x".join(map(str, s)))
def test_float_tolerance(oracle, shape, dist, ta, tb):
    """Floating-point data within the 1e-6 bounds at K up to 1024."""
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, 4, dist, seed=M + N + K + 2 * ta + tb)
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm("mfmawide", A, B, w.make_c(), M, N, K, ta, tb, label=w.name)
    P.check_padding(out, N)
    frob = P.check_close(out[:, :N], oracle.gemm(A, B, M, N, K, ta, tb), K, w.name)
    print(f"wide {w.name} relFrob={frob:.3g}")


@pytest.mark.parametrize("shape,ta,tb", [((4096, 4096, 1024), 0, 0), ((8192, 4096, 1024), 0, 0),
                                         ((8192, 4096, 1024), 0, 1), ((4096, 4096, 512), 1, 0),
                                         ((4096, 4096, 256), 1, 1)],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_auto_selects_it_at_full_size(oracle, shape, ta, tb):
    """256 and 512 tiles: the automatic choice runs this kernel (bit-for-bit
    equal to the direct call), and sampled entries meet the bounds."""
    M, N, K = shape
    w = gi.make_case(M, N, K, ta, tb, 0, "n01", seed=3 * M + K + ta + 2 * tb)
    A, B = w.make_a(), w.make_b()
    auto = P.run_gemm("auto", A, B, w.make_c(), M, N, K, ta, tb, label=w.name)
    wide = P.run_gemm("mfmawide", A, B, w.make_c(), M, N, K, ta, tb, label=w.name)
    assert np.array_equal(auto, wide)
    rows, cols = gi.sample_entries(M, N, 3000, seed=23)
    ref = oracle.entries(A, B, M, N, K, ta, tb, rows, cols)
    frob = P.check_close(wide[rows, cols], ref, K, f"{w.name} sampled")
    print(f"wide {w.name} sampled relFrob={frob:.3g}")


def _batched(w, A, B):
    import torch
    import dense_fp32_matrix_gemm_amd as g
    dA, dB, dC = P.to_device(A), P.to_device(B), P.to_device(w.make_c())
    P.note(f"wide batched {w.name} batch={w.batch} t{w.transA}{w.transB}")
    st = g.gemm_f32_strided_batched(w.M, w.N, w.K, dA.data_ptr(), w.lda_, w.stride_a,
                                    dB.data_ptr(), w.ldb_, w.stride_b, dC.data_ptr(), w.ldc_,
                                    w.stride_c, w.batch, w.transA, w.transB,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    flat = dC.cpu().numpy().reshape(w.batch, w.stride_c)
    body = flat[:, :w.M * w.ldc_].reshape(w.batch, w.M, w.ldc_)
    return body[:, :, :w.N], flat


@pytest.mark.parametrize("tb", [0, 1])
@pytest.mark.parametrize("dist", ["int8", "n01"])
def test_batched(dist, tb):
    """64 products of 512 x 512 x 64 (256 tiles; with B transposed this is
    the attention-score batch): the batched entry point selects this kernel;
    exact on integers, and on floats each product is bit-for-bit the direct
    single-product call and within the bounds."""
    w = gi.Workload("wide-batch", 512, 512, 64, 91 + tb, 92, dist, dist, transB=tb, batch=64,
                    ldc=512 + 4, gap=8)
    A, B = w.make_a(), w.make_b()
    got, flat = _batched(w, A, B)
    pad = np.concatenate([flat[:, :w.M * w.ldc_].reshape(w.batch, w.M, w.ldc_)[:, :, w.N:].reshape(-1),
                          flat[:, w.M * w.ldc_:].reshape(-1)])
    assert np.all(pad == np.float32(gi.OUTPUT_PAD))
    ref = oracle_pkg.gemm_ref_batched(A, B, w.M, w.N, w.K, 0, tb, w.lda_, w.stride_a, w.ldb_,
                                      w.stride_b, w.batch)
    b_rows = w.N if tb else w.K
    for b in (0, 1, 37, 63):
        if dist == "int8":
            P.check_exact(got[b], ref[b], f"batch[{b}]")
            continue
        P.check_close(got[b], ref[b], w.K, f"batch[{b}]")
        Ab = A.reshape(-1)[b * w.stride_a: b * w.stride_a + w.M * w.lda_].reshape(w.M, w.lda_)
        Bb = B.reshape(-1)[b * w.stride_b: b * w.stride_b + b_rows * w.ldb_].reshape(b_rows, w.ldb_)
        one = P.run_gemm("mfmawide", Ab, Bb, gi.output_matrix(w.M, w.N), w.M, w.N, w.K, 0, tb,
                         label=f"batch[{b}] alone")
        assert np.array_equal(one, got[b])


def test_fused_epilogue_selects_it(oracle):
    """bias + GELU on 4096 x 4096 x 64 (256 tiles), sampled against the
    oracle's product and epilogue; with integers and bias only, exact."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    M, N, K = 4096, 4096, 64
    for dist, act in (("int8", 0), ("n01", 1)):
        w = gi.make_case(M, N, K, 0, 0, 0, dist, seed=77)
        A, B = w.make_a(), w.make_b()
        bias = gi.stored_matrix(78, 1, N, dist=dist)[0]
        dA, dB, dC, db = P.to_device(A), P.to_device(B), P.to_device(w.make_c()), P.to_device(bias)
        P.note(f"wide fused {w.name} act={act}")
        st = g.gemm_f32_bias_act(M, N, K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_, dC.data_ptr(),
                                 w.ldc_, 0, 0, db.data_ptr(), act, torch.cuda.current_stream().cuda_stream)
        assert st == 0, g.gemm_f32_strerror(st)
        torch.cuda.synchronize()
        out = dC.cpu().numpy()
        if act == 0:
            P.check_exact(out, oracle.epilogue(oracle.gemm(A, B, M, N, K), bias, 0), "integer bias")
            continue
        rows, cols = gi.sample_entries(M, N, 3000, seed=29)
        pre = oracle.entries(A, B, M, N, K, 0, 0, rows, cols) + bias[cols].astype(np.float64)
        ref = oracle.epilogue(pre[None, :], None, 1)[0]
        err = np.abs(out[rows, cols].astype(np.float64) - ref)
        bound = 1.2 * (1e-6 * K + 1e-5 * np.abs(pre)) + 5e-7 * np.abs(pre)
        assert np.all(err <= bound)
        assert not np.any(np.isnan(out))
