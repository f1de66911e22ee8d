"""GPU parity of the strided-batched product against the CPU oracle.

Marked ``gpu``.  Expected values come only from ``oracle.gemm_ref_batched``
(the plain product applied to each matrix of the batch).
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


def run_batched(w: gi.Workload, A, B, C, batch=None):
    import torch
    import dense_fp32_matrix_gemm_amd as g
    batch = w.batch if batch is None else batch
    dA, dB, dC = P.to_device(A), P.to_device(B), P.to_device(C)
    P.note(f"batched {w.name} batch={batch} M={w.M} N={w.N} K={w.K} t{w.transA}{w.transB} "
           f"strides {w.stride_a} {w.stride_b} {w.stride_c}")
    st = g.gemm_f32_strided_batched(w.M, w.N, w.K, dA.data_ptr(), w.lda_, w.stride_a,
                                    dB.data_ptr(), w.ldb_, w.stride_b, dC.data_ptr(), w.ldc_,
                                    w.stride_c, batch, w.transA, w.transB,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def split_c(w: gi.Workload, out: np.ndarray):
    """(batch, M, N) results and the padding/gap floats of the flat output."""
    flat = out.reshape(w.batch, w.stride_c)
    body = flat[:, :w.M * w.ldc_].reshape(w.batch, w.M, w.ldc_)
    pad = np.concatenate([body[:, :, w.N:].reshape(-1), flat[:, w.M * w.ldc_:].reshape(-1)])
    return body[:, :, :w.N], pad


def reference(w: gi.Workload, A, B):
    return oracle_pkg.gemm_ref_batched(A, B, w.M, w.N, w.K, w.transA, w.transB, w.lda_,
                                       w.stride_a, w.ldb_, w.stride_b, w.batch)


@pytest.mark.parametrize("name", ["attn-qk", "attn-pv"])
def test_attention_workloads(name):
    w = gi.WORKLOADS[name]
    A, B = w.make_a(), w.make_b()
    out = run_batched(w, A, B, w.make_c())
    got, pad = split_c(w, out)
    assert np.all(pad == np.float32(gi.OUTPUT_PAD))
    ref = reference(w, A, B)
    for b in range(w.batch):
        P.check_close(got[b], ref[b], w.K, f"{name}[{b}]")


LAYOUT_CASES = [(ta, tb, gap, shared) for ta in (0, 1) for tb in (0, 1)
                for gap, shared in ((0, False), (5, False), (3, True))]


@pytest.mark.parametrize("ta,tb,gap,shared", LAYOUT_CASES)
@pytest.mark.parametrize("shape", [(33, 47, 29, 6), (130, 70, 65, 3), (257, 129, 40, 4)],
                         ids=lambda s: "x".join(map(str, s)))
def test_integer_exact_batched(ta, tb, gap, shared, shape):
    M, N, K, batch = shape
    w = gi.Workload(f"b{M}x{N}x{K}", M, N, K, 50 + M, 60 + N, "int8", "int8", ta, tb,
                    lda=(M if ta else K) + 1, ldb=(K if tb else N) + 2, ldc=N + 3,
                    batch=batch, gap=gap, shared_b=shared)
    A, B = w.make_a(), w.make_b()
    got, pad = split_c(w, run_batched(w, A, B, w.make_c()))
    assert np.all(pad == np.float32(gi.OUTPUT_PAD))
    ref = reference(w, A, B)
    for b in range(batch):
        P.check_exact(got[b], ref[b], f"{w.name}[{b}] t{ta}{tb} gap{gap} shared{shared}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_integer_exact_batched_paired_small_tiles(ta, tb):
    """More 64 x 64 tiles than CUs over the batch (4 x 4 x 20 = 320), with
    16-byte aligned leading dimensions and strides: the two-workgroups-per-CU
    tile with its copies into LDS, a partial last k stage (K = 70) and the
    k-slices' halved final exchange.  Exact against the oracle."""
    M, N, K, batch = 256, 200, 70, 20
    w = gi.Workload(f"b{M}x{N}x{K}p", M, N, K, 93, 94, "int8", "int8", ta, tb,
                    lda=(M if ta else K) + 2 + (2 if ta else 0), ldb=(K if tb else N) + (2 if tb else 4),
                    ldc=N + 4, batch=batch)
    assert w.lda_ % 4 == 0 and w.ldb_ % 4 == 0 and w.stride_a % 4 == 0 and w.stride_b % 4 == 0
    import dense_fp32_matrix_gemm_amd as g
    plan = g.gemm_f32_plan(M, N, K, 1 << 20, w.lda_, 1 << 20, w.ldb_, w.ldc_, ta, tb, w.stride_a,
                           w.stride_b, batch)
    assert g.PLANS[plan] == "mfma-64x64-pair", g.PLANS.get(plan, plan)
    A, B = w.make_a(), w.make_b()
    got, pad = split_c(w, run_batched(w, A, B, w.make_c()))
    assert np.all(pad == np.float32(gi.OUTPUT_PAD))
    ref = reference(w, A, B)
    for b in range(batch):
        P.check_exact(got[b], ref[b], f"{w.name}[{b}] t{ta}{tb}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("gap", [1, 3])
def test_integer_exact_batched_aligned_ld_odd_stride(ta, tb, gap):
    """Leading dimensions that are multiples of 4 with strides that are not:
    product 0 is 16-byte aligned, products 1.. are not, so every product must
    take the element-wise loads.  Exact against the oracle."""
    M, N, K, batch = 136, 200, 72, 5
    w = gi.Workload(f"b{M}x{N}x{K}a", M, N, K, 91, 92, "int8", "int8", ta, tb,
                    lda=(M if ta else K) + 4, ldb=(K if tb else N) + 8, ldc=N + 4,
                    batch=batch, gap=gap)
    assert w.lda_ % 4 == 0 and w.ldb_ % 4 == 0 and w.stride_a % 4 != 0 and w.stride_b % 4 != 0
    A, B = w.make_a(), w.make_b()
    got, pad = split_c(w, run_batched(w, A, B, w.make_c()))
    assert np.all(pad == np.float32(gi.OUTPUT_PAD))
    ref = reference(w, A, B)
    for b in range(batch):
        P.check_exact(got[b], ref[b], f"{w.name}[{b}] t{ta}{tb} gap{gap}")


def test_batch_zero_and_k_zero():
    w = gi.Workload("kz", 20, 30, 0, 1, 2, transB=0, batch=3, gap=2, lda=1, ldb=30)
    A = np.full((3, 20 * 1 + 2), np.nan, np.float32)
    B = np.full((3, 1 * 30 + 2), np.nan, np.float32)
    C = w.make_c()
    got, pad = split_c(w, run_batched(w, A, B, C))
    assert np.all(got == 0.0) and np.all(pad == np.float32(gi.OUTPUT_PAD))
    untouched = run_batched(w, A, B, C, batch=0)
    assert np.all(untouched == np.float32(gi.OUTPUT_PAD))


def test_batch_beyond_grid_y_limit():
    """More products than one launch's grid y allows (65535): split launches."""
    w = gi.Workload("many", 3, 5, 4, 70, 71, "int8", "int8", batch=70000)
    A, B = w.make_a(), w.make_b()
    got, _ = split_c(w, run_batched(w, A, B, w.make_c()))
    ref = reference(w, A, B)
    P.check_exact(got.reshape(-1, w.N), ref.reshape(-1, w.N), "batch 70000")


def test_bmm_views():
    """bmm() maps a transposed key view and an expanded (stride 0) operand."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    q = P.to_device(gi.stored_batch(81, 6, 100, 64, 64, 0, "n01").reshape(6, 100, 64))
    k = P.to_device(gi.stored_batch(82, 6, 120, 64, 64, 0, "n01").reshape(6, 120, 64))
    scores = g.bmm(q, k.transpose(1, 2)).cpu().numpy()
    ref = oracle_pkg.gemm_ref_batched(q.cpu().numpy(), k.cpu().numpy(), 100, 120, 64, 0, 1,
                                      64, 100 * 64, 64, 120 * 64, 6)
    for b in range(6):
        P.check_close(scores[b], ref[b], 64, f"q.k^T[{b}]")
    w = P.to_device(gi.stored_matrix(83, 64, 32, dist="n002"))
    out = g.bmm(q, w.unsqueeze(0).expand(6, 64, 32)).cpu().numpy()
    ref = oracle_pkg.gemm_ref_batched(q.cpu().numpy(), w.cpu().numpy(), 100, 32, 64, 0, 0,
                                      64, 100 * 64, 32, 0, 6)
    for b in range(6):
        P.check_close(out[b], ref[b], 64, f"q.W[{b}]")
