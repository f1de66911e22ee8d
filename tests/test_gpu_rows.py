"""GPU parity of the row reductions (include/rows_f32.h) against the oracle
(oracle/rows.py): causal and plain softmax, its gradient, the row
normalisation and its gradient.

Marked ``gpu``.  Expected values come only from the oracle (float64).

Tolerances, derived from FP32 arithmetic with unit roundoff u = 2^-24
(about 6e-8) and the inputs used here (|scale * x| below about 8, rows up
to 5000 long, wave sums of at most log2(64) + 13 levels):
  softmax          |dy| <= 1e-5 * y + 1e-8: the exponent's argument
                   (scale*x - max - log sum) carries a few u per term plus
                   the log of the sum's relative error, at most ~2e-6 in
                   all; exp turns that into a relative error.  Masked
                   entries must be exactly 0.
  softmax grad     |ddx| <= 1e-5 * |scale| * y * (|dy| + S) + 1e-9, S the
                   row's sum of |dy * y|: the row sum d is off by about
                   u * S * levels, and dy - d and the products add a few u.
  normalize        |dy| <= 1e-5 * (|y| + 1): mean and variance are off by
                   about u * levels relative to the row's scale, the root
                   and division by a few u.
  normalize grad   |ddx| <= 2e-5 * (|dx| + r * (|dy| + mean|dy| + |xhat| *
                   mean|dy * xhat|)) + 1e-9, r = 1 / sigma: each of the
                   three terms carries the normalize error above.
Padding columns of every output must keep their sentinel; runs repeat bit
for bit.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import parity as P
from oracle import rows as R

pytestmark = pytest.mark.gpu

PAD = np.float32(-5555.0)


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


def stored(seed, rows, width, ld, dist="n01", scale=1.0):
    x = gi.stored_matrix(seed, rows, width, ld, dist)
    if scale != 1.0:
        x[:, :width] *= np.float32(scale)
    return x


def out_buffer(rows, ld):
    return np.full((rows, ld), PAD, np.float32)


def call(fn, *args):
    import torch
    import dense_fp32_matrix_gemm_amd as g
    st = getattr(g, fn)(*args, torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"{fn} status {st}"
    torch.cuda.synchronize()


def check_padding(out, width):
    assert np.all(out[:, width:] == PAD), "wrote into the padding"


# ---------------------------------------------------------------- softmax ---

def run_softmax(x, rows, width, queries, causal, scale, ldy, offset=0):
    dx = P.to_device(np.concatenate([np.zeros(offset, np.float32), x.reshape(-1)]))
    dy = P.to_device(np.concatenate([np.zeros(offset, np.float32), out_buffer(rows, ldy).reshape(-1)]))
    P.note(f"softmax rows={rows} width={width} q={queries} causal={causal} ld={x.shape[1]}/{ldy} off={offset}")
    call("rows_softmax_f32", rows, width, queries, causal, scale, dx.data_ptr() + 4 * offset,
         x.shape[1], dy.data_ptr() + 4 * offset, ldy)
    return dy.cpu().numpy()[offset:].reshape(rows, ldy)


def check_softmax(got, ref, width):
    check_padding(got, width)
    y = got[:, :width].astype(np.float64)
    masked = ref == 0.0
    assert np.all(y[masked] == 0.0), "masked entries must be exactly 0"
    err = np.abs(y - ref)
    bound = 1e-5 * ref + 1e-8
    assert np.all(err <= bound), f"softmax: worst ratio {np.max(err / bound):.3g}"


SOFTMAX_CASES = [  # rows, width, queries, causal, scale, extra ld
    (7, 1, 1, 1, 1.0, 0), (33, 3, 3, 1, 1.0, 1), (64, 64, 64, 1, 0.125, 0), (65, 100, 5, 1, 1.0, 3),
    (40, 255, 255, 0, 0.5, 1), (30, 256, 256, 1, 0.125, 4), (30, 257, 7, 1, 1.0, 0),
    (24, 512, 512, 1, 0.125, 0), (24, 1000, 1, 1, 1.0, 2), (16, 1024, 1024, 0, 0.125, 4),
    (12, 2048, 2048, 1, 0.125, 0), (10, 4096, 4096, 1, 0.125, 4), (9, 4097, 4097, 1, 0.125, 1),
    (6, 5000, 3, 1, 0.25, 0), (40000, 32, 32, 1, 1.0, 0),
]


@pytest.mark.parametrize("case", SOFTMAX_CASES, ids=lambda c: "r{}w{}q{}c{}ld+{}".format(*c[:4], c[5]))
def test_softmax(case):
    rows, width, queries, causal, scale, extra = case
    x = stored(rows * 31 + width, rows, width, width + extra)
    got = run_softmax(x, rows, width, queries, causal, scale, width + extra)
    check_softmax(got, R.softmax(x, width, queries, scale, bool(causal)), width)


def test_softmax_never_reads_the_future_or_padding():
    rows, width, queries = 48, 300, 12
    x = stored(4, rows, width, width + 4)
    ref = R.softmax(x, width, queries, 0.3)
    pos = R.positions(rows, width, queries)
    for r in range(rows):
        x[r, pos[r] + 1:] = np.nan          # future and padding
    got = run_softmax(x, rows, width, queries, 1, 0.3, width + 4)
    check_softmax(got, ref, width)


def test_softmax_unaligned_and_in_place():
    import torch
    import dense_fp32_matrix_gemm_amd as g
    rows, width = 50, 512
    x = stored(5, rows, width, width)
    ref = R.softmax(x, width, width, 0.125)
    check_softmax(run_softmax(x, rows, width, width, 1, 0.125, width, offset=1), ref, width)
    d = P.to_device(x)
    P.note("softmax in place")
    out = g.softmax(d, 0.125, out=d)
    torch.cuda.synchronize()
    check_softmax(out.cpu().numpy(), ref, width)


def test_softmax_minus_infinity_scores():
    """Scores of -inf (an additive padding mask) before a lane's first finite
    score: the streamed path for rows longer than 4096 and the register path
    at 4096 both give the oracle's values, 0 at every -inf."""
    rows = 6
    for width, causal in ((4096, 0), (4097, 0), (5000, 0), (4100, 1)):
        x = stored(71, rows, width, width + 1)
        x[:, :130] = -np.inf                # every lane's first two scores
        x[::2, 300:900:7] = -np.inf         # scattered further on
        x[3, 4000:] = -np.inf
        queries = rows                      # causal: rows keep 4095..4100 columns
        ref = R.softmax(x, width, queries, 0.125, bool(causal))
        assert np.all(np.isfinite(ref)) and np.all(ref[:, :130] == 0.0)
        got = run_softmax(x, rows, width, queries, causal, 0.125, width + 1)
        assert not np.any(np.isnan(got)), f"width {width}: NaN"
        check_softmax(got, ref, width)


def test_softmax_attention_scores_full_size():
    """8 sequences x 8 heads x 512 queries over 512 keys, scale 1/8 (head size
    64): the scores of the batched attention product, checked on sampled rows."""
    rows, width = 8 * 8 * 512, 512
    x = stored(3000, rows, width, width)
    got = run_softmax(x, rows, width, width, 1, 0.125, width)
    pick = np.sort(np.random.default_rng(1).choice(rows, 600, replace=False))
    # row r's query is at position r % width; alone, the same row is the
    # first of a group of width - r % width queries, whose first position
    # is that one
    ref = np.stack([R.softmax(x[r:r + 1], width, width - r % width, 0.125)[0] for r in pick])
    check_softmax(got[pick], ref, width)


# ------------------------------------------------------- softmax gradient ---

@pytest.mark.parametrize("case", [(33, 3, 1.0, 0), (64, 256, 0.125, 4), (30, 257, 1.0, 1),
                                  (24, 1024, 0.125, 0), (10, 4096, 0.5, 4), (6, 5000, 0.25, 2),
                                  (30000, 64, 1.0, 0)],
                         ids=lambda c: "r{}w{}ld+{}".format(c[0], c[1], c[3]))
def test_softmax_backward(case):
    rows, width, scale, extra = case
    ld = width + extra
    x = stored(rows + 7 * width, rows, width, ld)
    y = np.full((rows, ld), np.nan, np.float32)
    y[:, :width] = R.softmax(x, width, max(1, width // 3), scale).astype(np.float32)
    dy = stored(rows + 11 * width, rows, width, ld)
    d_y, d_dy = P.to_device(y), P.to_device(dy)
    d_dx = P.to_device(out_buffer(rows, ld))
    P.note(f"softmax backward rows={rows} width={width}")
    call("rows_softmax_backward_f32", rows, width, scale, d_y.data_ptr(), ld, d_dy.data_ptr(), ld,
         d_dx.data_ptr(), ld)
    got = d_dx.cpu().numpy()
    check_padding(got, width)
    ref = R.softmax_backward(y, dy, width, scale)
    y64, g64 = y[:, :width].astype(np.float64), dy[:, :width].astype(np.float64)
    S = np.sum(np.abs(g64 * y64), axis=1, keepdims=True)
    bound = 1e-5 * abs(scale) * np.abs(y64) * (np.abs(g64) + S) + 1e-9
    err = np.abs(got[:, :width] - ref)
    assert np.all(err <= bound), f"worst ratio {np.max(err / bound):.3g}"


# -------------------------------------------------------------- normalize ---

def norm_bound(ref):
    return 1e-5 * (np.abs(ref) + 1.0)


@pytest.mark.parametrize("case", [(7, 1, 1e-5, 0), (33, 3, 1e-5, 1), (64, 100, 1e-3, 3),
                                  (40, 256, 1e-5, 0), (30, 257, 1e-5, 4), (24, 1024, 1e-5, 0),
                                  (12, 2048, 0.0, 4), (10, 4096, 1e-5, 0), (6, 6000, 1e-5, 1),
                                  (20000, 128, 1e-5, 0)],
                         ids=lambda c: "r{}n{}ld+{}".format(c[0], c[1], c[3]))
def test_normalize(case):
    rows, n, eps, extra = case
    ld = n + extra
    x = stored(rows + 3 * n, rows, n, ld, "u11", scale=3.0)
    x[:, :n] += np.float32(1.5)  # a row mean away from 0
    dx, dy = P.to_device(x), P.to_device(out_buffer(rows, ld))
    P.note(f"normalize rows={rows} n={n} eps={eps}")
    call("rows_normalize_f32", rows, n, eps, dx.data_ptr(), ld, dy.data_ptr(), ld)
    got = dy.cpu().numpy()
    check_padding(got, n)
    ref = R.normalize(x, n, eps) if n > 1 or eps > 0 else np.zeros((rows, n))
    err = np.abs(got[:, :n] - ref)
    assert np.all(err <= norm_bound(ref)), f"worst ratio {np.max(err / norm_bound(ref)):.3g}"


def test_normalize_hidden_states_full_size():
    """The transformer set's activations X[8192 x 1024], normalised (eps 1e-5)."""
    rows, n = 8192, 1024
    x = stored(2000, rows, n, n)
    dx, dy = P.to_device(x), P.to_device(out_buffer(rows, n))
    P.note("normalize full size")
    call("rows_normalize_f32", rows, n, 1e-5, dx.data_ptr(), n, dy.data_ptr(), n)
    got = dy.cpu().numpy()
    pick = np.random.default_rng(2).choice(rows, 500, replace=False)
    ref = R.normalize(x[pick], n, 1e-5)
    err = np.abs(got[pick] - ref)
    assert np.all(err <= norm_bound(ref))


@pytest.mark.parametrize("case", [(33, 3, 1e-5, 1), (64, 100, 1e-3, 3), (30, 257, 1e-5, 4),
                                  (24, 1024, 1e-5, 0), (10, 4096, 1e-5, 0), (6, 6000, 1e-5, 1),
                                  (20000, 128, 1e-5, 0)],
                         ids=lambda c: "r{}n{}ld+{}".format(c[0], c[1], c[3]))
def test_normalize_backward(case):
    rows, n, eps, extra = case
    ld = n + extra
    x = stored(rows + 5 * n, rows, n, ld, "u11", scale=2.0)
    dy = stored(rows + 9 * n, rows, n, ld)
    d_x, d_dy, d_dx = P.to_device(x), P.to_device(dy), P.to_device(out_buffer(rows, ld))
    P.note(f"normalize backward rows={rows} n={n}")
    call("rows_normalize_backward_f32", rows, n, eps, d_x.data_ptr(), ld, d_dy.data_ptr(), ld,
         d_dx.data_ptr(), ld)
    got = d_dx.cpu().numpy()
    check_padding(got, n)
    ref = R.normalize_backward(x, dy, n, eps)
    a = x[:, :n].astype(np.float64)
    g = dy[:, :n].astype(np.float64)
    sigma = np.sqrt(a.var(axis=1, keepdims=True) + eps)
    xhat = (a - a.mean(axis=1, keepdims=True)) / sigma
    bound = 2e-5 * (np.abs(ref) + (np.abs(g) + np.abs(g).mean(axis=1, keepdims=True)
                                   + np.abs(xhat) * np.abs(g * xhat).mean(axis=1, keepdims=True))
                    / sigma) + 1e-9
    err = np.abs(got[:, :n] - ref)
    assert np.all(err <= bound), f"worst ratio {np.max(err / bound):.3g}"


def test_rows_repeatable():
    import torch
    import dense_fp32_matrix_gemm_amd as g
    x = P.to_device(stored(8, 3000, 777, 777))
    first = None
    for r in range(5):
        P.note(f"rows repeat {r}")
        outs = [g.softmax(x, 0.2, queries=777), g.normalize(x, 1e-5),
                g.normalize_backward(x, x, 1e-5)]
        torch.cuda.synchronize()
        got = [o.cpu().numpy() for o in outs]
        if first is None:
            first = got
        for a, b in zip(first, got):
            assert np.array_equal(a, b)


def test_tensor_helpers_match_the_oracle():
    """The tensor-level wrappers (softmax, softmax_backward, normalize,
    normalize_backward) on padded views, against the oracle."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    rows, width = 96, 200
    x = stored(21, rows, width, width + 4)
    dy = stored(22, rows, width, width + 4)
    dx_t, ddy_t = P.to_device(x)[:, :width], P.to_device(dy)[:, :width]
    y = g.softmax(dx_t, 0.5, queries=8)
    g_soft = g.softmax_backward(y, ddy_t, 0.5)
    n = g.normalize(dx_t, 1e-4)
    g_norm = g.normalize_backward(dx_t, ddy_t, 1e-4)
    torch.cuda.synchronize()
    ref_y = R.softmax(x, width, 8, 0.5)
    check_softmax(np.concatenate([y.cpu().numpy(), np.full((rows, 1), PAD, np.float32)], 1),
                  ref_y, width)
    y32 = y.cpu().numpy()
    ref = R.softmax_backward(y32, dy, width, 0.5)
    S = np.sum(np.abs(dy[:, :width].astype(np.float64) * y32), axis=1, keepdims=True)
    assert np.all(np.abs(g_soft.cpu().numpy() - ref)
                  <= 1e-5 * 0.5 * np.abs(y32) * (np.abs(dy[:, :width]) + S) + 1e-9)
    refn = R.normalize(x, width, 1e-4)
    assert np.all(np.abs(n.cpu().numpy() - refn) <= norm_bound(refn))
    refb = R.normalize_backward(x, dy, width, 1e-4)
    assert np.all(np.abs(g_norm.cpu().numpy() - refb) <= 1e-4 * (np.abs(refb) + 1.0))


def test_tensor_helpers_refuse_mismatched_shapes():
    import dense_fp32_matrix_gemm_amd as g
    x = P.to_device(stored(23, 16, 32, 32))
    small = P.to_device(stored(24, 8, 32, 32))
    for call in (lambda: g.softmax(x, out=small), lambda: g.normalize(x, out=small),
                 lambda: g.softmax_backward(x, small), lambda: g.normalize_backward(x, small)):
        with pytest.raises(ValueError, match="shape"):
            call()
