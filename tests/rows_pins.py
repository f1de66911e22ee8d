"""Pins of the row-reduction oracle (oracle/rows.py), written as functions of
the module under test so that planted mistakes can be run through them too
(tests/test_rows_mutants.py).

Each pin checks the oracle against something other than itself: values
worked by hand, closed forms, scipy's softmax, torch's float64 layer_norm
and autograd (independent library routines of the same definitions), and
central finite differences of the oracle's own forward pass for the
gradients.  Each returns nothing and raises AssertionError on failure.
"""

from __future__ import annotations

import math

import numpy as np

import gemm_inputs as gi

PINS = []


def pin(fn):
    PINS.append(fn)
    return fn


def _scores(rows, width, ld, seed, dist="n01"):
    return gi.stored_matrix(seed, rows, width, ld, dist)


# ---------------------------------------------------------------- softmax ---

@pin
def positions_by_hand(R):
    # 4 rows of 2 queries each over 4 keys: the queries are positions 2 and 3
    assert list(R.positions(4, 4, 2)) == [2, 3, 2, 3]
    # training: as many queries as keys, query i at position i
    assert list(R.positions(6, 3, 3)) == [0, 1, 2, 0, 1, 2]


@pin
def softmax_by_hand(R):
    # no mask: exp(0) : exp(ln 3) = 1 : 3
    x = np.array([[0.0, math.log(3.0)]], np.float32)
    y = R.softmax(x, 2, 1, 1.0, causal=False)
    assert np.allclose(y, [[0.25, 0.75]], rtol=1e-7, atol=0)
    # causal, equal scores: row i spreads evenly over positions 0..i
    y = R.softmax(np.zeros((3, 3), np.float32), 3, 3, 1.0)
    want = np.array([[1, 0, 0], [1 / 2, 1 / 2, 0], [1 / 3, 1 / 3, 1 / 3]])
    assert np.allclose(y, want, rtol=1e-15, atol=0)
    # the scale multiplies the scores: scores 0 and ln(3)/2 with scale 2
    x = np.array([[0.0, math.log(3.0) / 2]], np.float32)
    assert np.allclose(R.softmax(x, 2, 1, 2.0, causal=False), [[0.25, 0.75]], rtol=1e-6)


@pin
def softmax_matches_scipy(R):
    from scipy.special import softmax as sp_softmax
    x = _scores(12, 37, 40, 5)
    for queries, scale in [(37, 0.125), (5, 1.0), (1, 0.5)]:
        y = R.softmax(x, 37, queries, scale)
        pos = R.positions(12, 37, queries)
        for r in range(12):
            keep = pos[r] + 1
            ref = sp_softmax(scale * x[r, :keep].astype(np.float64))
            assert np.allclose(y[r, :keep], ref, rtol=1e-13, atol=0)
            assert np.all(y[r, keep:] == 0.0)
    yf = R.softmax(x, 37, 37, 0.3, causal=False)
    assert np.allclose(yf, sp_softmax(0.3 * x[:, :37].astype(np.float64), axis=1), rtol=1e-13)


@pin
def softmax_ignores_masked_values(R):
    # the future may hold anything, even NaN: it is never read
    x = _scores(6, 9, 9, 6)
    clean = R.softmax(x, 9, 3, 0.7)
    dirty = x.copy()
    pos = R.positions(6, 9, 3)
    for r in range(6):
        dirty[r, pos[r] + 1:] = np.nan
    assert np.array_equal(R.softmax(dirty, 9, 3, 0.7), clean)
    assert np.allclose(clean.sum(axis=1), 1.0, rtol=1e-14)


@pin
def softmax_large_scores_do_not_overflow(R):
    x = np.array([[1000.0, 999.0, -1000.0]], np.float32)
    y = R.softmax(x, 3, 1, 1.0, causal=False)
    e = math.exp(-1.0)
    assert np.allclose(y, [[1 / (1 + e), e / (1 + e), 0.0]], rtol=1e-14, atol=1e-300)


def _fd_softmax(R, x64, dy, width, queries, scale, causal, h=1e-5):
    """Central differences of L = sum(dy * softmax(x)) in float64."""
    g = np.zeros_like(x64)
    for r in range(x64.shape[0]):
        for c in range(width):
            p, m = x64.copy(), x64.copy()
            p[r, c] += h
            m[r, c] -= h
            lp = np.sum(dy * R.softmax(p, width, queries, scale, causal))
            lm = np.sum(dy * R.softmax(m, width, queries, scale, causal))
            g[r, c] = (lp - lm) / (2 * h)
    return g


@pin
def softmax_backward_matches_finite_differences(R):
    rng = np.random.default_rng(3)
    for causal, queries in [(False, 7), (True, 7), (True, 3)]:
        x64 = rng.standard_normal((3, 7))
        dy = rng.standard_normal((3, 7))
        y = R.softmax(x64, 7, queries, 0.6, causal)
        dx = R.softmax_backward(y, dy, 7, 0.6)
        fd = _fd_softmax(R, x64, dy, 7, queries, 0.6, causal)
        assert np.allclose(dx, fd, rtol=1e-6, atol=1e-9), (causal, np.max(np.abs(dx - fd)))


@pin
def softmax_backward_matches_torch_autograd(R):
    import torch
    x = _scores(5, 16, 16, 8)
    dy = _scores(5, 16, 16, 9)
    t = torch.tensor(x.astype(np.float64), requires_grad=True)
    mask = torch.tensor(np.arange(16)[None, :] > R.positions(5, 16, 4)[:, None])
    z = (0.25 * t).masked_fill(mask, float("-inf"))
    out = torch.softmax(z, dim=1)
    out.backward(torch.tensor(dy.astype(np.float64)))
    y = R.softmax(x, 16, 4, 0.25)
    assert np.allclose(y, out.detach().numpy(), rtol=1e-13, atol=0)
    assert np.allclose(R.softmax_backward(y, dy, 16, 0.25), t.grad.numpy(), rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------- normalize ---

@pin
def normalize_by_hand(R):
    y = R.normalize(np.array([[1.0, 3.0]], np.float32), 2, 0.0)
    assert np.allclose(y, [[-1.0, 1.0]], rtol=1e-15)
    # epsilon inside the root: var = 1, eps = 3 -> divide by 2
    y = R.normalize(np.array([[1.0, 3.0]], np.float32), 2, 3.0)
    assert np.allclose(y, [[-0.5, 0.5]], rtol=1e-15)
    assert np.all(R.normalize(np.full((2, 5), 4.0, np.float32), 5, 1e-5) == 0.0)


@pin
def normalize_moments(R):
    x = _scores(7, 300, 301, 11, "u11") * np.float32(3.0)
    eps = 1e-5
    y = R.normalize(x, 300, eps)
    a = x[:, :300].astype(np.float64)
    var = a.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-14)
    assert np.allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-12)


@pin
def normalize_matches_torch(R):
    import torch
    x = _scores(9, 64, 66, 12)
    ref = torch.nn.functional.layer_norm(torch.tensor(x[:, :64].astype(np.float64)), (64,),
                                         eps=1e-3).numpy()
    assert np.allclose(R.normalize(x, 64, 1e-3), ref, rtol=1e-12, atol=1e-14)


@pin
def normalize_backward_matches_torch_and_differences(R):
    import torch
    x = _scores(4, 24, 24, 13)
    dy = _scores(4, 24, 24, 14)
    t = torch.tensor(x.astype(np.float64), requires_grad=True)
    torch.nn.functional.layer_norm(t, (24,), eps=1e-2).backward(torch.tensor(dy.astype(np.float64)))
    dx = R.normalize_backward(x, dy, 24, 1e-2)
    assert np.allclose(dx, t.grad.numpy(), rtol=1e-11, atol=1e-13)
    x64 = x.astype(np.float64)
    h = 1e-5
    for r in range(2):
        for c in range(24):
            p, m = x64.copy(), x64.copy()
            p[r, c] += h
            m[r, c] -= h
            fd = (np.sum(dy * R.normalize(p, 24, 1e-2)) - np.sum(dy * R.normalize(m, 24, 1e-2))) / (2 * h)
            assert abs(dx[r, c] - fd) <= 1e-6 * (1 + abs(fd))


@pin
def algorithmic_bytes_count_each_array_once(R):
    assert R.algorithmic_bytes("softmax", 10, 20) == 2 * 4 * 200
    assert R.algorithmic_bytes("softmax_backward", 10, 20) == 3 * 4 * 200
    assert R.algorithmic_bytes("normalize_backward", 3, 5) == 3 * 4 * 15


def run_all(R) -> None:
    for p in PINS:
        p(R)
