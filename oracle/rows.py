"""CPU oracle for the row reductions next to the GEMM: the causal softmax of
attention scores, the row normalisation, and the gradients of both.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
module; the HIP library shares nothing with it.

Every function is the plain definition in float64 (numpy), one row at a
time in the page's terms, from float32 inputs stored row-major with a
leading dimension.  The source is the Smallem page ("Rendre le GPU rapide"):

* section "Les kernels fusionnés": the causal softmax computes, for row r of
  a [rows x width] block of scores, the query's position
  ``width - queries + r % queries`` and gives every column beyond it the
  value 0; the other columns get exp(scale*a - row max - log of the row's
  sum of exponentials), the max and sum taken over the columns kept.  The
  same section names the normalisation ("Normalize", with an epsilon) and
  describes it as a mean, a subtraction, a square, a second mean, a root
  and a division; the backward passes of both have their own kernels there.
* section "Un warp par ligne": those row maxima, sums, means and variances
  are reductions along each row.

Readings where the page is silent (listed in the design doc): the variance is the
mean of squared deviations (population form); epsilon is added to it before
the root; the normalisation has no scale or shift parameters; the softmax
gradient is taken with respect to the unscaled scores, so it carries the
factor ``scale``; a non-causal softmax (every column kept) is the same
definition with the mask off.

Parity status: every function here is pinned in tests/test_rows_oracle.py
(closed forms, hand-worked cases, scipy's softmax, torch's float64
layer_norm and autograd, central finite differences of the forward).
"""

from __future__ import annotations

import numpy as np


def _rows(x: np.ndarray, width: int) -> np.ndarray:
    """The logical [rows x width] block of a stored float32 array, as float64."""
    if x.ndim != 2 or x.shape[1] < width:
        raise ValueError("stored array must be 2-D with at least `width` columns")
    return x[:, :width].astype(np.float64)


def positions(rows: int, width: int, queries: int) -> np.ndarray:
    """Position of the query each row belongs to: rows come in groups of
    ``queries`` consecutive query rows (one group per sequence and head), and
    the queries of a group are the last ``queries`` positions of a sequence
    of ``width`` keys."""
    if not 1 <= queries <= width:
        raise ValueError("need 1 <= queries <= width")
    r = np.arange(rows)
    return width - queries + r % queries


def softmax(x: np.ndarray, width: int, queries: int, scale: float,
            causal: bool = True) -> np.ndarray:
    """y[r][c] = exp(scale*x[r][c] - m_r - log s_r) for kept columns
    (c <= position of row r when causal, every c otherwise), 0 elsewhere;
    m_r the max of scale*x over the kept columns, s_r = sum over the kept
    columns of exp(scale*x - m_r)."""
    a = _rows(x, width)
    rows = a.shape[0]
    out = np.zeros((rows, width))
    pos = positions(rows, width, queries) if causal else np.full(rows, width - 1)
    for r in range(rows):
        keep = pos[r] + 1
        z = scale * a[r, :keep]
        m = np.max(z)
        log_sum = np.log(np.sum(np.exp(z - m)))
        out[r, :keep] = np.exp((z - m) - log_sum)
    return out


def softmax_backward(y: np.ndarray, dy: np.ndarray, width: int, scale: float) -> np.ndarray:
    """Gradient with respect to the unscaled scores x of a loss L, given the
    softmax output y and dL/dy: dx[r][c] = scale * y[r][c] * (dy[r][c] - d_r)
    with d_r = sum over c of dy[r][c] * y[r][c].  (Columns the forward pass
    masked hold y = 0, so their gradient is 0.)"""
    yy = _rows(y, width)
    g = _rows(dy, width)
    out = np.empty_like(yy)
    for r in range(yy.shape[0]):
        d = np.sum(g[r] * yy[r])
        out[r] = scale * yy[r] * (g[r] - d)
    return out


def normalize(x: np.ndarray, n: int, eps: float) -> np.ndarray:
    """y[r][c] = (x[r][c] - mu_r) / sqrt(var_r + eps), mu_r the mean of row r
    and var_r the mean of its squared deviations from mu_r."""
    a = _rows(x, n)
    out = np.empty_like(a)
    for r in range(a.shape[0]):
        mu = np.mean(a[r])
        dev = a[r] - mu
        var = np.mean(dev * dev)
        out[r] = dev / np.sqrt(var + eps)
    return out


def normalize_backward(x: np.ndarray, dy: np.ndarray, n: int, eps: float) -> np.ndarray:
    """Gradient of a loss with respect to x through y = normalize(x):
    with sigma = sqrt(var + eps) and xhat = (x - mu) / sigma,
    dx = (dy - mean(dy) - xhat * mean(dy * xhat)) / sigma, row by row
    (the derivative of the definition above, mu and var depending on x)."""
    a = _rows(x, n)
    g = _rows(dy, n)
    out = np.empty_like(a)
    for r in range(a.shape[0]):
        mu = np.mean(a[r])
        dev = a[r] - mu
        sigma = np.sqrt(np.mean(dev * dev) + eps)
        xhat = dev / sigma
        out[r] = (g[r] - np.mean(g[r]) - xhat * np.mean(g[r] * xhat)) / sigma
    return out


def algorithmic_bytes(op: str, rows: int, width: int) -> int:
    """Bytes an op must move at least once: each input read and the output
    written, 4 bytes per element (the HBM roofline's numerator)."""
    arrays = {"softmax": 2, "softmax_backward": 3, "normalize": 2, "normalize_backward": 3}[op]
    return 4 * arrays * rows * width
