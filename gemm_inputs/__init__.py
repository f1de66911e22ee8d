"""Seeded synthetic inputs for the FP32 GEMM workloads.

This module only decides shapes, leading dimensions, seeds, value
distributions and what sits in the padding of each row.  It performs no
matrix arithmetic: the CPU oracle and the HIP library both consume the arrays
it returns, and neither side's computation lives here.

Storage convention (row-major with a leading dimension): a stored matrix with
``rows`` rows, ``cols`` used columns and leading dimension ``ld >= cols`` is a
numpy float32 array of shape ``(rows, ld)``; element ``(r, c)`` sits at flat
offset ``r * ld + c``.  Columns ``cols .. ld-1`` are padding and are filled
with a sentinel (NaN for operands, so a kernel that reads padding into the
result is caught; -7777.0 for the output, so a kernel that writes padding is
caught).

Workloads
---------
The square and ragged cases use i.i.d. U(-1, 1) entries.  The transformer
set reproduces the three GEMMs of one GPT layer's MLP projection over 8192
tokens (forward X.W, backward dX = dY.W^T and dW = X^T.dY) with X, dY ~ N(0, 1)
and W ~ N(0, 0.02), the usual GPT initialisation scale.  These stand in for
the training run that the "Rendre le GPU rapide" (Smallem) page profiles,
whose data and model are not available.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

OPERAND_PAD = float("nan")
OUTPUT_PAD = -7777.0

# Value distributions by name.
DISTRIBUTIONS = ("u11", "n01", "n002", "int8")


def _draw(rng: np.random.Generator, dist: str, shape: Tuple[int, int]) -> np.ndarray:
    """Draw float64 values of the named distribution, then round to float32."""
    if dist == "u11":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "n01":
        x = rng.standard_normal(size=shape)
    elif dist == "n002":
        x = rng.normal(0.0, 0.02, size=shape)
    elif dist == "int8":
        # Integers in [-8, 8]: every product and every partial sum of up to
        # 2^18 of them is an exactly representable float32, so any summation
        # order gives the same bits.
        x = rng.integers(-8, 9, size=shape).astype(np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float32)


def stored_matrix(seed: int, rows: int, cols: int, ld: Optional[int] = None,
                  dist: str = "u11", pad: float = OPERAND_PAD) -> np.ndarray:
    """A seeded row-major float32 matrix of ``rows x cols`` with leading dim ``ld``.

    Returns an array of shape ``(rows, ld)`` whose first ``cols`` columns hold
    the values and whose remaining columns hold ``pad``.  ``rows == 0`` or
    ``cols == 0`` yields an empty (but correctly shaped) array.
    """
    ld = max(1, cols) if ld is None else ld
    if ld < cols:
        raise ValueError(f"ld={ld} < cols={cols}")
    rng = np.random.default_rng(seed)
    out = np.full((rows, ld), pad, dtype=np.float32)
    if rows and cols:
        out[:, :cols] = _draw(rng, dist, (rows, cols))
    return out


def stored_batch(seed: int, batch: int, rows: int, cols: int, ld: int, gap: int = 0,
                 dist: str = "u11", pad: float = OPERAND_PAD) -> np.ndarray:
    """``batch`` stored matrices, each rows x cols with leading dimension ld,
    laid out one after another with ``gap`` extra floats between them.

    Returns a float32 array of shape (batch, rows * ld + gap): row b is the
    flat storage of matrix b (stride rows * ld + gap floats); padding and
    gaps hold ``pad``.
    """
    rng = np.random.default_rng(seed)
    stride = rows * ld + gap
    out = np.full((batch, stride), pad, dtype=np.float32)
    if batch and rows and cols:
        vals = _draw(rng, dist, (batch * rows, cols)).reshape(batch, rows, cols)
        body = out[:, :rows * ld].reshape(batch, rows, ld)
        body[:, :, :cols] = vals
    return out


def output_matrix(rows: int, cols: int, ld: Optional[int] = None,
                  fill: float = OUTPUT_PAD) -> np.ndarray:
    """The output buffer: every element (including the padding) set to ``fill``."""
    ld = max(1, cols) if ld is None else ld
    return np.full((rows, ld), fill, dtype=np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One GEMM problem C[MxN] = op(A)[MxK] . op(B)[KxN] with its input recipe.

    ``transA``: 0 -> A stored M x K (lda >= K); 1 -> A stored K x M (lda >= M).
    ``transB``: 0 -> B stored K x N (ldb >= N); 1 -> B stored N x K (ldb >= K).
    ``lda/ldb/ldc`` of ``None`` mean packed.
    """

    name: str
    M: int
    N: int
    K: int
    seed_a: int
    seed_b: int
    dist_a: str = "u11"
    dist_b: str = "u11"
    transA: int = 0
    transB: int = 0
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    description: str = ""
    batch: int = 1        # > 1: a strided batch of independent products
    gap: int = 0          # extra floats between consecutive matrices of a batch
    shared_b: bool = False  # every product of the batch uses one B (stride 0)

    # -- stored shapes -------------------------------------------------
    @property
    def a_dims(self) -> Tuple[int, int]:
        return (self.K, self.M) if self.transA else (self.M, self.K)

    @property
    def b_dims(self) -> Tuple[int, int]:
        return (self.N, self.K) if self.transB else (self.K, self.N)

    @property
    def lda_(self) -> int:
        return self.lda if self.lda is not None else max(1, self.a_dims[1])

    @property
    def ldb_(self) -> int:
        return self.ldb if self.ldb is not None else max(1, self.b_dims[1])

    @property
    def ldc_(self) -> int:
        return self.ldc if self.ldc is not None else max(1, self.N)

    # Batch strides in floats (0 for a single product or a shared B).
    @property
    def stride_a(self) -> int:
        return self.a_dims[0] * self.lda_ + self.gap if self.batch > 1 else 0

    @property
    def stride_b(self) -> int:
        if self.batch == 1 or self.shared_b:
            return 0
        return self.b_dims[0] * self.ldb_ + self.gap

    @property
    def stride_c(self) -> int:
        return self.M * self.ldc_ + self.gap if self.batch > 1 else 0

    @property
    def flops(self) -> int:
        """2*M*N*K per product: one multiply and one add per (i, j, k) term."""
        return 2 * self.M * self.N * self.K * self.batch

    def make_a(self) -> np.ndarray:
        """Single product: (rows, lda).  Batch: (batch, stride_a) flat storage."""
        r, c = self.a_dims
        if self.batch > 1:
            return stored_batch(self.seed_a, self.batch, r, c, self.lda_, self.gap, self.dist_a)
        return stored_matrix(self.seed_a, r, c, self.lda_, self.dist_a)

    def make_b(self) -> np.ndarray:
        r, c = self.b_dims
        if self.batch > 1 and not self.shared_b:
            return stored_batch(self.seed_b, self.batch, r, c, self.ldb_, self.gap, self.dist_b)
        return stored_matrix(self.seed_b, r, c, self.ldb_, self.dist_b)

    def make_c(self) -> np.ndarray:
        if self.batch > 1:
            return np.full((self.batch, self.stride_c), OUTPUT_PAD, dtype=np.float32)
        return output_matrix(self.M, self.N, self.ldc_)

    def make(self) -> Dict[str, np.ndarray]:
        return {"A": self.make_a(), "B": self.make_b(), "C": self.make_c()}

    def abi_args(self) -> Dict[str, int]:
        return dict(M=self.M, N=self.N, K=self.K, lda=self.lda_, ldb=self.ldb_,
                    ldc=self.ldc_, transA=self.transA, transB=self.transB)

    def with_dist(self, dist: str, name_suffix: str = "-int") -> "Workload":
        """The same shapes and seeds with a different value distribution."""
        return dataclasses.replace(self, name=self.name + name_suffix,
                                   dist_a=dist, dist_b=dist)


# The transformer set draws three tensors once and reuses them across its
# three GEMMs, so X, W and dY keep one seed each.
SEED_X, SEED_W, SEED_DY = 2000, 2001, 2002

WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("S64", 64, 64, 64, 1000, 1001,
                 description="square 64^3, U(-1,1), packed, no transposes"),
        Workload("S1k", 1024, 1024, 1024, 1002, 1003,
                 description="square 1024^3, U(-1,1), packed"),
        Workload("S4k", 4096, 4096, 4096, 1004, 1005,
                 description="square 4096^3, U(-1,1), packed (headline size)"),
        Workload("R", 2049, 3071, 769, 1006, 1007, lda=769 + 3, ldb=3071 + 5,
                 ldc=3071 + 1,
                 description="ragged 2049x3071x769, U(-1,1), lda=K+3, ldb=N+5, ldc=N+1"),
        Workload("T-fwd", 8192, 4096, 1024, SEED_X, SEED_W, "n01", "n002",
                 description="forward X[8192x1024] . W[1024x4096]"),
        Workload("T-dX", 8192, 1024, 4096, SEED_DY, SEED_W, "n01", "n002",
                 transB=1,
                 description="backward dX = dY[8192x4096] . W^T (W stored 1024x4096)"),
        Workload("T-dW", 1024, 4096, 8192, SEED_X, SEED_DY, "n01", "n01",
                 transA=1,
                 description="backward dW = X^T . dY (X stored 8192x1024)"),
    ]
}

# Batched products of one attention layer over 8 sequences x 8 heads of
# 512 positions with head size 64: the scores Q . K^T (keys stored position
# by position, so transposed) and the weighted values P . V.  They stand in
# for the generation-cache product of the "Rendre le GPU rapide" page.
BATCHED: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("attn-qk", 512, 512, 64, 3000, 3001, "n01", "n01", transB=1, batch=64,
                 description="scores Q[64 x 512 x 64] . K^T (K stored 64 x 512 x 64)"),
        Workload("attn-pv", 512, 64, 512, 3002, 3003, "u11", "n01", batch=64,
                 description="values P[64 x 512 x 512] . V[64 x 512 x 64]"),
    ]
}
WORKLOADS.update(BATCHED)

# The workload the throughput metric is quoted on.
HEADLINE = "S4k"
TRANSFORMER_SET = ("T-fwd", "T-dX", "T-dW")


def sample_entries(M: int, N: int, count: int, seed: int = 7,
                   include_corners: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Seeded (row, col) positions of C to check one by one at full size.

    The corners and the last row/column are always included so that edge
    tiles are covered; the rest are uniform over [0, M) x [0, N).
    """
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, size=count))
    cols = list(rng.integers(0, N, size=count))
    if include_corners and M and N:
        for r, c in [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]:
            rows.append(r)
            cols.append(c)
        # a full last row and a full last column stretch of 64 entries
        for t in range(min(64, N)):
            rows.append(M - 1)
            cols.append(N - 1 - t)
        for t in range(min(64, M)):
            rows.append(M - 1 - t)
            cols.append(N - 1)
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


def shape_sweep(tile_sizes: Tuple[int, ...] = (32, 64, 128, 256), limit: int = 70,
                seed: int = 11, count: int = 40) -> List[Tuple[int, int, int]]:
    """Seeded (M, N, K) triples: tiny sizes plus tile boundaries +-1.

    Every size in 1..``limit`` appears in some position, and each tile size t
    contributes t-1, t, t+1 and 2t+1, so that both full and partial edge tiles
    are exercised in every dimension.
    """
    rng = np.random.default_rng(seed)
    bounds = sorted({v for t in tile_sizes for v in (t - 1, t, t + 1, 2 * t + 1)})
    small = list(range(1, limit + 1))
    shapes = set()
    for v in small:
        shapes.add((v, int(rng.choice(small)), int(rng.choice(small))))
        shapes.add((int(rng.choice(small)), v, int(rng.choice(small))))
        shapes.add((int(rng.choice(small)), int(rng.choice(small)), v))
    for v in bounds:
        shapes.add((v, v, v))
        shapes.add((v, int(rng.choice(bounds)), int(rng.choice(bounds))))
    for _ in range(count):
        shapes.add(tuple(int(rng.choice(bounds)) for _ in range(3)))
    return sorted(shapes)


def iter_layouts() -> Iterator[Tuple[int, int, int]]:
    """(transA, transB, extra_ld) combinations: both transposes, packed or padded."""
    for ta in (0, 1):
        for tb in (0, 1):
            for extra in (0, 3):
                yield ta, tb, extra


def make_case(M: int, N: int, K: int, transA: int, transB: int, extra_ld: int,
              dist: str, seed: int) -> Workload:
    """An ad-hoc workload for parity sweeps (padding of ``extra_ld`` per row)."""
    a_cols = M if transA else K
    b_cols = K if transB else N
    return Workload(f"case-{M}x{N}x{K}-t{transA}{transB}-p{extra_ld}-{dist}",
                    M, N, K, seed, seed + 1, dist, dist, transA, transB,
                    lda=max(1, a_cols) + extra_ld, ldb=max(1, b_cols) + extra_ld,
                    ldc=max(1, N) + extra_ld)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b) if b else 0


__all__ = [
    "OPERAND_PAD", "OUTPUT_PAD", "Workload", "WORKLOADS", "HEADLINE",
    "TRANSFORMER_SET", "stored_matrix", "output_matrix", "sample_entries",
    "shape_sweep", "iter_layouts", "make_case", "ceil_div",
]
