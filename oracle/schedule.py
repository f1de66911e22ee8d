"""Emulated memory-access schedules of the pages' GEMM kernels.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

The benchmark divides by two figures that come from the pages' cost model:
the operation count of a product and the bytes a naive kernel moves.  Rather
than retype those formulas, this module walks each kernel's thread and loop
structure on small problems, records every operand load, and counts.  The
tests then check the counts against the values the pages print and against
the closed forms the benchmark uses.

Kernels walked (all for square-tile multiples, as the pages write them):

* ``naive``: one thread per output element, each thread reading a full row
  of A and a full column of B ("3 . La memoire partagee", section 3.1).
* ``tiled``: a T x T block of threads per T x T output tile; per K step each
  thread copies one element of A and one of B into shared memory, then reads
  T elements of each shared tile (section 3.3; also the cuda-oxide book's
  tiled_sgemm and its summary table, whose double-buffered variant issues
  the same loads, only earlier).
* ``register_tiled``: BM x BN output tile per block, BK deep stages, each
  thread owning a TM x TN register tile and reading TM + TN shared values per
  k for TM * TN multiply-adds (section 3.4; the 4 x 4 patch of "Rendre le
  GPU rapide", section "Plusieurs sorties par thread").
"""

from __future__ import annotations

from collections import Counter
from dataclasses import dataclass, field
from typing import Dict, Tuple

FLOAT_BYTES = 4


@dataclass
class ScheduleCount:
    """What one emulated kernel launch did."""

    ops: int = 0                      # multiplies + adds
    global_loads: int = 0             # operand elements read from global memory
    shared_loads: int = 0             # operand elements read from shared memory
    per_thread_global: Counter = field(default_factory=Counter)
    per_thread_shared: Counter = field(default_factory=Counter)
    reads_of_element: Counter = field(default_factory=Counter)  # global reads per element

    @property
    def global_bytes(self) -> int:
        return self.global_loads * FLOAT_BYTES

    @property
    def intensity(self) -> float:
        """Operations per byte of global traffic."""
        return self.ops / self.global_bytes

    def thread_loads(self) -> Tuple[set, set]:
        """Distinct per-thread global and shared load counts."""
        return set(self.per_thread_global.values()), set(self.per_thread_shared.values())


def naive(M: int, N: int, K: int) -> ScheduleCount:
    """One thread per C[i][j]; k loop reads A[i][k] and B[k][j] from global memory."""
    c = ScheduleCount()
    for i in range(M):
        for j in range(N):
            thread = (i, j)
            for k in range(K):
                c.reads_of_element[("A", i, k)] += 1
                c.reads_of_element[("B", k, j)] += 1
                c.per_thread_global[thread] += 2
                c.global_loads += 2
                c.ops += 2        # one multiply, one add
    return c


def tiled(M: int, N: int, K: int, T: int) -> ScheduleCount:
    """T x T thread blocks; per step: one global load of A and of B per thread
    into shared tiles, barrier, T shared reads of each tile, barrier."""
    if M % T or N % T or K % T:
        raise ValueError("the pages' tiled kernel assumes tile multiples")
    c = ScheduleCount()
    for bi in range(M // T):
        for bj in range(N // T):
            for t in range(K // T):
                for ty in range(T):
                    for tx in range(T):
                        thread = (bi * T + ty, bj * T + tx)
                        c.reads_of_element[("A", bi * T + ty, t * T + tx)] += 1
                        c.reads_of_element[("B", t * T + ty, bj * T + tx)] += 1
                        c.per_thread_global[thread] += 2
                        c.global_loads += 2
                        # compute phase: As[ty][k] and Bs[k][tx] for k < T
                        c.per_thread_shared[thread] += 2 * T
                        c.shared_loads += 2 * T
                        c.ops += 2 * T
    return c


def register_tiled(M: int, N: int, K: int, BM: int, BN: int, BK: int,
                   TM: int, TN: int) -> ScheduleCount:
    """BM x BN tile per block of (BM/TM)*(BN/TN) threads, BK-deep stages.

    Each stage the block copies the BM x BK slice of A and the BK x BN slice
    of B to shared memory (each element once, spread over the threads); then
    for every k in the stage each thread reads TM values of A and TN of B and
    performs TM * TN multiply-adds (the outer product).
    """
    if M % BM or N % BN or K % BK or BM % TM or BN % TN:
        raise ValueError("the pages' register-tiled kernel assumes tile multiples")
    threads = (BM // TM) * (BN // TN)
    c = ScheduleCount()
    for bi in range(M // BM):
        for bj in range(N // BN):
            for t in range(K // BK):
                # cooperative copy: element e of the stage goes to thread e % threads
                stage = [("A", bi * BM + r, t * BK + q) for r in range(BM) for q in range(BK)]
                stage += [("B", t * BK + q, bj * BN + s) for q in range(BK) for s in range(BN)]
                for e, elem in enumerate(stage):
                    c.reads_of_element[elem] += 1
                    c.per_thread_global[(bi, bj, e % threads)] += 1
                    c.global_loads += 1
                for th in range(threads):
                    for _k in range(BK):
                        c.per_thread_shared[(bi, bj, th)] += TM + TN
                        c.shared_loads += TM + TN
                        c.ops += 2 * TM * TN
    return c


def outer_product_step(TM: int, TN: int) -> Dict[str, int]:
    """One k step of a TM x TN register tile: shared reads and multiply-adds."""
    reads = 0
    fmas = 0
    reg_a = [None] * TM
    reg_b = [None] * TN
    for i in range(TM):
        reg_a[i] = i
        reads += 1
    for j in range(TN):
        reg_b[j] = j
        reads += 1
    for i in range(TM):
        for j in range(TN):
            fmas += 1
    return {"shared_reads": reads, "fmas": fmas}
