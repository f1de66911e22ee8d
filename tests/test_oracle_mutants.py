"""Plant plausible mistakes in copies of the oracle and check the pins catch each.

Each mutant is the oracle's C source with one textual change (a dropped
term, a flipped sign, a swapped index, a transposed operand, a float
accumulator, a miscount, a wrong rounding), built with gcc into a temporary directory and run
through the same pins as the real oracle.  Every mutant must fail at least
one pin.  CPU only; the real oracle source is never modified.
"""

import os
import subprocess
import sys

import pytest

import gemm_inputs as gi
import oracle as oracle_pkg
import oracle_pins as pins
from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))

SOURCE = open(oracle_build.SOURCE).read()

MUTANTS = {
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k < K - 1; ++k)"),
    "dropped_first_term": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 1; k < K; ++k)"),
    "wrong_sign": ("s += op_a", "s -= op_a"),
    "a_not_transposed": ("return transA ? (double)A[k * lda + i] : (double)A[i * lda + k];",
                         "return transA ? (double)A[i * lda + k] : (double)A[i * lda + k];"),
    "a_index_swapped": ("return transA ? (double)A[k * lda + i] : (double)A[i * lda + k];",
                        "return transA ? (double)A[i * lda + k] : (double)A[k * lda + i];"),
    "b_index_swapped": ("return transB ? (double)B[j * ldb + k] : (double)B[k * ldb + j];",
                        "return transB ? (double)B[k * ldb + j] : (double)B[j * ldb + k];"),
    "b_uses_trans_a": ("op_b(B, ldb, transB, k, j)", "op_b(B, ldb, transA, k, j)"),
    "a_off_by_one": ("(double)A[i * lda + k];", "(double)A[i * lda + k + 1];"),
    "b_wrong_ld": ("(double)B[k * ldb + j];", "(double)B[k * (ldb - (ldb > 1)) + j];"),
    "float_accumulator": ("double s = 0.0;", "float s = 0.0f;"),
    "output_transposed": ("C[i * ldc + j] = dot(K, A, lda, transA, B, ldb, transB, i, j);",
                          "C[j * ldc + i] = dot(K, A, lda, transA, B, ldb, transB, i, j);"),
    "miscounted_macs": ("macs += K;", "macs += K - (K > 1);"),
    "miscounted_reads": ("reads += 2 * K;", "reads += K;"),
    "gelu_wrong_scale": ("erf(x / sqrt(2.0))", "erf(x / 2.0)"),
    "bias_by_row": ("(bias ? (double)bias[j] : 0.0)", "(bias ? (double)bias[i % N] : 0.0)"),
    "bf16_truncates": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;"),
    "bf16_ties_away": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    "bf16_ties_down": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x7FFFu;"),
    "bf16_low_bits_kept": ("u &= 0xFFFF0000u;", "u &= 0xFFFFFFFFu;"),
    "bf16_mask_too_wide": ("u &= 0xFFFF0000u;", "u &= 0xFFFE0000u;"),
    "bf16_a_not_rounded": ("const float a = round_bf16((float)op_a(A, lda, transA, i, k));",
                           "const float a = (float)op_a(A, lda, transA, i, k);"),
    "bf16_b_not_rounded": ("const float b = round_bf16((float)op_b(B, ldb, transB, k, j));",
                           "const float b = (float)op_b(B, ldb, transB, k, j);"),
    "bf16_b_transposed": ("round_bf16((float)op_b(B, ldb, transB, k, j))",
                          "round_bf16((float)op_b(B, ldb, 1 - transB, k, j))"),
}


def _all_pins(orc):
    def gemm(*a):
        return orc.gemm(*a)
    yield "identity", lambda: pins.pin_identity(gemm)
    yield "all_ones", lambda: pins.pin_all_ones(gemm)
    yield "rank_one", lambda: pins.pin_rank_one(gemm)
    yield "integer", lambda: pins.pin_integer_exact(gemm)
    yield "brute", lambda: pins.pin_brute_force(gemm, sizes=range(1, 4))
    yield "numpy_S64", lambda: pins.pin_numpy_f64(gemm, gi.WORKLOADS["S64"])
    yield "numpy_S1k", lambda: pins.pin_numpy_f64(gemm, gi.WORKLOADS["S1k"])
    yield "counts", lambda: pins.pin_counts(
        lambda A, B, M, N, K: orc.gemm(A, B, M, N, K, 0, 0, with_stats=True))
    yield "epilogue", lambda: pins.pin_epilogue(orc.epilogue)
    yield "bf16_round", lambda: pins.pin_bf16_rounding(orc.round_bf16)
    yield "bf16_gemm", lambda: pins.pin_bf16_gemm(orc.gemm_bf16)


def _caught(orc):
    caught = []
    for name, run in _all_pins(orc):
        try:
            run()
        except (AssertionError, ValueError):
            caught.append(name)
    return caught


def _caught_in_child(lib: str) -> str:
    """Run the pins on ``lib`` in a child process (a mutant may write out of
    bounds and crash).  Returns the names of the pins that failed, or a note
    that the mutant crashed, which also counts as caught."""
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle_mutants as t, oracle; "
            "print(','.join(t._caught(oracle.Oracle(%r))))" % (HERE, os.path.dirname(HERE), lib))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300)
    if r.returncode != 0:
        return f"crashed (status {r.returncode})"
    return r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    assert SOURCE.count(old) >= 1, f"mutation anchor for {mutant} not found in the oracle"
    src = tmp_path / "gemm_ref_mutant.c"
    src.write_text(SOURCE.replace(old, new))
    lib = oracle_build.build(str(src), str(tmp_path / "libmutant.so"))
    caught = _caught_in_child(lib)
    assert caught, f"no pin catches the mutant {mutant}"
    print(mutant, "->", caught)


def test_unmutated_copy_passes(tmp_path):
    """Control: the same harness on an unmodified copy catches nothing."""
    src = tmp_path / "gemm_ref_copy.c"
    src.write_text(SOURCE)
    lib = oracle_build.build(str(src), str(tmp_path / "libcopy.so"))
    assert _caught_in_child(lib) == ""
    assert os.path.exists(lib)
