"""The pages' operation and traffic counts, reproduced by walking the kernels.

``oracle.schedule`` emulates the naive, tiled and register-tiled kernels'
loop structure and counts every load; these tests check the counts against
the figures the pages print (``tests/golden/page_figures.json``) and against
the closed forms the benchmark divides by (``bench.py``).  CPU only.
"""

import json
import os

import pytest

from oracle import schedule

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
    PAGE = json.load(f)


@pytest.mark.parametrize("N", [4, 8, 16])
def test_naive_counts(N):
    g = PAGE["naive_counts"]
    c = schedule.naive(N, N, N)
    assert c.ops == g["ops_total_over_N3"] * N ** 3
    assert c.global_bytes == g["bytes_total_over_N3"] * N ** 3
    per_thread, _ = c.thread_loads()
    assert per_thread == {g["bytes_per_thread_over_N"] * N // 4}   # 2N floats = 8N bytes
    assert c.intensity == g["intensity_ops_per_byte"]
    # each element of A and of B is read N times
    assert set(c.reads_of_element.values()) == {g["reads_of_each_element_over_N"] * N}


def test_naive_rectangular_matches_bench_model():
    """The benchmark's naive byte model 8*M*N*K and flop count 2*M*N*K."""
    import bench
    for (M, N, K) in [(3, 5, 7), (8, 2, 9)]:
        c = schedule.naive(M, N, K)
        assert c.ops == bench.gemm_flops(M, N, K)
        assert c.global_bytes == bench.naive_model_bytes(M, N, K)


@pytest.mark.parametrize("N,T", [(8, 2), (16, 4), (32, 8), (64, 16)])
def test_tiled_counts(N, T):
    g = PAGE["tiled_counts"]
    c = schedule.tiled(N, N, N, T)
    naive = schedule.naive(N, N, N)
    assert c.ops == naive.ops
    assert c.global_bytes * T == g["bytes_total_over_N3_times_T"] * N ** 3
    assert c.intensity == g["intensity_over_T"] * T
    # every element is now read N / T times instead of N times
    assert set(c.reads_of_element.values()) == {N // T}


def test_tiled_figures_at_T32():
    g = PAGE["tiled_counts"]
    T = g["T"]
    N = 64
    c = schedule.tiled(N, N, N, T)
    assert c.intensity == g["intensity_at_T"]
    assert c.intensity / schedule.naive(N, N, N).intensity == g["gain_over_naive_at_T"]
    balance = PAGE["h100_naive_ceiling"]["machine_balance_ops_per_byte"]
    assert balance / c.intensity == g["below_balance_factor_at_T"]


def test_h100_naive_ceiling():
    """The worked H100 example: balance 20, naive 80x below it, 0.84 TFLOPS, 1.2 %."""
    g = PAGE["h100_naive_ceiling"]
    naive_i = schedule.naive(4, 4, 4).intensity
    balance = g["peak_fp32_flops"] / g["hbm_bytes_per_s"]
    assert round(balance) == g["machine_balance_ops_per_byte"]
    assert round(balance / naive_i) == g["below_balance_factor"]
    ceiling = g["hbm_bytes_per_s"] * naive_i
    assert round(ceiling / 1e12, 2) == g["naive_ceiling_tflops"]
    assert round(100 * ceiling / g["peak_fp32_flops"], 1) == g["naive_ceiling_pct_of_peak"]


def test_oxide_64x64_table():
    """Per-thread loads of a 64 x 64 product: naive 128 global; 16 x 16 tiles 8 global, 128 shared."""
    g = PAGE["oxide_64x64_table"]
    N = g["N"]
    n = schedule.naive(N, N, N)
    assert n.thread_loads() == ({g["naive_global_loads_per_thread"]}, set())
    t = schedule.tiled(N, N, N, g["tiled_TILE"])
    assert t.thread_loads() == ({g["tiled_global_loads_per_thread"]},
                                {g["tiled_shared_loads_per_thread"]})
    assert g["tiled_global_loads_per_thread"] == 2 * g["tiled_iterations"]
    assert n.global_bytes / t.global_bytes == g["traffic_cut_for_16x16_tiles"]


def test_register_tile_outer_product():
    g = PAGE["register_tile"]
    step = schedule.outer_product_step(g["TM"], g["TN"])
    assert step["shared_reads"] == g["shared_reads_per_k"]
    assert step["fmas"] == g["fmas_per_k"] == g["accumulator_registers"]
    assert step["fmas"] / step["shared_reads"] == g["compute_to_shared_ratio_after"]
    # the one-output-per-thread tiled kernel reads two shared values per FMA
    t = schedule.tiled(8, 8, 8, 4)
    assert (t.ops // 2) / t.shared_loads == g["compute_to_shared_ratio_before"]
    assert (g["BM"] // g["TM"]) * (g["BN"] // g["TN"]) == g["threads_per_block"]


def test_register_tile_global_intensity_reading():
    """Walk a scaled-down 128x128/BK8 kernel; the intensity is BM*BN/(2(BM+BN)).

    The page prints about 8 for 128 x 128; the walk gives 32, which is the
    reading the build uses (the page's extra factor 1/4 counts bytes twice).
    """
    g = PAGE["register_tile"]
    BM, BN, BK, TM, TN = g["BM"], g["BN"], g["BK"], g["TM"], g["TN"]
    c = schedule.register_tiled(BM, BN, 2 * BK, BM, BN, BK, TM, TN)
    assert c.intensity == g["reading_global_intensity"]
    assert c.intensity != g["printed_global_intensity"]
    import bench
    assert c.global_bytes == bench.tiled_model_bytes(BM, BN, 2 * BK, BM, BN)
    # smaller walk with rectangular tiles against the same closed form
    c2 = schedule.register_tiled(16, 8, 8, 8, 4, 2, 2, 2)
    assert c2.global_bytes == bench.tiled_model_bytes(16, 8, 8, 8, 4)


def test_smallem_patch():
    g = PAGE["smallem_patch"]
    step = schedule.outer_product_step(g["patch"], g["patch"])
    assert step["shared_reads"] == g["shared_reads_per_k"]
    assert step["fmas"] == g["products_per_k"]
    assert g["threads_per_side"] * g["patch"] == g["tile"]
    # one output per thread: 2 reads per product; 4x4 patch: 1 read per 2 products
    assert 2 / (step["shared_reads"] / step["fmas"]) == g["read_reduction_factor"]


def test_bank_model_fixture():
    """The padded transposed read of section 3.6, in the page's own bank model."""
    g = PAGE["bank_model"]
    banks = g["banks"]
    ty = 5
    unpadded = {(32 * tx + ty) % banks for tx in range(32)}
    padded = {(g["padded_row_length"] * tx + ty) % banks for tx in range(32)}
    assert len(unpadded) == 1 and banks // len(unpadded) == g["unpadded_transposed_read_ways"]
    assert len(padded) == banks
    assert 32 * g["bank_width_bytes"] == g["padding_cost_bytes"]


def test_occupancy_quiz():
    g = PAGE["occupancy_quiz"]
    blocks = g["smem_per_sm_kib"] // g["smem_per_block_kib"]
    assert blocks == g["resident_blocks"]
    assert 100 * blocks * g["threads_per_block"] / g["max_threads_per_sm"] == g["occupancy_pct"]
