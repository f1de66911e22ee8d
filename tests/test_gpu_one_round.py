"""GPU parity of the 128 x 128 tile for grids of one tile per CU (256
tiles), whose ring of four LDS stage buffers reads each stage's first k
group ahead, before the previous stage's last MFMAs, and leaves the partial
last stage to the register-staged path.

2048 x 2048 products (and one 2000 x 2000) with K from a single full stage
plus a partial one up to two thousand k, so that the ring runs no whole trip, one partial trip, and
several trips, each followed by a partial stage or not.  Leading dimensions
are multiples of 4 floats with padding, so that the copies go straight into
LDS.  Integers in [-8, 8]: every partial sum is exact, and the result must
match the oracle bit for bit.  Marked ``gpu``.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


def _up4(x):
    return (x + 3) // 4 * 4


# (K, algo): one full 32-k stage + 8, four + 7 and 31 + 8 with the 128 x 128
# tile forced (the automatic choice takes 64 x 64 tiles for products this
# short; forced, 256 tiles still take the one-tile-per-CU configuration);
# 32 + 13 and 64 + 5 as chosen automatically
# 32 + 13 and 64 + 5 as chosen automatically; and 2000 x 2000, whose edge
# tiles take the register-staged path beside the interior tiles' ring
CASES = [(2048, 40, "mfma128"), (2048, 135, "mfma128"), (2048, 1000, "mfma128"), (2048, 1037, "auto"),
         (2048, 2053, "auto"), (2000, 1037, "auto")]


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("MN,K,algo", CASES)
def test_one_round_tile_integer_exact(oracle, MN, K, algo, ta, tb):
    M = N = MN
    w = gi.Workload(f"one-round-{K}", M, N, K, 70 + K, 71 + K, "int8", "int8", ta, tb,
                    lda=_up4(M if ta else K) + 4, ldb=_up4(K if tb else N) + 4, ldc=N + 4)
    if algo == "auto":
        import dense_fp32_matrix_gemm_amd as g
        plan = g.gemm_f32_plan(M, N, K, 1 << 20, w.lda_, 1 << 20, w.ldb_, w.ldc_, ta, tb)
        assert g.PLANS[plan] == "mfma-128x128-one-round", g.PLANS.get(plan, plan)
    A, B = w.make_a(), w.make_b()
    out = P.run_gemm(algo, A, B, w.make_c(), M, N, K, ta, tb, label=f"{w.name} {algo} t{ta}{tb}")
    P.check_padding(out, N)
    P.check_exact(out[:, :N], oracle.gemm(A, B, M, N, K, ta, tb), f"{w.name} t{ta}{tb}")
