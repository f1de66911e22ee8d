"""GPU parity of the two-step mixed precision: gemm_f32_pack_bf16 (round an
FP32 operand to bf16 once, store it k-contiguous) and gemm_f32_bf16_packed
(the product of two packed operands, FP32 sums).

Marked ``gpu``.  Expected values come only from the oracle:
``oracle.round_bf16`` for the packed bits (the Smallem page's rounding,
"Rendre le GPU rapide", section "Les Tensor Cores"), and ``gemm_bf16`` /
``entries_bf16`` (the exact double sum of the products of the rounded
operands) for the product.

Acceptance bar: packing is bit-exact (integer work on bit patterns, the
rounding decision taken in FP32 on both sides) and leaves the padding
columns untouched; the product of small integers in [-8, 8] is exact; other
products meet the FP32 bar, |C_gpu - C_ref| <= 1e-6*K + 1e-5*|C_ref|
elementwise and relative Frobenius error <= 1e-6, against the
mixed-precision oracle.  Packed test operands are built on the host from
the oracle's rounding, so the product's tests do not rely on the pack
kernel; the end-to-end tests chain both.
"""

import numpy as np
import pytest

import gemm_inputs as gi
import parity as P

pytestmark = pytest.mark.gpu

SENTINEL = 0xABCD  # bit pattern left in padding columns by the host


@pytest.fixture(scope="module", autouse=True)
def device():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible GPU"
    import dense_fp32_matrix_gemm_amd as g
    return g.load()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def bf16_bits(oracle, x: np.ndarray) -> np.ndarray:
    """The oracle's rounding of x, as bf16 bit patterns (uint16)."""
    return (oracle.round_bf16(np.ascontiguousarray(x, np.float32)).view(np.uint32) >> 16).astype(np.uint16)


def _u16_device(x: np.ndarray, offset: int = 0):
    """A device copy of a uint16 array, ``offset`` elements into its buffer;
    returns (tensor, address of element 0)."""
    import torch
    flat = np.concatenate([np.full(offset, SENTINEL, np.uint16), np.ascontiguousarray(x).reshape(-1)])
    t = torch.from_numpy(flat.view(np.int16).copy()).cuda()
    return t, t.data_ptr() + 2 * offset


def _f32_device(x: np.ndarray, offset: int = 0):
    flat = np.concatenate([np.zeros(offset, np.float32), np.ascontiguousarray(x, np.float32).reshape(-1)])
    t = P.to_device(flat)
    return t, t.data_ptr() + 4 * offset


def _bit_patterns(rng, n, lo_exp=-100, hi_exp=100):
    """Float32 values of random sign, exponent in [lo_exp, hi_exp] and random
    significand bits; a third of them exact bf16 ties (low 16 bits 0x8000)."""
    sign = rng.integers(0, 2, n).astype(np.uint32) << 31
    exp = (rng.integers(lo_exp, hi_exp + 1, n) + 127).astype(np.uint32) << 23
    frac = rng.integers(0, 1 << 23, n).astype(np.uint32)
    tie = rng.random(n) < 1 / 3
    frac[tie] = (frac[tie] & 0x7F0000) | 0x8000
    return (sign | exp | frac).view(np.float32)


# ------------------------------------------------------------------- pack ---

def run_pack(x_stored, rows, cols, lds, trans, ldd, offs=(0, 0)):
    """Pack op(x) (x stored as given, leading dimension lds) into a rows x ldd
    uint16 buffer prefilled with SENTINEL; returns it on the host."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    src_t, src = _f32_device(x_stored, offs[0])
    dst_t, dst = _u16_device(np.full((rows, ldd), SENTINEL, np.uint16), offs[1])
    P.note(f"pack rows={rows} cols={cols} lds={lds} trans={trans} ldd={ldd} offs={offs}")
    st = g.gemm_f32_pack_bf16(rows, cols, src, lds, trans, dst, ldd, _stream())
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    return dst_t.cpu().numpy().view(np.uint16)[offs[1]:].reshape(rows, ldd)


PACK_SHAPES = [(1, 1), (3, 5), (64, 64), (65, 130), (200, 96), (257, 1000), (1000, 33), (3, 9000),
               (20000, 5)]


@pytest.mark.parametrize("shape", PACK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("trans", [0, 1])
@pytest.mark.parametrize("pad,offs", [((0, 0), (0, 0)), ((3, 8), (0, 0)), ((4, 5), (1, 1))])
def test_pack_bit_exact(oracle, shape, trans, pad, offs):
    """dst = bf16 bits of op(src), rounded as the page rounds; columns past
    cols untouched.  Padded leading dimensions and misaligned pointers take
    the element-wise paths."""
    rows, cols = shape
    rng = np.random.default_rng(rows * 131 + cols * 7 + trans)
    x = _bit_patterns(rng, rows * cols).reshape(rows, cols)  # op(src)
    flat, n = x.reshape(-1), min(4, x.size)
    flat[:n] = np.array([0.0, -0.0, np.inf, -np.inf], np.float32)[:n]
    stored = np.ascontiguousarray(x.T if trans else x)
    lds = stored.shape[1] + pad[0]
    buf = np.zeros((stored.shape[0], lds), np.float32)
    buf[:, :stored.shape[1]] = stored
    ldd = cols + pad[1]
    got = run_pack(buf, rows, cols, lds, trans, ldd, offs)
    want = bf16_bits(oracle, x)
    assert np.array_equal(got[:, :cols], want), f"pack {shape} t{trans}"
    assert np.all(got[:, cols:] == SENTINEL)


def test_pack_overflow_and_ties(oracle):
    """The largest floats round up to infinity; exact ties go to the even
    neighbour (both as the page's add-half-then-truncate rule gives)."""
    vals = np.array([3.4028235e38, -3.4028235e38, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                     -(1.0 + 2.0 ** -8), 2.0 ** -126], np.float32).reshape(1, -1)
    got = run_pack(vals, 1, vals.shape[1], vals.shape[1], 0, vals.shape[1])
    assert np.array_equal(got, bf16_bits(oracle, vals))
    assert got[0, 0] == 0x7F80 and got[0, 1] == 0xFF80  # +-inf
    assert got[0, 2] == 0x3F80 and got[0, 3] == 0x3F82  # ties to even


# ---------------------------------------------------------------- product ---

def run_packed(M, N, K, Ab, Bb, ldc, offs=(0, 0, 0)):
    """C = A . B^T on packed bit patterns Ab (M x lda) and Bb (N x ldb); C is
    M x ldc prefilled with the output pad value.  Returns C on the host."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    at, a = _u16_device(Ab, offs[0])
    bt, b = _u16_device(Bb, offs[1])
    c0 = np.full((M, ldc), gi.OUTPUT_PAD, np.float32)
    ct, c = _f32_device(c0, offs[2])
    lda, ldb = Ab.shape[1], Bb.shape[1]
    P.note(f"bf16_packed M={M} N={N} K={K} ld {lda} {ldb} {ldc} offs {offs}")
    st = g.gemm_f32_bf16_packed(M, N, K, a, lda, b, ldb, c, ldc, _stream())
    assert st == 0, g.gemm_f32_strerror(st)
    torch.cuda.synchronize()
    return ct.cpu().numpy()[offs[2]:].reshape(M, ldc)


def packed_case(oracle, M, N, K, dist, seed, pad=(0, 0)):
    """FP32 operands A (M x K) and B^T stored N x K from the seeded
    generators, their packed bits with leading dimensions K + pad, and the
    oracle's product."""
    A = gi.stored_matrix(seed, M, K, K, dist)[:, :K]
    Bt = gi.stored_matrix(seed + 1, N, K, K, dist)[:, :K]
    Ab = np.full((M, K + pad[0]), SENTINEL, np.uint16)
    Bb = np.full((N, K + pad[1]), SENTINEL, np.uint16)
    Ab[:, :K] = bf16_bits(oracle, A)
    Bb[:, :K] = bf16_bits(oracle, Bt)
    ref = oracle.gemm_bf16(np.ascontiguousarray(A), np.ascontiguousarray(Bt), M, N, K, 0, 1)
    return Ab, Bb, ref


# 4000 x 2000 and 3001 x 2817 take the 256 x 128 tile and 4097 x 4000 the
# 256 x 256 tile, each with partial tiles in M and N and a partial last
# stage; the others the 128 x 128 tile.
SHAPES = [(1, 1, 1), (37, 45, 29), (128, 128, 32), (129, 257, 95), (300, 200, 512),
          (1000, 1000, 1000), (2049, 700, 77), (4000, 2000, 100), (3001, 2817, 100),
          (4097, 4000, 100)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_integers_exact(oracle, shape):
    M, N, K = shape
    Ab, Bb, ref = packed_case(oracle, M, N, K, "int8", seed=5 * M + 3 * N + K)
    out = run_packed(M, N, K, Ab, Bb, N + 1)
    P.check_padding(out, N)
    P.check_exact(out[:, :N], ref, f"int {shape}")


@pytest.mark.parametrize("shape", SHAPES[1:], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dist", ["u11", "n01"])
def test_tolerance(oracle, shape, dist):
    M, N, K = shape
    Ab, Bb, ref = packed_case(oracle, M, N, K, dist, seed=13 * M + N + 7 * K)
    out = run_packed(M, N, K, Ab, Bb, N + 3)
    P.check_padding(out, N)
    P.check_close(out[:, :N], ref, K, f"{dist} {shape}")


@pytest.mark.parametrize("pad,offs", [((3, 5), (0, 0, 0)), ((0, 0), (1, 3, 1)), ((8, 16), (8, 0, 2))])
def test_unaligned_operands(oracle, pad, offs):
    """Leading dimensions that are not multiples of 8, or pointers that are
    not 16-byte aligned, stage every tile through registers; aligned padding
    keeps the copy path.  Same results either way."""
    M, N, K = 600, 520, 200
    Ab, Bb, ref = packed_case(oracle, M, N, K, "u11", seed=91, pad=pad)
    out = run_packed(M, N, K, Ab, Bb, N, offs)
    P.check_close(out[:, :N], ref, K, f"pad {pad} offs {offs}")


def test_long_k_takes_the_chunked_tile(oracle):
    """K beyond 16384: the small tile, summing runs of 128 k first."""
    M, N, K = 300, 260, 16500
    Ab, Bb, ref = packed_case(oracle, M, N, K, "u11", seed=17)
    out = run_packed(M, N, K, Ab, Bb, N)
    P.check_close(out[:, :N], ref, K, "long K")


def test_k_zero_writes_zeros():
    M, N = 70, 90
    out = run_packed(M, N, 0, np.zeros((M, 1), np.uint16), np.zeros((N, 1), np.uint16), N + 2)
    assert np.all(out[:, :N] == 0.0)
    P.check_padding(out, N)


# -------------------------------------------------------------- end to end ---

@pytest.mark.parametrize("name", ["S1k", "R"])
def test_pack_then_product_named(oracle, name):
    """Both steps on the GPU through the tensor helpers, for a named
    workload with its transposes and padded leading dimensions."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    w = gi.WORKLOADS[name]
    A, B = w.make_a(), w.make_b()
    a = P.to_device(A)[:, :(w.M if w.transA else w.K)]
    b = P.to_device(B)[:, :(w.K if w.transB else w.N)]
    a = a.t() if w.transA else a
    b = b.t() if w.transB else b
    P.note(f"pack+product {name}")
    out = g.matmul_bf16_packed(g.pack_bf16(a), g.pack_bf16(b.t()))
    torch.cuda.synchronize()
    ref = oracle.gemm_bf16(A, B, w.M, w.N, w.K, w.transA, w.transB)
    P.check_close(out.cpu().numpy(), ref, w.K, name)


@pytest.mark.parametrize("name", ["S4k", "T-fwd", "T-dX", "T-dW"])
def test_full_size_sampled(oracle, name):
    """Full-size products packed and multiplied in the benchmark's launch
    configuration, checked on sampled entries of the oracle."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    w = gi.WORKLOADS[name]
    A, B = w.make_a(), w.make_b()
    a = P.to_device(A)[:, :(w.M if w.transA else w.K)]
    b = P.to_device(B)[:, :(w.K if w.transB else w.N)]
    a = a.t() if w.transA else a
    b = b.t() if w.transB else b
    P.note(f"pack+product full size {name}")
    ap, bp = g.pack_bf16(a), g.pack_bf16(b.t())
    out = g.matmul_bf16_packed(ap, bp)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    rows, cols = gi.sample_entries(w.M, w.N, 2000, seed=31)
    ref = oracle.entries_bf16(A, B, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
    got = out[rows, cols].astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= P.ELEM_ABS * w.K + P.ELEM_REL * np.abs(ref)), name
    assert np.linalg.norm(err) <= P.FROB_REL * np.linalg.norm(ref), name
    assert not np.any(np.isnan(out))


def test_packed_agrees_with_fused_entry(oracle):
    """The two-step path and gemm_f32_bf16 compute the same thing: both
    within the bar of the same oracle on the same inputs."""
    import torch
    import dense_fp32_matrix_gemm_amd as g
    M, N, K = 700, 900, 640
    A = gi.stored_matrix(3, M, K, K, "n01")
    B = gi.stored_matrix(4, K, N, N, "n01")
    a, b = P.to_device(A), P.to_device(B)
    two = g.matmul_bf16_packed(g.pack_bf16(a), g.pack_bf16(b.t()))
    one = g.matmul_bf16(a, b)
    torch.cuda.synchronize()
    ref = oracle.gemm_bf16(A, B, M, N, K, 0, 0)
    P.check_close(two.cpu().numpy(), ref, K, "two-step")
    P.check_close(one.cpu().numpy(), ref, K, "fused")
