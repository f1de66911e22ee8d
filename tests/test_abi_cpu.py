"""The C ABI on the host: symbols, argument validation, Python-side layout logic.

CPU only: no test here launches a kernel.  Invalid arguments are rejected on
the host before any HIP call, so the codes are checked without a GPU.
"""

import ctypes
import os
import re

import pytest

import gemm_inputs as gi

import dense_fp32_matrix_gemm_amd as g
from dense_fp32_matrix_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]

BIG = 1 << 31
FAKE = 0x1000  # a non-NULL pointer value; never dereferenced by these tests


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(\w+)\s*\(", text, flags=re.M):
            if not m.group(0).lstrip().startswith(("#", "typedef", "enum", "struct")):
                names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert {"gemm_f32", "gemm_f32_naive", "gemm_f32_ex", "gemm_f32_strerror",
            "gemm_f32_version"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert set(_lib.SIGNATURES) == declared_functions()


def test_version(lib):
    assert g.gemm_f32_version() == 10700


def call(M=4, N=4, K=4, A=FAKE, lda=None, B=FAKE, ldb=None, C=FAKE, ldc=None,
         ta=0, tb=0, fn="gemm_f32", algo=None):
    lda = max(1, M if ta else K) if lda is None else lda
    ldb = max(1, K if tb else N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    args = [M, N, K, A, lda, B, ldb, C, ldc, ta, tb, None]
    if fn == "gemm_f32_ex":
        args.append(0 if algo is None else algo)
    return getattr(g, fn)(*args)


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_f32_naive", "gemm_f32_ex", "gemm_f32_bf16"])
@pytest.mark.parametrize("kwargs,code", [
    (dict(M=-1), -1), (dict(N=-1), -2), (dict(K=-1), -3),
    (dict(M=BIG), -1), (dict(N=BIG), -2), (dict(K=BIG), -3),
    (dict(A=None), -4), (dict(lda=3), -5), (dict(lda=BIG), -5),
    (dict(B=None), -6), (dict(ldb=3), -7),
    (dict(C=None), -8), (dict(ldc=3), -9), (dict(ldc=BIG), -9),
    (dict(ta=2), -10), (dict(tb=-1), -11),
    (dict(ta=1, lda=3, M=4, K=9), -5),      # transposed A: lda >= M
    (dict(tb=1, ldb=8, K=9), -7),           # transposed B: ldb >= K
    (dict(M=0, lda=0), -5),                 # lda >= 1 even when nothing is read
])
def test_invalid_arguments(fn, kwargs, code):
    assert call(fn=fn, **kwargs) == code
    assert g.gemm_f32_strerror(code).startswith(f"invalid argument {-code} ")


def test_invalid_algo():
    assert call(fn="gemm_f32_ex", algo=9) == -13
    assert call(fn="gemm_f32_ex", algo=-1) == -13


WIDE = g.ALGOS["mfmawide"]
ALIGNED = 0x10000  # 16-byte aligned, never dereferenced


@pytest.mark.parametrize("kwargs", [
    dict(M=300), dict(N=200),                        # not multiples of 256
    dict(K=1056), dict(K=40), dict(K=16),            # K above 1024 or not a multiple of 32
    dict(lda=66), dict(ldb=258),                     # leading dimensions not multiples of 4
    dict(ta=1, lda=258), dict(tb=1, ldb=66),         # the same with transposed operands
    dict(A=ALIGNED + 4), dict(B=ALIGNED + 8),        # operands not 16-byte aligned
], ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
def test_wide_refuses_problems_outside_its_domain(kwargs):
    """The 256 x 256 kernel runs only aligned products with M and N multiples
    of 256 and K a multiple of 32 up to 1024 (either transpose): anything
    else is -13, decided on the host before any HIP call."""
    args = dict(M=256, N=256, K=64, A=ALIGNED, B=ALIGNED, C=ALIGNED)
    args.update(kwargs)
    assert call(fn="gemm_f32_ex", algo=WIDE, **args) == -13


def test_wide_quick_returns_before_its_domain_check():
    """Empty outputs return 0 whatever the shape; K == 0 is the zero fill."""
    assert call(fn="gemm_f32_ex", algo=WIDE, M=0, N=300, K=40, A=None, C=None) == 0
    assert call(fn="gemm_f32_ex", algo=WIDE, M=300, N=0, K=40, B=None, C=None) == 0


@pytest.mark.parametrize("kwargs", [dict(M=0, A=None, C=None), dict(N=0, B=None, C=None),
                                    dict(M=0, N=0, A=None, B=None, C=None)])
def test_quick_return_without_launch(kwargs):
    """M == 0 or N == 0: nothing to write, status 0, no HIP call (works without a GPU)."""
    assert call(**kwargs) == 0
    assert call(fn="gemm_f32_ex", algo=1, **kwargs) == 0
    assert call(fn="gemm_f32_bf16", **kwargs) == 0


def test_strerror_is_total():
    for st in range(-20, 1):
        assert isinstance(g.gemm_f32_strerror(st), str)
    assert g.gemm_f32_strerror(0) == "success"
    assert g.gemm_f32_strerror(-99) == "unknown status"
    assert len(g.gemm_f32_strerror(100)) > 0   # a hipError_t, described by HIP


def test_launch_without_gpu_returns_hip_error():
    """Valid arguments on a host with no GPU: a positive hipError_t, not a crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; this case is for GPU-less hosts")
    st = call(M=2, N=2, K=2)
    assert st > 0
    assert isinstance(g.gemm_f32_strerror(st), str)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setenv("GEMM_F32_LIBRARY", str(tmp_path / "nope.so"))
    with pytest.raises(_lib.LibraryNotBuilt):
        _lib.load()


def test_operand_layout_from_strides():
    import torch
    x = torch.empty(6, 10)
    assert g.operand_layout(x) == (0, 10)
    assert g.operand_layout(x.t()) == (1, 10)               # 10 x 6 view of a 6 x 10 array
    assert g.operand_layout(x[:, :7]) == (0, 10)            # column slice keeps ld
    assert g.operand_layout(x[:, :7].t()) == (1, 10)
    with pytest.raises(ValueError):
        g.operand_layout(x[:, ::2])


def test_header_is_plain_c():
    """The public header compiles as C with no HIP headers on the include path."""
    import subprocess
    src = "#include \"gemm_f32.h\"\nint main(void){return gemm_f32_version() == 10700 ? 0 : 1;}\n"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), "-x", "c", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def bcall(M=4, N=4, K=4, A=FAKE, lda=None, sA=None, B=FAKE, ldb=None, sB=None, C=FAKE,
          ldc=None, sC=None, batch=3, ta=0, tb=0):
    lda = max(1, M if ta else K) if lda is None else lda
    ldb = max(1, K if tb else N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    sA = (K if ta else M) * lda if sA is None else sA
    sB = (N if tb else K) * ldb if sB is None else sB
    sC = M * ldc if sC is None else sC
    return g.gemm_f32_strided_batched(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch,
                                      ta, tb, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(M=-1), -1), (dict(N=-1), -2), (dict(K=-1), -3), (dict(A=None), -4),
    (dict(lda=3), -5), (dict(sA=-1), -6), (dict(B=None), -7), (dict(ldb=3), -8),
    (dict(sB=-4), -9), (dict(C=None), -10), (dict(ldc=3), -11), (dict(sC=-1), -12),
    (dict(sC=15), -12),                     # C products would overlap: 3*4 + 4 = 16 > 15
    (dict(batch=-1), -13), (dict(batch=BIG), -13), (dict(ta=3), -14), (dict(tb=2), -15),
])
def test_strided_batched_invalid_arguments(kwargs, code):
    assert bcall(**kwargs) == code


def test_strided_batched_quick_returns():
    """batch 0, or an empty product, writes nothing and touches no GPU."""
    assert bcall(batch=0, A=None, B=None, C=None) == 0
    assert bcall(M=0, A=None, C=None) == 0
    assert bcall(sA=0, sB=0, batch=0) == 0          # shared operands are allowed
    assert bcall(sC=16, batch=0) == 0


@pytest.mark.parametrize("kwargs,code", [
    (dict(M=-1), -1), (dict(A=None), -4), (dict(lda=3), -5), (dict(C=None), -8),
    (dict(ta=2), -10), (dict(act=2), -13), (dict(act=-1), -13),
])
def test_bias_act_invalid_arguments(kwargs, code):
    act = kwargs.pop("act", 1)
    M, K = kwargs.get("M", 4), 4
    args = dict(M=M, N=4, K=K, A=FAKE, lda=4, B=FAKE, ldb=4, C=FAKE, ldc=4, ta=0, tb=0)
    args.update(kwargs)
    st = g.gemm_f32_bias_act(args["M"], args["N"], args["K"], args["A"], args["lda"], args["B"],
                             args["ldb"], args["C"], args["ldc"], args["ta"], args["tb"], None,
                             act, None)
    assert st == code


def test_bias_act_quick_return():
    assert g.gemm_f32_bias_act(0, 4, 4, None, 4, FAKE, 4, None, 4, 0, 0, None, 1, None) == 0


# ------------------------------------------------------------- split k ---

def splitk(M=8, N=8, K=64, splits=2, ws=FAKE, ws_bytes=1 << 20, **kw):
    return g.gemm_f32_splitk(M, N, K, kw.get("A", FAKE), kw.get("lda", max(K, 1)),
                             kw.get("B", FAKE), kw.get("ldb", max(N, 1)), kw.get("C", FAKE),
                             kw.get("ldc", max(N, 1)), 0, 0,
                             splits, ws, ws_bytes, None)


def test_splitk_workspace_size():
    """Runs of ceil(K/splits) rounded up to 32; one M x N partial per run."""
    ws = g.gemm_f32_splitk_workspace_size
    assert ws(1024, 4096, 8192, 2) == 2 * 1024 * 4096 * 4
    assert ws(10, 10, 33, 2) == 2 * 10 * 10 * 4      # runs of 32: 32 + 1
    assert ws(10, 10, 100, 50) == 4 * 10 * 10 * 4    # capped at 32-k runs
    assert ws(10, 10, 100, 3) == 2 * 10 * 10 * 4     # ceil(100/3) = 34 -> runs of 64: 64 + 36
    assert ws(10, 10, 32, 4) == 0                    # one run: no workspace
    assert ws(10, 10, 0, 4) == 0 and ws(0, 10, 64, 2) == 0 and ws(10, 0, 64, 2) == 0
    assert ws(-1, 1, 1, 1) == -1 and ws(1, -1, 1, 1) == -2 and ws(1, 1, -1, 1) == -3
    assert ws(1, 1, 1, 0) == -12 and ws(1, 1, 1, -3) == -12


def test_splitk_argument_errors():
    assert splitk(splits=0) == -12
    assert splitk(ws=None) == -13
    assert splitk(ws_bytes=2 * 8 * 8 * 4 - 1) == -14
    assert splitk(M=-1) == -1 and splitk(lda=3) == -5
    assert "splits" in g.gemm_f32_strerror(-12)
    assert "workspace" in g.gemm_f32_strerror(-13) and "workspace" in g.gemm_f32_strerror(-14)


def test_splitk_quick_return_without_launch():
    assert splitk(M=0) == 0 and splitk(N=0) == 0
    assert splitk(M=0, ws=None, ws_bytes=0) == 0


def noalloc(M=8, N=8, K=64, splits=2, **kw):
    return g.gemm_f32_splitk_noalloc(M, N, K, kw.get("A", FAKE), kw.get("lda", max(K, 1)),
                                     kw.get("B", FAKE), kw.get("ldb", max(N, 1)),
                                     kw.get("C", FAKE), kw.get("ldc", max(N, 1)),
                                     kw.get("ta", 0), kw.get("tb", 0), splits, None)


def test_splitk_noalloc_argument_errors():
    """Checked on the host before the scratch lookup or any launch."""
    assert noalloc(splits=0) == -12 and noalloc(splits=-1) == -12
    assert noalloc(M=-1) == -1 and noalloc(N=-2) == -2 and noalloc(K=-3) == -3
    assert noalloc(lda=3) == -5 and noalloc(ldb=7) == -7 and noalloc(ldc=7) == -9
    assert noalloc(C=None) == -8 and noalloc(ta=2) == -10 and noalloc(tb=-1) == -11
    # the largest partial products the scratch holds, and one float more
    cap = _lib.SPLITK_SCRATCH_BYTES
    assert g.gemm_f32_splitk_workspace_size(1024, 4096, 8192, 4) == cap
    assert noalloc(M=1025, N=4096, K=8192, splits=4, lda=8192, ldb=4096, ldc=4096) == -12
    assert noalloc(M=4096, N=4096, K=4096, splits=2, lda=4096, ldb=4096, ldc=4096) == -12
    assert "SCRATCH" in g.gemm_f32_strerror(-12)


def test_splitk_noalloc_quick_returns_without_launch():
    assert noalloc(M=0) == 0 and noalloc(N=0) == 0
    # an empty output needs no partials, so no scratch limit applies
    assert noalloc(M=0, N=4096, K=8192, splits=4, lda=8192, ldb=4096, ldc=4096) == 0


def test_splitk_noalloc_scratch_limit_in_header():
    text = open(os.path.join(ROOT, "include", "gemm_f32.h")).read()
    m = re.search(r"#define GEMM_F32_SPLITK_SCRATCH_BYTES \((\d+)LL << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.SPLITK_SCRATCH_BYTES


# --------------------------------------------------------- row reductions ---

def test_rows_header_is_plain_c():
    import subprocess
    src = "#include \"rows_f32.h\"\nint main(void){return 0;}\n"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), "-x", "c", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_rows_argument_errors():
    sm = lambda **k: g.rows_softmax_f32(k.get("rows", 4), k.get("width", 8), k.get("q", 8),
                                        k.get("causal", 1), 1.0, k.get("x", FAKE),
                                        k.get("ldx", 8), k.get("y", FAKE), k.get("ldy", 8), None)
    assert sm(rows=-1) == -1 and sm(width=-1) == -2 and sm(width=BIG) == -2
    assert sm(q=0) == -3 and sm(q=9) == -3 and sm(causal=2) == -4
    assert sm(x=None) == -6 and sm(ldx=7) == -7 and sm(y=None) == -8 and sm(ldy=0) == -9
    assert sm(rows=0) == 0 and sm(width=0, ldx=1, ldy=1, q=5) == 0   # nothing to do, no launch
    sb = lambda **k: g.rows_softmax_backward_f32(4, k.get("width", 8), 1.0, k.get("y", FAKE), 8,
                                                 k.get("dy", FAKE), k.get("lddy", 8),
                                                 k.get("dx", FAKE), 8, None)
    assert sb(y=None) == -4 and sb(dy=None) == -6 and sb(lddy=3) == -7 and sb(dx=None) == -8
    nm = lambda **k: g.rows_normalize_f32(k.get("rows", 4), 8, k.get("eps", 1e-5),
                                          k.get("x", FAKE), 8, k.get("y", FAKE), k.get("ldy", 8),
                                          None)
    assert nm(eps=-1.0) == -3 and nm(eps=float("nan")) == -3 and nm(eps=float("inf")) == -3
    assert nm(x=None) == -4 and nm(y=None) == -6 and nm(ldy=2) == -7 and nm(rows=0) == 0
    nb = lambda **k: g.rows_normalize_backward_f32(4, 8, 1e-5, k.get("x", FAKE), 8,
                                                   k.get("dy", FAKE), 8, k.get("dx", FAKE),
                                                   k.get("lddx", 8), None)
    assert nb(x=None) == -4 and nb(dy=None) == -6 and nb(dx=None) == -8 and nb(lddx=1) == -9


def test_tensor_helpers_refuse_host_tensors():
    """The tensor-level helpers check dtype and device before any library
    call: a host tensor's pointer must never reach a kernel."""
    import torch
    x = torch.ones(4, 4)
    for call in (lambda: g.matmul(x, x), lambda: g.linear(x, x), lambda: g.matmul_splitk(x, x, 2),
                 lambda: g.bmm(x[None], x[None]), lambda: g.softmax(x), lambda: g.normalize(x),
                 lambda: g.softmax_backward(x, x), lambda: g.normalize_backward(x, x),
                 lambda: g.matmul_bf16(x, x), lambda: g.pack_bf16(x)):
        with pytest.raises(ValueError, match="device tensor"):
            call()
    xb = x.to(torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        g.matmul_bf16_packed(xb, xb)
    with pytest.raises(TypeError, match="bfloat16"):
        g.matmul_bf16_packed(x, x)
    with pytest.raises(TypeError, match="float32"):
        g.matmul(x.double(), x.double())


# ------------------------------------------------------------- packed bf16 ---

def pack(rows=4, cols=6, src=FAKE, lds=None, trans=0, dst=FAKE, ldd=None):
    lds = max(1, rows if trans else cols) if lds is None else lds
    ldd = max(1, cols) if ldd is None else ldd
    return g.gemm_f32_pack_bf16(rows, cols, src, lds, trans, dst, ldd, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(rows=-1), -1), (dict(rows=BIG), -1), (dict(cols=-1), -2), (dict(cols=BIG), -2),
    (dict(src=None), -3), (dict(lds=5), -4), (dict(lds=BIG), -4),
    (dict(trans=1, lds=3), -4),            # transposed: src stored cols x rows, lds >= rows
    (dict(trans=2), -5), (dict(trans=-1), -5),
    (dict(dst=None), -6), (dict(ldd=5), -7), (dict(ldd=BIG), -7),
    (dict(rows=0, ldd=0), -7),             # ldd >= 1 even when nothing is written
])
def test_pack_bf16_invalid_arguments(kwargs, code):
    assert pack(**kwargs) == code


def test_pack_bf16_quick_return_without_launch():
    assert pack(rows=0, src=None, dst=None) == 0
    assert pack(cols=0, src=None, dst=None, lds=1, ldd=1) == 0


def packed(M=4, N=4, K=4, A=FAKE, lda=None, B=FAKE, ldb=None, C=FAKE, ldc=None):
    lda = max(1, K) if lda is None else lda
    ldb = max(1, K) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return g.gemm_f32_bf16_packed(M, N, K, A, lda, B, ldb, C, ldc, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(M=-1), -1), (dict(N=BIG), -2), (dict(K=-1), -3), (dict(K=BIG), -3),
    (dict(A=None), -4), (dict(lda=3), -5), (dict(lda=BIG), -5),
    (dict(B=None), -6), (dict(ldb=3), -7),  # B is N x K: ldb >= K
    (dict(N=9, ldb=3), -7),
    (dict(C=None), -8), (dict(ldc=3), -9), (dict(ldc=BIG), -9),
])
def test_bf16_packed_invalid_arguments(kwargs, code):
    assert packed(**kwargs) == code
    assert g.gemm_f32_strerror(code).startswith(f"invalid argument {-code} ")


def test_bf16_packed_quick_return_without_launch():
    assert packed(M=0, A=None, C=None) == 0
    assert packed(N=0, B=None, C=None) == 0


# ---------------------------------------------------------------- plans ---

def plan(M, N, K, ta=0, tb=0, A=ALIGNED, B=ALIGNED, lda=None, ldb=None, ldc=None, sA=0, sB=0, batch=1):
    lda = max(1, M if ta else K) if lda is None else lda
    ldb = max(1, K if tb else N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    code = g.gemm_f32_plan(M, N, K, A, lda, B, ldb, ldc, ta, tb, sA, sB, batch)
    return g.PLANS.get(code, code)


WORKLOAD_PLANS = {
    "S64": "mfma-64x64", "S1k": "mfma-64x64", "R": "mfma-64x64-pair", "S4k": "mfma-256x128",
    "T-fwd": "mfma-256x256", "T-dX": "mfma-256x128", "T-dW": "mfma-128x128-one-round",
    "attn-qk": "mfma-256x256", "attn-pv": "mfma-128x64",
}


@pytest.mark.parametrize("name", sorted(WORKLOAD_PLANS))
def test_plan_of_each_workload(name):
    """The automatic choice for every benchmark workload, decided on the
    host (operands 16-byte aligned, as device allocations are)."""
    w = gi.WORKLOADS[name]
    got = plan(w.M, w.N, w.K, w.transA, w.transB, lda=w.lda_, ldb=w.ldb_, ldc=w.ldc_,
               sA=w.stride_a, sB=w.stride_b, batch=w.batch)
    assert got == WORKLOAD_PLANS[name]


def test_plan_rules_at_their_edges():
    # 256 x 256 tile: K <= 1024, aligned operands and leading dimensions, >= 256 tiles
    assert plan(8192, 4096, 1024) == "mfma-256x256"
    assert plan(8192, 4096, 1024, tb=1) == "mfma-256x256"
    assert plan(8192, 4096, 1056) == "mfma-256x128"           # K above 1024
    assert plan(8192, 4096, 1024, A=ALIGNED + 4) == "mfma-256x128"  # A not 16-byte aligned
    assert plan(8192, 4096, 1024, lda=1026) == "mfma-256x128"       # lda not a multiple of 4
    assert plan(4096, 2048, 1024) == "mfma-128x128"           # 128 wide tiles: too few
    # batched: the strides must keep every product aligned
    assert plan(512, 512, 64, tb=1, sA=512 * 64, sB=512 * 64, batch=64) == "mfma-256x256"
    assert plan(512, 512, 64, tb=1, sA=512 * 64 + 1, sB=512 * 64, batch=64) == "mfma-128x128-kk"
    # 256 x 128: 384 tiles, or whole rounds of 256 when K >= 2048
    assert plan(8192, 1024, 4096, tb=1) == "mfma-256x128"
    assert plan(8192, 1024, 1024, tb=1, A=ALIGNED + 4) == "mfma-128x128-kk"
    # 128 x 128: one round or more, and the k-contiguous layout
    assert plan(1024, 4096, 8192, ta=1) == "mfma-128x128-one-round"
    assert plan(2048, 4096, 8192, ta=1) == "mfma-256x128"    # 256 large tiles: a whole round
    assert plan(1536, 4096, 8192, ta=1) == "mfma-128x128"    # 384 tiles, 192 large ones
    assert plan(2048, 2048, 2048, tb=1) == "mfma-128x128-kk"
    # narrow outputs: N <= 64 and at least 256 tiles of 128 rows
    assert plan(512, 64, 512, sA=512 * 512, sB=512 * 64, batch=64) == "mfma-128x64"
    assert plan(512, 65, 512, sA=512 * 512, sB=512 * 65, batch=64) == "mfma-64x64-pair"  # 1024 small tiles
    assert plan(512, 64, 512, sA=512 * 512, sB=512 * 64, batch=63) == "mfma-64x64-pair"  # 504 small tiles
    # small tiles: one workgroup per CU up to one tile per CU, two sharing a CU beyond
    assert plan(1024, 1024, 1024) == "mfma-64x64"             # 256 small tiles
    assert plan(1088, 1024, 1024) == "mfma-64x64-pair"        # 272
    assert plan(256, 64, 512, sA=256 * 512, sB=512 * 64, batch=64) == "mfma-64x64"  # 256 (batched)
    # degenerate shapes
    assert plan(0, 64, 64) == "nothing" and plan(64, 0, 64) == "nothing"
    assert plan(64, 64, 0) == "zero-fill"


@pytest.mark.parametrize("kwargs,code", [
    (dict(M=-1), -1), (dict(N=-1), -2), (dict(K=-1), -3), (dict(lda=3), -5), (dict(ldb=3), -7),
    (dict(ldc=3), -8), (dict(ta=2), -9), (dict(tb=-1), -10), (dict(sA=-1), -11), (dict(sB=-1), -12),
    (dict(batch=0), -13),
])
def test_plan_invalid_arguments(kwargs, code):
    args = dict(M=4, N=4, K=4)
    args.update(kwargs)
    assert g.gemm_f32_plan(args["M"], args["N"], args["K"], ALIGNED, args.get("lda", 4), ALIGNED,
                           args.get("ldb", 4), args.get("ldc", 4), args.get("ta", 0), args.get("tb", 0),
                           args.get("sA", 0), args.get("sB", 0), args.get("batch", 1)) == code
