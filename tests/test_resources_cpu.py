"""Register, scratch and LDS use of every kernel, read from the compiler.

CPU only.  Each ``csrc/*.hip`` is compiled for gfx950 with the library's own
flags plus ``-Rpass-analysis=kernel-resource-usage`` (the compiler's report
of registers, scratch, occupancy and LDS per kernel) and ``-S`` (the AMD
assembly of the code built here).  Checked:

* no kernel touches scratch memory (per-lane spill space) inside a loop:
  every accumulator, fragment and copy address stays in registers, so a
  configuration change that spills in its k loop fails here before it costs
  time on the GPU.  Outside the loops a kernel may park at most a value or
  two there; the large tiles and the 256 x 256 and mixed-precision kernels
  use none at all;
* no SGPR spills in the product kernels, and no dynamic stack;
* the occupancy and LDS footprint each tile configuration is designed
  around: the 256 x 128 and 256 x 256 FP32 tiles run one workgroup of 8
  waves per CU (2 waves per SIMD), the 128 x 128 tile two workgroups
  (4 waves per SIMD, at most 64 KB of LDS each), the 64 x 64 ring four,
  and the 64 x 64 tile with 128-k stages (grids of about one tile per CU)
  one workgroup with 128 KB of LDS.

The report's figures are printed, so ``pytest -s`` shows the table.
"""

import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from dense_fp32_matrix_gemm_amd import build as B

pytestmark = pytest.mark.slow


def _compile(src: str, tmp: str):
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = [B.HIPCC, *B.COMMON, f"-I{B.INCLUDE}", f"-I{B.CSRC}", "--offload-device-only", "-S",
           src, "-o", out, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr, open(out).read()


def _parse(remarks: str):
    kernels, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s*(.*?)\s*\[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            cur = {"mangled": text.split(":", 1)[1].strip()}
            kernels.append(cur)
        elif cur is not None and ":" in text:
            k, v = text.rsplit(":", 1)
            cur[k.strip()] = v.strip()
    return kernels


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    out = []
    for n in r.stdout.splitlines():
        n = re.sub(r"(\w+::)*\(anonymous namespace\)::", "", n)
        out.append(n[:n.index("(")] if "(" in n else n)
    return out


@pytest.fixture(scope="module")
def report():
    srcs = B.sources()
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            results = list(ex.map(lambda s: _compile(s, tmp), srcs))
    kernels, asm = [], {}
    for src, (remarks, text) in zip(srcs, results):
        ks = _parse(remarks)
        for k in ks:
            k["file"] = os.path.basename(src)
        kernels += ks
        asm[os.path.basename(src)] = text
    for k, name in zip(kernels, _demangle([k["mangled"] for k in kernels])):
        k["name"] = name
    return kernels, asm


def test_every_kernel_was_reported(report):
    kernels, _ = report
    names = " ".join(k["name"] for k in kernels)
    for family in ("mfma_kernel", "wide_kernel", "fma_kernel", "naive_kernel", "tiled_kernel",
                   "bf16_kernel", "packed_kernel", "splitk_reduce_kernel", "zero_fill_kernel"):
        assert family in names, family


# Scratch (per-lane spill memory) the compiler may use outside every loop:
# a value or two computed before a kernel's k loop and needed after it.
SCRATCH_LIMIT = 16  # bytes per lane: at most four values


def test_scratch_use(report):
    kernels, _ = report
    rows = [f"{k['VGPRs']:>4} VGPR {k['AGPRs']:>3} AGPR  scratch {k['ScratchSize [bytes/lane]']:>3}  "
            f"occ {k['Occupancy [waves/SIMD]']}  LDS {k['LDS Size [bytes/block]']:>6}  {k['name']}"
            for k in kernels]
    print("\n".join(rows))
    over = [k["name"] for k in kernels if int(k["ScratchSize [bytes/lane]"]) > SCRATCH_LIMIT]
    assert not over, "kernels beyond the scratch limit:\n" + "\n".join(over)
    # the k loops of the large tiles, and every 256 x 256 and mixed-precision
    # kernel, use none at all
    for k in kernels:
        cfg = _config(k["name"])
        big = cfg is not None and cfg[0] * cfg[1] >= 256 * 128
        if big or k["file"] in ("gemm_mfma_wide.hip", "gemm_bf16.hip", "gemm_bf16_packed.hip"):
            assert int(k["ScratchSize [bytes/lane]"]) == 0, k["name"]


def _loops(lines):
    """(first, last) line of every backward branch's range: the loops."""
    labels = {}
    for i, ln in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+):", ln)
        if m:
            labels[m.group(1)] = i
    spans = []
    for i, ln in enumerate(lines):
        m = re.search(r"\bs_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)", ln)
        if m and m.group(1) in labels and labels[m.group(1)] <= i:
            spans.append((labels[m.group(1)], i))
    return spans


def test_no_scratch_access_inside_any_loop(report):
    """Read from the instructions: whatever scratch a kernel uses is touched
    only before or after its loops, never per stage, so accumulators,
    fragments and copy addresses all stay in registers."""
    _, asm = report
    for f, text in asm.items():
        lines = text.splitlines()
        starts = [i for i, ln in enumerate(lines) if re.match(r"^_Z\w+:", ln)] + [len(lines)]
        for a, b in zip(starts, starts[1:]):
            body = lines[a:b]
            spans = _loops(body)
            hits = [i for i, ln in enumerate(body) if re.search(r"^\s*scratch_(load|store)", ln)
                    and any(x <= i <= y for x, y in spans)]
            assert not hits, f"{f} {body[0]}: {[body[i].strip() for i in hits[:3]]}"


def test_no_sgpr_spills_in_the_products_and_no_dynamic_stack(report):
    """The product kernels keep every scalar in a scalar register.  The row
    kernels that hold a long row in registers (up to 64 values per lane)
    need more column masks than there are scalar registers; the compiler
    parks the rest in lanes of a vector register (no memory: their scratch
    size is 0, checked above)."""
    kernels, _ = report
    for k in kernels:
        assert k["Dynamic Stack"] == "False", k["name"]
        if k["file"] != "rows.hip":
            assert int(k["SGPRs Spill"]) == 0, k["name"]


def _config(name):
    m = re.search(r"Config<([\d, ]+)>", name)
    return tuple(int(x) for x in m.group(1).split(",")) if m else None


def test_fp32_tile_occupancy_and_lds(report):
    kernels, _ = report
    seen = set()
    for k in kernels:
        occ, lds = int(k["Occupancy [waves/SIMD]"]), int(k["LDS Size [bytes/block]"])
        regs = int(k["VGPRs"]) + int(k["AGPRs"])
        if k["name"].startswith("void wide_kernel"):
            # 256 x 256: two 64 KB stage buffers, 8 waves in one workgroup per CU
            assert lds == 128 * 1024 and occ >= 2 and regs <= 256, k["name"]
            seen.add("256x256")
            continue
        if not k["name"].startswith("void mfma_kernel"):
            continue
        cfg = _config(k["name"])
        bm, bn, wpe, nbuf = cfg[0], cfg[1], cfg[5], cfg[10]
        assert occ >= min(wpe, 2), k["name"]
        stagger = len(cfg) > 14 and cfg[14] == 1
        if (bm, bn) == (256, 128):
            # at most 144 KB of stage buffers (four of 24 KB): one workgroup per CU
            assert lds <= 3 * 48 * 1024 and occ == 2 and regs <= 256, k["name"]
            seen.add("256x128")
        elif (bm, bn) == (128, 128) and nbuf == 2 and not stagger:
            # two workgroups per CU: 4 waves per SIMD, 64 KB of LDS each
            assert lds <= 64 * 1024 and occ >= 4 and regs <= 128, k["name"]
            seen.add("128x128")
        elif (bm, bn) == (128, 128) and cfg[2] == 16:
            # 16-k stages in four buffers: 64 KB, two workgroups per CU
            assert lds <= 64 * 1024 and occ >= 4 and regs <= 128, k["name"]
            seen.add("128x128")
        elif (bm, bn) == (128, 128) and cfg[2] == 32 and nbuf == 4:
            # one tile per CU: four 32 KB stage buffers, one workgroup
            assert lds <= 128 * 1024 and occ >= 2, k["name"]
            seen.add("128x128")
        elif (bm, bn) == (64, 64) and nbuf == 4:
            # grids of about one tile per CU: four 32 KB stage buffers (128 KB),
            # one workgroup (two waves per SIMD) per CU
            assert lds <= 128 * 1024 and occ >= 2, k["name"]
            seen.add("64x64")
        elif (bm, bn) == (64, 64):
            # more tiles than CUs: two workgroups share a CU
            assert lds <= 64 * 1024 and occ >= 4, k["name"]
            seen.add("64x64")
    assert seen == {"256x256", "256x128", "128x128", "64x64"}
