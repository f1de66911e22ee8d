"""Build the HIP library ``libgemm_f32.so`` for gfx950, in-tree.

Every ``csrc/*.hip`` translation unit is compiled by hipcc to an object in
``_build/`` (in parallel), then linked into a shared library next to this
file, where the Python binding loads it.  Run ``python -m
dense_fp32_matrix_gemm_amd.build`` or call ``build()``.

Flags: ``-O3``; packed FP32 instructions are disabled for device code
(``-packed-fp32-ops``), so the compiler emits scalar ``v_fma_f32`` /
``v_add_f32``; the matrix-core path is unaffected.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys
from typing import List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libgemm_f32.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources() -> List[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Evidence builds: the same sources with one design choice undone, written
# next to the library under their own names (load one with the environment
# variable GEMM_F32_LIBRARY).  Not used by the package itself.
ABLATIONS = {
    "noswizzle": ["-DGEMM_MFMA_SWIZZLE=0"],  # MFMA kernel LDS rows without the XOR swizzle
    "nopad": ["-DGEMM_FMA_PAD=0"],           # vector-FMA kernel LDS rows without padding
    "fmanoswizzle": ["-DGEMM_FMA_SWIZZLE=0"],  # vector-FMA kernel: transposed tiles unswizzled
    "singlebuffer": ["-DGEMM_MFMA_SINGLE_BUFFER=1"],  # MFMA kernel: copy/barrier/compute/barrier
    # MFMA kernel, 256 x 128 tile, one running accumulator instead of chunked
    # sums (misses the 1e-6 error bound: what the chunking costs)
    "nochunk": ["-DGEMM_MFMA_HUGE_CONFIG=256,128,16,4,2,2,4,1,1,1,4,0,1,0,0,1"],
    # race detection: every stage buffer holds NaN between its release and
    # its refill (FP32 MFMA, 256 x 256 and packed bf16 kernels; same results)
    "poison": ["-DGEMM_LDS_POISON=1"],
}


def _compile(src: str, verbose: bool, extra: List[str], build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the device feature flag; drop that note
    noise = [ln for ln in r.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose: bool = False, output: Optional[str] = None,
          extra_flags: Optional[List[str]] = None, jobs: Optional[int] = None,
          ablation: Optional[str] = None) -> str:
    """Compile and link the library (or one of the ABLATIONS, as
    libgemm_f32_<name>.so); returns the path of the ``.so``."""
    extra = list(extra_flags or [])
    build_dir = BUILD_DIR
    if ablation is not None:
        extra += ABLATIONS[ablation]
        build_dir = os.path.join(BUILD_DIR, ablation)
        output = output or os.path.join(PKG, f"libgemm_f32_{ablation}.so")
    output = output or LIBRARY
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    jobs = jobs or min(len(srcs), 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, build_dir), srcs))
    tmp = output + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    abl = sys.argv[sys.argv.index("--ablation") + 1] if "--ablation" in sys.argv else None
    print(build(verbose="-v" in sys.argv, ablation=abl))
