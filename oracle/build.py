"""Build the CPU oracle library (plain C, gcc, OpenMP).

TEST INFRASTRUCTURE: see the header of ``gemm_ref.c``.  This build shares no
flags, headers or steps with the HIP library's build.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gemm_ref.c")
LIBRARY = os.path.join(HERE, "libgemm_ref.so")

# -O2 without -ffast-math: gcc keeps the k-ordered double sum as written.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY, verbose: bool = False) -> str:
    """Compile ``source`` into the shared library ``output`` and return its path."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, source, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
