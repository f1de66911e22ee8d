"""Host-side pieces of bench.py that the GPU run relies on.  CPU only."""

import os

import bench

CSRC = os.path.join(os.path.dirname(bench.__file__), "dense_fp32_matrix_gemm_amd", "csrc")


def test_code_text_drops_comments_keeps_literals():
    src = 'int a = 1; // note\n/* block\n note */ const char *s = "x // y /* z */";\nchar q = \'\\\'\';  b  =  2;'
    assert bench.code_text(src) == 'int a = 1; const char *s = "x // y /* z */"; char q = \'\\\'\'; b = 2;'


def test_comment_edits_keep_a_kernel_digest_and_code_edits_change_it():
    with open(os.path.join(CSRC, "gemm_mfma.hip"), encoding="utf-8") as f:
        src = f.read()
    base = bench.code_text(src)
    commented = src.replace("{", "{ // an added note\n", 1).replace(";", "; /* another */", 1)
    assert bench.code_text(commented) == base
    assert bench.code_text(src.replace("kWave", "kWave2", 1)) != base


def test_every_listed_source_exists():
    for files in bench.KERNEL_SOURCES.values():
        for name in files:
            assert os.path.exists(os.path.join(CSRC, name)), name
    assert len(bench.source_digest("gemm_f32_mfma")) == 16
