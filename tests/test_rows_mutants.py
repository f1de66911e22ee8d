"""Plant plausible mistakes in copies of the row-reduction oracle and check
that the pins catch each one (CPU only; the real source is never modified).

Each mutant is oracle/rows.py with one textual change -- a mask off by one,
a dropped scale, a sample instead of a population variance, epsilon outside
the root, a dropped gradient term, a log-sum taken without the max -- loaded
as a fresh module and run through every pin; at least one must fail.
"""

import os
import types

import pytest

import rows_pins
from oracle import rows as R

SOURCE = open(R.__file__).read()

MUTANTS = {
    "position_off_by_one": ("return width - queries + r % queries", "return width - queries + r % queries - 1"),
    "mask_drops_own_position": ("keep = pos[r] + 1", "keep = pos[r]"),
    "mask_keeps_one_future": ("keep = pos[r] + 1", "keep = min(pos[r] + 2, width)"),
    "scale_dropped": ("z = scale * a[r, :keep]", "z = a[r, :keep]"),
    "logsum_without_max": ("log_sum = np.log(np.sum(np.exp(z - m)))", "log_sum = np.log(np.sum(np.exp(z)))"),
    "softmax_grad_without_scale": ("out[r] = scale * yy[r] * (g[r] - d)", "out[r] = yy[r] * (g[r] - d)"),
    "softmax_grad_sign": ("out[r] = scale * yy[r] * (g[r] - d)", "out[r] = scale * yy[r] * (g[r] + d)"),
    "sample_variance": ("        var = np.mean(dev * dev)\n", "        var = np.sum(dev * dev) / (n - 1)\n"),
    "eps_outside_root": ("out[r] = dev / np.sqrt(var + eps)", "out[r] = dev / (np.sqrt(var) + eps)"),
    "norm_grad_drops_mean": ("(g[r] - np.mean(g[r]) - xhat * np.mean(g[r] * xhat)) / sigma",
                             "(g[r] - xhat * np.mean(g[r] * xhat)) / sigma"),
    "norm_grad_drops_projection": ("(g[r] - np.mean(g[r]) - xhat * np.mean(g[r] * xhat)) / sigma",
                                   "(g[r] - np.mean(g[r])) / sigma"),
    "bytes_miscount": ('"softmax_backward": 3', '"softmax_backward": 2'),
}


def mutant_module(old, new):
    assert SOURCE.count(old) >= 1, f"mutation target missing: {old!r}"
    mod = types.ModuleType("rows_mutant")
    mod.__file__ = R.__file__
    exec(compile(SOURCE.replace(old, new, 1), "rows_mutant", "exec"), mod.__dict__)
    return mod


def test_unmodified_copy_passes():
    rows_pins.run_all(mutant_module("import numpy as np", "import numpy as np"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mod = mutant_module(old, new)
    with pytest.raises(Exception):
        rows_pins.run_all(mod)
