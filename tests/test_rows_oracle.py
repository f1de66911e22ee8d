"""The row-reduction oracle (oracle/rows.py) against its pins (CPU only)."""

import pytest

import rows_pins
from oracle import rows as R


@pytest.mark.parametrize("pin", rows_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(R)


def test_bench_row_byte_model_matches_the_oracle():
    """bench.py keeps its own copy of the row-reduction byte model (it may
    not import the oracle outside its CPU-baseline leg); both must agree."""
    import bench
    for op in ("softmax", "softmax_backward", "normalize", "normalize_backward"):
        for rows, width in ((1, 1), (32768, 512), (8192, 1024)):
            assert bench.row_bytes(op, rows, width) == R.algorithmic_bytes(op, rows, width)
