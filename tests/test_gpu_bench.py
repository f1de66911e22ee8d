"""The benchmark's output contract: ``bench.py`` run as the driver runs it
prints one JSON line with the required fields, the roofline and CPU-baseline
objects, and a passing sampled parity.  Marked ``gpu`` (the runs use the
device); ``--gpus`` above 1 is refused without touching it (CPU test).
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

REQUIRED = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"}
ROOFLINE = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def run_bench(*args, timeout=240):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def check_line(d, steps, warmup):
    assert REQUIRED <= set(d), REQUIRED - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert ROOFLINE <= set(roof), ROOFLINE - set(roof)
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9


@pytest.mark.gpu
def test_default_line_with_cpu_baseline():
    """The headline run (4096^3 FP32), short: every field, the CPU-baseline
    leg and a passing sampled parity."""
    d = run_bench("--steps", "3", "--warmup", "3")
    check_line(d, 3, 3)
    assert d["config"]["workload"] == "S4k" and d["dtype"] == "f32"
    assert d["roofline"]["bound"] == "mfma" and d["roofline"]["peak"] == 157.3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert d["parity"]["ok"] and d["parity"]["relfrob_3000_sampled"] <= 1e-6
    assert "torch.mm" in d["context"] and "relfrob_3000_sampled" in d["context"]["torch.mm"]
    cold = d["context"]["cold_cache"]
    assert cold["tflops"] > 0 and cold["scratch_mb"] == 512
    ws = d["windows_summary"]
    assert len(d["windows_ms_per_step"]) == 3 and ws["min_ms"] <= ws["median_ms"]
    assert ws["value_at_min"] >= ws["value_at_median"] > 0


@pytest.mark.gpu
@pytest.mark.parametrize("args,bound", [(("--rows", "softmax"), "hbm"),
                                        (("--algo", "bf16packed"), "mfma"),
                                        (("--workload", "attn-qk"), "mfma"),
                                        (("--algo", "naive", "--workload", "S1k"), "hbm")])
def test_other_lines(args, bound):
    d = run_bench(*args, "--steps", "2", "--warmup", "2", "--no-context")
    check_line(d, 2, 2)
    assert d["roofline"]["bound"] == bound
    assert d["parity"]["ok"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
    assert r.stdout.strip() == ""
