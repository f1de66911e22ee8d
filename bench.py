"""Throughput of the FP32 GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload S4k] [--algo auto]

One step is one C = A.B of the workload (default: the 4096^3 square
product the throughput metric is quoted on), with A, B and C resident in
HBM before timing starts.  At least W untimed steps (300 if W is not
given), and in either case at least 0.3 s of them, so that the timed steps
run at a settled clock (the line reports W and the calls actually made),
then exactly K steps between
two device synchronisations, timed with HIP events recorded on the stream
the library launches on (PyTorch's current stream).  Prints ONE JSON line.

Besides the metric the line carries:
  roofline      the GEMM kernel against the MI355X FP32 matrix peak
                (157.3 TFLOP/s), with HBM traffic from rocprofv3 counters
                when the committed counter summary matches these sources;
  cpu_baseline  the CPU oracle timed on a bounded row-panel of the same
                product on this host's cores (a reported baseline, not a target);
  context       the other kernel families (vector FMA, LDS-tiled, naive with
                its 1/4 flop-per-byte HBM model) and torch.mm on the same
                inputs, for comparison;
  parity        a sampled check of the timed result against the oracle.

cpu_baseline and parity form the CPU-baseline leg, the only part of this
script that runs the oracle (skipped with --no-cpu-baseline).

``--algo bf16`` times the mixed-precision entry point instead (operands
rounded to bf16, FP32 sums) against the dense bf16 matrix peak (2.5 PFLOP/s);
``--algo bf16packed`` times the product of operands packed beforehand
(gemm_f32_pack_bf16, outside the timed region, like a framework's bf16
copies of its weights), and reports the packing kernels' time and the
end-to-end rate beside it.

``--copy-probe`` instead runs a plain device copy of known size, the
scale reference for the HBM byte counters.  ``--gpus`` above 1 exits:
this benchmark measures one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

MI355X_FP32_PEAK_TFLOPS = 157.3   # 256 CU x 2.4 GHz x 256 FLOP/clk/CU (matrix and packed vector)
MI355X_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak (published; no structured sparsity)
MI355X_HBM_TBPS = 8.0
PROFILES = os.path.join(ROOT, "profiles")


# -------------------------------------------------- algorithmic work models ---

def gemm_flops(M: int, N: int, K: int) -> int:
    """2*M*N*K: a multiply and an add per (i, j, k) term."""
    return 2 * M * N * K


def naive_model_bytes(M: int, N: int, K: int) -> int:
    """The naive kernel's traffic model: every term reads one float of A and
    one of B from HBM (8 bytes per multiply-add), caches ignored."""
    return 8 * M * N * K


def tiled_model_bytes(M: int, N: int, K: int, BM: int, BN: int) -> int:
    """Global->shared traffic of a BM x BN-tiled product: each of the
    ceil(M/BM)*ceil(N/BN) tiles reads a BM x K panel of A and a K x BN panel of B."""
    tiles = -(-M // BM) * -(-N // BN)
    return 4 * K * tiles * (BM + BN)


def compulsory_bytes(M: int, N: int, K: int) -> int:
    """Read A and B once, write C once."""
    return 4 * (M * K + K * N + M * N)


# The sources each kernel family is compiled from (its own file plus the
# shared headers); a counter summary stays valid while these are unchanged.
KERNEL_SOURCES = {
    "gemm_f32_mfma": ["gemm_mfma.hip", "gemm_mfma_wide.hip", "tile_common.hpp", "gemm_internal.hpp"],
    "gemm_f32_fma": ["gemm_fma.hip", "tile_common.hpp", "gemm_internal.hpp"],
    "gemm_f32_tiled": ["gemm_simple.hip", "gemm_internal.hpp"],
    "gemm_f32_naive": ["gemm_simple.hip", "gemm_internal.hpp"],
    "gemm_f32_bf16": ["gemm_bf16.hip", "tile_common.hpp", "gemm_internal.hpp"],
    "gemm_f32_bf16packed": ["gemm_bf16_packed.hip", "tile_common.hpp", "gemm_internal.hpp"],
    "rows_softmax_f32": ["rows.hip", "gemm_internal.hpp", "../../include/rows_f32.h"],
}


def code_text(src: str) -> str:
    """C++ source without its comments and with runs of white space made one
    space: what the compiler sees, so that editing a comment does not change
    a kernel's digest.  String and character literals are kept as written."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(kernel: str = "gemm_f32_mfma") -> str:
    """Hash of the code (comments excluded) of the sources of one kernel
    family; counter summaries are valid only for this digest."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_fp32_matrix_gemm_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        p = os.path.join(csrc, name)
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """Per-launch HBM bytes from profiles/traffic_<kernel>_<workload>.md, or None
    if absent or taken from different sources."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if kernel not in KERNEL_SOURCES or fields.get("source_digest") != source_digest(kernel):
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ runner ---

def _timed(fn, steps: int, warmup: int):
    """Average ms per call of fn over `steps` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _window_summary(windows, work):
    """Median and fastest of the timed windows (ms per step), and the rate
    at each (work per step / time, in the line's unit)."""
    import statistics
    med, fast = statistics.median(windows), min(windows)
    return {"median_ms": med, "min_ms": fast,
            "value_at_median": work / (med * 1e-3) / 1e12, "value_at_min": work / (fast * 1e-3) / 1e12}


def _timed_cold(fn, reps: int = 30, scratch_mb: int = 512):
    """Mean ms of fn when each launch follows a scratch write larger than the
    caches; each launch is bracketed by its own HIP events on the current
    stream (the fills run between them, so the GPU never idles)."""
    import torch
    scratch = torch.empty(scratch_mb << 18, dtype=torch.float32, device="cuda")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        scratch.fill_(float(i))
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / reps
    del scratch
    return ms


def _timed_windows(fn, steps: int, windows: int = 3):
    """The timed region: exactly ``steps`` calls between two synchronisations,
    with HIP events also splitting them into ``windows`` consecutive windows.
    Returns (ms per call over all steps, [ms per call in each window])."""
    import torch
    torch.cuda.synchronize()
    bounds = [round(i * steps / windows) for i in range(windows + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    events[0].record()
    for w in range(windows):
        for _ in range(bounds[w + 1] - bounds[w]):
            fn()
        events[w + 1].record()
    torch.cuda.synchronize()
    per = [events[w].elapsed_time(events[w + 1]) / max(bounds[w + 1] - bounds[w], 1)
           for w in range(windows)]
    return events[0].elapsed_time(events[-1]) / steps, per


def _warm_up(fn, warmup, min_launches: int = 300, min_seconds: float = 0.3):
    """Run the untimed warm-up: at least ``warmup`` calls (``min_launches``
    when not given) and, either way, at least ``min_seconds`` of them.  The
    clock ramps up over the first tenths of a second of load, so a fixed
    handful of launches (a few ms of a 1 ms kernel) would time the ramp, not
    the kernel.  Returns (calls made, seconds spent)."""
    import torch
    want = min_launches if warmup is None else warmup
    done, t0 = 0, time.perf_counter()
    while done < want or time.perf_counter() - t0 < min_seconds:
        for _ in range(10):
            fn()
        done += 10
        torch.cuda.synchronize()
    return done, time.perf_counter() - t0


def _timed_warm(fn, steps: int):
    """A comparison timing: about 0.3 s of warm-up (at least 10 calls), then
    ``steps`` timed calls; ms per call."""
    _warm_up(fn, None, min_launches=10)
    return _timed(fn, steps, 0)


def _lscpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sampled_parity(w, A, B, c_host, mixed: bool, bias, act: int) -> dict:
    """Part of the CPU-baseline leg: 256 sampled entries of the timed result
    (the last product of a batch) against the oracle, to the FP32 bar."""
    import numpy as np
    import gemm_inputs as gi
    import oracle
    orc = oracle.load()
    rows, cols = gi.sample_entries(w.M, w.N, 256, seed=23)
    a0, b0, c0 = A, B, c_host
    if w.batch > 1:
        last = w.batch - 1
        a0 = A[last, :w.a_dims[0] * w.lda_].reshape(w.a_dims[0], w.lda_)
        b0 = B if w.shared_b else B[last, :w.b_dims[0] * w.ldb_].reshape(w.b_dims[0], w.ldb_)
        c0 = c0[last, :w.M * w.ldc_].reshape(w.M, w.ldc_)
    entries = orc.entries_bf16 if mixed else orc.entries
    ref = entries(a0, b0, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
    if bias is not None:
        ref = orc.epilogue((ref + bias[cols].astype(np.float64))[None, :], None, act)[0]
    got = c0[rows, cols].astype(np.float64)
    ratio = np.abs(got - ref) / (1e-6 * w.K + 1e-5 * np.abs(ref))
    return {"entries": int(rows.size), "max_err_over_bound": float(np.max(ratio)),
            "ok": bool(np.all(ratio <= 1.0))}


def sampled_relfrob(w, A, B, results, count: int = 3000) -> list:
    """Part of the CPU-baseline leg: the relative Frobenius error of each
    M x N result against the oracle over the same ``count`` sampled entries."""
    import numpy as np
    import gemm_inputs as gi
    import oracle
    rows, cols = gi.sample_entries(w.M, w.N, count, seed=17)
    ref = oracle.load().entries(A, B, w.M, w.N, w.K, w.transA, w.transB, rows, cols)
    return [float(np.linalg.norm(r[rows, cols].astype(np.float64) - ref) / np.linalg.norm(ref))
            for r in results]


def cpu_baseline(w, target_s: float = 12.0, mixed: bool = False) -> dict:
    """The oracle, as it stands, on a row panel of the workload's product
    (its mixed-precision function when ``mixed``)."""
    import numpy as np
    import oracle
    orc = oracle.load()
    A, B = w.make_a(), w.make_b()

    def run(rows: int) -> float:
        # a panel of `rows` rows of C: the same product restricted to A's first rows
        a_panel = A[:, :rows] if w.transA else A[:rows]
        t0 = time.perf_counter()
        fn = orc.gemm_bf16 if mixed else orc.gemm
        fn(np.ascontiguousarray(a_panel), B, rows, w.N, w.K, w.transA, w.transB)
        return time.perf_counter() - t0

    probe_rows = max(1, min(w.M, 16))
    t_probe = run(probe_rows)
    rows = int(min(w.M, max(probe_rows, target_s / max(t_probe, 1e-9) * probe_rows)))
    t = run(rows)
    tflops = gemm_flops(rows, w.N, w.K) / t / 1e12
    # context: numpy's float64 product (the host BLAS) on the same panel
    a64 = np.ascontiguousarray(A[:, :rows].T if w.transA else A[:rows], dtype=np.float64)[:, :w.K]
    b64 = (B[:w.N, :w.K].T if w.transB else B[:w.K, :w.N]).astype(np.float64)
    t0 = time.perf_counter()
    a64 @ b64
    t_np = time.perf_counter() - t0
    return {"value": tflops, "unit": "TFLOPS", "cores": orc.threads(), "kind": "oracle",
            "numpy_f64_matmul_same_panel": {"tflops": gemm_flops(rows, w.N, w.K) / t_np / 1e12,
                                            "seconds": t_np, "note": "context, not the oracle"},
            "sample": f"first {rows} of {w.M} rows of C ({w.name}: {w.M}x{w.N}x{w.K}), "
                      f"{t:.1f} s, FP64-accumulating triple loop"
                      f"{' on bf16-rounded operands' if mixed else ''}, OpenMP over rows",
            "host_cpu": _lscpu_model(), "os_cpu_count": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def copy_probe(mib: int = 1024, reps: int = 5) -> None:
    """A plain device copy of `mib` MiB, the scale reference for FETCH/WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "bytes_written": n * 4, "reps": reps}))


# Row-reduction workloads: the causal softmax of one attention layer's scores
# (8 sequences x 8 heads x 512 queries over 512 keys, head size 64, so scale
# 1/8) with its gradient, and the normalisation of the transformer set's
# activations X[8192 x 1024] with its gradient.
ROW_OPS = {
    "softmax": dict(rows=8 * 8 * 512, width=512, seed=3000, fn="rows_softmax_f32"),
    "softmax-bwd": dict(rows=8 * 8 * 512, width=512, seed=3000, fn="rows_softmax_backward_f32"),
    "normalize": dict(rows=8192, width=1024, seed=2000, fn="rows_normalize_f32"),
    "normalize-bwd": dict(rows=8192, width=1024, seed=2000, fn="rows_normalize_backward_f32"),
}


def row_bytes(op: str, rows: int, width: int) -> int:
    """Algorithmic bytes of a row reduction: each input read once and the
    output written once, 4 bytes per element (one input for the forward
    passes, two for the gradients)."""
    inputs = 2 if op.endswith("backward") else 1
    return 4 * (inputs + 1) * rows * width


def rows_oracle_leg(op, x, dy, got, rows, width, scale, eps):
    """The CPU-baseline leg of a row-reduction run, the only place it runs
    the oracle: 64 sampled rows of the timed result against it, and the
    oracle itself timed on the first 1024 rows (about 10 s, one core)."""
    import numpy as np
    from oracle import rows as R
    pick = np.sort(np.random.default_rng(5).choice(rows, 64, replace=False))
    if op == "softmax":
        # a row's causal mask follows its index r: alone, it is a group of
        # width - r % width queries
        ref = np.stack([R.softmax(x[r:r + 1], width, width - r % width, scale)[0] for r in pick])
        bound = 1e-5 * ref + 1e-8
    elif op == "softmax_backward":
        ref = R.softmax_backward(x[pick], dy[pick], width, scale)
        S = np.sum(np.abs(dy[pick].astype(np.float64) * x[pick]), axis=1, keepdims=True)
        bound = 1e-5 * scale * np.abs(x[pick]) * (np.abs(dy[pick]) + S) + 1e-9
    elif op == "normalize":
        ref = R.normalize(x[pick], width, eps)
        bound = 1e-5 * (np.abs(ref) + 1.0)
    else:
        ref = R.normalize_backward(x[pick], dy[pick], width, eps)
        a64, g64 = x[pick].astype(np.float64), dy[pick].astype(np.float64)
        sigma = np.sqrt(a64.var(axis=1, keepdims=True) + eps)
        xhat = (a64 - a64.mean(axis=1, keepdims=True)) / sigma
        bound = 2e-5 * (np.abs(ref) + (np.abs(g64) + np.abs(g64).mean(axis=1, keepdims=True)
                                       + np.abs(xhat) * np.abs(g64 * xhat).mean(axis=1, keepdims=True))
                        / sigma) + 1e-9
    ratio = np.abs(got[pick] - ref) / bound
    parity = {"rows": int(len(pick)), "max_err_over_bound": float(np.max(ratio)),
              "ok": bool(np.all(ratio <= 1.0))}
    sample = 1024
    fn = {"softmax": lambda: R.softmax(x[:sample], width, width, scale),
          "softmax_backward": lambda: R.softmax_backward(x[:sample], dy[:sample], width, scale),
          "normalize": lambda: R.normalize(x[:sample], width, eps),
          "normalize_backward": lambda: R.normalize_backward(x[:sample], dy[:sample], width, eps)}[op]
    reps, t = 0, 0.0
    t0 = time.perf_counter()
    while t < 10.0:
        fn()
        reps += 1
        t = time.perf_counter() - t0
    cpu = {"value": row_bytes(op, sample, width) * reps / t / 1e9, "unit": "GB/s",
           "cores": 1, "kind": "oracle",
           "sample": f"first {sample} of {rows} rows, {reps} repetitions in {t:.1f} s "
                     "(numpy float64, one row at a time)"}
    return parity, cpu


def rows_main(args) -> int:
    """Time one row reduction on its workload: algorithmic bytes (each input
    read once, the output written once) over the mean launch time, against
    the HBM roofline."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import gemm_inputs as gi
    import dense_fp32_matrix_gemm_amd as g

    spec = ROW_OPS[args.rows]
    rows, width = spec["rows"], spec["width"]
    g.load()
    scale, eps = 0.125, 1e-5
    if args.rows == "softmax-bwd":
        # the forward output y: seeded values in [0, 2/width), the range of a
        # row of probabilities (the gradient is defined for any y)
        x = (gi.stored_matrix(spec["seed"] + 1, rows, width, dist="u11") + np.float32(1.0)) \
            * np.float32(1.0 / width)
    else:
        x = gi.stored_matrix(spec["seed"], rows, width, dist="n01")
    dy = gi.stored_matrix(spec["seed"] + 2, rows, width, dist="n01")
    dx, ddy = torch.from_numpy(x).cuda(), torch.from_numpy(dy).cuda()
    out = torch.empty_like(dx)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    calls = {
        "softmax": lambda: g.rows_softmax_f32(rows, width, width, 1, scale, dx.data_ptr(), width,
                                              out.data_ptr(), width, s),
        "softmax-bwd": lambda: g.rows_softmax_backward_f32(rows, width, scale, dx.data_ptr(), width,
                                                           ddy.data_ptr(), width, out.data_ptr(),
                                                           width, s),
        "normalize": lambda: g.rows_normalize_f32(rows, width, eps, dx.data_ptr(), width,
                                                  out.data_ptr(), width, s),
        "normalize-bwd": lambda: g.rows_normalize_backward_f32(rows, width, eps, dx.data_ptr(),
                                                               width, ddy.data_ptr(), width,
                                                               out.data_ptr(), width, s),
    }
    call = calls[args.rows]

    def step():
        st = call()
        if st != 0:
            raise g.GemmError(st)

    op = {"softmax": "softmax", "softmax-bwd": "softmax_backward", "normalize": "normalize",
          "normalize-bwd": "normalize_backward"}[args.rows]
    nbytes = row_bytes(op, rows, width)
    torch.cuda.synchronize()
    warm_calls, warm_s = _warm_up(step, args.warmup)
    args.warmup = args.warmup if args.warmup is not None else warm_calls
    ms, windows = _timed_windows(step, args.steps)
    value = nbytes / (ms * 1e-3) / 1e9

    parity = cpu = None
    if not args.no_cpu_baseline:
        parity, cpu = rows_oracle_leg(op, x, dy, out.cpu().numpy(), rows, width, scale, eps)

    line = {
        "metric": f"row reduction HBM throughput ({op}, algorithmic bytes / s)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_calls_made": warm_calls, "warmup_seconds": warm_s,
        "ms_per_step": ms, "windows_ms_per_step": windows, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.rows, "rows": rows, "width": width,
                   "scale": scale if "softmax" in op else None, "eps": eps if "normalize" in op else None,
                   "causal": True if op == "softmax" else None, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": value, "peak": MI355X_HBM_TBPS * 1000,
                     "unit": "GB/s", "frac": value / (MI355X_HBM_TBPS * 1000),
                     "traffic": read_traffic(spec["fn"], args.rows),
                     "kernel": spec["fn"], "bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
        "parity": parity,
        "library": os.path.relpath(g.library_path(), ROOT),
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches before timing, at least this many and at least 0.3 s of them (default 300)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--algo", default="auto",
                    choices=["auto", "mfma", "mfma256", "mfma128", "mfma64", "mfmawide", "fma", "tiled", "naive", "bf16",
                             "bf16packed"],
                    help="kernel family; bf16 times the mixed-precision entry point "
                         "(operands rounded to bf16, FP32 sums), bf16packed its two-step form "
                         "on operands packed beforehand")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--epilogue", default="none", choices=["none", "bias", "gelu"],
                    help="time the fused C = act(A.B + bias) entry point instead")
    ap.add_argument("--splitk", type=int, default=0,
                    help="time gemm_f32_splitk with this many runs of k (partials plus their sum)")
    ap.add_argument("--rows", default=None, choices=sorted(ROW_OPS),
                    help="time a row reduction (GB/s against the HBM roofline) instead of a GEMM")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the GEMM has no multi-GPU path in this library.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import gemm_inputs as gi
    import dense_fp32_matrix_gemm_amd as g

    if args.copy_probe:
        copy_probe()
        return 0
    if args.rows:
        return rows_main(args)

    torch.backends.cuda.matmul.allow_tf32 = False
    name = args.workload or gi.HEADLINE
    w = gi.WORKLOADS[name]
    lib_path = g.library_path()
    g.load()  # fail loudly now if the HIP library is missing

    A, B, C = w.make_a(), w.make_b(), w.make_c()
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.from_numpy(C).cuda()
    stream = torch.cuda.current_stream()
    mixed = args.algo in ("bf16", "bf16packed")
    packed = args.algo == "bf16packed"
    algo_id = g.ALGOS["auto" if mixed else args.algo]

    batched = w.batch > 1
    if batched and args.algo not in ("auto", "mfma"):
        print("batched workloads run on the MFMA path only", file=sys.stderr)
        return 2
    fused = args.epilogue != "none"
    if mixed and batched:
        print("the mixed-precision entry point takes single products", file=sys.stderr)
        return 2
    if fused and (batched or args.algo not in ("auto", "mfma")):
        print("the fused epilogue runs single products on the MFMA path", file=sys.stderr)
        return 2
    splitk = args.splitk > 0
    if splitk and (batched or fused or mixed or args.algo not in ("auto", "mfma")):
        print("--splitk times single FP32 products on the MFMA path", file=sys.stderr)
        return 2
    ws_bytes = g.gemm_f32_splitk_workspace_size(w.M, w.N, w.K, args.splitk) if splitk else 0
    dws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda") if splitk else None
    bias = gi.stored_matrix(2003, 1, w.N, dist="n002")[0] if fused else None
    dbias = torch.from_numpy(bias).cuda() if fused else None
    act = g.ACT_GELU if args.epilogue == "gelu" else g.ACT_NONE
    # op(A) (M x K) and op(B) (K x N) as views of the stored operands
    op_a = dA.reshape(-1, A.shape[-1])[:, :w.a_dims[1]] if not batched else None
    op_b = dB.reshape(-1, B.shape[-1])[:, :w.b_dims[1]] if not batched else None
    if not batched:
        op_a = op_a.t() if w.transA else op_a
        op_b = op_b.t() if w.transB else op_b
    if packed:
        pa = g.pack_bf16(op_a)       # M x K, k along the rows
        pb = g.pack_bf16(op_b.t())   # N x K
        torch.cuda.synchronize()

    def step(algo=algo_id, plain=False):
        if splitk and not plain:
            st = g.gemm_f32_splitk(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                                   dC.data_ptr(), w.ldc_, w.transA, w.transB, args.splitk,
                                   dws.data_ptr(), ws_bytes, stream.cuda_stream)
        elif fused:
            st = g.gemm_f32_bias_act(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                                     dC.data_ptr(), w.ldc_, w.transA, w.transB, dbias.data_ptr(),
                                     act, stream.cuda_stream)
        elif packed and algo == algo_id and not plain:
            st = g.gemm_f32_bf16_packed(w.M, w.N, w.K, pa.data_ptr(), pa.stride(0), pb.data_ptr(),
                                        pb.stride(0), dC.data_ptr(), w.ldc_, stream.cuda_stream)
        elif mixed and algo == algo_id:
            st = g.gemm_f32_bf16(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                                 dC.data_ptr(), w.ldc_, w.transA, w.transB, stream.cuda_stream)
        elif batched:
            st = g.gemm_f32_strided_batched(
                w.M, w.N, w.K, dA.data_ptr(), w.lda_, w.stride_a, dB.data_ptr(), w.ldb_,
                w.stride_b, dC.data_ptr(), w.ldc_, w.stride_c, w.batch, w.transA, w.transB,
                stream.cuda_stream)
        else:
            st = g.gemm_f32_ex(w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_,
                               dC.data_ptr(), w.ldc_, w.transA, w.transB, stream.cuda_stream,
                               algo)
        if st != 0:
            raise g.GemmError(st)

    flops = w.flops
    torch.cuda.synchronize()
    warm_calls, warm_s = _warm_up(step, args.warmup)
    args.warmup = args.warmup if args.warmup is not None else warm_calls
    ms, windows = _timed_windows(step, args.steps)
    value = flops / (ms * 1e-3) / 1e12

    c_host = dC.cpu().numpy()

    kernel = "gemm_f32_" + ("mfma" if args.algo in ("auto", "mfma256", "mfma128", "mfma64", "mfmawide")
                            else args.algo)
    peak = MI355X_BF16_PEAK_TFLOPS if mixed else MI355X_FP32_PEAK_TFLOPS
    roofline = {"bound": "mfma", "achieved": value, "peak": peak,
                "unit": "TFLOP/s", "frac": value / peak,
                "traffic": read_traffic(kernel, name),
                "kernel": kernel, "flops_per_launch": flops,
                "compulsory_bytes": compulsory_bytes(w.M, w.N, w.K) * w.batch}
    roofline["peak_basis"] = ("dense bf16 matrix-core peak, published" if mixed else
                              "FP32 MFMA: 256 flop/clk/CU x 256 CUs x 2.4 GHz")
    if args.algo == "naive":
        model = naive_model_bytes(w.M, w.N, w.K) / (ms * 1e-3) / 1e9
        roofline.update(bound="hbm", achieved=model, peak=MI355X_HBM_TBPS * 1000,
                        unit="GB/s", frac=model / (MI355X_HBM_TBPS * 1000),
                        peak_basis="the pages' naive model: every operand read from HBM at 8.0 TB/s, "
                                   "8 bytes per multiply-add (1/4 flop per byte)",
                        measured_limiter="load latency: each wave waits for its k-th loads before the "
                                         "next, one load in flight per wave (profiles/naive_S4k.md)")
    elif args.algo == "fma":
        # The kernel issues plain v_fmac_f32 (packed FP32 is disabled in every
        # build); gfx950 completes one wave64 v_fmac_f32 per 2 cycles per SIMD,
        # so its peak is 64 lanes x 2 flop / 2 cycles x 4 SIMDs x 256 CUs x
        # 2.4 GHz, the same 157.3 TFLOP/s (the kernel's own counters show more
        # than one instruction per 4 cycles per SIMD).
        roofline.update(bound="alu", peak_basis="plain v_fmac_f32 (VOP2): one wave64 instruction per "
                        "2 cycles per SIMD, 64 x 2 flop / 2 x 4 SIMDs x 256 CUs x 2.4 GHz")

    context = None
    vendor_host = None  # torch.mm's result, for the accuracy comparison
    if not args.no_context and batched:
        def view(x, rows, cols, ld, stride, trans):
            v = x[:, :rows * ld].reshape(-1, rows, ld)[:, :, :cols]
            v = v.expand(w.batch, rows, cols) if stride == 0 else v
            return (v.transpose(1, 2) if trans else v).contiguous()
        ta = view(dA.reshape(-1, A.shape[-1]), *w.a_dims, w.lda_, w.stride_a, w.transA)
        tb = view(dB.reshape(-1, B.shape[-1]), *w.b_dims, w.ldb_, w.stride_b, w.transB)
        out = torch.empty((w.batch, w.M, w.N), dtype=torch.float32, device="cuda")
        tms = _timed_warm(lambda: torch.bmm(ta, tb, out=out), 20)
        context = {"torch.bmm (contiguous copies)": {"tflops": flops / (tms * 1e-3) / 1e12,
                                                     "ms": tms}}
    elif not args.no_context and fused:
        ta = dA[:, :w.a_dims[1]]
        tb = dB[:, :w.b_dims[1]]
        ta = ta.t() if w.transA else ta
        tb = tb.t() if w.transB else tb
        out = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

        def unfused():
            torch.addmm(dbias, ta, tb, out=out)
            if act == g.ACT_GELU:
                torch.nn.functional.gelu(out)
        tms = _timed_warm(unfused, 50)
        plain = _timed_warm(lambda: g.gemm_f32_ex(
            w.M, w.N, w.K, dA.data_ptr(), w.lda_, dB.data_ptr(), w.ldb_, dC.data_ptr(), w.ldc_,
            w.transA, w.transB, stream.cuda_stream, g.ALGOS["mfma"]), 50)
        context = {"torch addmm+gelu (unfused)": {"tflops": flops / (tms * 1e-3) / 1e12,
                                                  "ms": tms},
                   "gemm_f32 without epilogue": {"tflops": flops / (plain * 1e-3) / 1e12,
                                                 "ms": plain}}
    elif not args.no_context and splitk:
        plain = _timed_warm(lambda: step(g.ALGOS["mfma"], plain=True), 50)
        ta = dA[:, :w.a_dims[1]]
        tb = dB[:, :w.b_dims[1]]
        ta = ta.t() if w.transA else ta
        tb = tb.t() if w.transB else tb
        out = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        tms = _timed_warm(lambda: torch.mm(ta, tb, out=out), 50)
        context = {"gemm_f32 (one product)": {"tflops": flops / (plain * 1e-3) / 1e12, "ms": plain},
                   "torch.mm": {"tflops": flops / (tms * 1e-3) / 1e12, "ms": tms},
                   "workspace_bytes": ws_bytes}
    elif not args.no_context and mixed:
        ta, tb = op_a, op_b
        ha, hb = ta.to(torch.bfloat16), tb.to(torch.bfloat16)
        out16 = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        t16 = _timed_warm(lambda: torch.mm(ha, hb, out=out16), 20)
        t32 = _timed_warm(lambda: torch.mm(ta, tb, out=out), 20)
        mine = _timed_warm(lambda: step(g.ALGOS["mfma"]), 20)
        context = {"torch.mm bf16 (operands pre-converted, bf16 output)":
                   {"tflops": flops / (t16 * 1e-3) / 1e12, "ms": t16},
                   "torch.mm f32": {"tflops": flops / (t32 * 1e-3) / 1e12, "ms": t32},
                   "gemm_f32 (FP32 MFMA)": {"tflops": flops / (mine * 1e-3) / 1e12, "ms": mine}}
        # the vendor product with the same output precision as ours (FP32 C
        # from bf16 operands), where this PyTorch offers it
        try:
            torch.mm(ha, hb, out_dtype=torch.float32)
            t16f = _timed_warm(lambda: torch.mm(ha, hb, out_dtype=torch.float32), 20)
            context["torch.mm bf16 operands, FP32 output (out_dtype)"] = {
                "tflops": flops / (t16f * 1e-3) / 1e12, "ms": t16f,
                "note": "allocates its output on every call"}
        except (RuntimeError, TypeError) as e:
            context["torch.mm bf16 operands, FP32 output (out_dtype)"] = {"unavailable": str(e).split("\n")[0][:160]}
        if packed:
            # the packing kernels (HBM-bound: 4 bytes read, 2 written per
            # element) and the fused one-step entry point on the same inputs
            tpa = _timed_warm(lambda: g.pack_bf16(op_a, out=pa), 20)
            tpb = _timed_warm(lambda: g.pack_bf16(op_b.t(), out=pb), 20)
            fused1 = _timed_warm(lambda: step(algo_id, plain=True), 20)
            pbytes = 6 * (w.M * w.K + w.N * w.K)
            context.update({
                "pack A and B (gemm_f32_pack_bf16)": {"ms": tpa + tpb, "gbps": pbytes / ((tpa + tpb) * 1e-3) / 1e9},
                "pack + product (end to end)": {"tflops": flops / ((ms + tpa + tpb) * 1e-3) / 1e12,
                                                "ms": ms + tpa + tpb},
                "gemm_f32_bf16 (one step, converts on every read)": {"tflops": flops / (fused1 * 1e-3) / 1e12,
                                                                     "ms": fused1}})
    elif not args.no_context:
        context = {}
        for other in ("mfma", "fma", "tiled", "naive"):
            if other == args.algo or (other == "mfma" and args.algo == "auto"):
                continue
            reps = 3 if other == "naive" else 10
            # the naive kernel takes tens of ms at full size: warm up by count
            oms = (_timed(lambda: step(g.ALGOS[other]), reps, 1) if other == "naive"
                   else _timed_warm(lambda: step(g.ALGOS[other]), reps))
            entry = {"tflops": flops / (oms * 1e-3) / 1e12, "ms": oms}
            if other == "naive":
                gbps = naive_model_bytes(w.M, w.N, w.K) / (oms * 1e-3) / 1e9
                roof = MI355X_HBM_TBPS * 1e12 / 4 / 1e12
                entry.update(model_gbps=gbps, model_roofline_tflops=roof,
                             frac_of_model_roofline=entry["tflops"] / roof)
            context[other] = entry
        # the vendor library through PyTorch, same shapes (a labelled comparison)
        ta = dA[:, :w.a_dims[1]]
        tb = dB[:, :w.b_dims[1]]
        ta = ta.t() if w.transA else ta
        tb = tb.t() if w.transB else tb
        out = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        tms = _timed_warm(lambda: torch.mm(ta, tb, out=out), 20)
        context["torch.mm"] = {"tflops": flops / (tms * 1e-3) / 1e12, "ms": tms}
        vendor_host = out.cpu().numpy()
        # cold cache: each launch after a 512 MB scratch write, which evicts
        # A, B and C from L2 and the 256 MB Infinity Cache
        cms = _timed_cold(lambda: step(algo_id))
        context["cold_cache"] = {"tflops": flops / (cms * 1e-3) / 1e12, "ms": cms, "scratch_mb": 512,
                                 "launches": 30, "note": "each launch timed alone after a 512 MB write"}

    # The CPU-baseline leg, the only place this script runs the oracle: the
    # oracle timed on a sample of the workload, and a sampled check of the
    # timed result against it.
    cpu = parity = None
    if not args.no_cpu_baseline:
        parity = sampled_parity(w, A, B, c_host, mixed, bias if fused else None, act)
        if vendor_host is not None:
            # the same accuracy measure for our result and the vendor's, on
            # the same 3000 sampled entries
            mine, theirs = sampled_relfrob(w, A, B, (c_host[:, :w.N], vendor_host))
            parity["relfrob_3000_sampled"] = mine
            context["torch.mm"]["relfrob_3000_sampled"] = theirs
            context["torch.mm"]["meets_1e-6_bound"] = bool(theirs <= 1e-6)
        if not batched:
            cpu = cpu_baseline(w, mixed=mixed)

    line = {
        "metric": ("mixed-precision GEMM TFLOPS (2MNK/s; bf16 operands packed beforehand, FP32 sums)"
                   if packed else
                   "mixed-precision GEMM TFLOPS (2MNK/s; bf16 operands, FP32 sums)" if mixed else
                   "FP32 GEMM TFLOPS (2MNK/s) and % of MI355X FP32 peak at N=4096"),
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls_made": warm_calls,
        "warmup_seconds": warm_s,
        "ms_per_step": ms,
        "windows_ms_per_step": windows,
        "windows_summary": _window_summary(windows, flops),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mixed else "f32",
        "data": "synthetic",
        "config": {"workload": name, "batch": w.batch, "M": w.M, "N": w.N, "K": w.K,
                   "lda": w.lda_,
                   "ldb": w.ldb_, "ldc": w.ldc_, "transA": w.transA, "transB": w.transB,
                   "inputs": w.description, "seeds": [w.seed_a, w.seed_b],
                   "algo": args.algo, "epilogue": args.epilogue, "splitk": args.splitk,
                   "parallelism": "single GPU"},
        "pct_of_peak": 100.0 * value / peak,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "context": context,
        "parity": parity,
        "library": os.path.relpath(lib_path, ROOT),
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
