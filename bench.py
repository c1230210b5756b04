"""Benchmark of the dense GEMM hot path on one MI355X.

One step is one gemm() call through the C ABI on the full workload: host
checks, path and tile selection, and the matrix-core kernel with its fused
epilogue (inputs already resident in HBM). The default workload is the
compute-bound 8192^3 bf16 case with B stored [N,K] (transB = 1), alpha = 1,
beta = 0.

Prints ONE JSON line with TFLOP/s (2MNK/t), the roofline of the kernel
(measured with HIP events on the stream the kernel runs on), the oracle's
max relative error on sampled rows, and the CPU oracle timed on a bounded
sample of the same workload on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--shape M,N,K,dtype,tA,tB[,alpha,beta[,lda[,ldb]]]]
                  [--no-cpu-baseline] [--cpu-seconds S]
  python bench.py --copy-calibration   # plain copy of known size (counter scale)
  python bench.py --library-context    # the same workload on PyTorch's own GEMM
                                       # (hipBLASLt on ROCm): context, not a result
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0,  # MI355X dense MFMA, published
               "f32_bf16": 2500.0, "f32_f16": 2500.0}  # rounded operands run on the same cores
PEAK_HBM_GBS = 8000.0
PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 MFMA, published
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, published
COPY_CAL_BYTES = 1 << 30
DIST_TEXT = {"uniform": "uniform[-1, 1]", "normal": "normal(0, 1)",
             "normal_invsqrtk": "normal(0, 1/sqrt(K))"}


def kernel_sources_digest(files) -> str:
    """Digest of a kernel's source files (paths relative to the package's
    csrc/), to tell whether counters stored for that kernel are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_tile_amd", "csrc")
    for name in sorted(files):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed counter summary, or None if the summary is missing or was taken
    on different sources of that kernel (the summary names its source files
    and their digest)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    files = vals.get("kernel_source_files", "").split()
    try:
        if not files or vals.get("kernel_sources_digest") != kernel_sources_digest(files):
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError, OSError):
        return None


class ClockSampler:
    """Samples the GPU's shader clock and socket power on a host thread.

    Source: the amdgpu metrics table through amdsmi (current gfx clock of each
    XCD, socket power), else the driver's pp_dpm_sclk current level and hwmon
    power1_input. The firmware refreshes these about once a second, so a
    reading describes the second before it: only a sustained run of a second
    or more gives a figure that belongs to the kernel."""

    def __init__(self, period_s: float = 0.02):
        import glob
        import threading
        self.period = period_s
        self.samples = []  # (t, mean MHz over XCDs, per-XCD MHz or None, W or None)
        self.source = None
        self._smi = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = (amdsmi, amdsmi.amdsmi_get_processor_handles()[0])
            self.source = "amdsmi gpu metrics (current_gfxclks per XCD, current_socket_power)"
        except Exception:  # amdsmi missing or no device: the sysfs files below
            self._smi = None
        self.sclk = next(iter(sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))), None)
        dev = os.path.dirname(self.sclk) if self.sclk else None
        hw = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))) if dev else []
        self.power = os.path.join(hw[0], "power1_input") if hw else None
        self.cap = os.path.join(hw[0], "power1_cap") if hw else None
        if self._smi is None and self.sclk:
            self.source = "amdgpu pp_dpm_sclk current level, hwmon power1_input"
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self.t0 = None

    def _read_sysfs(self):
        mhz = w = None
        # One line per clock level ("1: 2400Mhz"); the current one ends in "*".
        with open(self.sclk) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    mhz = float(line.split()[1].lower().replace("mhz", ""))
        if self.power:
            with open(self.power) as f:
                w = float(f.read()) / 1e6
        return mhz, None, w

    def _read_smi(self):
        amdsmi, h = self._smi
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        per = [float(v) for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float))
               and 0 < v < 10000]
        if not per and isinstance(m.get("current_gfxclk"), (int, float)):
            per = [float(m["current_gfxclk"])]
        w = m.get("current_socket_power")
        w = float(w) if isinstance(w, (int, float)) else None
        return (sum(per) / len(per) if per else None), (per or None), w

    def _run(self):
        while not self._stop.is_set():
            try:
                mhz, per, w = self._read_smi() if self._smi else self._read_sysfs()
                if mhz:
                    self.samples.append((time.perf_counter() - self.t0, mhz, per, w))
            except Exception:  # a sensor read that fails is skipped
                pass
            time.sleep(self.period)

    def __enter__(self):
        self.t0 = time.perf_counter()
        if self._smi or self.sclk:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self, after_s: float = 0.0):
        ss = [x for x in self.samples if x[0] >= after_s]
        if not ss:
            return None
        mhz = [x[1] for x in ss]
        out = {"sclk_mhz_mean": round(sum(mhz) / len(mhz), 1), "sclk_mhz_min": min(mhz),
               "sclk_mhz_max": max(mhz), "samples": len(ss), "source": self.source}
        per = [x[2] for x in ss if x[2]]
        if per and all(len(p) == len(per[0]) for p in per):
            out["sclk_mhz_per_xcd_mean"] = [round(sum(p[i] for p in per) / len(per), 1)
                                            for i in range(len(per[0]))]
        w = [x[3] for x in ss if x[3] is not None]
        if w:
            out["power_w_mean"] = round(sum(w) / len(w), 1)
        try:
            with open(self.cap) as f:
                out["power_cap_w"] = float(f.read()) / 1e6
        except (OSError, TypeError, ValueError):
            pass
        return out


def warm_up(step, steps: int, seconds: float):
    """Runs `steps` untimed steps, then more until `seconds` have passed since
    the first (host syncs every ~20 ms). Returns what was run."""
    import torch
    t0 = time.perf_counter()
    n = 0
    for _ in range(steps):
        step()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < seconds:
        t1 = time.perf_counter()
        k = 0
        while time.perf_counter() - t1 < 0.02:
            step()
            k += 1
            if k % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        n += k
    return {"steps": n, "seconds": round(time.perf_counter() - t0, 3)}


def sustained_clock(step, stream, ms_per_step: float, seconds: float, settle_s: float = 1.0):
    """Runs `step` back to back for `seconds` (untimed for the result; the
    same call as the timed steps) and returns the clock and power sampled
    after the first `settle_s` seconds, with the mean time per step over that
    part (HIP events on the launch stream)."""
    import torch
    chunk = max(1, int(20.0 / max(ms_per_step, 1e-3)))  # ~20 ms between host syncs
    e0 = e1 = None
    n = 0
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            if e0 is None and time.perf_counter() - t0 >= settle_s:
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                n = 0
            for _ in range(chunk):
                step()
            n += chunk
            torch.cuda.synchronize()
        if e0 is not None:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            torch.cuda.synchronize()
    out = clk.summary(after_s=settle_s) or {}
    out["window_s"] = seconds
    out["settle_s"] = settle_s
    if e0 is not None and n:
        out["ms_per_step"] = round(e0.elapsed_time(e1) / n, 5)
        out["steps"] = n
    return out


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, inp, seconds: float):
    """Time the oracle (as it stands) on a bounded row sample of the workload."""
    import numpy as np

    import oracle
    import workloads

    lda, ldb, ldc, _ = cfg.lds()
    C = inp.C.numpy().reshape(-1) if inp.C is not None else None
    if cfg.dtype.startswith("f32_"):  # float32 operands, rounded by the oracle itself
        ref = oracle.gemm_reference_f32
        dt = 0 if cfg.dtype == "f32_f16" else 1
        A, B = inp.A.numpy().reshape(-1), inp.B.numpy().reshape(-1)
    else:
        ref = oracle.gemm_reference
        dt = workloads.DTYPE_CODE[cfg.dtype]
        A = workloads.bits_u16(inp.A).reshape(-1)
        B = workloads.bits_u16(inp.B).reshape(-1)

    def timed(nrows):
        rows = np.arange(nrows)
        t0 = time.perf_counter()
        ref(cfg.M, cfg.N, cfg.K, dt, cfg.transA, cfg.transB, cfg.alpha, cfg.beta, A, lda, B, ldb,
            C, ldc, rows=rows, with_bound=False)
        return time.perf_counter() - t0

    # Two short probes give a fixed cost (operand decode) and a per-row cost;
    # the measured call is then sized to take about `seconds`.
    r0, r1 = min(cfg.M, 64), min(cfg.M, 256)
    t0 = timed(r0)
    rows, t = r0, t0
    if r1 > r0:
        t1 = timed(r1)
        per_row = max((t1 - t0) / (r1 - r0), 1e-6)
        fixed = max(t0 - r0 * per_row, 0.0)
        rows = int(min(cfg.M, max(r1, (seconds - fixed) / per_row)))
        rows = max(r1, rows // 64 * 64) if rows < cfg.M else cfg.M
        t = timed(rows) if rows != r1 else t1
    flops = 2.0 * rows * cfg.N * cfg.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of D ({rows}x{cfg.N}x{cfg.K}, fp64 numpy oracle "
                      f"incl. operand decode), {t:.1f} s"}


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    n = COPY_CAL_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_CAL_BYTES,
                      "copy_calibration_bytes_written": COPY_CAL_BYTES, "launches": 3}))


def bench_i8(args):
    """The int8 form on 8192^3 NT (A [M,K], B [N,K], alpha 1, beta 0): integer
    ops per second against the int8 matrix-core peak; bit-exact oracle check
    on sampled rows."""
    import numpy as np
    import torch

    import dense_gemm_tile_amd as dgt
    import workloads
    M = N = K = 8192
    A, B = workloads.make_i8_inputs(M, N, K, 0, 1, 1007)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    Ad, Bd = A.to(dev), B.to(dev)
    D = torch.empty((M, N), dtype=torch.int32, device=dev)

    def step():
        dgt.gemm_i8(M, N, K, 0, 1, 1, 0, Ad, K, Bd, K, None, N, D, N, stream=stream)

    warm_up(step, args.warmup, args.warmup_seconds)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    clock = sustained_clock(step, stream, ms, args.clock_seconds) if args.clock_seconds > 0 else None
    if clock and "ms_per_step" in clock:
        clock["tops"] = round(2.0 * M * N * K / (clock["ms_per_step"] * 1e-3) / 1e12, 2)
    ok = None
    if not args.no_check:
        import oracle
        rows = np.array([0, 1, 127, 128, 4095, 4096, 8191])
        ref = oracle.gemm_reference_i8(M, N, K, 0, 1, 1, 0, A.numpy().reshape(-1), K,
                                       B.numpy().reshape(-1), K, rows=rows)
        ok = bool(np.array_equal(D[rows].cpu().numpy(), ref))
        if not ok:
            print("PARITY FAILURE on sampled rows", file=sys.stderr)
            sys.exit(1)
    tops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "TOP/s (2MNK/t) int8 -> int32 M=N=K=8192", "value": round(tops, 2),
        "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic (seed 1007; uniform int8)",
        "config": {"workload": "gemm8192_i8_nt", "M": M, "N": N, "K": K, "transA": 0,
                   "transB": 1, "alpha": 1, "beta": 0, "parallelism": "single GPU"},
        "oracle_bit_exact_sampled_rows": ok, "path": dgt.gemm_last_path(), "clock": clock,
        "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TOP/s", "frac": round(tops / PEAK_INT8_TOPS, 4), "traffic": None},
    }), flush=True)


def bench_fp8(args):
    """The 8-bit float form (OCP E4M3) on 8192^3 NT, alpha 1, beta 0: TFLOP/s
    against the fp8 matrix-core peak; oracle check on sampled rows."""
    import numpy as np
    import torch

    import dense_gemm_tile_amd as dgt
    import workloads
    M = N = K = 8192
    A, B = workloads.make_fp8_inputs(M, N, K, 0, 1, 4, 1008)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    Ad, Bd = A.to(dev), B.to(dev)
    D = torch.empty((M, N), dtype=torch.float32, device=dev)

    def step():
        dgt.gemm(M, N, K, "f8e4m3", 0, 1, 1.0, 0.0, Ad, K, Bd, K, None, N, D, N, stream=stream)

    warm_up(step, args.warmup, args.warmup_seconds)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    clock = sustained_clock(step, stream, ms, args.clock_seconds) if args.clock_seconds > 0 else None
    if clock and "ms_per_step" in clock:
        clock["tflops"] = round(2.0 * M * N * K / (clock["ms_per_step"] * 1e-3) / 1e12, 2)
    max_rel = None
    if not args.no_check:
        import oracle
        rows = np.array([0, 1, 127, 128, 4095, 4096, 8191])
        D_ref, bound = oracle.gemm_reference(M, N, K, 4, 0, 1, 1.0, 0.0, A.numpy().reshape(-1),
                                             K, B.numpy().reshape(-1), K, rows=rows)
        rep = oracle.check(D[rows].cpu().numpy().astype(np.float64), D_ref, bound)
        if not rep["ok"]:
            print(f"PARITY FAILURE on sampled rows: {rep}", file=sys.stderr)
            sys.exit(1)
        max_rel = rep["max_rel_err"]
    tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "TFLOP/s (2MNK/t) fp8 e4m3 M=N=K=8192", "value": round(tf, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f8e4m3",
        "data": "synthetic (seed 1008; uniform over finite E4M3 codes)",
        "config": {"workload": "gemm8192_f8e4m3_nt", "M": M, "N": N, "K": K, "transA": 0,
                   "transB": 1, "alpha": 1.0, "beta": 0.0, "parallelism": "single GPU"},
        "oracle_max_rel_err": max_rel, "path": dgt.gemm_last_path(), "clock": clock,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None},
    }), flush=True)


# Workloads whose operands fit in the 256 MB MALL: their hot time (operands left in
# L2/MALL by the previous call) and cold time (a 1 GiB buffer written between calls)
# differ, so both are reported.
PER_CALL_DEFAULT = ("atom16x8x16", "gemm512", "ragged4097x1000x1032_tn")


def per_call_timing(step, stream, n):
    """Median and minimum of n individually timed calls, hot and cold.

    Each call sits between its own pair of HIP events on the launch stream. Hot:
    calls back to back. Cold: a 1 GiB fill between calls (outside the event pair)
    evicts L2 and the MALL, so the operands come from HBM."""
    import torch

    def run(scrub):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (e0, e1) in enumerate(evs):
            if scrub is not None:
                scrub.fill_(float(i & 7))
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        return {"median_us": round(ts[n // 2], 3), "min_us": round(ts[0], 3)}

    hot = run(None)
    with torch.cuda.stream(stream):
        scrub = torch.empty(1 << 28, dtype=torch.float32, device=stream.device)
        cold = run(scrub)
    del scrub
    return {"samples": n, "hot": hot, "cold": cold}


def library_context(args, cfg, A, B, C, D, stream):
    """The same call on PyTorch's own GEMM (hipBLASLt on ROCm), f32 output from
    16-bit operands, for context only. The operands are views of the same
    stored buffers (a transposed view where the flag says so); the library
    picks its own kernel. beta != 0 goes through addmm with the same C."""
    import torch
    if cfg.dtype not in ("bf16", "f16"):
        print("library context covers 16-bit operands only", file=sys.stderr)
        sys.exit(2)
    opA = A[:, : cfg.M].t() if cfg.transA else A[:, : cfg.K]
    opB = B[:, : cfg.K].t() if cfg.transB else B[:, : cfg.N]
    Dv = D[:, : cfg.N]
    if cfg.beta != 0.0:
        Cv = C[:, : cfg.N]  # the same storage as Dv for the in-place workloads

        def step():
            torch.addmm(Cv, opA, opB, beta=cfg.beta, alpha=cfg.alpha,
                        out_dtype=torch.float32, out=Dv)
    elif cfg.alpha == 1.0:
        def step():
            torch.mm(opA, opB, out_dtype=torch.float32, out=Dv)
    else:
        def step():
            torch.mm(opA, opB, out_dtype=torch.float32, out=Dv)
            Dv.mul_(cfg.alpha)
    with torch.cuda.stream(stream):
        warm = warm_up(step, args.warmup, args.warmup_seconds)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = evs[0].elapsed_time(evs[-1]) / args.steps
        clock = sustained_clock(step, stream, ms, args.clock_seconds) if args.clock_seconds > 0 else None
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    tflops = float(cfg.flops) / (ms * 1e-3) / 1e12
    if clock and "ms_per_step" in clock:
        clock["tflops"] = round(float(cfg.flops) / (clock["ms_per_step"] * 1e-3) / 1e12, 2)
    print(json.dumps({
        "context": True,
        "library": f"torch {torch.__version__} mm/addmm, out_dtype=float32",
        "metric": "TFLOP/s (2MNK/t)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "ms_per_step": round(ms, 5),
        "warmup_run": warm,
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 5), "min": round(step_ms[0], 5),
                    "max": round(step_ms[-1], 5)},
        "pct_of_mfma_peak": round(100.0 * tflops / PEAK_TFLOPS[cfg.dtype], 2),
        "clock": clock,
        "config": {"workload": cfg.name, "M": cfg.M, "N": cfg.N, "K": cfg.K,
                   "transA": cfg.transA, "transB": cfg.transB, "alpha": cfg.alpha,
                   "beta": cfg.beta},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gemm8192_nt")
    ap.add_argument("--shape", default=None,
                    help="an ad-hoc workload instead: M,N,K,dtype,transA,transB[,alpha,beta"
                         "[,lda[,ldb]]] "
                         "(normal(0,1) inputs, seed 7; for tile-choice measurements)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="after the --warmup steps, keep running untimed steps until this many "
                         "seconds of warmup have passed: an idle GPU sits at a sleep clock and "
                         "ramps up over about a second of load (0: the --warmup steps only)")
    ap.add_argument("--clock-seconds", type=float, default=2.5,
                    help="length of the sustained run after the timed steps over which the "
                         "clock and power are read (0: skip)")
    ap.add_argument("--library-context", action="store_true",
                    help="time PyTorch's own GEMM (hipBLASLt on ROCm) on the same operands "
                         "instead of this library, for context; prints a line marked "
                         '"context": true')
    ap.add_argument("--per-call", type=int, default=None,
                    help="samples of per-call hot and cold timing (default: 200 for the "
                         "workloads that fit in the MALL, 0 otherwise)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(an M-split of the output tiles needs no collective, only a "
              "broadcast of op(B)). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload == "gemm8192_i8_nt":
        bench_i8(args)
        return
    if args.workload == "gemm8192_f8e4m3_nt":
        bench_fp8(args)
        return

    import numpy as np
    import torch

    import dense_gemm_tile_amd as dgt
    import workloads

    if args.shape:
        f = args.shape.split(",")
        alpha, beta = (float(f[6]), float(f[7])) if len(f) >= 8 else (1.0, 0.0)
        lda = int(f[8]) if len(f) >= 9 else None
        ldb = int(f[9]) if len(f) >= 10 else None
        name = f"shape{f[0]}x{f[1]}x{f[2]}_{f[3]}_{f[4]}{f[5]}"
        if lda is not None or ldb is not None:
            name += f"_lda{lda}_ldb{ldb}"
        cfg = workloads.Config(name, int(f[0]), int(f[1]), int(f[2]), f[3], int(f[4]), int(f[5]),
                               alpha, beta, "normal", 7, lda=lda, ldb=ldb)
    else:
        cfg = {**workloads.CONFIGS, **workloads.EXTRA_CONFIGS}[args.workload]
    lda, ldb, ldc, ldd = cfg.lds()
    inp = workloads.make_inputs(cfg)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    A, B = inp.A.to(dev), inp.B.to(dev)
    C0 = inp.C.to(dev) if inp.C is not None else None
    if cfg.inplace:
        D = C0.clone()
        C = D
    else:
        D = torch.empty((cfg.M, ldd), dtype=torch.float32, device=dev)
        C = C0

    def step():
        dgt.gemm(cfg.M, cfg.N, cfg.K, cfg.dtype, cfg.transA, cfg.transB, cfg.alpha, cfg.beta,
                 A, lda, B, ldb, C, ldc, D, ldd, stream=stream)

    if args.library_context:
        library_context(args, cfg, A, B, C, D, stream)
        return

    warm = warm_up(step, args.warmup, args.warmup_seconds)
    path = dgt.gemm_last_path()

    # The timed steps, back to back, with a HIP event on the launch stream
    # before the first and after every step (events do not serialise the
    # stream): whole-region time and each step's own time.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = gpu_ms / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))

    n_per_call = args.per_call
    if n_per_call is None:
        n_per_call = 200 if cfg.name in PER_CALL_DEFAULT else 0
    per_call = per_call_timing(step, stream, n_per_call) if n_per_call > 0 else None

    # Clock and power: the sensors refresh about once a second, far longer
    # than the timed steps, so they are read over a sustained run of the same
    # step after the timed region (its own time per step reported beside).
    clock = sustained_clock(step, stream, ms_per_step, args.clock_seconds) \
        if args.clock_seconds > 0 else None
    if clock and "ms_per_step" in clock:
        clock["tflops"] = round(float(cfg.flops) / (clock["ms_per_step"] * 1e-3) / 1e12, 2)

    # Parity of what was timed: a fresh call, then sampled rows against the oracle.
    max_rel = None
    if not args.no_check:
        import oracle
        if cfg.inplace:
            D.copy_(C0)
        step()
        torch.cuda.synchronize()
        rng = np.random.default_rng(0)
        rows = np.unique(np.concatenate([[0, cfg.M - 1], rng.integers(0, cfg.M, 14)]))
        Cn = inp.C.numpy().reshape(-1) if inp.C is not None else None
        if cfg.dtype.startswith("f32_"):
            D_ref, bound = oracle.gemm_reference_f32(
                cfg.M, cfg.N, cfg.K, 0 if cfg.dtype == "f32_f16" else 1, cfg.transA, cfg.transB,
                cfg.alpha, cfg.beta, inp.A.numpy().reshape(-1), lda, inp.B.numpy().reshape(-1),
                ldb, Cn, ldc, rows=rows)
        else:
            D_ref, bound = oracle.gemm_reference(
                cfg.M, cfg.N, cfg.K, workloads.DTYPE_CODE[cfg.dtype], cfg.transA, cfg.transB,
                cfg.alpha, cfg.beta, workloads.bits_u16(inp.A).reshape(-1), lda,
                workloads.bits_u16(inp.B).reshape(-1), ldb, Cn, ldc, rows=rows)
        got = D[rows, : cfg.N].cpu().numpy().astype(np.float64)
        rep = oracle.check(got, D_ref, bound)
        if not rep["ok"]:
            print(f"PARITY FAILURE on sampled rows: {rep}", file=sys.stderr)
            sys.exit(1)
        max_rel = rep["max_rel_err"]

    flops = float(cfg.flops)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    traffic = stored_traffic(cfg.name)
    # Algorithmic bytes: A and B once (16-bit), C once when beta != 0, D once.
    esz = 4.0 if cfg.dtype.startswith("f32_") else 2.0
    alg_bytes = esz * (cfg.M * cfg.K + cfg.K * cfg.N) + 4.0 * cfg.M * cfg.N * (2 if cfg.beta != 0 else 1)
    if flops / alg_bytes >= (peak * 1e12) / (PEAK_HBM_GBS * 1e9):
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4), "traffic": traffic}
    else:
        gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    out = {
        "metric": "TFLOP/s (2MNK/t) bf16 M=N=K=8192 + % of MFMA peak; oracle max rel err",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic (seed {cfg.seed}; A, B {DIST_TEXT[cfg.dist]} in {cfg.dtype})",
        "config": {"workload": cfg.name, "M": cfg.M, "N": cfg.N, "K": cfg.K,
                   "transA": cfg.transA, "transB": cfg.transB, "alpha": cfg.alpha,
                   "beta": cfg.beta, "parallelism": "single GPU"},
        "pct_of_mfma_peak": round(100.0 * tflops / peak, 2),
        "oracle_max_rel_err": max_rel,
        "path": path,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 5), "min": round(step_ms[0], 5),
                    "max": round(step_ms[-1], 5)},
        "clock": clock,
        "roofline": roofline,
    }
    if per_call is not None:
        for k in ("hot", "cold"):
            per_call[k]["gbs_at_median"] = round(alg_bytes / (per_call[k]["median_us"] * 1e-6) / 1e9, 1)
        out["per_call"] = per_call
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
