#!/usr/bin/env python3
"""Benchmark of the gfx950 FP32 SGEMM: TFLOP/s = 2MNK / t at M = N = K = 4096.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sq4096]
                    [--variant V] [--cpu-seconds S] [--no-cpu-baseline]
                    [--copy-calibration-mib N]
    python bench.py --sweep VARIANTS --sweep-sizes SIZES [--rounds R]

A step is one SGEMM call (the whole path: one kernel launch over the
device-resident A, B and C).  The GPU idles at a low shader clock and takes
tens of milliseconds of load to reach its steady clock; the clock cannot be
locked on this machine (the pages lock theirs at 2002 MHz for the same
reason, "gpu_matmul", Results).  So before the W warm-up steps the bench
runs untimed steps for --settle-seconds of wall time (the count and time
are in the JSON line).  Then W untimed warm-up steps, then exactly K timed
steps, back to back, between two device synchronisations; a pair of HIP
events on the stream the kernel is launched on brackets them, and the
per-launch kernel time of the roofline is their elapsed time over K (an
event around every call would put its own marker in the queue).  A second,
untimed pass of K calls with events around each reports the spread of
single calls (kernel_ms).  The
shader clock the power firmware reports (per XCD; its table refreshes about
once a second) is read at idle, just before and just after the timed
steps.  Prints one JSON line.

--sweep times the given variant ids (comma separated; -1 = the automatic
choice, "mm" = torch.mm in FP32 for context, "op:TN" and the like = sgemm_op
with the operands stored transposed as named, "lowp:bf16" / "lowp:f16" =
sgemm_lowp on the same values in that 16-bit type ("lowp:bf16:V" forces
sgemm_lowp_ex variant V, "lowp:bf16:op:TN" and the like run sgemm_lowp_op
with the operands stored transposed as named), "mm:bf16" / "mm:f16" =
torch.mm in that type, 16-bit output, for context; "batch:B:TN" and the
like = sgemm_strided_batched over B copies of the problem, stored as
named, TFLOP/s over all B, "batch:B:NN:bf16" the same through
sgemm_lowp on 16-bit copies) on problems of the given sizes
("N" for N^3 or "MxNxK"; packed row-major, so lda = K and ldb = ldc = N), interleaved round by round in one process so that clock drift hits
every variant alike (after half a second of untimed calls per size, for
the clock): each round times a batch of back-to-back calls of every
variant under one HIP event pair, and one JSON line per (size, variant)
gives the median over the rounds of the time per call.  It is the
evidence behind the automatic tile choice.

The CPU baseline times the fp64 oracle on a bounded slab of rows of the
same problem (host cores, OpenMP over rows) and checks the GPU result on
that slab.  --copy-calibration-mib adds plain device copies of known size
after the timed region, so that one profiler run reads the HBM counters of
the GEMM and of a copy whose byte count is known.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SGEMM TFLOP/s (2MNK/t) at M=N=K=4096 FP32; % of MI355X FP32 matrix peak"
# FP32 SGEMM rates the source pages report on NVIDIA cards, all at
# M = N = K = 4096: their vendor library and their pipelined kernel on an
# RTX 3060 with clocks locked at 2002 MHz ("gpu_matmul", Results), and the
# 32x32 shared-memory tile on a T4 ("V1. Shared Memory Tiling", section 6,
# benchmark table).  Quoted on the bench line for context; other hardware,
# not a target.
PAGES_CONTEXT = {
    "note": "FP32 SGEMM at 4096^3 as the source pages report it on NVIDIA cards; context, not a target",
    "rtx3060_vendor_library_tflops": 8.69,
    "rtx3060_pipelined_kernel_tflops": 9.66,
    "rtx3060_locked_clock_mhz": 2002,
    "rtx3060_source": "gpu_matmul, Results",
    "t4_shared_memory_tile32_tflops": 0.695,
    "t4_source": "V1. Shared Memory Tiling, section 6",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sgemm_sq4096.txt")


# The translation unit the timed 4096^3 kernel (the lean 128x128x32 kernel)
# is compiled from, with the headers it includes.
KERNEL_SOURCES = ("sgemm_kernels.hpp", "sgemm_lean.hpp", "sgemm_lean.hip")


def kernel_source_hash():
    """Hash of the timed kernel's sources: a counter record taken on other
    kernel code no longer describes the kernel that runs (the record also
    names the variant, so a change of the automatic choice voids it too)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp32_sgemm_tuning_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(variant_name):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is absent or was taken on other kernel sources or variant."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash() or vals.get("variant") != variant_name:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(A, B, Cin, C_gpu, w, target_seconds):
    """Time the oracle on leading row slabs of the problem until about
    target_seconds of CPU work; check the GPU rows of that slab."""
    import numpy as np

    import oracle
    threads = oracle.max_threads()
    rows, spent, flop = 0, 0.0, 0
    max_ratio, nonfinite = 0.0, False
    step = 8
    while spent < target_seconds and rows < w.M:
        r1 = min(rows + step, w.M)
        t0 = time.perf_counter()
        ref = oracle.sgemm_ref(A[rows:r1], B, None if Cin is None else Cin[rows:r1], alpha=w.alpha, beta=w.beta)
        dt = time.perf_counter() - t0
        spent += dt
        flop += 2 * (r1 - rows) * w.N * w.K
        err = np.abs(C_gpu[rows:r1].astype(np.float64) - ref)
        tol = 1e-3 + 1e-4 * np.abs(ref)
        ratio = err / tol
        if np.all(np.isfinite(ratio)):
            max_ratio = max(max_ratio, float(ratio.max()))
        else:                        # a NaN or Inf anywhere in the slab is a failure
            nonfinite = True
        rows = r1
        if dt < target_seconds / 8:
            step *= 2
    # the same oracle on one thread, over a small leading slab (about a tenth
    # of the time budget): its rate, extrapolated to the whole problem
    oracle.set_threads(1)
    one_spent, one_rows = 0.0, 0
    while one_spent < target_seconds / 10 and one_rows < w.M:
        r_end = min(one_rows + 8, w.M)
        t0 = time.perf_counter()
        oracle.sgemm_ref(A[one_rows:r_end], B, None if Cin is None else Cin[one_rows:r_end], alpha=w.alpha,
                         beta=w.beta)
        one_spent += time.perf_counter() - t0
        one_rows = r_end
    oracle.set_threads(threads)
    one_rate = 2.0 * one_rows * w.N * w.K / one_spent / 1e9 if one_spent > 0 else None
    return {
        "value": flop / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of C ({rows}x{w.N}x{w.K}, {flop / 1e9:.1f} GFLOP) of the same "
                  f"problem, fp64 oracle, {spent:.1f} s",
        "seconds": spent,
        "single_thread_gflops": one_rate,
        "single_thread_sample": f"rows 0..{one_rows - 1} of {w.M} ({100.0 * one_rows / w.M:.1f}% of C), "
                                f"{one_spent:.2f} s on one thread; the rate is that slab's, not a full run",
        "single_thread_full_problem_s_extrapolated": (2.0 * w.M * w.N * w.K / (one_rate * 1e9)) if one_rate else None,
        "cpu_model": cpu_model(),
        "cpu_simd": cpu_simd(),
        "nproc": os.cpu_count(),
        "parity_on_sample_max_err_over_tol": None if nonfinite else max_ratio,
        "parity_on_sample_ok": bool(not nonfinite and max_ratio <= 1.0),
    }


class GpuClock:
    """The shader clock (MHz, mean over the XCDs) and socket power (W) that
    the power firmware reports, through amdsmi; None where unavailable.
    The firmware refreshes this table about once a second, so a reading
    describes the last second or so, not an instant."""

    def __init__(self, pci_bus_id=None):
        self.handle = None
        self.max_mhz = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if pci_bus_id is not None and len(handles) > 1:
                handles = [h for h in handles
                           if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == pci_bus_id] or handles
            self.amdsmi = amdsmi
            self.handle = handles[0]
            self.max_mhz = amdsmi.amdsmi_get_clock_info(self.handle, amdsmi.AmdSmiClkType.GFX).get("max_clk")
        except Exception:        # no amdsmi, or no permission: the line says null
            self.handle = None

    def read(self):
        if self.handle is None:
            return None
        try:
            m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
            power = m.get("current_socket_power")
            return {"sclk_mhz": round(sum(clks) / len(clks), 1) if clks else m.get("current_gfxclk"),
                    "sclk_mhz_per_xcd": clks or None,
                    "socket_power_w": power if isinstance(power, (int, float)) else None,
                    "hotspot_c": m.get("temperature_hotspot")}
        except Exception:
            return None


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where absent)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_simd():
    """The host CPU's vector extensions that bear on an fp64 loop (from the
    flags line of /proc/cpuinfo; None where absent)."""
    wanted = ("sse4_2", "avx", "avx2", "fma", "avx512f", "avx512dq", "avx512vl")
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("flags"):
                have = set(line.split(":", 1)[1].split())
                return [f for f in wanted if f in have]
    except OSError:
        pass
    return None


def parse_shape(text):
    """'4096' -> (4096, 4096, 4096); '3001x4999x2047' -> (3001, 4999, 2047)."""
    parts = [int(x) for x in text.lower().split("x")]
    if len(parts) == 1:
        parts *= 3
    if len(parts) != 3 or min(parts) < 1:
        raise SystemExit(f"bad --sweep-sizes entry {text!r}")
    return tuple(parts)


def sweep(variants, sizes, rounds, settle_s=0.5):
    import statistics

    import torch

    from fp32_sgemm_tuning_amd import SgemmError, capi, sgemm, sgemm_lowp, sgemm_op
    from fp32_sgemm_tuning_amd.inputs import make_problem
    torch.backends.cuda.matmul.allow_tf32 = False
    capi.load()
    for M, N, K in sizes:
        A, B, _ = make_problem(M, N, K, 7)
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        dC = torch.empty((M, N), device="cuda")
        flop = 2 * M * N * K
        reps = max(5, min(200, int(2e11 / max(flop, 1))))

        stored, half, batched = {}, {}, {}
        for v in variants:
            if isinstance(v, str) and v.startswith("op:"):
                ta, tb = v[3] == "T", v[4] == "T"
                stored[v] = (dA.t().contiguous() if ta else dA, dB.t().contiguous() if tb else dB, ta, tb)
            if isinstance(v, str) and v.startswith("batch:"):
                parts = v.split(":")
                nb, ops = parts[1:3]
                ta, tb = ops[0] == "T", ops[1] == "T"
                a1 = dA.t().contiguous() if ta else dA
                b1 = dB.t().contiguous() if tb else dB
                if len(parts) > 3:           # 16-bit inputs
                    t = {"bf16": torch.bfloat16, "f16": torch.float16}[parts[3]]
                    a1, b1 = a1.to(t), b1.to(t)
                batched[v] = (a1.unsqueeze(0).repeat(int(nb), 1, 1), b1.unsqueeze(0).repeat(int(nb), 1, 1),
                              torch.empty((int(nb), M, N), device="cuda"), ta, tb)
            if isinstance(v, str) and v.split(":")[0] in ("lowp", "mm") and ":" in v:
                parts = v.split(":")
                t = {"bf16": torch.bfloat16, "f16": torch.float16}[parts[1]]
                a16, b16 = dA.to(t), dB.to(t)
                if len(parts) > 3 and parts[2] == "op":
                    a16 = a16.t().contiguous() if parts[3][0] == "T" else a16
                    b16 = b16.t().contiguous() if parts[3][1] == "T" else b16
                half[v] = (a16, b16, torch.empty((M, N), dtype=t, device="cuda"))

        def label(v):
            if v == "mm":
                return "torch.mm fp32"
            if v in stored:
                return "sgemm_op " + v[3:5]
            if v in batched:
                parts = v.split(":")
                if len(parts) > 3:
                    return f"sgemm_lowp_strided_batched {parts[3]} {parts[1]} x {parts[2]}"
                return f"sgemm_strided_batched {parts[1]} x {parts[2]}"
            if v in half:
                if v.startswith("lowp"):
                    parts = v.split(":")
                    if len(parts) > 3 and parts[2] == "op":
                        return f"sgemm_lowp_op {parts[1]} {parts[3]}"
                    var = int(parts[2]) if len(parts) > 2 else capi.sgemm_lowp_select_variant(
                        M, N, K, half[v][0].data_ptr(), K, half[v][1].data_ptr(), N)
                    return f"sgemm_lowp {parts[1]} {capi.sgemm_lowp_variant_name(var)}"
                return "torch.mm " + v.split(":")[1]
            if v == -1:
                return "auto:" + capi.sgemm_variant_name(capi.sgemm_select_variant(
                    M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dC.data_ptr(), N))
            return capi.sgemm_variant_name(v)

        def run(v):
            if v == "mm":
                torch.mm(dA, dB, out=dC)
            elif v in half:
                a16, b16, c16 = half[v]
                if v.startswith("lowp"):
                    parts = v.split(":")
                    if len(parts) > 3 and parts[2] == "op":
                        sgemm_lowp(a16, b16, dC, trans_a=parts[3][0] == "T", trans_b=parts[3][1] == "T")
                    else:
                        sgemm_lowp(a16, b16, dC, variant=int(parts[2]) if len(parts) > 2 else None)
                else:
                    torch.mm(a16, b16, out=c16)
            elif v in stored:
                sa, sb, ta, tb = stored[v]
                sgemm_op(sa, sb, dC, trans_a=ta, trans_b=tb)
            elif v in batched:
                sa, sb, sc, ta, tb = batched[v]
                if sa.dtype == torch.float32:
                    sgemm_op(sa, sb, sc, trans_a=ta, trans_b=tb)
                else:
                    sgemm_lowp(sa, sb, sc, trans_a=ta, trans_b=tb)
            else:
                sgemm(dA, dB, dC, variant=None if v == -1 else v)
        usable = []
        for v in variants:
            try:
                for _ in range(3):
                    run(v)
                usable.append(v)
            except SgemmError as e:      # e.g. a 128-bit variant on unaligned rows
                print(json.dumps({"sweep": label(v), "variant": v, "shape": f"{M}x{N}x{K}",
                                  "skipped": str(e)}), flush=True)
        torch.cuda.synchronize()
        # clock settle: the usable variants in turn for settle_s of wall time
        t_settle = time.perf_counter()
        while usable and time.perf_counter() - t_settle < settle_s:
            for v in usable:
                run(v)
            torch.cuda.synchronize()
        # each round times a batch of `reps` back-to-back calls of every
        # variant under one event pair (no marker between the calls)
        times = {v: [] for v in usable}
        for _ in range(rounds):
            for v in usable:
                st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                st.record()
                for _ in range(reps):
                    run(v)
                en.record()
                torch.cuda.synchronize()
                times[v].append(st.elapsed_time(en) / reps)
        for v in usable:
            ms = statistics.median(times[v])
            f = flop * (int(v.split(":")[1]) if v in batched else 1)
            print(json.dumps({"sweep": label(v), "variant": v, "shape": f"{M}x{N}x{K}", "median_ms": round(ms, 5),
                              "tflops": round(f / ms / 1e9, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sq4096")
    ap.add_argument("--variant", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--settle-seconds", type=float, default=1.5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--sweep", default=None)
    ap.add_argument("--sweep-sizes", default="4096")
    ap.add_argument("--rounds", type=int, default=4)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU per process; --gpus {args.gpus} is not supported "
              "(row-slab sharding across GPUs is described in the design notes but not built)",
              file=sys.stderr)
        sys.exit(2)

    if args.sweep is not None:
        def variant_arg(v):
            if v == "mm" or ":" in v:
                return v
            try:
                return int(v)
            except ValueError:        # a variant name
                from fp32_sgemm_tuning_amd import capi
                names = {capi.sgemm_variant_name(i): i for i in capi.all_variants()}
                if v not in names:
                    raise SystemExit(f"unknown variant {v!r}")
                return names[v]
        variants = [variant_arg(v) for v in args.sweep.split(",")]
        sweep(variants, [parse_shape(x) for x in args.sweep_sizes.split(",")], args.rounds,
              settle_s=min(args.settle_seconds, 0.5))
        return

    import numpy as np
    import torch

    from fp32_sgemm_tuning_amd import capi, model, sgemm
    from fp32_sgemm_tuning_amd.inputs import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    capi.load()
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    A, B, Cin = workload_inputs(w)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC0 = torch.from_numpy(Cin).to(dev) if Cin is not None else None
    dC = dC0.clone() if dC0 is not None else torch.empty((w.M, w.N), device=dev)
    variant = args.variant
    chosen = variant if variant is not None else capi.sgemm_select_variant(
        w.M, w.N, w.K, dA.data_ptr(), w.K, dB.data_ptr(), w.N, w.beta, dC.data_ptr(), w.N)
    variant_name = capi.sgemm_variant_name(chosen)
    stream = torch.cuda.current_stream(dev)

    props = torch.cuda.get_device_properties(dev)
    clock = GpuClock(getattr(props, "pci_bus_id", None))
    clock_idle = clock.read()

    # Correctness run on pristine C (beta != 0 reads it), kept for the CPU check.
    sgemm(dA, dB, dC, alpha=w.alpha, beta=w.beta, variant=variant)
    torch.cuda.synchronize()
    C_first = dC.cpu().numpy()

    # Clock settle: untimed steps until the shader clock has left idle and
    # held under load for a while (--settle-seconds of wall time).
    settle_steps, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(8):
            sgemm(dA, dB, dC, alpha=w.alpha, beta=w.beta, variant=variant)
        settle_steps += 8
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle

    for _ in range(args.warmup):
        sgemm(dA, dB, dC, alpha=w.alpha, beta=w.beta, variant=variant)
    # The timed steps run back to back, as a caller's stream of products
    # would; one pair of HIP events on the launching stream brackets them
    # (an event around every call would add its own marker to the queue:
    # about 0.8% of a 4096^3 step, half of a 512^3 one).
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    clock_before = clock.read()
    t0 = time.perf_counter()
    region[0].record(stream)
    for _ in range(args.steps):
        sgemm(dA, dB, dC, alpha=w.alpha, beta=w.beta, variant=variant)
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock_after = clock.read()
    region_ms = region[0].elapsed_time(region[1])

    # Spread of single calls: a second pass of the same steps with an event
    # pair around each call (not the timed region).
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        sgemm(dA, dB, dC, alpha=w.alpha, beta=w.beta, variant=variant)
        ends[i].record(stream)
    torch.cuda.synchronize()
    kernel_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    flop = w.flops
    ms_per_step = wall / args.steps * 1e3
    value = flop / (wall / args.steps) / 1e12
    avg_kernel_s = region_ms / args.steps / 1e3        # per launch, back to back in the timed region
    achieved = flop / avg_kernel_s / 1e12
    peak = model.MI355X_FP32_MATRIX_TFLOPS
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_fp32_matrix_peak": round(100.0 * value / peak, 2),
        "config": {
            "workload": w.describe(),
            "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta, "seed": w.seed,
            "layout": "row-major, lda=K, ldb=ldc=N",
            "variant": variant_name,
            "parallelism": "single GPU",
        },
        "timed_region_ms_per_launch": round(region_ms / args.steps, 5),
        "kernel_ms": {"mean": round(float(kernel_ms.mean()), 5), "median": round(float(np.median(kernel_ms)), 5),
                      "min": round(float(kernel_ms.min()), 5), "max": round(float(kernel_ms.max()), 5),
                      "first_quarter_mean": round(float(kernel_ms[:max(1, len(kernel_ms) // 4)].mean()), 5),
                      "last_quarter_mean": round(float(kernel_ms[-max(1, len(kernel_ms) // 4):].mean()), 5),
                      "source": "HIP events around each call on the launching stream, in a second pass of "
                                "the same steps after the timed region"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(variant_name),
            "traffic_source": "rocprofv3 FETCH_SIZE and WRITE_SIZE per launch, scaled by a device copy of "
                              "known size, from " + os.path.relpath(TRAFFIC_FILE, ROOT) +
                              " (null unless taken on these kernel sources and this variant)",
        },
        "clock_settle": {"steps": settle_steps, "seconds": round(settle_s, 3),
                         "why": "the shader clock idles near 100 MHz and ramps up over tens of ms of load; it "
                                "cannot be locked here"},
        "gpu_clock": {"idle": clock_idle, "before_timed": clock_before, "after_timed": clock_after,
                      "max_sclk_mhz": clock.max_mhz,
                      "source": "amdsmi gpu_metrics (power firmware, refreshed about once a second)"},
        "device": {
            "name": torch.cuda.get_device_name(dev),
            "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "memory_bytes": props.total_memory,
            # peak check: CUs x 256 FP32 MFMA FLOP per clock per CU x the
            # highest shader clock the firmware allows
            "peak_from_cus_and_max_sclk_tflops": (round(props.multi_processor_count * 256 * clock.max_mhz * 1e6
                                                        / 1e12, 2) if clock.max_mhz else None),
        },
        "kernel_source_sha256": kernel_source_hash(),
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(A, B, Cin, C_first, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
