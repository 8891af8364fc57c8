"""Kernel-time evidence for the split-K factor of small grids, and the fit
of the cost model that chooses it.

Three steps:

    # 1. one process per forced factor S (0 = the automatic choice), under a
    #    kernel trace; each shape runs a settle phase and CALLS timed calls,
    #    framed by two small fills so the trace can be cut per shape
    SGEMM_SPLITK=S rocprofv3 --kernel-trace --output-format csv -d DIR -o run -- \\
        python3 -m fp32_sgemm_tuning_amd.splitk_fit run --variant lean_64x64x64_w4x1_splitk \\
        --shapes 512,768x768x2048,... [--calls 150] > RUN.jsonl
    # 2. cut the trace: median kernel duration per shape
    python3 -m fp32_sgemm_tuning_amd.splitk_fit cut DIR/.../run_kernel_trace.csv RUN.jsonl > CUT.jsonl
    # 3. fit the model's constants to every CUT.jsonl and score the choice
    python3 -m fp32_sgemm_tuning_amd.splitk_fit fit CUT.jsonl [CUT.jsonl ...]

Why kernel time: below about 25 us a call is bound by the host (Python,
the C call and the launch take about 12 us), so timing calls with events
hides what a split saves inside the kernel; a caller that repeats such
products captures them in a HIP graph, where the kernel time is what is
paid.  The factor is a tuning parameter chosen from measurements, as the
block-tile parameters are in the "gpu_matmul" blog (1D Blocktiling, its
autotuner); splitting K itself is not on the pages: it spreads a grid of
fewer tiles than the 256 compute units hold over the whole chip.

`model_cost` and `choose` restate the library's split_cost() and
choose_splits() (csrc/sgemm.hip) so the fit scores exactly the rule the
library runs; a CPU test checks the two agree on a grid of shapes.
"""
import argparse
import csv
import json
import math
import statistics
import sys
import time

CUS = 256
SPLIT_MAX = 16
MAX_SPLIT_TILES = 4096        # 64 MiB of partials over 64x64 tiles of FP32
FLOOR = 0.15                  # operand-traffic floor, steps per tile-step of (bm + bn) / (bm * bn)
THRESHOLD = 0.95              # a split is taken when it costs at most this share of no split
MIN_KT_PER_SPLIT = 2
# The library's constants (csrc/sgemm.hip: kBlockFixed, kSplitFixed,
# kSplitPerPartial), in K-tile steps.
LIB_PARAMS = {"block_fixed": 2.8, "split_fixed": 1.7, "per_partial": 0.45}


def _cd(a, b):
    return -(-a // b)


def _shape(s):
    p = [int(x) for x in s.split("x")]
    return (p[0],) * 3 if len(p) == 1 else tuple(p)


def model_cost(M, N, K, S, bm=64, bn=64, bk=64, block_fixed=2.8, split_fixed=1.7, per_partial=0.45, batch=1):
    """Modelled time of an M x N x K grid (`batch` of them in one strided
    batch) split S ways, in K-tile steps."""
    tiles = _cd(M, bm) * _cd(N, bn) * batch
    kt = _cd(K, bk)
    r = _cd(tiles * S, CUS)
    busiest = r * _cd(kt, S) + _cd(r, 2) * block_fixed
    floor = FLOOR * tiles * kt * (bm + bn) / (bm * bn)
    partials = split_fixed + per_partial * S if S > 1 else 0.0
    return max(busiest, floor) + partials


def choose(M, N, K, bm=64, bn=64, bk=64, batch=1, **params):
    """The factor the library's automatic choice takes (1 = no split); a
    strided batch counts its problems' tiles together."""
    params = {**LIB_PARAMS, **params, "batch": batch}
    tiles = _cd(M, bm) * _cd(N, bn) * batch
    kt = _cd(K, bk)
    fit = MAX_SPLIT_TILES * 64 * 64 // (bm * bn)
    if tiles > MAX_SPLIT_TILES or kt < 2 or tiles >= 2 * CUS:
        return 1
    base = model_cost(M, N, K, 1, bm, bn, bk, **params)
    best, best_cost = 1, base
    for s in range(2, SPLIT_MAX + 1):
        if s > kt // MIN_KT_PER_SPLIT or s * tiles > fit:
            break
        c = model_cost(M, N, K, s, bm, bn, bk, **params)
        if c < best_cost:
            best, best_cost = s, c
    return best if best_cost <= THRESHOLD * base else 1


def run(args):
    """Time one variant on each shape (the factor comes from SGEMM_SPLITK in
    the environment); prints one JSON line per shape."""
    import os
    import torch
    from fp32_sgemm_tuning_amd import capi
    capi.load()
    auto = os.environ.get("SGEMM_SPLITK", "0").strip() in ("", "0")
    ids = [v for v in capi.all_variants() if capi.sgemm_variant_name(v) == args.variant]
    if not ids:
        sys.exit(f"unknown variant {args.variant}")
    vid = ids[0]
    h = torch.cuda.current_stream().cuda_stream
    mark = torch.empty(64, device="cuda")
    for i, (M, N, K) in enumerate(_shape(s) for s in args.shapes.split(",")):
        A = torch.randn(M, K, device="cuda")
        B = torch.randn(K, N, device="cuda")
        C = torch.empty(M, N, device="cuda")
        call = (M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C.data_ptr(), N, h, vid)
        st = capi.sgemm_ex(*call)
        if st != capi.SGEMM_STATUS_OK:
            sys.exit(f"{M}x{N}x{K}: {capi.sgemm_strerror(st)}")
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle_seconds:
            for _ in range(50):
                capi.sgemm_ex(*call)
            torch.cuda.synchronize()
        mark[:i + 1].fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(args.calls):
            capi.sgemm_ex(*call)
        torch.cuda.synchronize()
        mark[:i + 1].fill_(2.0)
        torch.cuda.synchronize()
        print(json.dumps({"shape": f"{M}x{N}x{K}", "variant": args.variant, "auto": auto,
                          "split": capi.sgemm_split_factor(vid, M, N, K), "calls": args.calls}), flush=True)


def cut(args):
    """Median kernel duration of the timed calls of every shape of a run."""
    runs = [json.loads(l) for l in open(args.run) if l.startswith("{")]
    rows = sorted(csv.DictReader(open(args.trace)), key=lambda r: int(r["Start_Timestamp"]))
    segs, cur, fills = [], None, 0
    for r in rows:
        name = r["Kernel_Name"]
        if "FillFunctor" in name:          # torch's fill: the marks around each shape's timed calls
            fills += 1
            if fills % 2 == 1:
                cur = []
            else:
                segs.append(cur)
                cur = None
        elif cur is not None and "sgemm" in name:
            cur.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if len(segs) != len(runs):
        sys.exit(f"{len(segs)} marked segments for {len(runs)} shapes")
    for rec, d in zip(runs, segs):
        rec.update({"launches": len(d), "median_us": round(statistics.median(d) / 1e3, 3),
                    "min_us": round(min(d) / 1e3, 3)})
        print(json.dumps(rec))


def load_cuts(paths):
    """{shape: {split: median_us}} from cut outputs (the first measurement
    of a factor is kept when forcing different S clamps to the same one),
    and {shape: (split, median_us)} of runs of the automatic choice."""
    forced, auto = {}, {}
    for p in paths:
        for l in open(p):
            if not l.startswith("{"):
                continue
            r = json.loads(l)
            if r.get("auto"):
                auto[r["shape"]] = (r["split"], r["median_us"])
            else:
                forced.setdefault(r["shape"], {}).setdefault(r["split"], r["median_us"])
    return forced, auto


def decision_loss(forced, params):
    """Per shape, the measured time at the factor the model chooses over the
    fastest measured factor (shapes whose chosen factor was not measured
    are left out)."""
    out = {}
    for shape, d in forced.items():
        s = choose(*_shape(shape), **params)
        if s in d:
            out[shape] = d[s] / min(d.values())
    return out


def fit(args):
    """Least-squares fit of the model's constants (log residuals) to every
    forced-factor measurement; scores the library's constants and the fitted
    ones by decision_loss, and the automatic choice's own runs against the
    fastest forced factor of the same shape.  --out writes all of it, with
    the measurements, as one JSON file."""
    from scipy.optimize import least_squares
    forced, auto = load_cuts(args.cuts)
    pts = [(_shape(k), s, t) for k, d in forced.items() for s, t in d.items()]
    names = ("step_us", "block_fixed", "split_fixed", "per_partial")

    def resid(p):
        prm = dict(zip(names[1:], p[1:]))
        return [math.log(p[0] * model_cost(*shp, s, **prm) / t) for shp, s, t in pts]

    r = least_squares(resid, [0.85, 3.0, 3.0, 0.3], bounds=([0.1, 0, 0, 0], [5, 20, 20, 10]))
    res = resid(r.x)
    fitted = dict(zip(names, (round(float(x), 3) for x in r.x)))
    summary = {"fitted": fitted, "points": len(pts), "shapes": len(forced),
               "log_residual_rms": round(math.sqrt(sum(x * x for x in res) / len(res)), 4)}
    print(json.dumps(summary))
    scores = {}
    for label, prm in (("library", LIB_PARAMS), ("fitted", {k: fitted[k] for k in names[1:]})):
        loss = decision_loss(forced, prm)
        scores[label] = {"params": prm, "scored_shapes": len(loss),
                         "mean_over_best": round(statistics.mean(loss.values()), 4),
                         "worst_over_best": round(max(loss.values()), 4),
                         "worst_shape": max(loss, key=loss.get)}
        print(json.dumps({"constants": label, **scores[label]}))
    auto_runs = {}
    for shape, (s, t) in auto.items():
        d = forced.get(shape, {})
        if d:
            best = min(d, key=d.get)
            auto_runs[shape] = {"split": s, "median_us": t, "best_forced_split": best, "best_forced_us": d[best],
                                "unsplit_us": d.get(1), "over_best": round(t / d[best], 4)}
    if auto_runs:
        over = [a["over_best"] for a in auto_runs.values()]
        print(json.dumps({"automatic_choice_runs": len(over), "mean_over_best": round(statistics.mean(over), 4),
                          "worst_over_best": round(max(over), 4)}))
    if args.out:
        with open(args.out, "w") as f:
            json.dump({"about": "Split-K factor of small grids on MI355X (gfx950): median kernel-trace duration "
                                "(us) of one variant per shape and forced factor, the automatic choice's own "
                                "runs, the least-squares fit of the cost model's constants, and how the "
                                "library's constants choose on these shapes.",
                       "command": args.command, "fit": summary, "scores": scores, "automatic_choice": auto_runs,
                       "times_us": {k: {str(s): t for s, t in sorted(d.items())} for k, d in forced.items()}},
                      f, indent=1, sort_keys=True)
            f.write("\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("run")
    a.add_argument("--variant", default="lean_64x64x64_w4x1_splitk")
    a.add_argument("--shapes", required=True)
    a.add_argument("--calls", type=int, default=150)
    a.add_argument("--settle-seconds", type=float, default=0.15)
    c = sub.add_parser("cut")
    c.add_argument("trace")
    c.add_argument("run")
    f = sub.add_parser("fit")
    f.add_argument("cuts", nargs="+")
    f.add_argument("--out")
    f.add_argument("--command", default="")
    args = ap.parse_args()
    {"run": run, "cut": cut, "fit": fit}[args.cmd](args)


if __name__ == "__main__":
    main()
