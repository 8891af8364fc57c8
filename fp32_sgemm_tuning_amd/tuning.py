"""The tile-choice evidence as data: the tuning table the automatic choice is
checked against.

    python -m fp32_sgemm_tuning_amd.tuning --sweep SWEEP.jsonl \\
        --resources fp32_sgemm_tuning_amd/_build/resource_usage.txt \\
        --counters-4096 DIR [DIR ...] --workload-counters DIR [DIR ...] \\
        --command "the sweep command" --out profiles/tuning_fp32.json

The table holds, per problem shape (packed row-major FP32, alpha = 1,
beta = 0), the time per call of every lean variant and of the automatic
choice from an interleaved sweep (bench.py --sweep, one process, clock
settled; the median over rounds of batches of back-to-back calls), the
resources of every kernel instantiation from the
build's resource report, whether each variant passes cfg_valid(), hardware
counters per variant at 4096^3, and the MFMA-busy share of the automatic
choice on every workload.  The autotuner of the "gpu_matmul" blog (1D
Blocktiling) filters its candidate configurations with a validity check
before timing them; cfg_valid() is that filter for this hardware: a tile
must fit the 160 KiB of LDS of a compute unit and keep every value in
registers (no scratch).
"""
import argparse
import csv
import glob
import json
import os
import re
import statistics

LDS_LIMIT = 160 * 1024          # bytes of LDS per compute unit on gfx950
CUS = 256
SIMDS = 4 * CUS
PEAK_TFLOPS = 157.3
# Measurement spread the table's comparisons allow.  The same plan (same
# variant, split and shape) timed in interleaved sweeps on different boxes
# (each call between its own event pair, as the sweep timed them then)
# measured up to 7.9% apart for kernels of 50-400 us (1088^2 x 2048 on the
# 64x64x64 split kernel: 53.1 and 57.3 us; 3072^3 and 1600^3 6.5-6.6%), the
# median over 41 such pairs 1.5%; kernels under 50 us, which launch and
# first-load latency set, up to 19% (512^3: 12.8 and 15.3 us).
SPREAD = 0.07
SPREAD_SHORT = 0.15
SHORT_US = 50.0

_TILE = re.compile(r"^lean_(dw_)?(\d+)x(\d+)x(\d+)_w(\d+)x(\d+)(_splitk)?$")


def variant_tile(name):
    """(BM, BN, BK, WAVES_M, WAVES_N, DW) of a lean variant name, else None."""
    m = _TILE.match(name)
    if not m:
        return None
    return (int(m.group(2)), int(m.group(3)), int(m.group(4)), int(m.group(5)), int(m.group(6)), bool(m.group(1)))


def parse_resource_usage(text):
    """{mangled kernel: {vgpr, agpr, scratch, lds, occupancy}} from the
    compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    fields = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
              "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        if cur is None:
            continue
        for label, key in fields.items():
            m = re.search(r"remark:\s+" + re.escape(label) + r": (\d+)", line)
            if m:
                cur[key] = int(m.group(1))
    return out


def lean_template_args(mangled):
    """Template arguments of a sgemm_lean_kernel instantiation: ints then
    bools, (BM, BN, BK, WM, WN, BETA0, EDGE, SPLIT, DW, TA, TB); else None."""
    if "sgemm_lean_kernel" not in mangled:
        return None
    args = re.findall(r"L([ib])(\d+)E", mangled.split("sgemm_lean_kernel", 1)[1])
    vals = [int(v) if t == "i" else bool(int(v)) for t, v in args]
    return tuple(vals) if len(vals) == 11 else None


def cfg_valid(instances):
    """A tile configuration is valid when every instantiation of it fits the
    LDS of a compute unit and spills nothing to scratch."""
    return bool(instances) and all(r.get("lds", 0) <= LDS_LIMIT and r.get("scratch", 0) == 0 for r in instances)


def variant_resources(name, resources):
    """Resource records of every instantiation of a lean variant's tile and
    load width (plain and split forms, all epilogue, edge and operand forms)."""
    tile = variant_tile(name)
    if tile is None:
        return []
    bm, bn, bk, wm, wn, dw = tile
    out = []
    for mangled, r in resources.items():
        a = lean_template_args(mangled)
        if a and a[:5] == (bm, bn, bk, wm, wn) and a[8] == dw:
            out.append(r)
    return out


def _counter_medians(dirs):
    """{(template args of the lean kernel): {counter: median}} over the
    counter_collection CSVs of rocprofv3 runs."""
    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                a = _demangled_args(row["Kernel_Name"])
                if a is None:
                    continue
                vals.setdefault(a, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return {a: {c: statistics.median(v) for c, v in cs.items()} for a, cs in vals.items()}


def _demangled_args(name):
    """Template arguments from a demangled kernel name as rocprofv3 prints it
    ("void sgemm_mi355x::sgemm_lean_kernel<128, 128, 32, 2, 2, true, ...>")."""
    m = re.search(r"sgemm_lean_kernel<([^>]*)>", name)
    if not m:
        return None
    parts = [p.strip() for p in m.group(1).split(",")]
    vals = [p == "true" if p in ("true", "false") else int(p) for p in parts]
    return tuple(vals) if len(vals) == 11 else None


def _mfma_busy(c):
    if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or "GRBM_GUI_ACTIVE" not in c:
        return None
    return c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8 * SIMDS)


def build_table(sweep_lines, resources, counters_4096, workload_counters, command):
    shapes = {}
    for line in sweep_lines:
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        if "median_ms" not in r:
            continue
        entry = shapes.setdefault(r["shape"], {"times_us": {}})
        if r["sweep"].startswith("auto:"):
            entry["auto_variant"] = r["sweep"][5:]
            entry["auto_us"] = round(r["median_ms"] * 1e3, 2)
        else:
            entry["times_us"][r["sweep"]] = round(r["median_ms"] * 1e3, 2)
    names = sorted({v for e in shapes.values() for v in e["times_us"]} |
                   {e["auto_variant"] for e in shapes.values() if "auto_variant" in e})
    variants = {}
    for n in names:
        inst = variant_resources(n, resources)
        tile = variant_tile(n)
        variants[n] = {
            "tile": None if tile is None else {"bm": tile[0], "bn": tile[1], "bk": tile[2], "waves_m": tile[3],
                                               "waves_n": tile[4], "four_byte_loads": tile[5]},
            "instantiations": len(inst),
            "max_vgpr": max((r.get("vgpr", 0) for r in inst), default=None),
            "max_agpr": max((r.get("agpr", 0) for r in inst), default=None),
            "max_scratch_bytes_per_lane": max((r.get("scratch", 0) for r in inst), default=None),
            "lds_bytes": max((r.get("lds", 0) for r in inst), default=None),
            "min_occupancy_waves_per_simd": min((r.get("occupancy", 0) for r in inst), default=None),
            "cfg_valid": cfg_valid(inst),
        }
    c4096 = _counter_medians(counters_4096)
    for n, v in variants.items():
        t = variant_tile(n)
        if t is None:
            continue
        # the whole-tile, beta = 0, unsplit instantiation that 4096^3 runs
        key = (t[0], t[1], t[2], t[3], t[4], True, False, False, t[5], False, False)
        c = c4096.get(key)
        if c:
            v["at_4096"] = {
                "mfma_busy": None if _mfma_busy(c) is None else round(_mfma_busy(c), 4),
                "fetch_bytes": c.get("FETCH_SIZE") and round(c["FETCH_SIZE"] * 1024 * 2.0),
                "write_bytes": c.get("WRITE_SIZE") and round(c["WRITE_SIZE"] * 1024),
                "non_mfma_valu_per_mfma": (round((c["SQ_INSTS_VALU"] - c["SQ_INSTS_VALU_MFMA_MOPS_F32"] / 4) /
                                                 (c["SQ_INSTS_VALU_MFMA_MOPS_F32"] / 4), 4)
                                           if "SQ_INSTS_VALU" in c and c.get("SQ_INSTS_VALU_MFMA_MOPS_F32") else None),
                "lds_bank_conflicts": c.get("SQ_LDS_BANK_CONFLICT"),
            }
    for shape, e in shapes.items():
        M, N, K = (int(x) for x in shape.split("x"))
        # the automatic plan, timed under both names in the same sweep
        both = [t for t in (e.get("auto_us"), e["times_us"].get(e.get("auto_variant"))) if t]
        if both:
            e["auto_plan_us"] = round(sum(both) / len(both), 2)
        valid = {n: t for n, t in e["times_us"].items() if variants.get(n, {}).get("cfg_valid")}
        if valid:
            best = min(valid, key=valid.get)
            e["best_variant"] = best
            e["best_us"] = valid[best]
            e["best_tflops"] = round(2.0 * M * N * K / (valid[best] * 1e-6) / 1e12, 2)
    wl = {}
    for d in workload_counters:
        name = os.path.basename(os.path.normpath(d))
        c = _counter_medians([d])
        if c:
            # the kernel with the most MFMA work is the product's own
            key = max(c, key=lambda a: c[a].get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0))
            busy = _mfma_busy(c[key])
            wl[name] = {"kernel_template_args": list(key), "mfma_busy": None if busy is None else round(busy, 4)}
    return {
        "about": "Tile-choice evidence for the FP32 SGEMM on MI355X (gfx950): per shape, the time per call "
                 "(median over rounds of back-to-back batches) of every lean variant and of the automatic "
                 "choice; per variant, resources and the "
                 "cfg_valid filter (LDS <= 160 KiB, no scratch); counters at 4096^3.",
        "sweep_command": command,
        "spread": SPREAD,
        "spread_short": SPREAD_SHORT,
        "short_us": SHORT_US,
        "lds_limit_bytes": LDS_LIMIT,
        "peak_tflops": PEAK_TFLOPS,
        "variants": variants,
        "shapes": shapes,
        "workload_mfma_busy": wl,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sweep", required=True)
    ap.add_argument("--resources", required=True)
    ap.add_argument("--counters-4096", nargs="*", default=[])
    ap.add_argument("--workload-counters", nargs="*", default=[])
    ap.add_argument("--command", default="")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    table = build_table(open(args.sweep).read().splitlines(), parse_resource_usage(open(args.resources).read()),
                        args.counters_4096, args.workload_counters, args.command)
    with open(args.out, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"{args.out}: {len(table['shapes'])} shapes, {len(table['variants'])} variants")


if __name__ == "__main__":
    main()
