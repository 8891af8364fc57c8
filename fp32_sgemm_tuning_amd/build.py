"""Build libsgemm.so (HIP, gfx950) in-tree with hipcc, and its race-check
twin libsgemm_poison.so.

    python -m fp32_sgemm_tuning_amd.build [--isa]

libsgemm_poison.so is the same library with the lean FP32 and the 16-bit
kernel units compiled with SGEMM_LDS_POISON=1: every LDS stage is filled
with NaN bits as soon as its last reader has passed its barrier, so a
missing barrier gives a wrong result (tests only; the C-ABI object is the
normal build's).

Flags: -O3 for gfx950 only, packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``; the host pass warns
that it does not know the feature, which is harmless), and the kernel
resource report (VGPR/AGPR/spill/LDS/occupancy) written to
``_build/resource_usage.txt``.  ``--isa`` also keeps the gfx950 assembly in
``_build/``.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsgemm.so")
POISON_LIB = os.path.join(PKG, "libsgemm_poison.so")
BUILD_DIR = os.path.join(PKG, "_build")
# (source, extra flags): each translation unit is compiled on its own (in
# parallel), then linked into one shared library.  The sgemm_lean*.hip units
# keep MFMA results in ordinary VGPRs; that flag is per translation unit and
# would make the shared header's 256-accumulator kernels spill.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
UNITS = [
    ("sgemm.hip", []),
    ("sgemm_lean.hip", VGPR_FORM),
    ("sgemm_lean_split.hip", VGPR_FORM),
    ("sgemm_lean_ops.hip", VGPR_FORM),
    ("sgemm_lean_split_t.hip", VGPR_FORM),
    ("sgemm_lowp.hip", VGPR_FORM),
]
SOURCES = [os.path.join(CSRC, u) for u, _ in UNITS]
# units rebuilt with the LDS poison for the race-check library (the rest of
# that library is the normal build's sgemm.o)
POISON_UNITS = [(u, extra + ["-DSGEMM_LDS_POISON=1"]) for u, extra in UNITS if u != "sgemm.hip"]
DEPS = SOURCES + [os.path.join(CSRC, h) for h in ("sgemm_kernels.hpp", "sgemm_lean.hpp")] + \
    [os.path.join(INCLUDE, "sgemm.h")]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def needs_build() -> bool:
    if not (os.path.exists(LIB) and os.path.exists(POISON_LIB)):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(POISON_LIB))
    return any(os.path.getmtime(p) > t for p in DEPS)


def _link(objs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True, cwd=BUILD_DIR)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError(f"hipcc link failed ({r.returncode})")
    os.replace(tmp, out)


def build(verbose: bool = False, isa: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs, objs, poison_objs = [], [], []
    jobs = [(u, extra, "") for u, extra in UNITS] + [(u, extra, "_poison") for u, extra in POISON_UNITS]
    for unit, extra, suffix in jobs:
        obj = os.path.join(BUILD_DIR, os.path.splitext(unit)[0] + suffix + ".o")
        cmd = [HIPCC, *HIP_FLAGS, *extra, "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, unit), "-o", obj]
        if isa and not suffix:
            cmd += ["-save-temps"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((unit + suffix, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                      text=True, cwd=BUILD_DIR)))
        (poison_objs if suffix else objs).append(obj)
    report, poison_report, failed = [], [], []
    for unit, p in procs:
        out, err = p.communicate()
        (poison_report if unit.endswith("_poison") else report).append(f"==== {unit}\n{err}")
        if p.returncode != 0:
            failed.append((unit, err))
    # the product library's kernels, and the race-check build's apart (same names)
    with open(os.path.join(BUILD_DIR, "resource_usage.txt"), "w") as f:
        f.write("\n".join(report))
    with open(os.path.join(BUILD_DIR, "resource_usage_poison.txt"), "w") as f:
        f.write("\n".join(poison_report))
    for unit, err in failed:
        sys.stderr.write(err)
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(u for u, _ in failed))
    _link(objs, LIB, verbose)
    # the race-check library: the normal C-ABI object and the poisoned kernels
    _link([objs[0]] + poison_objs, POISON_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, isa="--isa" in sys.argv))
