"""Build libsgemm.so (HIP, gfx950) in-tree with hipcc.

    python -m fp32_sgemm_tuning_amd.build [--isa]

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
    ("sgemm_lowp.hip", VGPR_FORM),
]
SOURCES = [os.path.join(CSRC, u) for u, _ in UNITS]
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
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


def build(verbose: bool = False, isa: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    procs, objs = [], []
    for unit, extra in UNITS:
        obj = os.path.join(BUILD_DIR, os.path.splitext(unit)[0] + ".o")
        cmd = [HIPCC, *HIP_FLAGS, *extra, "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, unit), "-o", obj]
        if isa:
            cmd += ["-save-temps"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((unit, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                                             cwd=BUILD_DIR)))
        objs.append(obj)
    report, failed = [], []
    for unit, p in procs:
        out, err = p.communicate()
        report.append(f"==== {unit}\n{err}")
        if p.returncode != 0:
            failed.append((unit, err))
    with open(os.path.join(BUILD_DIR, "resource_usage.txt"), "w") as f:
        f.write("\n".join(report))
    for unit, err in failed:
        sys.stderr.write(err)
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(u for u, _ in failed))
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True, cwd=BUILD_DIR)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError(f"hipcc link failed ({r.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, isa="--isa" in sys.argv))
