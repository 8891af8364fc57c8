"""Checks on the gfx950 assembly of the split-K kernels (CPU only: hipcc
cross-compiles).

The lean kernels stream their K tiles with direct-to-LDS buffer loads and
wait for them once per K tile.  If the compiler cannot tell those LDS writes
apart from the kernel's LDS reads (it could not while the split-K ticket was
a second __shared__ variable), it puts a wait for every outstanding load after
each direct load, which serialises the loads of the K loop.  This test builds
the split-K translation unit to assembly and counts, per kernel, the direct
loads followed within a few instructions by a full `vmcnt(0)` wait.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp32_sgemm_tuning_amd", "csrc")


def _device_asm(unit, tmp_path):
    from fp32_sgemm_tuning_amd import build as b
    hipcc = b.HIPCC if os.path.exists(b.HIPCC) else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    extra = dict(b.UNITS)[unit]
    out = os.path.join(str(tmp_path), unit + ".s")
    cmd = [hipcc, *b.HIP_FLAGS, *extra, "--cuda-device-only", "-S", os.path.join(CSRC, unit), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _waits_after_direct_loads(asm):
    """{kernel symbol: (direct loads, loads followed by a vmcnt(0) wait before
    the next direct load, within 8 lines)}."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        lines = asm[m.end():end].splitlines()
        loads = waits = 0
        for i, line in enumerate(lines):
            if not line.rstrip().endswith(" lds"):
                continue
            loads += 1
            for nxt in lines[i + 1:i + 8]:
                if "vmcnt(0)" in nxt:
                    waits += 1
                    break
                if nxt.rstrip().endswith(" lds"):
                    break
        if loads:
            out[m.group(1)] = (loads, waits)
    return out


def test_split_k_loop_keeps_loads_in_flight(tmp_path):
    asm = _device_asm("sgemm_lean_split.hip", tmp_path)
    kernels = _waits_after_direct_loads(asm)
    split = {k: v for k, v in kernels.items() if "sgemm_lean_kernel" in k}
    assert len(split) >= 20, sorted(kernels)
    # the K-remainder prologue and the edge paths may wait once or twice; a
    # serialised K loop waits after every load (17 of 32 in the 64x64x64
    # kernel before the ticket moved into the kernel's LDS buffer)
    bad = {k: v for k, v in split.items() if v[1] > 4}
    assert not bad, bad
