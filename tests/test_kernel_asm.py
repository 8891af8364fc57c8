"""Checks on the gfx950 assembly of the lean kernels (CPU only: hipcc
cross-compiles).

The lean kernels stream their K tiles with direct-to-LDS buffer loads and
wait for them once per K tile.
- If the compiler cannot tell those LDS writes apart from the kernel's LDS
  reads (it could not while the split-K ticket was a second __shared__
  variable), it puts a wait for every outstanding load after each direct
  load, which serialises the loads of the K loop.
- If a buffer descriptor ends up in vector registers (a wave-uniform value
  merged through divergent control flow), every load using it runs inside a
  waterfall loop (read the first lane, compare, mask, repeat).
Both cost a large share of the kernel's speed and neither shows in results,
so the tests build the translation units to assembly and look for them.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp32_sgemm_tuning_amd", "csrc")


def _device_asm(builds, tmp_path):
    """Device assembly of each build {key: (unit, extra flags)}, compiled in
    parallel: {key: text}."""
    from fp32_sgemm_tuning_amd import build as b
    hipcc = b.HIPCC if os.path.exists(b.HIPCC) else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    procs = {}
    for key, (unit, extra) in builds.items():
        out = os.path.join(str(tmp_path), key + ".s")
        cmd = [hipcc, *b.HIP_FLAGS, *dict(b.UNITS)[unit], *extra, "--cuda-device-only", "-S",
               os.path.join(CSRC, unit), "-o", out]
        procs[key] = (out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    texts = {}
    for key, (out, proc) in procs.items():
        _, err = proc.communicate()
        assert proc.returncode == 0, err[-2000:]
        texts[key] = open(out).read()
    return texts


@pytest.fixture(scope="module")
def asm_builds(tmp_path_factory):
    """The lean units as the library builds them, and the plain lean unit
    as the race-check library builds it."""
    return _device_asm({"sgemm_lean.hip": ("sgemm_lean.hip", []),
                        "sgemm_lean_split.hip": ("sgemm_lean_split.hip", []),
                        "sgemm_lean_split_t.hip": ("sgemm_lean_split_t.hip", []),
                        "poison:sgemm_lean.hip": ("sgemm_lean.hip", ["-DSGEMM_LDS_POISON=1"])},
                       tmp_path_factory.mktemp("asm"))


@pytest.fixture(scope="module")
def lean_asm(asm_builds):
    return {k: v for k, v in asm_builds.items() if not k.startswith("poison:")}


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


def _kernels(asm):
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end].splitlines()


def _waterfall_loops(lines):
    """Loops (a label and a branch back to it) of under 40 lines holding a
    buffer access and a v_readfirstlane: the shape of a waterfall loop."""
    n = 0
    for h, line in enumerate(lines):
        if "Loop Header" not in line:
            continue
        label = line.split(":")[0]
        back = [i for i, x in enumerate(lines) if "s_cbranch" in x and x.strip().endswith(label)]
        if not back:
            continue
        body = lines[h:back[-1] + 1]
        if len(body) < 40 and any("v_readfirstlane" in x for x in body) and any("buffer_" in x for x in body):
            n += 1
    return n


def test_no_waterfall_loops(lean_asm):
    """Every buffer descriptor of the lean kernels (plain and split-K, every
    edge and alignment form) stays in scalar registers."""
    bad = {}
    count = 0
    for unit, asm in lean_asm.items():
        for name, lines in _kernels(asm):
            if "sgemm_lean_kernel" not in name:
                continue
            count += 1
            w = _waterfall_loops(lines)
            if w:
                bad[name] = w
    assert count >= 60
    assert not bad, bad


def test_split_k_loop_keeps_loads_in_flight(lean_asm):
    kernels = _waits_after_direct_loads(lean_asm["sgemm_lean_split.hip"])
    kernels.update(_waits_after_direct_loads(lean_asm["sgemm_lean_split_t.hip"]))
    split = {k: v for k, v in kernels.items() if "sgemm_lean_kernel" in k}
    assert len(split) >= 32, sorted(kernels)
    # the K-remainder prologue and the edge paths may wait once or twice; a
    # serialised K loop waits after every load (17 of 32 in the 64x64x64
    # kernel before the ticket moved into the kernel's LDS buffer)
    bad = {k: v for k, v in split.items() if v[1] > 4}
    assert not bad, bad


def test_race_check_build_poisons_the_stages(lean_asm, asm_builds):
    """The lean kernels fill LDS only through direct loads, so the normal
    build has no LDS write instruction in them at all; the race-check build
    (SGEMM_LDS_POISON=1, as libsgemm_poison.so is built) writes the NaN
    bits with ds_write before every stage's refill."""
    def ds_writes(asm):
        return {name: sum("ds_write" in x for x in lines) for name, lines in _kernels(asm)
                if "sgemm_lean_kernel" in name}
    plain = ds_writes(lean_asm["sgemm_lean.hip"])
    poisoned = ds_writes(asm_builds["poison:sgemm_lean.hip"])
    assert plain and set(plain) == set(poisoned)
    assert all(n == 0 for n in plain.values()), plain
    assert all(n > 0 for n in poisoned.values()), poisoned
