"""Host-side check of the kernel's LDS A-stage layouts (no GPU needed): the
loader assignment and the LDS offsets are bijections, every 8-loader write
group fills one 128-byte LDS row, and every 16-lane ds_read_b128 pass of a
fragment read hits 16 distinct bank slots (tests/layout_check.hip)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_lds_layouts(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "layout_check"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "fp32_sgemm_tuning_amd", "csrc"),
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "layout_check.hip"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok") == 5, r.stdout
