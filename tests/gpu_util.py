"""Helpers shared by the GPU tests: device transfer, the elementwise parity
check against the oracle, and device-resident problem setup."""
import numpy as np

ATOL = 1e-3
RTOL = 1e-4


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def to_dev(x, torch):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def check_close(C_gpu, C_ref, what=""):
    """|C - C_ref| <= 1e-3 + 1e-4 |C_ref| elementwise (C_ref in fp64)."""
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    assert C_gpu.shape == C_ref.shape, (C_gpu.shape, C_ref.shape)
    err = np.abs(C_gpu - C_ref)
    tol = ATOL + RTOL * np.abs(C_ref)
    bad = ~(err <= tol)             # NaN counts as a failure
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(int(v) for v in i)}: got {C_gpu[tuple(i)]!r} want {C_ref[tuple(i)]!r}"
                           for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} entries out of tolerance; "
                             f"max err {np.nanmax(err):.3e}; first: {detail}")
    return float(err.max()) if err.size else 0.0, float((err / tol).max()) if err.size else 0.0


def padded_device(x, ld, torch, fill=float("nan"), offset=0):
    """Device copy of x (rows x cols) inside a buffer with leading dimension ld,
    starting `offset` floats into the allocation; returns (view, buffer)."""
    rows, cols = x.shape
    buf = torch.full((offset + rows * ld + 16,), fill, dtype=torch.float32, device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(to_dev(x, torch))
    return view, buf
