"""MI355X-native FP32 SGEMM (C = alpha*A*B + beta*C, row-major) for gfx950.

The GEMM runs in hand-written HIP kernels in ``libsgemm.so`` (C ABI in
include/sgemm.h, raw binding in :mod:`.capi`).  This module marshals torch
tensors into that call: device pointers, leading dimensions and the current
HIP stream.  PyTorch only supplies device memory and streams.
"""
from . import capi

__all__ = ["sgemm", "SgemmError", "capi", "variant_names"]


class SgemmError(RuntimeError):
    def __init__(self, status: int):
        msg = capi.sgemm_strerror(status)
        if status == capi.SGEMM_STATUS_HIP_ERROR:
            msg += ": " + capi.sgemm_last_hip_error()
        super().__init__(f"sgemm failed with status {status}: {msg}")
        self.status = status


def _ld(t, name):
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    # A single row (or an empty matrix) has no meaningful row stride; keep a
    # padded view's stride when it is valid, else use the packed one.
    if rows > 1 or t.stride(0) >= max(cols, 1):
        return t.stride(0)
    return max(cols, 1)


def sgemm(A, B, C=None, alpha=1.0, beta=0.0, variant=None, stream=None):
    """C = alpha * A @ B + beta * C on the current device; returns C.

    A [M,K], B [K,N], C [M,N] are float32 CUDA/HIP tensors with unit column
    stride (padded rows are fine).  With C None a new tensor is allocated
    (then beta must be 0).  ``variant`` forces a kernel variant (tests and
    sweeps); ``stream`` is a torch stream (default: the current stream).
    """
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(M, N)}")
    lda, ldb, ldc = _ld(A, "A"), _ld(B, "B"), _ld(C, "C")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    args = (M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
            float(beta), C.data_ptr(), ldc, s.cuda_stream)
    with torch.cuda.device(A.device):
        if variant is None:
            st = capi.sgemm(*args)
        else:
            st = capi.sgemm_ex(*args, int(variant))
    if st != capi.SGEMM_STATUS_OK:
        raise SgemmError(st)
    return C


def variant_names():
    return [capi.sgemm_variant_name(v) for v in range(capi.sgemm_num_variants())]
