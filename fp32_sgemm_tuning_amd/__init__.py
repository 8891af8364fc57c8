"""MI355X-native FP32 SGEMM (C = alpha*A*B + beta*C, row-major) for gfx950.

The GEMM runs in hand-written HIP kernels in ``libsgemm.so`` (C ABI in
include/sgemm.h, raw binding in :mod:`.capi`).  This module marshals torch
tensors into that call: device pointers, leading dimensions and the current
HIP stream.  PyTorch only supplies device memory and streams.
"""
import contextlib

from . import capi

__all__ = ["sgemm", "sgemm_op", "sgemm_lowp", "SgemmError", "capi", "variant_names"]


class SgemmError(RuntimeError):
    def __init__(self, status: int):
        msg = capi.sgemm_strerror(status)
        if status == capi.SGEMM_STATUS_HIP_ERROR:
            msg += ": " + capi.sgemm_last_hip_error()
        super().__init__(f"sgemm failed with status {status}: {msg}")
        self.status = status


def _ld(t, name, dtypes=None):
    import torch
    if t.dtype not in (dtypes or (torch.float32,)):
        raise TypeError(f"{name} must be " + " or ".join(str(d).replace("torch.", "") for d in (dtypes or (torch.float32,))))
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
    _same_device(A, B, C)
    with _device_ctx(A.device):
        args = (M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
                float(beta), C.data_ptr(), ldc, _stream_handle(A.device, stream))
        if variant is None:
            st = capi.sgemm(*args)
        else:
            st = capi.sgemm_ex(*args, int(variant))
    if st != capi.SGEMM_STATUS_OK:
        raise SgemmError(st)
    return C


def _same_device(A, B, C):
    if not (A.device == B.device == C.device):
        raise ValueError(f"A, B and C must be on one device, got {A.device}, {B.device}, {C.device}")


def _device_ctx(device):
    """A context with `device` current; nothing to do when it already is."""
    import torch
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _stream_handle(device, stream):
    """The HIP stream handle of `stream` (a torch stream), else of the
    device's current stream."""
    if stream is not None:
        return stream.cuda_stream
    import torch
    idx = device.index if device.index is not None else torch.cuda.current_device()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(idx)
    return torch.cuda.current_stream(idx).cuda_stream


def variant_names():
    return [capi.sgemm_variant_name(v) for v in range(capi.sgemm_num_variants())]


def _mat(t, name, dtypes=None):
    """(rows, cols, ld) of a row-major matrix view, or of each matrix of a
    3-D batch view (then also the batch stride)."""
    import torch
    if t.dtype not in (dtypes or (torch.float32,)):
        raise TypeError(f"{name} has type {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() == 2:
        return t.shape[0], t.shape[1], _ld(t, name, dtypes), 0
    if t.dim() == 3:
        rows, cols = t.shape[1], t.shape[2]
        if cols > 1 and t.stride(2) != 1:
            raise ValueError(f"{name} must have unit column stride (row-major)")
        ld = t.stride(1) if rows > 1 or t.stride(1) >= max(cols, 1) else max(cols, 1)
        return rows, cols, ld, t.stride(0) if t.shape[0] > 1 else 0
    raise ValueError(f"{name} must be 2-D or 3-D")


def sgemm_op(A, B, C=None, alpha=1.0, beta=0.0, trans_a=False, trans_b=False, stream=None):
    """C = alpha * op(A) @ op(B) + beta * C with op(X) = X or X^T, row-major;
    returns C.

    A and B are the stored matrices: with trans_a, A is [K,M]; with trans_b,
    B is [N,K].  3-D tensors ([batch, rows, cols], any batch stride, one of A
    and B may have batch 1 to be shared) run as one strided batch.
    """
    import torch
    batched = A.dim() == 3 or B.dim() == 3 or (C is not None and C.dim() == 3)
    ra, ca, lda, sa = _mat(A, "A")
    rb, cb, ldb, sb = _mat(B, "B")
    M, K = (ca, ra) if trans_a else (ra, ca)
    K2, N = (cb, rb) if trans_b else (rb, cb)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: op(A) is {M}x{K}, op(B) is {K2}x{N}")
    batch = max(A.shape[0] if A.dim() == 3 else 1, B.shape[0] if B.dim() == 3 else 1)
    for t, name in ((A, "A"), (B, "B")):
        if t.dim() == 3 and t.shape[0] not in (1, batch):
            raise ValueError(f"{name} has batch {t.shape[0]}, expected 1 or {batch}")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((batch, M, N) if batched else (M, N), dtype=torch.float32, device=A.device)
    rc, cc, ldc, sc = _mat(C, "C")
    _same_device(A, B, C)
    if (rc, cc) != (M, N) or (C.dim() == 3 and C.shape[0] != batch):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(batch, M, N) if batched else (M, N)}")
    op_a = capi.SGEMM_OP_T if trans_a else capi.SGEMM_OP_N
    op_b = capi.SGEMM_OP_T if trans_b else capi.SGEMM_OP_N
    with _device_ctx(A.device):
        h = _stream_handle(A.device, stream)
        if batched:
            st = capi.sgemm_strided_batched(op_a, op_b, M, N, K, float(alpha), A.data_ptr(), lda, sa,
                                            B.data_ptr(), ldb, sb, float(beta), C.data_ptr(), ldc, sc, batch, h)
        else:
            st = capi.sgemm_op(op_a, op_b, M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
                               float(beta), C.data_ptr(), ldc, h)
    if st != capi.SGEMM_STATUS_OK:
        raise SgemmError(st)
    return C


def sgemm_lowp(A, B, C=None, alpha=1.0, beta=0.0, variant=None, stream=None, trans_a=False, trans_b=False):
    """C = alpha * op(A) @ op(B) + beta * C with bfloat16 or float16 A and B
    (one type for both, unit column stride) and FP32 accumulation; C is
    float32 (allocated when None, then beta must be 0); returns C.  op(X) =
    X, or X^T with trans_a / trans_b (then A is stored [K,M], B [N,K]).  3-D
    tensors ([batch, rows, cols], any batch stride, one of A and B may have
    batch 1 to be shared) run as one strided batch.  ``variant`` forces a
    kernel variant of a single untransposed problem (tests and sweeps)."""
    import torch
    codes = {torch.bfloat16: capi.SGEMM_DTYPE_BF16, torch.float16: capi.SGEMM_DTYPE_F16}
    batched = A.dim() == 3 or B.dim() == 3 or (C is not None and C.dim() == 3)
    ra, ca, lda, sa = _mat(A, "A", tuple(codes))
    rb, cb, ldb, sb = _mat(B, "B", tuple(codes))
    if B.dtype != A.dtype:
        raise TypeError(f"A is {A.dtype} but B is {B.dtype}")
    M, K = (ca, ra) if trans_a else (ra, ca)
    K2, N = (cb, rb) if trans_b else (rb, cb)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: op(A) is {M}x{K}, op(B) is {K2}x{N}")
    batch = max(A.shape[0] if A.dim() == 3 else 1, B.shape[0] if B.dim() == 3 else 1)
    for t, name in ((A, "A"), (B, "B")):
        if t.dim() == 3 and t.shape[0] not in (1, batch):
            raise ValueError(f"{name} has batch {t.shape[0]}, expected 1 or {batch}")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((batch, M, N) if batched else (M, N), dtype=torch.float32, device=A.device)
    rc, cc, ldc, sc = _mat(C, "C")
    if (rc, cc) != (M, N) or (C.dim() == 3 and C.shape[0] != batch):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(batch, M, N) if batched else (M, N)}")
    _same_device(A, B, C)
    op_a = capi.SGEMM_OP_T if trans_a else capi.SGEMM_OP_N
    op_b = capi.SGEMM_OP_T if trans_b else capi.SGEMM_OP_N
    with _device_ctx(A.device):
        h = _stream_handle(A.device, stream)
        if batched:
            st = capi.sgemm_lowp_strided_batched(codes[A.dtype], op_a, op_b, M, N, K, float(alpha), A.data_ptr(),
                                                 lda, sa, B.data_ptr(), ldb, sb, float(beta), C.data_ptr(), ldc, sc,
                                                 batch, h)
        elif trans_a or trans_b:
            st = capi.sgemm_lowp_op(codes[A.dtype], op_a, op_b, M, N, K, float(alpha), A.data_ptr(), lda,
                                    B.data_ptr(), ldb, float(beta), C.data_ptr(), ldc, h,
                                    capi.SGEMM_VARIANT_AUTO if variant is None else int(variant))
        else:
            args = (codes[A.dtype], M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb,
                    float(beta), C.data_ptr(), ldc, h)
            st = capi.sgemm_lowp(*args) if variant is None else capi.sgemm_lowp_ex(*args, int(variant))
    if st != capi.SGEMM_STATUS_OK:
        raise SgemmError(st)
    return C
