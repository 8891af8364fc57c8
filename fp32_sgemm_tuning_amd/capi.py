"""ctypes binding of libsgemm.so with the C ABI's own names and signatures
(include/sgemm.h).  Argument marshalling only: every step of the GEMM runs in
the library's HIP kernels.  There is no fallback: if the library is missing
or does not load, every call raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsgemm.so")
# The race-check build (LDS stages poisoned with NaN between their last read
# and their refill); for tests.
POISON_LIB_PATH = os.path.join(PKG, "libsgemm_poison.so")

SGEMM_STATUS_OK = 0
SGEMM_STATUS_INVALID_DIM = -1
SGEMM_STATUS_NULL_POINTER = -2
SGEMM_STATUS_HIP_ERROR = -3
SGEMM_STATUS_INVALID_VARIANT = -4
SGEMM_STATUS_UNSUPPORTED = -5
SGEMM_STATUS_INVALID_OP = -6
SGEMM_STATUS_INVALID_DTYPE = -7
SGEMM_STATUS_SCRATCH_TOO_SMALL = -8

SGEMM_WORKSPACE_BYTES = 64 * 1024 * 1024 + 16 * 1024
SGEMM_MAX_STREAM_WORKSPACES = 8
SGEMM_MAX_COPY_BUFFERS = 2
SGEMM_MAX_COPY_BUFFER_BYTES = 4 << 30
SGEMM_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024 + 16 * 1024

SGEMM_DTYPE_BF16 = 1
SGEMM_DTYPE_F16 = 2

SGEMM_OP_N = 0
SGEMM_OP_T = 1

SGEMM_VARIANT_AUTO = -1
SGEMM_VARIANT_SIMPLE = 0
SGEMM_VARIANT_DB128_VEC = 1
SGEMM_VARIANT_DB128_SCALAR = 2

# Every symbol include/sgemm.h declares.
EXPORTS = ("sgemm", "sgemm_ex", "sgemm_select_variant", "sgemm_num_variants",
           "sgemm_variant_name", "sgemm_variant_info", "sgemm_split_factor", "sgemm_strerror",
           "sgemm_last_hip_error", "sgemm_version", "sgemm_op", "sgemm_strided_batched", "sgemm_cm",
           "sgemm_cm_strided_batched", "sgemm_lowp", "sgemm_lowp_ex", "sgemm_lowp_select_variant",
           "sgemm_lowp_variant_name", "sgemm_lowp_split_factor", "sgemm_tail_split", "sgemm_lowp_op",
           "sgemm_lowp_strided_batched", "sgemm_workspace_bytes", "sgemm_release_workspaces",
           "sgemm_noalloc")

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsgemm.so (once) and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A separate handle on a build of the library at `path` (the race-check
    build, for tests), with the signatures declared; not the module's own."""
    # libsgemm.so needs libamdhip64.so.7.  PyTorch-ROCm ships its own copy of
    # that runtime under the same soname; whichever copy is loaded first is
    # the one the whole process uses.  Import torch first so this library
    # binds to torch's runtime and the process holds exactly one HIP runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise LibraryMissing(
            f"{path} is not built; run `python -m fp32_sgemm_tuning_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    i, f, vp, cp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_char_p
    gemm_args = [i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    lib.sgemm.argtypes = gemm_args
    lib.sgemm.restype = i
    lib.sgemm_noalloc.argtypes = gemm_args
    lib.sgemm_noalloc.restype = i
    lib.sgemm_ex.argtypes = gemm_args + [i]
    lib.sgemm_ex.restype = i
    lib.sgemm_select_variant.argtypes = [i, i, i, vp, i, vp, i, f, vp, i]
    lib.sgemm_select_variant.restype = i
    lib.sgemm_num_variants.argtypes = []
    lib.sgemm_num_variants.restype = i
    lib.sgemm_variant_name.argtypes = [i]
    lib.sgemm_variant_name.restype = cp
    ip = ctypes.POINTER(ctypes.c_int)
    lib.sgemm_variant_info.argtypes = [i, ip, ip, ip, ip]
    lib.sgemm_variant_info.restype = i
    ll = ctypes.c_longlong
    op_args = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    batched_args = [i, i, i, i, i, f, vp, i, ll, vp, i, ll, f, vp, i, ll, i, vp]
    for name, args in (("sgemm_op", op_args), ("sgemm_cm", op_args),
                       ("sgemm_strided_batched", batched_args), ("sgemm_cm_strided_batched", batched_args)):
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = i
    lib.sgemm_lowp.argtypes = [i, i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    lib.sgemm_lowp.restype = i
    lib.sgemm_lowp_ex.argtypes = [i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, i]
    lib.sgemm_lowp_ex.restype = i
    lib.sgemm_lowp_op.argtypes = [i, i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, i]
    lib.sgemm_lowp_op.restype = i
    lib.sgemm_lowp_strided_batched.argtypes = [i, i, i, i, i, i, f, vp, i, ll, vp, i, ll, f, vp, i, ll, i, vp]
    lib.sgemm_lowp_strided_batched.restype = i
    lib.sgemm_lowp_select_variant.argtypes = [i, i, i, vp, i, vp, i]
    lib.sgemm_lowp_select_variant.restype = i
    lib.sgemm_lowp_split_factor.argtypes = [i, i, i, i]
    lib.sgemm_lowp_split_factor.restype = i
    lib.sgemm_lowp_variant_name.argtypes = [i]
    lib.sgemm_lowp_variant_name.restype = cp
    lib.sgemm_tail_split.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_int)]
    lib.sgemm_tail_split.restype = i
    lib.sgemm_split_factor.argtypes = [i, i, i, i]
    lib.sgemm_split_factor.restype = i
    lib.sgemm_strerror.argtypes = [i]
    lib.sgemm_strerror.restype = cp
    lib.sgemm_last_hip_error.argtypes = []
    lib.sgemm_last_hip_error.restype = cp
    lib.sgemm_version.argtypes = []
    lib.sgemm_version.restype = i
    lib.sgemm_workspace_bytes.argtypes = []
    lib.sgemm_workspace_bytes.restype = ll
    lib.sgemm_release_workspaces.argtypes = []
    lib.sgemm_release_workspaces.restype = i
    return lib


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream):
    """Raw C call; pointers and stream are integers (device addresses / hipStream_t)."""
    return load().sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream):
    """sgemm with split-K partials in the library's static scratch: no allocation."""
    return load().sgemm_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant):
    return load().sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)


def sgemm_select_variant(M, N, K, A, lda, B, ldb, beta, C, ldc):
    return load().sgemm_select_variant(M, N, K, A, lda, B, ldb, beta, C, ldc)


def sgemm_num_variants():
    return load().sgemm_num_variants()


def sgemm_variant_name(variant):
    s = load().sgemm_variant_name(variant)
    return None if s is None else s.decode()


def sgemm_variant_info(variant):
    """(status, bm, bn, bk, needs_vec) of a variant."""
    v = [ctypes.c_int(0) for _ in range(4)]
    st = load().sgemm_variant_info(variant, *[ctypes.byref(x) for x in v])
    return (st,) + tuple(x.value for x in v)


def sgemm_op(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream):
    return load().sgemm_op(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_cm(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream):
    return load().sgemm_cm(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_strided_batched(op_a, op_b, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch, stream):
    return load().sgemm_strided_batched(op_a, op_b, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc,
                                        batch, stream)


def sgemm_cm_strided_batched(op_a, op_b, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch, stream):
    return load().sgemm_cm_strided_batched(op_a, op_b, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc,
                                           batch, stream)


def sgemm_lowp(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream):
    return load().sgemm_lowp(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_lowp_ex(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant):
    return load().sgemm_lowp_ex(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)


def sgemm_lowp_op(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant):
    return load().sgemm_lowp_op(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)


def sgemm_lowp_strided_batched(dtype, op_a, op_b, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch,
                               stream):
    return load().sgemm_lowp_strided_batched(dtype, op_a, op_b, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C,
                                             ldc, sc, batch, stream)


def sgemm_lowp_select_variant(M, N, K, A, lda, B, ldb):
    return load().sgemm_lowp_select_variant(M, N, K, A, lda, B, ldb)


def sgemm_lowp_variant_name(variant):
    s = load().sgemm_lowp_variant_name(variant)
    return None if s is None else s.decode()


def sgemm_lowp_split_factor(variant, M, N, K):
    return load().sgemm_lowp_split_factor(variant, M, N, K)


def lowp_variants():
    """Every sgemm_lowp_ex variant id."""
    n = 0
    while sgemm_lowp_variant_name(n) is not None:
        n += 1
    return list(range(n))


def sgemm_tail_split(variant, M, N, K):
    """(S, tiles of the second launch) of the last-wave split; S == 1: one launch."""
    t = ctypes.c_int(0)
    s = load().sgemm_tail_split(variant, M, N, K, ctypes.byref(t))
    return s, t.value


def sgemm_split_factor(variant, M, N, K):
    return load().sgemm_split_factor(variant, M, N, K)


def all_variants():
    """Every variant id the library offers."""
    return list(range(sgemm_num_variants()))


def sgemm_strerror(status):
    return load().sgemm_strerror(status).decode()


def sgemm_last_hip_error():
    return load().sgemm_last_hip_error().decode()


def sgemm_version():
    return load().sgemm_version()


def sgemm_workspace_bytes():
    return load().sgemm_workspace_bytes()


def sgemm_release_workspaces():
    return load().sgemm_release_workspaces()
