"""The C-ABI library without a GPU: it loads, exports every symbol that
include/sgemm.h declares, and rejects bad arguments before any HIP call.

Nothing here launches a kernel: every call below returns from the argument
checks, which run before the library touches the HIP runtime.
"""
import os
import re

import pytest

from fp32_sgemm_tuning_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")

# Fake device addresses: only inspected for alignment, never dereferenced.
AL = 0x10000          # 16-byte aligned
MIS = 0x10004         # 4-byte aligned only


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgemm\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return capi.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert set(declared) == set(capi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), f"libsgemm.so does not export {name}"


def test_variant_info(lib):
    for v in capi.all_variants():
        st, bm, bn, bk, vec = capi.sgemm_variant_info(v)
        assert st == capi.SGEMM_STATUS_OK
        assert bm % 16 == 0 and bn % 16 == 0 and bk % 4 == 0 and vec in (0, 1)
        assert f"{bm}x{bn}x{bk}" in capi.sgemm_variant_name(v)
    assert capi.sgemm_variant_info(capi.sgemm_num_variants())[0] == capi.SGEMM_STATUS_INVALID_VARIANT
    assert capi.sgemm_variant_info(capi.SGEMM_VARIANT_DB128_VEC)[1:] == (128, 128, 32, 1)
    assert capi.sgemm_variant_info(capi.SGEMM_VARIANT_DB128_SCALAR)[1:] == (128, 128, 32, 0)
    assert capi.sgemm_variant_info(capi.SGEMM_VARIANT_SIMPLE)[4] == 0


def test_version_and_variants(lib):
    assert capi.sgemm_version() >= 1
    n = capi.sgemm_num_variants()
    assert n >= 3
    names = [capi.sgemm_variant_name(v) for v in range(n)]
    assert all(names) and len(set(names)) == n
    assert capi.sgemm_variant_name(n) is None
    assert capi.sgemm_variant_name(-1) is None
    assert capi.sgemm_last_hip_error() == ""


@pytest.mark.parametrize("status", [0, -1, -2, -3, -4, -5, -6, -7, -8])
def test_strerror_known(status):
    s = capi.sgemm_strerror(status)
    assert s and s != "unknown status"


def test_strerror_unknown():
    assert capi.sgemm_strerror(42) == "unknown status"


GOOD = dict(M=8, N=8, K=8, alpha=1.0, A=AL, lda=8, B=AL, ldb=8, beta=0.0, C=AL, ldc=8, stream=None)


def _call(**kw):
    a = {**GOOD, **kw}
    return capi.sgemm(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"], a["ldb"],
                      a["beta"], a["C"], a["ldc"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(lda=7), dict(ldb=7), dict(ldc=7),
    dict(K=0, lda=0), dict(N=0, ldb=0), dict(N=0, ldc=0),
])
def test_invalid_dimensions(kw):
    assert _call(**kw) == capi.SGEMM_STATUS_INVALID_DIM


@pytest.mark.parametrize("kw", [dict(A=None), dict(B=None), dict(C=None)])
def test_null_pointers(kw):
    assert _call(**kw) == capi.SGEMM_STATUS_NULL_POINTER


def test_empty_extents_are_noops():
    # M == 0 or N == 0: OK without launching, even with NULL pointers.
    assert _call(M=0, A=None, C=None) == capi.SGEMM_STATUS_OK
    assert _call(N=0, B=None, C=None) == capi.SGEMM_STATUS_OK
    # K == 0 needs only C (A and B are never read)
    assert capi.sgemm_select_variant(4, 4, 0, None, 1, None, 4, 1.0, AL, 4) >= 0


def test_forced_variant_checks():
    a = GOOD
    args = (a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"], a["ldb"], a["beta"], a["C"],
            a["ldc"], None)
    assert capi.sgemm_ex(*args, capi.sgemm_num_variants()) == capi.SGEMM_STATUS_INVALID_VARIANT
    assert capi.sgemm_ex(*args, -2) == capi.SGEMM_STATUS_INVALID_VARIANT
    # a 128-bit variant forced on misaligned data is refused before launch
    mis = list(args)
    mis[4] = MIS
    assert capi.sgemm_ex(*mis, capi.SGEMM_VARIANT_DB128_VEC) == capi.SGEMM_STATUS_UNSUPPORTED
    odd = list(args)
    odd[5] = 9
    assert capi.sgemm_ex(*odd, capi.SGEMM_VARIANT_DB128_VEC) == capi.SGEMM_STATUS_UNSUPPORTED


def _needs_vec(v):
    return capi.sgemm_variant_info(v)[4] == 1


def _name(v):
    return capi.sgemm_variant_name(v)


@pytest.mark.parametrize("shape,expected", [
    # 128x128 grid of at most 256 tiles: the 64x64x64 tile (split-capable)
    ((4, 4, 4), "lean_64x64x64_w4x1_splitk"),
    ((64, 64, 64), "lean_64x64x64_w4x1_splitk"),
    ((1024, 1024, 64), "lean_64x64x64_w4x1_splitk"),
    ((1024, 1024, 1024), "lean_64x64x64_w4x1_splitk"),
    ((1536, 1536, 1536), "lean_64x64x64_w4x1_splitk"),
    # (half the two-per-CU slots or fewer)
    ((2048, 2048, 2048), "lean_64x64x64_w4x1_splitk"),
    ((2000, 2000, 500), "lean_64x64x64_w4x1_splitk"),
    # last wave of 128x128 tiles fuller than that of 64x64 tiles less 3%
    # (the split-capable form: whole waves launch the plain kernel, a partly
    # filled last wave may split)
    ((4096, 4096, 4096), "lean_128x128x32_w2x2_splitk"),
    ((8192, 8192, 8192), "lean_128x128x32_w2x2_splitk"),
    ((4096, 4000, 100), "lean_128x128x32_w2x2_splitk"),
    ((6000, 6000, 6000), "lean_128x128x32_w2x2_splitk"),
    # short K (at most 256) on at least one full wave of 64x64 tiles: the
    # 32-deep K tile; fewer tiles, or longer K, keep the 64-deep one
    ((2944, 2944, 256), "lean_64x64x32_w4x1_splitk"),
    ((2048, 2048, 128), "lean_64x64x32_w4x1_splitk"),
    ((1536, 1536, 256), "lean_64x64x32_w4x1_splitk"),
    ((1024, 1024, 256), "lean_64x64x64_w4x1_splitk"),
    ((2944, 2944, 512), "lean_64x64x64_w4x1_splitk"),
    ((4096, 4096, 256), "lean_128x128x32_w2x2_splitk"),
    # a partly empty last wave of 128x128 tiles
    ((3072, 3072, 3072), "lean_64x64x64_w4x1_splitk"),
    ((2560, 2560, 2560), "lean_64x64x64_w4x1_splitk"),
    ((1920, 1536, 1024), "lean_64x64x64_w4x1_splitk"),
])
def test_variant_selection_by_shape(shape, expected):
    """Aligned operands take a lean variant chosen by the size of the grid and
    the fill of the last wave of tiles over the 256 CUs."""
    M, N, K = shape
    v = capi.sgemm_select_variant(M, N, K, AL, K, AL, N, 0.0, AL, N)
    assert _name(v) == expected, (shape, _name(v))
    assert _needs_vec(v)


def test_split_factors():
    """K is split only for grids under one full wave of resident blocks (512
    tiles of the variant's own tile), by the factor of least modelled cost
    (busiest CU, operand-traffic floor, a fixed and a per-split cost of the
    hand-off), at most 16, into splits of at least two K tiles, and only
    when that saves at least 5%."""
    names = {capi.sgemm_variant_name(v): v for v in capi.all_variants()}
    v128, v64 = names["lean_128x128x32_w2x2_splitk"], names["lean_64x64x64_w4x1_splitk"]
    f = capi.sgemm_split_factor
    assert f(v128, 1024, 1024, 1024) == 4          # 64 tiles, 32 K tiles: one block per CU
    assert f(v128, 512, 512, 512) == 8             # 16 tiles, 16 K tiles: two K tiles per split
    assert f(v128, 64, 64, 4096) == 16
    assert f(v128, 1536, 1536, 1536) == 3          # 144 tiles
    assert f(v128, 1920, 1536, 1024) == 1          # 180 tiles
    assert f(v128, 1024, 1024, 128) == 1           # 4 K tiles: too few to gain
    assert f(v64, 1024, 1024, 1024) == 1           # 256 tiles of 64x64: every CU busy
    assert f(v64, 512, 512, 2048) == 4             # 64 tiles, 32 K tiles of 64
    assert f(v64, 768, 768, 4096) == 5             # 144 tiles: 720 blocks, three per CU at most
    assert f(v64, 640, 640, 4096) == 5             # 100 tiles: 500 blocks
    assert f(v64, 1152, 1152, 2048) == 3           # 324 tiles
    assert f(v64, 1280, 1280, 2048) == 1           # 400 tiles: too little to gain
    assert f(v64, 1024, 1024, 8192) == 1           # 256 tiles: the operand traffic bounds every S
    assert f(v64, 256, 256, 8192) == 16            # 128 K tiles: eight per split
    assert f(v64, 512, 512, 512) == 4              # 64 tiles, 8 K tiles: two per split
    assert f(v64, 384, 384, 384) == 3              # 36 tiles, 6 K tiles
    assert f(v64, 256, 256, 256) == 1              # 16 tiles, 4 K tiles: the fixed costs eat the gain
    assert f(v64, 1216, 1216, 2048) == 2
    assert f(v64, 2048, 2048, 64) == 1             # whole waves: left to the last-wave split
    for v in (v128, v64):
        for (M, N, K) in [(100, 100, 10000), (300, 200, 500), (1, 1, 100000), (900, 700, 3000)]:
            s = f(v, M, N, K)
            st, bm, bn, bk, _ = capi.sgemm_variant_info(v)
            tiles = -(-M // bm) * -(-N // bn)
            assert 1 <= s <= 16 and (s == 1 or (tiles < 512 and -(-K // bk) >= 2 * s)), (v, M, N, K, s)
    # variants without split-K, bad ids, bad sizes
    assert f(names["lean_128x128x32_w2x2"], 64, 64, 4096) == 1
    assert f(capi.sgemm_num_variants(), 64, 64, 64) == capi.SGEMM_STATUS_INVALID_VARIANT
    assert f(v128, -1, 64, 64) == capi.SGEMM_STATUS_INVALID_DIM


def test_variant_selection_by_alignment():
    """Operands that do not allow 128-bit access take the lean kernel with
    4-byte loads, on the tile the aligned case would use."""
    sel = capi.sgemm_select_variant
    assert _needs_vec(sel(64, 64, 64, AL, 64, AL, 64, 0.0, AL, 64))
    for args in [(MIS, 64, AL, 64, AL, 64), (AL, 64, MIS, 64, AL, 64), (AL, 64, AL, 64, MIS, 64),
                 (AL, 66, AL, 64, AL, 64)]:
        a, lda, b, ldb, c, ldc = args
        assert _name(sel(64, 64, 64, a, lda, b, ldb, 0.0, c, ldc)) == "lean_dw_64x64x64_w4x1_splitk"
    assert _name(sel(4096, 4096, 4095, AL, 4095, AL, 4096, 0.0, AL, 4096)) == "lean_dw_128x128x32_w2x2"
    assert _name(sel(3072, 3072, 3071, AL, 3071, AL, 3072, 0.0, AL, 3072)) == "lean_dw_64x64x64_w4x1_splitk"
    # the ragged workload's leading dimensions (2047, 4999) are not multiples of 4
    assert not _needs_vec(sel(3001, 4999, 2047, AL, 2047, AL, 4999, -0.5, AL, 4999))
    # aligned, padded operands whose K or N is not a multiple of 4: the
    # 16-byte kernels would need whole chunks at the edge
    assert _name(sel(1024, 1024, 1023, AL, 1024, AL, 1024, 0.0, AL, 1024)) == "lean_dw_64x64x64_w4x1_splitk"
    assert _name(sel(4096, 4094, 4096, AL, 4096, AL, 4096, 0.0, AL, 4096)) == "lean_dw_128x128x32_w2x2"
    assert _name(sel(1024, 1024, 1024, AL, 1024, AL, 1024, 0.0, AL, 1024)) == "lean_64x64x64_w4x1_splitk"
    assert sel(-1, 4, 4, AL, 4, AL, 4, 0.0, AL, 4) == capi.SGEMM_STATUS_INVALID_DIM


def test_single_hip_runtime_in_process():
    """Loading the library must not bring in a second HIP runtime next to the
    one PyTorch ships (same soname, different build): the binding imports
    torch first, so exactly one libamdhip64 is mapped and it is torch's."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from fp32_sgemm_tuning_amd import capi\n"
            "capi.load()\n"
            "import torch, os\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(paths)); print(list(paths)[0]); print(os.path.dirname(torch.__file__))\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    n, path, torch_dir = r.stdout.split("\n")[:3]
    assert n == "1", r.stdout
    assert os.path.realpath(path).startswith(os.path.realpath(torch_dir)), (path, torch_dir)


def _op(fn, op_a, op_b, M, N, K, lda, ldb, ldc, A=AL, B=AL, C=AL, batch=None, strides=(0, 0, 0)):
    if batch is None:
        return fn(op_a, op_b, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, None)
    sa, sb, sc = strides
    return fn(op_a, op_b, M, N, K, 1.0, A, lda, sa, B, ldb, sb, 0.0, C, ldc, sc, batch, None)


N_, T_ = capi.SGEMM_OP_N, capi.SGEMM_OP_T


@pytest.mark.parametrize("op_a,op_b,lda,ldb,ok", [
    # row-major: lda >= K (or M when A is transposed), ldb >= N (or K)
    (N_, N_, 7, 5, True), (N_, N_, 6, 5, False), (N_, N_, 7, 4, False),
    (T_, N_, 3, 5, True), (T_, N_, 2, 5, False),
    (N_, T_, 7, 7, True), (N_, T_, 7, 6, False),
    (T_, T_, 3, 7, True),
])
def test_op_leading_dimension_checks(op_a, op_b, lda, ldb, ok):
    """M = 3, N = 5, K = 7: the required leading dimensions follow the stored
    shape of each operand.  Invalid calls return before any HIP call; the
    valid ones are not run here (no GPU), only the invalid ones are."""
    if not ok:
        assert _op(capi.sgemm_op, op_a, op_b, 3, 5, 7, lda, ldb, 5) == capi.SGEMM_STATUS_INVALID_DIM


def test_op_codes_and_batches():
    assert _op(capi.sgemm_op, 2, N_, 3, 5, 7, 7, 5, 5) == capi.SGEMM_STATUS_INVALID_OP
    assert _op(capi.sgemm_op, N_, -1, 3, 5, 7, 7, 5, 5) == capi.SGEMM_STATUS_INVALID_OP
    sb = capi.sgemm_strided_batched
    # empty batches and empty extents are no-ops, even with NULL pointers
    assert _op(sb, N_, N_, 3, 5, 7, 7, 5, 5, batch=0, A=None, B=None, C=None) == capi.SGEMM_STATUS_OK
    assert _op(sb, T_, N_, 0, 5, 7, 1, 5, 5, batch=3, A=None, C=None) == capi.SGEMM_STATUS_OK
    # negative batch, too large a batch, overlapping C problems, negative strides
    assert _op(sb, N_, N_, 3, 5, 7, 7, 5, 5, batch=-1) == capi.SGEMM_STATUS_INVALID_DIM
    assert _op(sb, N_, N_, 3, 5, 7, 7, 5, 5, batch=65536) == capi.SGEMM_STATUS_INVALID_DIM
    assert _op(sb, N_, N_, 3, 5, 7, 7, 5, 5, batch=2, strides=(21, 35, 14)) == capi.SGEMM_STATUS_INVALID_DIM
    assert _op(sb, N_, N_, 3, 5, 7, 7, 5, 5, batch=2, strides=(-21, 35, 15)) == capi.SGEMM_STATUS_INVALID_DIM
    assert _op(sb, N_, N_, 3, 5, 7, 7, 5, 5, batch=2, strides=(21, 35, 15), C=None) == \
        capi.SGEMM_STATUS_NULL_POINTER


@pytest.mark.parametrize("op_a,op_b,lda,ldb,ldc,ok", [
    # column-major: lda >= M (or K when transposed), ldb >= K (or N), ldc >= M
    (N_, N_, 3, 7, 3, True), (N_, N_, 2, 7, 3, False), (N_, N_, 3, 6, 3, False), (N_, N_, 3, 7, 2, False),
    (T_, N_, 7, 7, 3, True), (T_, N_, 6, 7, 3, False),
    (N_, T_, 3, 5, 3, True), (N_, T_, 3, 4, 3, False),
])
def test_column_major_leading_dimension_checks(op_a, op_b, lda, ldb, ldc, ok):
    if not ok:
        assert _op(capi.sgemm_cm, op_a, op_b, 3, 5, 7, lda, ldb, ldc) == capi.SGEMM_STATUS_INVALID_DIM


def test_lowp_argument_checks():
    """The 16-bit-input entry point: type code first, then the checks of sgemm()."""
    f = capi.sgemm_lowp
    bf, hf = capi.SGEMM_DTYPE_BF16, capi.SGEMM_DTYPE_F16
    for bad in (0, 3, -1):
        assert f(bad, 8, 8, 8, 1.0, AL, 8, AL, 8, 0.0, AL, 8, None) == capi.SGEMM_STATUS_INVALID_DTYPE
    assert f(bf, -1, 8, 8, 1.0, AL, 8, AL, 8, 0.0, AL, 8, None) == capi.SGEMM_STATUS_INVALID_DIM
    assert f(bf, 8, 8, 8, 1.0, AL, 7, AL, 8, 0.0, AL, 8, None) == capi.SGEMM_STATUS_INVALID_DIM
    assert f(hf, 8, 8, 8, 1.0, AL, 8, AL, 7, 0.0, AL, 8, None) == capi.SGEMM_STATUS_INVALID_DIM
    assert f(hf, 8, 8, 8, 1.0, AL, 8, AL, 8, 0.0, AL, 7, None) == capi.SGEMM_STATUS_INVALID_DIM
    assert f(bf, 8, 8, 8, 1.0, None, 8, AL, 8, 0.0, AL, 8, None) == capi.SGEMM_STATUS_NULL_POINTER
    assert f(bf, 8, 8, 8, 1.0, AL, 8, AL, 8, 0.0, None, 8, None) == capi.SGEMM_STATUS_NULL_POINTER
    # empty extents: OK without launching, even with NULL pointers
    assert f(hf, 0, 8, 8, 1.0, None, 8, None, 8, 0.0, None, 8, None) == capi.SGEMM_STATUS_OK
    assert f(bf, 8, 0, 8, 1.0, None, 8, None, 1, 0.0, None, 1, None) == capi.SGEMM_STATUS_OK


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_16bit_inputs_are_16bit_values(dtype):
    """The 16-bit-input problems hold values that the 16-bit type represents
    exactly (a round trip through torch's conversion changes nothing)."""
    import numpy as np
    import torch
    from fp32_sgemm_tuning_amd.inputs import make_problem, make_problem_16bit
    A, B, C = make_problem_16bit(33, 17, 65, seed=1, dtype=dtype, dist="normal", with_c=True)
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    for x in (A, B):
        assert x.dtype == np.float32
        assert np.array_equal(torch.from_numpy(x).to(t).float().numpy(), x)
    A32, B32, C32 = make_problem(33, 17, 65, seed=1, dist="normal", with_c=True)
    assert np.array_equal(C, C32)
    # the 16-bit values are the FP32 draws to within the type's precision
    rel = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -10
    assert np.all(np.abs(A - A32) <= rel * np.abs(A32) + 2.0 ** -24)


def test_lowp_variants_and_selection():
    """Forced 16-bit variants: unknown ids and operands outside a variant's
    fast path are refused before anything is enqueued; the automatic choice
    takes the plain kernel for shapes the fast kernels do not take."""
    bf = capi.SGEMM_DTYPE_BF16
    ids = capi.lowp_variants()
    assert len(ids) >= 2 and capi.sgemm_lowp_variant_name(0).startswith("lowp_simple")
    assert capi.sgemm_lowp_variant_name(len(ids)) is None and capi.sgemm_lowp_variant_name(-1) is None
    ex = capi.sgemm_lowp_ex
    assert ex(bf, 64, 64, 64, 1.0, AL, 64, AL, 64, 0.0, AL, 64, None, len(ids)) == capi.SGEMM_STATUS_INVALID_VARIANT
    assert ex(bf, 64, 64, 64, 1.0, AL, 64, AL, 64, 0.0, AL, 64, None, -2) == capi.SGEMM_STATUS_INVALID_VARIANT
    for v in ids[1:]:
        # K below one K tile, K or N not a multiple of 8, misaligned A, odd lda
        for M, N, K, A, lda, ldb in ((64, 64, 16, AL, 16, 64), (64, 64, 100, AL, 100, 64), (64, 60, 64, AL, 64, 60),
                                     (64, 64, 64, AL + 2, 64, 64), (64, 64, 64, AL, 68, 64)):
            assert ex(bf, M, N, K, 1.0, A, lda, AL, ldb, 0.0, AL, N, None, v) == capi.SGEMM_STATUS_UNSUPPORTED
    sel = capi.sgemm_lowp_select_variant
    assert sel(64, 64, 16, AL, 16, AL, 64) == 0
    assert capi.sgemm_lowp_variant_name(sel(64, 64, 32, AL, 32, AL, 64)).endswith(
        ("x32_s4", "x32_s4_alt", "simple_64x64"))
    assert sel(3001, 4999, 2047, AL, 2047, AL, 4999) == 0
    assert sel(4096, 4096, 4096, AL, 4096, AL, 4096) > 0
    assert sel(4096, 4096, 4096, AL + 2, 4096, AL, 4096) == 0
    assert sel(-1, 4, 4, AL, 4, AL, 4) == capi.SGEMM_STATUS_INVALID_DIM


def test_lowp_split_factors():
    """16-bit split-K: only the 128x128 kernel splits; small grids with long K
    split, full grids and short K do not; the factor respects the slots and
    the 64 MiB workspace."""
    f = capi.sgemm_lowp_split_factor
    names = {capi.sgemm_lowp_variant_name(v): v for v in capi.lowp_variants()}
    v128, valt, v256x128 = names["lowp_128x128x64_s2"], names["lowp_256x256x32_s4_alt"], names["lowp_256x128x64_s3"]
    assert f(v128, 2048, 2048, 8192) == 2          # 256 tiles in 512 slots, long K
    assert f(v128, 1024, 1024, 8192) == 8
    assert f(v128, 4096, 4096, 4096) == 1          # a full grid
    assert f(v128, 512, 512, 256) == 1             # 4 K tiles: too short to split
    for v in (valt, v256x128):                     # no split-K form
        assert f(v, 2048, 2048, 8192) == 1 and f(v, 256, 256, 65536) == 1
    for M, N, K in ((2048, 2048, 8192), (512, 512, 65536), (256, 256, 4096), (1000, 3000, 5000), (64, 64, 1 << 20)):
        s = f(v128, M, N, K)
        tiles = -(-M // 128) * -(-N // 128)
        assert 1 <= s <= 16
        assert s == 1 or (s * tiles <= 512 and s * tiles * 128 * 128 * 4 <= 64 << 20 and -(-K // 64) >= 8 * s)
    assert f(len(names), 8, 8, 8) == capi.SGEMM_STATUS_INVALID_VARIANT
    assert f(v128, -1, 8, 8) == capi.SGEMM_STATUS_INVALID_DIM


def test_tail_split_plan():
    """A grid of whole waves (512 workgroup slots) plus a partly filled last
    wave runs as two launches, the last wave's tiles with K split (at least
    three K tiles per split), where the cost model says that saves 5%: the
    plans measured faster split (1536^3, 2560x2624x2560) split, those
    measured slower (1550x1572x1000, 2944^2 x 256) do not; the
    any-alignment 64x64 kernel too."""
    names = {capi.sgemm_variant_name(v): v for v in capi.all_variants()}
    v64, v128 = names["lean_64x64x64_w4x1_splitk"], names["lean_128x128x32_w2x2_splitk"]
    t = capi.sgemm_tail_split
    assert t(v64, 1536, 1536, 1536) == (4, 64)      # 576 tiles = 512 + 64
    assert t(v64, 2560, 2624, 2560) == (2, 104)     # 1640 tiles = 3 waves + 104
    assert t(v64, 1550, 1572, 1000) == (1, 0)       # 625 tiles, 16 K tiles: too short to gain
    assert t(v64, 1550, 1570, 1000) == (1, 0)       # N not a multiple of 4: no lean kernel
    assert t(v128, 2944, 2944, 256) == (1, 0)       # 529 tiles, 8 K tiles: too short
    assert t(v128, 3072, 3072, 3072) == (4, 64)     # 576 tiles of 128x128, 96 K tiles
    assert t(v64, 2048, 2048, 2048) == (1, 0)       # whole waves
    assert t(v128, 4096, 4096, 4096) == (1, 0)
    assert t(v128, 6016, 6016, 6016) == (3, 161)    # 2209 tiles of 128x128, 188 K tiles
    assert t(v128, 7744, 7744, 7744) == (5, 137)
    assert t(v64, 1664, 1664, 1664) == (1, 0)       # 676 tiles: last wave a third full
    assert t(v64, 1600, 1600, 1600) == (2, 113)     # 625 tiles: 113 left, 25 K tiles
    assert t(v64, 1792, 1792, 1792) == (1, 0)       # 784 tiles: last wave over half full
    assert t(v64, 2944, 2944, 128) == (1, 0)        # 2116 tiles, 2 K tiles
    assert t(v64, 512, 512, 4096) == (1, 0)         # a small grid splits K as a whole instead
    assert t(v64, 1536, 1536, 64) == (1, 0)         # one K tile
    assert t(names["lean_64x64x64_w4x1"], 1536, 1536, 1536) == (1, 0)   # no split-K form
    vdw = names["lean_dw_64x64x64_w4x1_splitk"]
    assert t(vdw, 1535, 1537, 1535) == (2, 88)      # 600 tiles = 1 wave + 88
    assert t(vdw, 3001, 4999, 2047) == (1, 0)       # 3713 tiles = 7 waves + 129: two per CU would remain
    assert t(vdw, 1536, 1536, 1535) == (4, 64)      # K not a multiple of 4: the 4-byte kernel takes it
    assert t(len(names), 8, 8, 8)[0] == capi.SGEMM_STATUS_INVALID_VARIANT
    assert t(v64, -1, 8, 8)[0] == capi.SGEMM_STATUS_INVALID_DIM
    # the automatic choice at 1536^3 is the split-capable 64x64 kernel
    assert capi.sgemm_variant_name(capi.sgemm_select_variant(1536, 1536, 1536, AL, 1536, AL, 1536, 0.0, AL,
                                                              1536)) == "lean_64x64x64_w4x1_splitk"


def test_lowp_op_argument_checks():
    """Transposed 16-bit operands: op codes, the leading dimensions of the
    stored operands, and variants not built for transposes."""
    f = capi.sgemm_lowp_op
    bf, T, N_ = capi.SGEMM_DTYPE_BF16, capi.SGEMM_OP_T, capi.SGEMM_OP_N
    auto = capi.SGEMM_VARIANT_AUTO
    assert f(bf, 2, N_, 8, 8, 8, 1.0, AL, 8, AL, 8, 0.0, AL, 8, None, auto) == capi.SGEMM_STATUS_INVALID_OP
    assert f(9, T, N_, 8, 8, 8, 1.0, AL, 8, AL, 8, 0.0, AL, 8, None, auto) == capi.SGEMM_STATUS_INVALID_DTYPE
    # A stored K x M: lda >= M; B stored N x K: ldb >= K
    assert f(bf, T, N_, 16, 8, 4, 1.0, AL, 15, AL, 8, 0.0, AL, 8, None, auto) == capi.SGEMM_STATUS_INVALID_DIM
    assert f(bf, N_, T, 8, 8, 16, 1.0, AL, 16, AL, 15, 0.0, AL, 8, None, auto) == capi.SGEMM_STATUS_INVALID_DIM
    assert f(bf, T, T, 8, 8, 8, 1.0, None, 8, AL, 8, 0.0, AL, 8, None, auto) == capi.SGEMM_STATUS_NULL_POINTER
    assert f(bf, T, T, 0, 8, 8, 1.0, None, 1, None, 8, 0.0, None, 8, None, auto) == capi.SGEMM_STATUS_OK
    names = {capi.sgemm_lowp_variant_name(v): v for v in capi.lowp_variants()}
    for n in ("lowp_128x128x64_s2", "lowp_256x128x64_s3", "lowp_256x256x32_s4"):
        assert f(bf, T, N_, 256, 256, 256, 1.0, AL, 256, AL, 256, 0.0, AL, 256, None, names[n]) == \
            capi.SGEMM_STATUS_UNSUPPORTED
    assert f(bf, T, N_, 256, 256, 256, 1.0, AL, 256, AL, 256, 0.0, AL, 256, None, len(names)) == \
        capi.SGEMM_STATUS_INVALID_VARIANT


def test_header_constants_match_binding():
    """The limits the header states for the library's kept device memory are
    the binding's (the C side asserts its own at compile time)."""
    text = open(HEADER).read()
    for name in ("SGEMM_WORKSPACE_BYTES", "SGEMM_MAX_STREAM_WORKSPACES", "SGEMM_MAX_COPY_BUFFERS",
                 "SGEMM_MAX_COPY_BUFFER_BYTES", "SGEMM_NOALLOC_SCRATCH_BYTES"):
        m = re.search(r"#define\s+%s\s+(.+?)(?:/\*|$)" % name, text, flags=re.M)
        assert m, name
        value = eval(m.group(1).replace("ll", ""), {})
        assert value == getattr(capi, name), (name, value)
