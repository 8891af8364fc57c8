"""GPU write-footprint checks: every kernel path writes exactly the M x N
outputs of C and nothing around them.

C lives in a buffer filled with a canary value: guard bands before and after
it, the padding columns [N, ldc) of every row and, in strided batches, the
gap between problems.  After a call every canary must be intact and C must
match the fp64 oracle element by element.  The cases cover the automatic
choice on the paths it takes (16-byte and 4-byte lean kernels, split-K, the
last-wave split), every lean and split-K variant forced, and the 16-bit
kernels, including the path that copies unaligned 16-bit operands into
zero-padded buffers and runs the fast kernels with the true N (N not a
multiple of 4, C rows 16-byte aligned).
"""
import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import capi, sgemm, sgemm_lowp
from fp32_sgemm_tuning_amd.inputs import make_problem, make_problem_16bit
from gpu_util import check_close, padded_device, torch_cuda

pytestmark = pytest.mark.gpu

CANARY = -12345.0
GUARD = 1024


def canary_c(torch, Cin, ldc, batch=1, sC=None):
    """C (batch x M x N view, strides sC, ldc, 1) inside a canary-filled
    buffer with guard bands; Cin (M x N, or batch x M x N) copied in.
    Returns (buffer, view, mask of the elements C covers)."""
    M, N = Cin.shape[-2:]
    sC = M * ldc if sC is None else sC
    span = (batch - 1) * sC + (M - 1) * ldc + N
    total = 2 * GUARD + span
    buf = torch.full((total,), CANARY, dtype=torch.float32, device="cuda")
    C = torch.as_strided(buf, (batch, M, N), (sC, ldc, 1), GUARD)
    src = np.broadcast_to(Cin, (batch, M, N))
    for z in range(batch):
        C[z].copy_(torch.from_numpy(np.ascontiguousarray(src[z])))
    starts = GUARD + np.add.outer(np.arange(batch) * sC, np.arange(M) * ldc).ravel()
    mask = np.zeros(total, bool)
    idx = np.add.outer(starts, np.arange(N)).ravel()
    mask[idx] = True
    return buf, C, mask


def assert_canaries(buf, mask, what):
    host = buf.cpu().numpy()
    bad = np.flatnonzero((host != CANARY) & ~mask)
    if bad.size:
        raise AssertionError(f"{what}: {bad.size} elements outside C were written; first at buffer offset "
                             f"{int(bad[0]) - GUARD} from C's base (value {host[bad[0]]!r})")


def _names():
    try:
        return {capi.sgemm_variant_name(v): v for v in capi.all_variants()}
    except capi.LibraryMissing:      # collection without a built library
        return {}


NAMES = _names()
LEAN = sorted(v for n, v in NAMES.items() if n.startswith("lean_"))

# (M, N, K, ldc, what the automatic choice does there)
AUTO_CASES = [
    (130, 133, 70, 140, "4-byte lean kernel, N and K not multiples of 4"),
    (255, 129, 257, 132, "4-byte lean kernel"),
    (197, 260, 1028, 268, "16-byte lean kernel, ragged M, K remainder"),
    (1000, 1000, 1000, 1012, "16-byte 64x64 kernel, split K"),
    (509, 515, 8191, 520, "4-byte 64x64 kernel, split K"),
    (1536, 1532, 1000, 1540, "last wave split into a second launch"),
    (1535, 1537, 1535, 1540, "4-byte kernel, last wave split"),
    (4095, 4092, 256, 4096, "16-byte 128x128 kernel, ragged M and N"),
]


@pytest.mark.parametrize("M,N,K,ldc,what", AUTO_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in AUTO_CASES])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (-0.5, 1.5)], ids=["b0", "b1"])
def test_auto_footprint(M, N, K, ldc, what, ab):
    torch = torch_cuda()
    alpha, beta = ab
    print(f"[canary] auto {M}x{N}x{K} ldc={ldc} ({what}) beta={beta}", flush=True)
    A, B, Cin = make_problem(M, N, K, seed=M + 5 * N + K, dist="normal", with_c=True)
    dA, _ = padded_device(A, (K + 3) // 4 * 4, torch)
    dB, _ = padded_device(B, (N + 3) // 4 * 4, torch)
    buf, C, mask = canary_c(torch, Cin, ldc)
    sgemm(dA, dB, C[0], alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    assert_canaries(buf, mask, f"auto {M}x{N}x{K}")
    ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
    check_close(C[0].cpu().numpy(), ref, f"auto {M}x{N}x{K} beta={beta}")


@pytest.mark.parametrize("variant", LEAN, ids=lambda v: capi.sgemm_variant_name(v))
@pytest.mark.parametrize("shape", [(197, 260, 1028), (130, 260, 2000), (64, 68, 64)],
                         ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_lean_variant_footprint(variant, shape):
    """Every lean variant forced (its split-K form splits where the model
    says so), ragged M and N with K and N multiples of 4, padded ldc."""
    torch = torch_cuda()
    M, N, K = shape
    A, B, Cin = make_problem(M, N, K, seed=2 * M + N + K, dist="normal", with_c=True)
    dA, _ = padded_device(A, K + 4, torch)
    dB, _ = padded_device(B, N + 4, torch)
    buf, C, mask = canary_c(torch, Cin, N + 8)
    sgemm(dA, dB, C[0], alpha=0.75, beta=-1.25, variant=variant)
    torch.cuda.synchronize()
    name = capi.sgemm_variant_name(variant)
    assert_canaries(buf, mask, f"{name} {shape}")
    check_close(C[0].cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=0.75, beta=-1.25), f"{name} {shape}")


TAIL_FORCED = [(3072, 3072, 3072, "lean_128x128x32_w2x2_splitk"), (1600, 1600, 1600, "lean_64x64x64_w4x1_splitk")]


@pytest.mark.parametrize("M,N,K,name", TAIL_FORCED, ids=[c[3] for c in TAIL_FORCED])
def test_tail_split_footprint(M, N, K, name):
    torch = torch_cuda()
    v = NAMES[name]
    assert capi.sgemm_tail_split(v, M, N, K)[0] > 1
    A, B, Cin = make_problem(M, N, K, seed=M + N, dist="normal", with_c=True)
    dA, _ = padded_device(A, K, torch)
    dB, _ = padded_device(B, N, torch)
    buf, C, mask = canary_c(torch, Cin, N + 12)
    sgemm(dA, dB, C[0], alpha=1.5, beta=0.5, variant=v)
    torch.cuda.synchronize()
    assert_canaries(buf, mask, f"{name} {M}x{N}x{K}")
    check_close(C[0].cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=1.5, beta=0.5), f"{name} {M}x{N}x{K}")


def _dev16(torch, x, dtype, ld):
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    rows, cols = x.shape
    buf = torch.full((rows * ld + 16,), float("nan"), dtype=t, device="cuda")
    view = buf[:rows * ld].view(rows, ld)[:, :cols]
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)).to(t))
    return view


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ldc", [1000, 1004])
def test_lowp_copied_n_not_multiple_of_4(dtype, ldc):
    """Unaligned 16-bit operands are copied and the fast kernel runs with
    N = 999 on 16-byte aligned C rows: the last vector of every row straddles
    N, and no column past N may be written."""
    torch = torch_cuda()
    M, N, K = 1001, 999, 1003
    A, B, Cin = make_problem_16bit(M, N, K, seed=5, dtype=dtype, dist="normal", with_c=True)
    dA, dB = _dev16(torch, A, dtype, K), _dev16(torch, B, dtype, N)
    assert capi.sgemm_lowp_select_variant(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N) == 0
    for alpha, beta in ((1.0, 0.0), (1.25, -0.75)):
        print(f"[canary] lowp copied {dtype} {M}x{N}x{K} ldc={ldc} beta={beta}", flush=True)
        buf, C, mask = canary_c(torch, Cin, ldc)
        assert C.data_ptr() % 16 == 0
        sgemm_lowp(dA, dB, C[0], alpha=alpha, beta=beta)
        torch.cuda.synchronize()
        assert_canaries(buf, mask, f"lowp copied {dtype} ldc={ldc} beta={beta}")
        ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
        check_close(C[0].cpu().numpy(), ref, f"lowp copied {dtype} ldc={ldc} beta={beta}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("gap", [0, 1])
def test_lowp_batched_copied_footprint(dtype, gap):
    """A strided batch of copied 16-bit problems with N = 999 and C problems
    packed back to back (stride (M-1)*ldc + N, plus `gap` canaries): with
    gap 1 every problem's C is 16-byte aligned; with gap 0 problem 4 is, and
    it is the last, so a store past its N lands in the guard band."""
    torch = torch_cuda()
    M, N, K, ldc, batch = 257, 999, 1003, 1000, 5
    sC = (M - 1) * ldc + N + gap
    A, B, Cin = make_problem_16bit(M, N, K, seed=9, dtype=dtype, dist="normal", with_c=True)
    # a different A per problem: A scaled by powers of two stays exact
    A3 = np.stack([A * s for s in (1.0, 2.0, -1.0, 4.0, -2.0)]).astype(np.float32)
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    dA = torch.from_numpy(A3).to(t).cuda()
    assert np.array_equal(dA.float().cpu().numpy(), A3)
    dB = _dev16(torch, B, dtype, N)
    buf, C, mask = canary_c(torch, Cin, ldc, batch=batch, sC=sC)
    print(f"[canary] lowp batched copied {dtype} gap={gap}", flush=True)
    sgemm_lowp(dA, dB.unsqueeze(0), C, alpha=0.5, beta=2.0)
    torch.cuda.synchronize()
    assert_canaries(buf, mask, f"lowp batched copied {dtype} gap={gap}")
    got = C.cpu().numpy()
    for z in range(batch):
        check_close(got[z], oracle.sgemm_ref(A3[z], B, Cin, alpha=0.5, beta=2.0), f"problem {z}")


LOWP_FAST = [(200, 136, 256), (129, 264, 72), (300, 520, 1000)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", LOWP_FAST, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_lowp_variant_footprint(dtype, shape):
    """Every 16-bit variant forced on ragged tiles with padded, aligned C."""
    torch = torch_cuda()
    M, N, K = shape
    A, B, Cin = make_problem_16bit(M, N, K, seed=M + N, dtype=dtype, dist="normal", with_c=True)
    dA, dB = _dev16(torch, A, dtype, K), _dev16(torch, B, dtype, N)
    ref = oracle.sgemm_ref(A, B, Cin, alpha=-1.0, beta=0.25)
    for v in capi.lowp_variants():
        buf, C, mask = canary_c(torch, Cin, N + 4)
        sgemm_lowp(dA, dB, C[0], alpha=-1.0, beta=0.25, variant=v)
        torch.cuda.synchronize()
        what = f"lowp {dtype} {capi.sgemm_lowp_variant_name(v)} {shape}"
        assert_canaries(buf, mask, what)
        check_close(C[0].cpu().numpy(), ref, what)
