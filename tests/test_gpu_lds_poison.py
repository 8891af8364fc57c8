"""Race check: the parity shapes through the race-check build of the library
(libsgemm_poison.so), whose lean FP32 and 16-bit kernels fill every LDS
stage with NaN bits as soon as its last reader has passed the barrier that
frees it (before the direct loads that refill it are issued) and hold the
split-K ticket word at an invalid value between its two barriers.  A
missing or misplaced barrier then makes a wave read NaN or a wrong ticket,
so the result goes wrong whatever the timing.  Every case is compared with
the fp64 oracle and, bit for bit, with the normal build on the same inputs.
"""
import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import capi
from fp32_sgemm_tuning_amd.inputs import make_problem, make_problem_16bit
from gpu_util import check_close, padded_device, torch_cuda

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 1, 1), (7, 5, 3), (64, 64, 64), (127, 129, 31), (128, 128, 32), (129, 127, 33), (256, 384, 96),
    (300, 200, 500), (131, 517, 1029), (256, 256, 64), (256, 512, 128), (512, 768, 320), (200, 300, 256),
    (17, 260, 320), (520, 772, 192), (256, 256, 100), (130, 200, 36), (300, 260, 1028), (256, 128, 68),
]
# the automatic choice where it splits K or the last wave of tiles
SPLIT_SHAPES = [(256, 256, 16384), (640, 640, 4096), (767, 767, 4095), (509, 515, 8191), (1536, 1532, 1000),
                (1535, 1537, 1535)]


def _lib():
    try:
        return capi.open_library(capi.POISON_LIB_PATH)
    except capi.LibraryMissing:
        pytest.fail("libsgemm_poison.so is not built")


def _names():
    try:
        return {capi.sgemm_variant_name(v): v for v in capi.all_variants()}
    except capi.LibraryMissing:      # collection without a built library
        return {}


LEAN = ["auto"] + sorted(n for n in _names() if n.startswith("lean_"))


def _up4(n):
    return max(4, (n + 3) // 4 * 4)


def _fp32_case(torch, P, variant, M, N, K, alpha, beta, seed):
    A, B, Cin = make_problem(M, N, K, seed=seed, dist="normal", with_c=True)
    dA, _ = padded_device(A, _up4(K), torch)
    dB, _ = padded_device(B, _up4(N), torch)
    h = torch.cuda.current_stream().cuda_stream
    outs = []
    for lib in (P, capi.load()):
        dC, _ = padded_device(Cin, _up4(N), torch)
        if beta == 0.0:
            dC.fill_(float("nan"))
        args = (M, N, K, alpha, dA.data_ptr(), _up4(K), dB.data_ptr(), _up4(N), beta, dC.data_ptr(), _up4(N), h)
        st = lib.sgemm(*args) if variant is None else lib.sgemm_ex(*args, variant)
        assert st == 0, capi.sgemm_strerror(st)
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
    ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
    check_close(outs[0], ref, f"poisoned {variant} {M}x{N}x{K} beta={beta}")
    assert np.array_equal(outs[0], outs[1]), f"poisoned build differs from the normal one: {M}x{N}x{K}"


@pytest.mark.parametrize("name", LEAN)
@pytest.mark.parametrize("ab", [(1.0, 0.0), (1.5, -0.5)], ids=["b0", "b1"])
def test_lean_variants_poisoned(name, ab):
    torch = torch_cuda()
    P = _lib()
    variant = None if name == "auto" else _names()[name]
    print(f"[poison] {name} {ab}", flush=True)
    for M, N, K in SHAPES:
        _fp32_case(torch, P, variant, M, N, K, ab[0], ab[1], seed=M * 7 + N * 3 + K)


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_split_and_tail_poisoned(shape):
    """Split-K (ticket word included) and the last-wave split, automatic
    choice, with beta = 0 over NaN C and beta != 0."""
    torch = torch_cuda()
    P = _lib()
    M, N, K = shape
    for alpha, beta in ((1.0, 0.0), (0.5, -1.5)):
        _fp32_case(torch, P, None, M, N, K, alpha, beta, seed=M + 2 * N + K)


LOWP_SHAPES = [(128, 128, 64), (256, 256, 192), (200, 136, 256), (129, 264, 72), (300, 520, 1000),
               (512, 384, 192), (1024, 1024, 2048)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ops", ["NN", "TN", "NT", "TT"])
def test_lowp_poisoned(dtype, ops):
    """Every 16-bit variant (the alternating kernels for transposed
    operands), forced, on whole and ragged tiles and a split-K grid."""
    torch = torch_cuda()
    P = _lib()
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    code = capi.SGEMM_DTYPE_BF16 if dtype == "bf16" else capi.SGEMM_DTYPE_F16
    ta, tb = ops[0] == "T", ops[1] == "T"
    variants = [v for v in capi.lowp_variants() if v > 0 and (ops == "NN" or v in (4, 5))]
    h = torch.cuda.current_stream().cuda_stream
    for M, N, K in LOWP_SHAPES:
        if ta and M % 8:             # a transposed A needs M in whole 16-byte chunks
            continue
        A, B, Cin = make_problem_16bit(M, N, K, seed=M + N + K, dtype=dtype, dist="normal", with_c=True)
        dA = torch.from_numpy(np.ascontiguousarray(A.T if ta else A)).to(t).cuda()
        dB = torch.from_numpy(np.ascontiguousarray(B.T if tb else B)).to(t).cuda()
        lda, ldb = (M if ta else K), (K if tb else N)
        ref = oracle.sgemm_ref(A, B, Cin, alpha=-1.25, beta=0.5)
        for v in variants:
            outs = []
            for lib in (P, capi.load()):
                dC = torch.from_numpy(Cin).cuda()
                st = lib.sgemm_lowp_op(code, int(ta), int(tb), M, N, K, -1.25, dA.data_ptr(), lda, dB.data_ptr(),
                                       ldb, 0.5, dC.data_ptr(), N, h, v)
                assert st == 0, (v, capi.sgemm_strerror(st))
                torch.cuda.synchronize()
                outs.append(dC.cpu().numpy())
            what = f"poisoned lowp {dtype} {ops} {capi.sgemm_lowp_variant_name(v)} {M}x{N}x{K}"
            check_close(outs[0], ref, what)
            assert np.array_equal(outs[0], outs[1]), what + ": differs from the normal build"


@pytest.mark.parametrize("ops", ["TN", "NT", "TT"])
@pytest.mark.parametrize("shape", [(512, 512, 4096), (516, 772, 4100), (1536, 1536, 1536)],
                         ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_transposed_split_poisoned(ops, shape):
    """Transposed operands on grids that split K (the first two) or the last
    wave (1536^3), through sgemm_op, beta != 0."""
    torch = torch_cuda()
    P = _lib()
    M, N, K = shape
    ta, tb = ops[0] == "T", ops[1] == "T"
    A, B, Cin = make_problem(M, N, K, seed=M + 5 * N + K, dist="normal", with_c=True)
    dA = torch.from_numpy(np.ascontiguousarray(A.T if ta else A)).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B.T if tb else B)).cuda()
    lda, ldb = (M if ta else K), (K if tb else N)
    h = torch.cuda.current_stream().cuda_stream
    outs = []
    for lib in (P, capi.load()):
        dC = torch.from_numpy(Cin).cuda()
        st = lib.sgemm_op(int(ta), int(tb), M, N, K, 0.75, dA.data_ptr(), lda, dB.data_ptr(), ldb, -0.5,
                          dC.data_ptr(), N, h)
        assert st == 0, capi.sgemm_strerror(st)
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
    what = f"poisoned transposed split {ops} {M}x{N}x{K}"
    check_close(outs[0], oracle.sgemm_ref(A, B, Cin, alpha=0.75, beta=-0.5), what)
    assert np.array_equal(outs[0], outs[1]), what + ": differs from the normal build"
