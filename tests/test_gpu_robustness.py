"""GPU robustness: guard bands around C stay untouched, padding columns of C
(j in [N, ldc)) are never written, work on a non-default stream is ordered on
that stream, repeated calls give identical bits, and error statuses surface
as exceptions without writing anything."""
import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import SgemmError, capi, sgemm
from fp32_sgemm_tuning_amd.inputs import make_problem
from gpu_util import check_close, padded_device, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

CANARY = -12345.0


@pytest.mark.parametrize("variant", [capi.SGEMM_VARIANT_SIMPLE, capi.SGEMM_VARIANT_DB128_VEC,
                                     capi.SGEMM_VARIANT_DB128_SCALAR])
@pytest.mark.parametrize("shape", [(130, 133, 70), (255, 129, 257), (1, 1, 5)])
def test_guard_bands_and_ldc_padding(variant, shape):
    torch = torch_cuda()
    M, N, K = shape
    ldc = (N + 4 + 3) // 4 * 4          # padded, still a multiple of 4
    guard = 1024
    A, B, Cin = make_problem(M, N, K, 41, dist="normal", with_c=True)
    dA, _ = padded_device(A, (K + 3) // 4 * 4, torch)
    dB, _ = padded_device(B, (N + 3) // 4 * 4, torch)
    buf = torch.full((2 * guard + M * ldc,), CANARY, dtype=torch.float32, device="cuda")
    C = buf[guard:guard + M * ldc].view(M, ldc)[:, :N]
    C.copy_(to_dev(Cin, torch))
    sgemm(dA, dB, C, alpha=0.5, beta=1.5, variant=variant)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:guard] == CANARY), "write before C"
    assert np.all(host[guard + M * ldc:] == CANARY), "write after C"
    assert np.all(host[guard:guard + M * ldc].reshape(M, ldc)[:, N:] == CANARY), "write into ldc padding"
    ref = oracle.sgemm_ref(A, B, Cin, alpha=0.5, beta=1.5)
    check_close(C.cpu().numpy(), ref, "guard-band case")


@pytest.mark.parametrize("variant", list(range(capi.sgemm_num_variants())))
def test_whole_tiles_with_padded_leading_dimensions(variant):
    """Whole 256x256 tiles (so every variant runs its unguarded path) with
    lda, ldb and ldc all larger than the logical width: the kernels must step
    rows by the leading dimensions and leave C's padding and surroundings
    alone."""
    torch = torch_cuda()
    M, N, K = 256, 512, 192
    lda, ldb, ldc = K + 8, N + 4, N + 12
    guard = 1024
    A, B, Cin = make_problem(M, N, K, 43, dist="normal", with_c=True)
    dA, _ = padded_device(A, lda, torch)
    dB, _ = padded_device(B, ldb, torch)
    buf = torch.full((2 * guard + M * ldc,), CANARY, dtype=torch.float32, device="cuda")
    C = buf[guard:guard + M * ldc].view(M, ldc)[:, :N]
    C.copy_(to_dev(Cin, torch))
    sgemm(dA, dB, C, alpha=-0.75, beta=0.25, variant=variant)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:guard] == CANARY), "write before C"
    assert np.all(host[guard + M * ldc:] == CANARY), "write after C"
    assert np.all(host[guard:guard + M * ldc].reshape(M, ldc)[:, N:] == CANARY), "write into ldc padding"
    ref = oracle.sgemm_ref(A, B, Cin, alpha=-0.75, beta=0.25)
    check_close(C.cpu().numpy(), ref, f"whole tiles, padded ld, variant {variant}")


def test_non_default_stream_ordering():
    torch = torch_cuda()
    A, B, _ = make_problem(512, 512, 512, 42)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    s = torch.cuda.Stream()
    C = torch.zeros((512, 512), device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        # make the inputs on this stream, then the GEMM, then a dependent op
        A2 = dA * 2.0
        sgemm(A2, dB, C)
        D = C * 0.5
    s.synchronize()
    ref = oracle.sgemm_ref(A, B)
    check_close(D.cpu().numpy(), ref, "stream-ordered")


def test_explicit_stream_argument():
    torch = torch_cuda()
    A, B, _ = make_problem(300, 200, 100, 43)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    s = torch.cuda.Stream()
    C = torch.empty((300, 200), device="cuda")
    torch.cuda.synchronize()
    sgemm(dA, dB, C, stream=s)
    s.synchronize()
    check_close(C.cpu().numpy(), oracle.sgemm_ref(A, B), "explicit stream")


def test_deterministic_repeats():
    torch = torch_cuda()
    A, B, _ = make_problem(1024, 1024, 1024, 44)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    first = sgemm(dA, dB).clone()
    for _ in range(5):
        again = sgemm(dA, dB)
        torch.cuda.synchronize()
        assert torch.equal(first, again)


def test_errors_raise_and_write_nothing():
    torch = torch_cuda()
    C = torch.full((8, 8), CANARY, device="cuda")
    A = torch.ones((8, 8), device="cuda")
    B = torch.ones((8, 8), device="cuda")
    with pytest.raises(SgemmError) as e:
        sgemm(A, B, C, variant=99)
    assert e.value.status == capi.SGEMM_STATUS_INVALID_VARIANT
    st = capi.sgemm(8, 8, 8, 1.0, A.data_ptr(), 7, B.data_ptr(), 8, 0.0, C.data_ptr(), 8, None)
    assert st == capi.SGEMM_STATUS_INVALID_DIM
    torch.cuda.synchronize()
    assert torch.all(C == CANARY)
