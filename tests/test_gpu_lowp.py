"""GPU parity of the 16-bit-input entry point (sgemm_lowp: BF16 or FP16 A
and B, FP32 accumulation and C) against the fp64 CPU oracle.

Every product of two 16-bit values is exact in FP32, so the operation is the
FP32 GEMM of the same values widened: the oracle receives those values as
float32 arrays and the parity bar is the FP32 one, |C - C_ref| <= 1e-3 +
1e-4 |C_ref| elementwise.  The inputs are drawn as for the FP32 workloads and
made 16-bit values by the input module (bf16: low 16 bits cleared; f16:
rounded); the device copies are those exact values.
"""
import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import SgemmError, capi, sgemm_lowp
from fp32_sgemm_tuning_amd.inputs import make_problem_16bit, sample_indices
from gpu_util import check_close, torch_cuda

pytestmark = pytest.mark.gpu

DTYPES = ["bf16", "f16"]


def _tdtype(torch, dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def _dev16(x, dtype, torch, ld=None, offset=0, fill=float("nan")):
    """Device 16-bit copy of the float32 array x (whose values are 16-bit
    values), inside a buffer with leading dimension ld (padding = fill),
    starting `offset` elements into the allocation."""
    rows, cols = x.shape
    ld = cols if ld is None else ld
    t16 = torch.from_numpy(np.ascontiguousarray(x)).to(_tdtype(torch, dtype))
    assert np.array_equal(t16.float().numpy(), x), "input values are not 16-bit values"
    buf = torch.full((offset + rows * ld + 16,), fill, dtype=_tdtype(torch, dtype), device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(t16.to("cuda"))
    return view, buf


# (M, N, K): fast path (16-byte aligned, lda/ldb/N/K multiples of 8, K >= 64)
# with whole tiles, odd and even K-tile counts, ragged M and N edges and a K
# remainder tile taken first; then shapes that take the plain kernel.
FAST_SHAPES = [
    (128, 128, 64), (128, 128, 128), (256, 256, 192), (256, 384, 512),
    (200, 136, 256), (1, 8, 64), (129, 264, 72), (300, 520, 1000), (777, 1032, 136),
]
PLAIN_SHAPES = [(1, 1, 1), (7, 5, 3), (64, 64, 56), (130, 131, 129), (3001, 4999, 2047)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", FAST_SHAPES + PLAIN_SHAPES)
def test_lowp_shapes(dtype, shape):
    torch = torch_cuda()
    M, N, K = shape
    print(f"[lowp] {dtype} {M}x{N}x{K}", flush=True)
    A, B, Cin = make_problem_16bit(M, N, K, seed=M + 7 * N + 13 * K, dtype=dtype, dist="normal", with_c=True)
    dA, _ = _dev16(A, dtype, torch)
    dB, _ = _dev16(B, dtype, torch)
    for alpha, beta in ((1.0, 0.0), (1.5, -0.5)):
        dC = torch.from_numpy(Cin).to("cuda") if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
        sgemm_lowp(dA, dB, dC, alpha=alpha, beta=beta)
        torch.cuda.synchronize()
        ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
        check_close(dC.cpu().numpy(), ref, f"{dtype} {shape} alpha={alpha} beta={beta}")


try:
    LOWP_VARIANTS = capi.lowp_variants()
except capi.LibraryMissing:      # collection without a built library
    LOWP_VARIANTS = [0, 1]

VARIANT_SHAPES = [(256, 256, 128), (300, 520, 1000), (129, 264, 72), (512, 384, 192), (1, 8, 64)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("variant", LOWP_VARIANTS)
def test_lowp_variants(dtype, variant):
    """Every kernel variant, forced, on whole and ragged tiles, odd and even
    K-tile counts (the multi-stage pipelines' wrap-around) and a K
    remainder."""
    torch = torch_cuda()
    for M, N, K in VARIANT_SHAPES:
        print(f"[lowp] {dtype} variant {variant} {M}x{N}x{K}", flush=True)
        A, B, Cin = make_problem_16bit(M, N, K, seed=3 * M + N + K, dtype=dtype, dist="normal", with_c=True)
        dA, _ = _dev16(A, dtype, torch)
        dB, _ = _dev16(B, dtype, torch)
        dC = torch.from_numpy(Cin).to("cuda")
        sgemm_lowp(dA, dB, dC, alpha=-1.25, beta=0.5, variant=variant)
        torch.cuda.synchronize()
        check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=-1.25, beta=0.5),
                    f"{dtype} variant {variant} {M}x{N}x{K}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_lowp_unaligned_c(dtype):
    """C rows that are not 16-byte aligned take 32-bit C access."""
    torch = torch_cuda()
    M, N, K = 130, 136, 128
    A, B, Cin = make_problem_16bit(M, N, K, seed=17, dtype=dtype, with_c=True)
    dA, _ = _dev16(A, dtype, torch)
    dB, _ = _dev16(B, dtype, torch)
    for ldc, off in ((N + 1, 0), (N, 1)):
        buf = torch.full((off + M * ldc + 8,), float("nan"), device="cuda")
        dC = buf[off:off + M * ldc].view(M, ldc)[:, :N]
        dC.copy_(torch.from_numpy(Cin))
        sgemm_lowp(dA, dB, dC, alpha=2.0, beta=-1.0)
        torch.cuda.synchronize()
        check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=2.0, beta=-1.0), f"ldc={ldc} off={off}")
        pad = buf[off:off + M * ldc].view(M, ldc)[:, N:]
        assert torch.isnan(pad).all(), "a column past N was written"


@pytest.mark.parametrize("dtype", DTYPES)
def test_lowp_padded_rows_and_misalignment(dtype):
    """Leading dimensions beyond the row length, NaN in every padding
    element (never read), and operands that start off a 16-byte boundary or
    have leading dimensions that are not multiples of 8 (plain kernel)."""
    torch = torch_cuda()
    M, N, K = 200, 264, 200
    A, B, Cin = make_problem_16bit(M, N, K, seed=11, dtype=dtype, with_c=True)
    ref = oracle.sgemm_ref(A, B, Cin, alpha=0.75, beta=1.25)
    for lda, ldb, off in ((208, 272, 0), (K + 3, N + 5, 0), (208, 272, 1), (K, N, 3)):
        print(f"[lowp] {dtype} {M}x{N}x{K} lda={lda} ldb={ldb} offset={off}", flush=True)
        dA, _ = _dev16(A, dtype, torch, ld=lda, offset=off)
        dB, _ = _dev16(B, dtype, torch, ld=ldb, offset=off)
        dC = torch.from_numpy(Cin).to("cuda")
        sgemm_lowp(dA, dB, dC, alpha=0.75, beta=1.25)
        torch.cuda.synchronize()
        check_close(dC.cpu().numpy(), ref, f"{dtype} lda={lda} ldb={ldb} offset={off}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_lowp_sq4096_sampled(dtype):
    """The 4096^3 square product with 16-bit inputs, checked on a seeded
    sample of outputs plus the corners and on the first and last 128-row
    tile rows in full."""
    torch = torch_cuda()
    M = N = K = 4096
    print(f"[lowp] {dtype} 4096^3 (sampled)", flush=True)
    A, B, _ = make_problem_16bit(M, N, K, seed=2, dtype=dtype)
    dA, _ = _dev16(A, dtype, torch)
    dB, _ = _dev16(B, dtype, torch)
    I, J = sample_indices(M, N, 2)
    ref = oracle.sgemm_ref_sampled(A, B, I, J)
    for v in LOWP_VARIANTS[1:]:
        print(f"[lowp] {dtype} 4096^3 variant {v}", flush=True)
        check_close(sgemm_lowp(dA, dB, variant=v).cpu().numpy()[I, J], ref, f"{dtype} 4096^3 variant {v} sample")
    C = sgemm_lowp(dA, dB).cpu().numpy()
    check_close(C[I, J], ref, f"{dtype} 4096^3 sample")
    for r0 in (0, M - 128):
        sl = slice(r0, r0 + 128)
        check_close(C[sl], oracle.sgemm_ref(np.ascontiguousarray(A[sl]), B), f"{dtype} 4096^3 rows {r0}..")


@pytest.mark.parametrize("dtype", DTYPES)
def test_lowp_special_values(dtype):
    """K == 0 (C = beta*C), empty M, and exact small-integer products that
    any summation order gives bit for bit."""
    torch = torch_cuda()
    t = _tdtype(torch, dtype)
    C0 = torch.full((5, 8), 3.0, device="cuda")
    st = capi.sgemm_lowp(capi.SGEMM_DTYPE_BF16 if dtype == "bf16" else capi.SGEMM_DTYPE_F16, 5, 8, 0, 1.0,
                         C0.data_ptr(), 1, C0.data_ptr(), 8, -2.0, C0.data_ptr(), 8,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == capi.SGEMM_STATUS_OK
    assert torch.equal(C0, torch.full((5, 8), -6.0, device="cuda"))
    empty = sgemm_lowp(torch.empty((0, 64), dtype=t, device="cuda"), torch.empty((64, 8), dtype=t, device="cuda"))
    assert empty.shape == (0, 8)
    rng = np.random.default_rng(5)
    M, N, K = 256, 128, 320
    A = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    B = rng.integers(-8, 9, size=(K, N)).astype(np.float32)
    C = sgemm_lowp(torch.from_numpy(A).to(t).cuda(), torch.from_numpy(B).to(t).cuda()).cpu().numpy()
    assert np.array_equal(C.astype(np.float64), oracle.sgemm_ref(A, B))


def test_lowp_rejects_mixed_types():
    torch = torch_cuda()
    a = torch.zeros((8, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        sgemm_lowp(a, a.half())
    with pytest.raises(TypeError):
        sgemm_lowp(a.float(), a.float())
    assert capi.sgemm_lowp(9, 8, 8, 8, 1.0, a.data_ptr(), 8, a.data_ptr(), 8, 0.0, a.data_ptr(), 8, None) == \
        capi.SGEMM_STATUS_INVALID_DTYPE
    with pytest.raises(ValueError):
        sgemm_lowp(a, torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda"))


def test_lowp_operand_over_2gib():
    """B of 131072 x 8192 BF16 values (2 GiB): every K tile gets its own
    descriptor base, so the fast kernels take operands past the 31-bit
    buffer range; the automatic choice and the alternating 256x256 kernel,
    sampled against the oracle, corners included."""
    torch = torch_cuda()
    M, N, K = 256, 8192, 131072
    A, B, _ = make_problem_16bit(M, N, K, seed=23, dtype="bf16")
    assert B.size * 2 >= 2 ** 31
    dA = torch.from_numpy(A).to(torch.bfloat16).cuda()
    dB = torch.from_numpy(B).to(torch.bfloat16).cuda()
    I, J = sample_indices(M, N, 23, n=512)
    ref = oracle.sgemm_ref_sampled(A, B, I, J)
    del B
    for v in (None, capi.SGEMM_VARIANT_AUTO, 4):
        print(f"[lowp] 2 GiB operand variant {v}", flush=True)
        C = sgemm_lowp(dA, dB, variant=v)
        torch.cuda.synchronize()
        check_close(C.cpu().numpy()[I, J], ref, f"2 GiB operand, variant {v}")


SPLIT_SHAPES = [(2048, 2048, 2048), (512, 768, 8192), (300, 520, 4104), (1000, 1000, 3000)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_lowp_split_k(dtype):
    """Split-K on small grids with long K (the 128x128 two-stage and
    alternating kernels, forced, and the automatic choice; the 256x256
    alternating kernel, which does not split, on the same shapes): parity
    with the oracle, bit-identical repeats (the partials are added in a
    fixed order) and a factor above one where the shape calls for it."""
    torch = torch_cuda()
    names = {capi.sgemm_lowp_variant_name(v): v for v in capi.lowp_variants()}
    for M, N, K in SPLIT_SHAPES:
        A, B, Cin = make_problem_16bit(M, N, K, seed=M + N + K, dtype=dtype, dist="normal", with_c=True)
        dA, _ = _dev16(A, dtype, torch)
        dB, _ = _dev16(B, dtype, torch)
        ref = oracle.sgemm_ref(A, B, Cin, alpha=0.5, beta=1.5)
        for v in (None, names["lowp_128x128x64_s2"], names["lowp_128x128x64_s4_alt"], names["lowp_256x256x32_s4_alt"]):
            s = capi.sgemm_lowp_split_factor(v if v is not None else capi.sgemm_lowp_select_variant(
                M, N, K, dA.data_ptr(), K, dB.data_ptr(), N), M, N, K)
            print(f"[lowp] split {dtype} {M}x{N}x{K} variant {v} factor {s}", flush=True)
            outs = []
            for _ in range(2):
                dC = torch.from_numpy(Cin).to("cuda")
                sgemm_lowp(dA, dB, dC, alpha=0.5, beta=1.5, variant=v)
                torch.cuda.synchronize()
                outs.append(dC.cpu().numpy())
            check_close(outs[0], ref, f"{dtype} {M}x{N}x{K} variant {v} split {s}")
            assert np.array_equal(outs[0], outs[1]), "split-K result changed between calls"
    assert capi.sgemm_lowp_split_factor(names["lowp_128x128x64_s2"], 512, 768, 8192) > 1
    assert capi.sgemm_lowp_split_factor(names["lowp_128x128x64_s2"], 1000, 1000, 3000) > 1
    alt = names["lowp_128x128x64_s4_alt"]
    assert capi.sgemm_lowp_split_factor(alt, 512, 768, 8192) > 1            # 24 tiles
    assert capi.sgemm_lowp_split_factor(alt, 1000, 1000, 3000) > 1
    assert capi.sgemm_lowp_split_factor(alt, 300, 520, 4104) == 1           # 15 tiles: the two-stage kernel's
    assert capi.sgemm_lowp_split_factor(names["lowp_256x256x32_s4_alt"], 512, 768, 8192) == 1


OP_SHAPES = [(256, 512, 192), (304, 520, 1000), (129, 264, 72), (512, 256, 4104), (300, 200, 130)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans_a,trans_b", [(True, False), (False, True), (True, True)])
def test_lowp_transposed_operands(dtype, trans_a, trans_b):
    """op(A) / op(B) with the operands stored transposed (A as K x M, B as
    N x K), on the automatic choice and on each variant built for them (the
    two alternating kernels and the plain kernel); NaN in every padding
    element of the stored operands; whole and ragged tiles, K remainders,
    and shapes whose contiguous extents are not multiples of 8 (plain
    kernel)."""
    torch = torch_cuda()
    names = {capi.sgemm_lowp_variant_name(v): v for v in capi.lowp_variants()}
    forced = [None, names["lowp_256x256x32_s4_alt"], names["lowp_128x128x64_s4_alt"], names["lowp_simple_64x64"]]
    for M, N, K in OP_SHAPES:
        A, B, Cin = make_problem_16bit(M, N, K, seed=5 * M + N + 3 * K, dtype=dtype, dist="normal", with_c=True)
        sa = np.ascontiguousarray(A.T) if trans_a else A           # stored operands
        sb = np.ascontiguousarray(B.T) if trans_b else B
        lda = sa.shape[1] + (8 if sa.shape[1] % 8 == 0 else 3)
        ldb = sb.shape[1] + (8 if sb.shape[1] % 8 == 0 else 5)
        dA, _ = _dev16(sa, dtype, torch, ld=lda)
        dB, _ = _dev16(sb, dtype, torch, ld=ldb)
        ref = oracle.sgemm_ref(A, B, Cin, alpha=1.25, beta=-0.5)
        for v in forced:
            print(f"[lowp] op {dtype} ta={trans_a} tb={trans_b} {M}x{N}x{K} variant {v}", flush=True)
            dC = torch.from_numpy(Cin).to("cuda")
            try:
                sgemm_lowp(dA, dB, dC, alpha=1.25, beta=-0.5, variant=v, trans_a=trans_a, trans_b=trans_b)
            except SgemmError as e:
                # a fast variant forced on operands outside its fast path
                assert v not in (None, names["lowp_simple_64x64"]) and e.status == capi.SGEMM_STATUS_UNSUPPORTED
                continue
            torch.cuda.synchronize()
            check_close(dC.cpu().numpy(), ref, f"{dtype} ta={trans_a} tb={trans_b} {M}x{N}x{K} variant {v}")


@pytest.mark.parametrize("trans_a,trans_b", [(True, False), (False, True), (True, True)])
def test_lowp_transposed_sq4096_sampled(trans_a, trans_b):
    torch = torch_cuda()
    M = N = K = 4096
    print(f"[lowp] op bf16 4096^3 ta={trans_a} tb={trans_b} (sampled)", flush=True)
    A, B, _ = make_problem_16bit(M, N, K, seed=2, dtype="bf16")
    dA = torch.from_numpy(np.ascontiguousarray(A.T) if trans_a else A).to(torch.bfloat16).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B.T) if trans_b else B).to(torch.bfloat16).cuda()
    C = sgemm_lowp(dA, dB, trans_a=trans_a, trans_b=trans_b).cpu().numpy()
    I, J = sample_indices(M, N, 2)
    check_close(C[I, J], oracle.sgemm_ref_sampled(A, B, I, J), f"4096^3 ta={trans_a} tb={trans_b} sample")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans_a,trans_b,shared_b", [(False, False, False), (False, False, True), (True, False, False),
                                                       (False, True, True), (True, True, False)])
def test_lowp_strided_batched(dtype, trans_a, trans_b, shared_b):
    """Strided batches of 16-bit problems (one launch, blockIdx.z), batch
    strides with gaps between the problems, B shared by all problems
    (stride 0), transposed operands; every problem against the oracle.
    Shapes: one on the fast kernels, one on the plain kernel."""
    torch = torch_cuda()
    t = _tdtype(torch, dtype)
    batch = 3
    for M, N, K in ((256, 264, 136), (130, 70, 50)):
        print(f"[lowp] batched {dtype} ta={trans_a} tb={trans_b} shared_b={shared_b} {M}x{N}x{K}", flush=True)
        probs = [make_problem_16bit(M, N, K, seed=100 + z, dtype=dtype, dist="normal", with_c=True) for z in range(batch)]
        if shared_b:
            probs = [(a, probs[0][1], c) for a, _, c in probs]
        sa = [np.ascontiguousarray(a.T) if trans_a else a for a, _, _ in probs]
        sb = [np.ascontiguousarray(b.T) if trans_b else b for _, b, _ in probs]
        # batch strides with a gap of 8 elements after each problem
        def stack(xs):
            r, c = xs[0].shape
            buf = torch.full((len(xs), r * c + 8), float("nan"), dtype=t, device="cuda")
            view = buf[:, :r * c].view(len(xs), r, c)
            for z, x in enumerate(xs):
                view[z].copy_(torch.from_numpy(x).to(t))
            return view
        dA = stack(sa)
        dB = stack(sb[:1]) if shared_b else stack(sb)
        dC = torch.from_numpy(np.stack([c for _, _, c in probs])).cuda()
        sgemm_lowp(dA, dB, dC, alpha=0.5, beta=2.0, trans_a=trans_a, trans_b=trans_b)
        torch.cuda.synchronize()
        C = dC.cpu().numpy()
        for z, (a, b, c) in enumerate(probs):
            check_close(C[z], oracle.sgemm_ref(a, b, c, alpha=0.5, beta=2.0), f"problem {z}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans_a,trans_b", [(False, False), (True, False), (False, True)], ids=["NN", "TN", "NT"])
def test_lowp_strided_batched_unaligned_strides(dtype, trans_a, trans_b):
    """Batch strides that are not multiples of 8 elements (problem 0 aligned,
    later problems not) on a shape the fast kernels take for one problem:
    every problem against the oracle, NaN in the gaps between problems."""
    torch = torch_cuda()
    t = _tdtype(torch, dtype)
    batch, (M, N, K) = 3, (256, 264, 136)
    print(f"[lowp] batched odd strides {dtype} ta={trans_a} tb={trans_b}", flush=True)
    probs = [make_problem_16bit(M, N, K, seed=200 + z, dtype=dtype, dist="normal", with_c=True) for z in range(batch)]
    sa = [np.ascontiguousarray(a.T) if trans_a else a for a, _, _ in probs]
    sb = [np.ascontiguousarray(b.T) if trans_b else b for _, b, _ in probs]

    def stack(xs, gap):
        r, c = xs[0].shape
        buf = torch.full((len(xs) * (r * c + gap),), float("nan"), dtype=t, device="cuda")
        view = buf.as_strided((len(xs), r, c), (r * c + gap, c, 1))
        for z, x in enumerate(xs):
            view[z].copy_(torch.from_numpy(x).to(t))
        return view
    dA, dB = stack(sa, 3), stack(sb, 5)
    dC = torch.from_numpy(np.stack([c for _, _, c in probs])).cuda()
    sgemm_lowp(dA, dB, dC, alpha=0.5, beta=2.0, trans_a=trans_a, trans_b=trans_b)
    torch.cuda.synchronize()
    C = dC.cpu().numpy()
    for z, (a, b, c) in enumerate(probs):
        check_close(C[z], oracle.sgemm_ref(a, b, c, alpha=0.5, beta=2.0), f"odd strides, problem {z}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape,lds,off", [((1001, 999, 1003), (1003, 999), 0), ((640, 1030, 700), (703, 1037), 1),
                                           ((520, 264, 2048), (2049, 264), 0)],
                         ids=["K-and-N-odd", "misaligned", "lda-odd"])
def test_lowp_copied_operands(dtype, shape, lds, off):
    """Operands the fast kernels cannot take, in problems large enough to be
    copied into zero-padded aligned buffers first: parity with the oracle
    for beta = 0 (NaN C) and beta != 0, NaN in the callers' padding, twice
    in a row (the second call reuses the copy buffer)."""
    torch = torch_cuda()
    M, N, K = shape
    lda, ldb = lds
    A, B, Cin = make_problem_16bit(M, N, K, seed=M + N + K, dtype=dtype, with_c=True)
    dA, _ = _dev16(A, dtype, torch, ld=lda, offset=off)
    dB, _ = _dev16(B, dtype, torch, ld=ldb, offset=off)
    print(f"[lowp copy] {dtype} {M}x{N}x{K} lda={lda} ldb={ldb} offset={off}", flush=True)
    for beta in (0.0, -0.5):
        ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=1.25, beta=beta)
        for _ in range(2):
            dC = torch.from_numpy(Cin).to("cuda") if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
            sgemm_lowp(dA, dB, dC, alpha=1.25, beta=beta)
            torch.cuda.synchronize()
            check_close(dC.cpu().numpy(), ref, f"{dtype} {shape} beta={beta}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ops", [(True, False), (False, True), (True, True)], ids=["TN", "NT", "TT"])
def test_lowp_copied_transposed_operands(dtype, ops):
    """Transposed 16-bit operands the fast kernels cannot take (odd leading
    dimensions, K and N not multiples of 8), copied into zero-padded
    row-major buffers: parity with the oracle, NaN in the callers' padding."""
    torch = torch_cuda()
    ta, tb = ops
    M, N, K = 901, 1003, 777
    A, B, Cin = make_problem_16bit(M, N, K, seed=M + N + K + 2 * ta + tb, dtype=dtype, with_c=True)
    sA = np.ascontiguousarray(A.T) if ta else A
    sB = np.ascontiguousarray(B.T) if tb else B
    dA, _ = _dev16(sA, dtype, torch, ld=sA.shape[1] + 3)
    dB, _ = _dev16(sB, dtype, torch, ld=sB.shape[1] + 5)
    print(f"[lowp copy op] {dtype} TA={ta} TB={tb}", flush=True)
    for beta in (0.0, 1.5):
        dC = torch.from_numpy(Cin).to("cuda") if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
        sgemm_lowp(dA, dB, dC, alpha=0.5, beta=beta, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=0.5, beta=beta),
                    f"{dtype} op TA={ta} TB={tb} beta={beta}")


@pytest.mark.parametrize("dtype,ops,shared", [(d, o, "none") for d in DTYPES for o in ("NN", "TN", "NT", "TT")] +
                         [("bf16", "NN", "A"), ("bf16", "TT", "B"), ("f16", "TN", "B"), ("f16", "NT", "A")])
def test_lowp_batched_copied_operands(dtype, ops, shared):
    """Strided batches of 16-bit problems the fast kernels cannot take (odd
    leading dimensions and strides, K and N not multiples of 8), large
    enough to be copied into zero-padded buffers (per problem, or once for
    an operand of stride 0): every problem against the oracle, NaN in the
    gaps between stored problems never read, C between problems never
    written."""
    torch = torch_cuda()
    t = _tdtype(torch, dtype)
    ta, tb = ops[0] == "T", ops[1] == "T"
    batch, (M, N, K) = 3, (640, 517, 701)
    probs = [make_problem_16bit(M, N, K, seed=400 + z, dtype=dtype, dist="normal", with_c=True) for z in range(batch)]
    if shared == "A":
        probs = [(probs[0][0], b, c) for _, b, c in probs]
    if shared == "B":
        probs = [(a, probs[0][1], c) for a, _, c in probs]
    sa = [np.ascontiguousarray(a.T) if ta else a for a, _, _ in probs]
    sb = [np.ascontiguousarray(b.T) if tb else b for _, b, _ in probs]

    def stack(xs, pad, gap, one):
        r, c = xs[0].shape
        ld = c + pad
        n = 1 if one else len(xs)
        buf = torch.full((n * (r * ld + gap),), float("nan"), dtype=t, device="cuda")
        view = buf.as_strided((len(xs), r, c), (0 if one else r * ld + gap, ld, 1))
        for z in range(n):
            view[z].copy_(torch.from_numpy(xs[z]).to(t))
        return view
    dA = stack(sa, 1, 3, shared == "A")
    dB = stack(sb, 3, 5, shared == "B")
    sc = M * N + 7
    bufC = torch.full((batch * sc,), float("nan"), device="cuda")
    dC = bufC.as_strided((batch, M, N), (sc, N, 1))
    for z, (_, _, c) in enumerate(probs):
        dC[z].copy_(torch.from_numpy(c))
    print(f"[lowp] batched copy {dtype} {ops} shared={shared}", flush=True)
    sgemm_lowp(dA, dB, dC, alpha=0.5, beta=-1.0, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    host = bufC.cpu().numpy()
    for z, (a, b, c) in enumerate(probs):
        check_close(host[z * sc:z * sc + M * N].reshape(M, N), oracle.sgemm_ref(a, b, c, alpha=0.5, beta=-1.0),
                    f"batched copy {dtype} {ops} shared={shared} problem {z}")
        assert np.isnan(host[z * sc + M * N:(z + 1) * sc]).all(), "write between C problems"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("batch,M,N,K,shared_b", [(4, 256, 256, 4096, False), (3, 128, 256, 8192, True),
                                                  (8, 128, 128, 4096, False), (2, 200, 264, 2056, False)],
                         ids=lambda x: str(x))
def test_lowp_strided_batched_split(dtype, batch, M, N, K, shared_b):
    """Strided batches of untransposed 16-bit problems whose tiles together
    leave the chip mostly idle split K (the 128x128 two-stage kernel's
    split-K, each problem's partials and counters after those of the
    problems before it): every problem against the oracle, repeats bit for
    bit, beta != 0 and beta = 0."""
    torch = torch_cuda()
    t = _tdtype(torch, dtype)
    print(f"[lowp] batched split {dtype} {batch} x {M}x{N}x{K} shared_b={shared_b}", flush=True)
    probs = [make_problem_16bit(M, N, K, seed=300 + z, dtype=dtype, dist="normal", with_c=True) for z in range(batch)]
    if shared_b:
        probs = [(a, probs[0][1], c) for a, _, c in probs]
    dA = torch.from_numpy(np.stack([a for a, _, _ in probs])).to(t).cuda()
    dB = torch.from_numpy(probs[0][1][None] if shared_b else np.stack([b for _, b, _ in probs])).to(t).cuda()
    for alpha, beta in ((0.75, -1.5), (1.0, 0.0)):
        outs = []
        for _ in range(2):
            dC = torch.from_numpy(np.stack([c for _, _, c in probs])).cuda()
            if beta == 0.0:
                dC.fill_(float("nan"))
            sgemm_lowp(dA, dB, dC, alpha=alpha, beta=beta)
            torch.cuda.synchronize()
            outs.append(dC.cpu().numpy())
        for z, (a, b, c) in enumerate(probs):
            check_close(outs[0][z], oracle.sgemm_ref(a, b, c if beta != 0.0 else None, alpha=alpha, beta=beta),
                        f"batched split problem {z} beta={beta}")
        assert np.array_equal(outs[0], outs[1]), "split result changed between calls"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ops", [(True, False), (False, True), (True, True)], ids=["TN", "NT", "TT"])
@pytest.mark.parametrize("shape", [(384, 256, 8192), (200, 264, 4104)], ids=lambda s: "x".join(map(str, s)))
def test_lowp_transposed_long_k_split(dtype, ops, shape):
    """Transposed operands on a grid of few tiles with long K: the 128x128
    alternating kernel splits K (the split-K hand-off on the stream's
    workspace).  Parity with the oracle, NaN in the padding of the stored
    operands, beta = 0 (NaN C) and beta != 0, twice in a row (the
    workspace's counters reset by the first call), bit-identical
    repeats."""
    torch = torch_cuda()
    ta, tb = ops
    M, N, K = shape
    A, B, Cin = make_problem_16bit(M, N, K, seed=M + N + K + 2 * ta + tb, dtype=dtype, dist="normal", with_c=True)
    sA = np.ascontiguousarray(A.T) if ta else A
    sB = np.ascontiguousarray(B.T) if tb else B
    dA, _ = _dev16(sA, dtype, torch, ld=sA.shape[1] + 8)
    dB, _ = _dev16(sB, dtype, torch, ld=sB.shape[1] + 16)
    print(f"[lowp long-K split op] {dtype} TA={ta} TB={tb} {M}x{N}x{K}", flush=True)
    for beta in (0.0, -0.75):
        ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=1.5, beta=beta)
        outs = []
        for _ in range(2):
            dC = torch.from_numpy(Cin).to("cuda") if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
            sgemm_lowp(dA, dB, dC, alpha=1.5, beta=beta, trans_a=ta, trans_b=tb)
            torch.cuda.synchronize()
            outs.append(dC.cpu().numpy())
            check_close(outs[-1], ref, f"{dtype} TA={ta} TB={tb} {shape} beta={beta}")
        assert np.array_equal(outs[0], outs[1]), "result changed between calls"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ops,shared", [("TN", "B"), ("NT", "A"), ("TT", "none")])
def test_lowp_batched_transposed_long_k_split(dtype, ops, shared):
    """A strided batch of transposed long-K problems on few tiles: the
    128x128 alternating kernel splits K over the problems' tiles together
    (each problem's partials and counters after those of the problems
    before it), an operand of stride 0 shared; every problem against the
    oracle, C between problems never written."""
    torch = torch_cuda()
    t = _tdtype(torch, dtype)
    ta, tb = ops[0] == "T", ops[1] == "T"
    batch, (M, N, K) = 3, (256, 128, 4096)
    probs = [make_problem_16bit(M, N, K, seed=900 + z, dtype=dtype, dist="normal", with_c=True) for z in range(batch)]
    if shared == "A":
        probs = [(probs[0][0], b, c) for _, b, c in probs]
    if shared == "B":
        probs = [(a, probs[0][1], c) for a, _, c in probs]
    sa = [np.ascontiguousarray(a.T) if ta else a for a, _, _ in probs]
    sb = [np.ascontiguousarray(b.T) if tb else b for _, b, _ in probs]

    def stack(xs, one):
        r, c = xs[0].shape
        ld, gap = c + 8, 64
        n = 1 if one else len(xs)
        buf = torch.full((n * (r * ld + gap),), float("nan"), dtype=t, device="cuda")
        view = buf.as_strided((len(xs), r, c), (0 if one else r * ld + gap, ld, 1))
        for z in range(n):
            view[z].copy_(torch.from_numpy(xs[z]).to(t))
        return view
    dA = stack(sa, shared == "A")
    dB = stack(sb, shared == "B")
    sc = M * N + 8
    bufC = torch.full((batch * sc,), float("nan"), device="cuda")
    dC = bufC.as_strided((batch, M, N), (sc, N, 1))
    for z, (_, _, c) in enumerate(probs):
        dC[z].copy_(torch.from_numpy(c))
    print(f"[lowp] batched long-K op {dtype} {ops} shared={shared}", flush=True)
    sgemm_lowp(dA, dB, dC, alpha=0.5, beta=2.0, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    host = bufC.cpu().numpy()
    for z, (a, b, c) in enumerate(probs):
        check_close(host[z * sc:z * sc + M * N].reshape(M, N), oracle.sgemm_ref(a, b, c, alpha=0.5, beta=2.0),
                    f"batched long-K {dtype} {ops} shared={shared} problem {z}")
        assert np.isnan(host[z * sc + M * N:(z + 1) * sc]).all(), "write between C problems"
