"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle,
element by element, |C - C_ref| <= 1e-3 + 1e-4 |C_ref|.

Workloads: the five SGEMM configurations (256^3, 1024^3, 4096^3 with
beta = 0 and with alpha = 0.5, beta = 2, the ragged 3001 x 4999 x 2047 with
alpha = 1.5, beta = -0.5, and 512^3 / 2048^3 / 8192^3).  Every configuration
but 8192^3 is compared on every element (the compiled fp64 oracle takes
about a second and a half for 4096^3 on 16 host threads); 8192^3 is compared
on a seeded 4096-entry sample plus the four corners.
"""
import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import capi, sgemm
from fp32_sgemm_tuning_amd.inputs import WORKLOADS, make_problem, sample_indices, workload_inputs
from gpu_util import check_close, padded_device, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

FULL = ["sq256", "sq512", "sq1024", "sq2048", "ragged", "sq4096", "sq4096_beta"]
SAMPLED = ["sq8192"]


def _run(w, torch):
    A, B, Cin = workload_inputs(w)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    dC = to_dev(Cin, torch) if Cin is not None else torch.empty((w.M, w.N), device="cuda")
    sgemm(dA, dB, dC, alpha=w.alpha, beta=w.beta)
    torch.cuda.synchronize()
    return A, B, Cin, dC.cpu().numpy()


@pytest.mark.parametrize("name", FULL)
def test_workload_full(name):
    torch = torch_cuda()
    w = WORKLOADS[name]
    print(f"[parity] {w.describe()}", flush=True)
    A, B, Cin, C = _run(w, torch)
    ref = oracle.sgemm_ref(A, B, Cin, alpha=w.alpha, beta=w.beta)
    check_close(C, ref, name)


@pytest.mark.parametrize("name", SAMPLED)
def test_workload_sampled(name):
    torch = torch_cuda()
    w = WORKLOADS[name]
    print(f"[parity] {w.describe()} (sampled)", flush=True)
    A, B, Cin, C = _run(w, torch)
    I, J = sample_indices(w.M, w.N, w.seed)
    ref = oracle.sgemm_ref_sampled(A, B, I, J, Cin, alpha=w.alpha, beta=w.beta)
    check_close(C[I, J], ref, name + " sample")


try:
    ALL_VARIANTS = capi.all_variants()
except capi.LibraryMissing:      # collection without a built library
    ALL_VARIANTS = [0, 1, 2]


def _up4(n):
    return max(4, (n + 3) // 4 * 4)


SHAPES = [
    (1, 1, 1), (1, 129, 3), (7, 5, 3), (16, 64, 16), (64, 64, 64), (127, 129, 31),
    (128, 128, 32), (129, 127, 33), (256, 384, 96), (300, 200, 500), (131, 517, 1029),
    # whole 256x256 tiles with one, two and five 64-deep K tiles (odd and even
    # counts of the two-stage loop)
    (256, 256, 64), (256, 512, 128), (512, 768, 320),
    # K a whole number of 64-deep tiles, N a multiple of 4, M and N ragged:
    # the direct-to-LDS kernels' edge path (out-of-range buffer loads)
    (200, 300, 256), (17, 260, 320), (1, 4, 64), (520, 772, 192),
    # K a multiple of 4 but not of the K tile: the K remainder tile (with
    # NaN in A's padding columns when lda > K)
    (256, 256, 100), (130, 200, 36), (300, 260, 1028), (256, 128, 68),
]


@pytest.mark.parametrize("variant", ALL_VARIANTS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (1.5, -0.5)], ids=["b0", "b1"])
def test_variant_shapes(variant, shape, ab):
    torch = torch_cuda()
    M, N, K = shape
    alpha, beta = ab
    A, B, Cin = make_problem(M, N, K, seed=M * 7 + N * 3 + K, dist="normal", with_c=True)
    # Leading dimensions rounded up to a multiple of 4 (so the 128-bit variant
    # applies); the padding columns hold NaN, so a read past column K-1 of A
    # would poison the result.
    dA, _ = padded_device(A, _up4(K), torch)
    dB, _ = padded_device(B, _up4(N), torch)
    dC, _ = padded_device(Cin, _up4(N), torch)
    if beta == 0.0:
        dC.fill_(float("nan"))       # must never be read
    sgemm(dA, dB, dC, alpha=alpha, beta=beta, variant=variant)
    torch.cuda.synchronize()
    ref = oracle.sgemm_ref(A, B, Cin, alpha=alpha, beta=beta)
    check_close(dC.cpu().numpy(), ref, f"variant {variant} {shape} {ab}")


ANY_ALIGN_VARIANTS = [v for v in ALL_VARIANTS if capi.sgemm_variant_info(v)[4] == 0]
UNALIGNED_SHAPES = [(203, 157, 301), (130, 67, 77), (1, 3, 129), (300, 129, 64), (256, 256, 256),
                    (129, 131, 1001)]


@pytest.mark.parametrize("variant", ANY_ALIGN_VARIANTS)
@pytest.mark.parametrize("shape", UNALIGNED_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_unaligned_views(variant, shape):
    """Odd leading dimensions and base pointers 4 bytes off 16-byte alignment,
    with K and N not multiples of 4 (the 4-byte direct-load kernels' exact
    edges) and NaN in every padding element."""
    torch = torch_cuda()
    M, N, K = shape
    A, B, Cin = make_problem(M, N, K, 31, dist="normal", with_c=True)
    dA, _ = padded_device(A, K + 3, torch, offset=1)
    dB, _ = padded_device(B, N + 5, torch, offset=3)
    dC, bufC = padded_device(Cin, N + 1, torch, offset=1)
    auto = capi.sgemm_select_variant(M, N, K, dA.data_ptr(), K + 3, dB.data_ptr(), N + 5, 0.75,
                                     dC.data_ptr(), N + 1)
    assert capi.sgemm_variant_info(auto)[4] == 0
    sgemm(dA, dB, dC, alpha=1.25, beta=0.75, variant=variant)
    torch.cuda.synchronize()
    ref = oracle.sgemm_ref(A, B, Cin, alpha=1.25, beta=0.75)
    check_close(dC.cpu().numpy(), ref, "unaligned")
    # padding columns of C stay NaN (never written)
    pad = bufC[1:1 + M * (N + 1)].view(M, N + 1)[:, N]
    assert torch.isnan(pad).all()


@pytest.mark.parametrize("n", [256, 4096])
def test_auto_matches_forced_variant_bitwise(n):
    """Auto dispatch picks a 128-bit variant for packed aligned tensors and
    gives the same bits as forcing that variant."""
    torch = torch_cuda()
    A, B, _ = make_problem(n, n, n, 0)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    auto = sgemm(dA, dB)
    v = capi.sgemm_select_variant(n, n, n, dA.data_ptr(), n, dB.data_ptr(), n, 0.0, auto.data_ptr(), n)
    assert capi.sgemm_variant_info(v)[4] == 1
    forced = sgemm(dA, dB, variant=v)
    torch.cuda.synchronize()
    assert torch.equal(auto, forced)


def test_aligned_vs_scalar_variant_agree():
    """128-bit and 32-bit load paths of the same tile compute the same sums."""
    torch = torch_cuda()
    A, B, Cin = make_problem(384, 256, 320, 5, with_c=True)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    c1 = to_dev(Cin, torch)
    c2 = c1.clone()
    sgemm(dA, dB, c1, alpha=0.5, beta=2.0, variant=capi.SGEMM_VARIANT_DB128_VEC)
    sgemm(dA, dB, c2, alpha=0.5, beta=2.0, variant=capi.SGEMM_VARIANT_DB128_SCALAR)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    np.testing.assert_array_equal(c1.cpu().numpy(), c2.cpu().numpy())


SPLIT_SHAPES = [(1024, 1024, 1024), (512, 512, 512), (64, 64, 4096), (1024, 1024, 8192),
                (130, 260, 2000), (256, 256, 4100)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SPLIT_SHAPES])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (-0.75, 1.25)], ids=["b0", "b1"])
def test_split_k(shape, ab):
    """The 128x128x32 split-K variant on small tile grids with long K splits
    K; the result matches the oracle element by element, repeats bit for bit
    (partials are added in split order, whichever block arrives last), and
    agrees with the unsplit kernel of the same tile within the tolerance."""
    torch = torch_cuda()
    M, N, K = shape
    alpha, beta = ab
    A, B, Cin = make_problem(M, N, K, seed=M + N + K, dist="normal", with_c=True)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    C0 = to_dev(Cin, torch)
    v = [x for x in ALL_VARIANTS if capi.sgemm_variant_name(x) == "lean_128x128x32_w2x2_splitk"][0]
    assert capi.sgemm_split_factor(v, M, N, K) > 1, shape
    outs = []
    for _ in range(3):
        c = C0.clone()
        sgemm(dA, dB, c, alpha=alpha, beta=beta, variant=v)
        outs.append(c)
    plain = C0.clone()
    sgemm(dA, dB, plain, alpha=alpha, beta=beta, variant=24)
    torch.cuda.synchronize()
    ref = oracle.sgemm_ref(A, B, Cin, alpha=alpha, beta=beta)
    check_close(outs[0].cpu().numpy(), ref, f"split-K {shape}")
    check_close(plain.cpu().numpy(), ref, f"unsplit {shape}")
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "split-K result changed between identical calls"


AUTO_SPLIT_CASES = [
    # (M, N, K, split factor the automatic choice takes)
    (256, 256, 16384, 16),        # 256 K tiles over 16 splits
    (640, 640, 4096, 5),
    (1152, 1152, 2048, 3),
    (512, 512, 512, 4),           # two K tiles per split
    (384, 384, 384, 3),
    (767, 767, 4095, 5),          # any alignment: 4-byte loads, K remainder
    (509, 515, 8191, 7),
]


@pytest.mark.parametrize("M,N,K,S", AUTO_SPLIT_CASES, ids=[f"{m}x{n}x{k}" for m, n, k, _ in AUTO_SPLIT_CASES])
def test_auto_split_factors(M, N, K, S):
    """The automatic choice on grids where the split-K cost model splits K:
    the factor is the expected one, the result matches the oracle element by
    element for beta = 0 (NaN in C) and beta != 0, and repeats bit for bit."""
    torch = torch_cuda()
    A, B, Cin = make_problem(M, N, K, seed=M + 2 * N + K, dist="normal", with_c=True)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    probe = torch.empty((M, N), device="cuda")
    v = capi.sgemm_select_variant(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, probe.data_ptr(), N)
    assert capi.sgemm_split_factor(v, M, N, K) == S, (capi.sgemm_variant_name(v), S)
    print(f"[auto split] {M}x{N}x{K} {capi.sgemm_variant_name(v)} S={S}", flush=True)
    for alpha, beta in ((1.0, 0.0), (0.5, -1.5)):
        ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
        outs = []
        for _ in range(2):
            dC = to_dev(Cin, torch) if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
            sgemm(dA, dB, dC, alpha=alpha, beta=beta)
            torch.cuda.synchronize()
            outs.append(dC.cpu().numpy())
        check_close(outs[0], ref, f"auto split {M}x{N}x{K} beta={beta}")
        assert np.array_equal(outs[0], outs[1])


def test_split_k_on_two_streams():
    """Two split-K calls in flight on two streams use separate workspaces."""
    torch = torch_cuda()
    A, B, _ = make_problem(512, 512, 4096, 77)
    A2, B2, _ = make_problem(512, 512, 4096, 78)
    v = capi.sgemm_select_variant(512, 512, 4096, 16, 4096, 16, 512, 0.0, 16, 512)
    assert capi.sgemm_split_factor(v, 512, 512, 4096) > 1
    dA, dB, dA2, dB2 = (to_dev(x, torch) for x in (A, B, A2, B2))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            c1 = sgemm(dA, dB)
        with torch.cuda.stream(s2):
            c2 = sgemm(dA2, dB2)
        outs.append((c1, c2))
    torch.cuda.synchronize()
    check_close(outs[0][0].cpu().numpy(), oracle.sgemm_ref(A, B), "stream 1")
    check_close(outs[0][1].cpu().numpy(), oracle.sgemm_ref(A2, B2), "stream 2")
    for c1, c2 in outs[1:]:
        assert torch.equal(c1, outs[0][0]) and torch.equal(c2, outs[0][1])


SPLIT_VARIANTS = [v for v in ALL_VARIANTS if capi.sgemm_variant_name(v).endswith("_splitk")]


@pytest.mark.parametrize("variant", SPLIT_VARIANTS)
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (130, 260, 2000), (256, 256, 4100), (200, 100, 512)],
                         ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_split_k_variants_forced(variant, shape):
    """Every split-K tile shape, forced: oracle parity with beta != 0 and
    bit-identical repeats."""
    torch = torch_cuda()
    M, N, K = shape
    A, B, Cin = make_problem(M, N, K, seed=3 * M + N + K, dist="normal", with_c=True)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    C0 = to_dev(Cin, torch)
    c1, c2 = C0.clone(), C0.clone()
    sgemm(dA, dB, c1, alpha=0.5, beta=-1.5, variant=variant)
    sgemm(dA, dB, c2, alpha=0.5, beta=-1.5, variant=variant)
    torch.cuda.synchronize()
    check_close(c1.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=0.5, beta=-1.5),
                f"{capi.sgemm_variant_name(variant)} {shape}")
    assert torch.equal(c1, c2)


def test_operand_over_2gib():
    """B of 65536 x 8192 floats (2 GiB): the lean kernel gives every K tile
    its own descriptor base, so operands past the 31-bit buffer range stay on
    it; sampled against the oracle, corners included."""
    torch = torch_cuda()
    M, N, K = 128, 8192, 65536
    A, B, _ = make_problem(M, N, K, 21)
    assert B.nbytes >= 2 ** 31
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    C = sgemm(dA, dB)
    torch.cuda.synchronize()
    I, J = sample_indices(M, N, 21, n=512)
    check_close(C.cpu().numpy()[I, J], oracle.sgemm_ref_sampled(A, B, I, J), "2 GiB operand")


TAIL_CASES = [
    # (M, N, K, variant name): the grid is whole waves plus a last wave at
    # most a quarter full, which runs as a second launch with K split
    (1536, 1536, 1536, None),
    (2560, 2624, 2560, "lean_64x64x64_w4x1_splitk"),
    (3072, 3072, 3072, "lean_128x128x32_w2x2_splitk"),
    (1600, 1600, 1600, "lean_64x64x64_w4x1_splitk"),
    # the any-alignment kernel: K and N not multiples of 4
    (1535, 1537, 1535, "lean_dw_64x64x64_w4x1_splitk"),
]


@pytest.mark.parametrize("M,N,K,name", TAIL_CASES)
def test_last_wave_split(M, N, K, name):
    """Two launches over disjoint tiles of C, the second split-K: parity with
    the oracle for beta = 0 over NaN C and for beta != 0, and bit-identical
    repeats."""
    torch = torch_cuda()
    names = {capi.sgemm_variant_name(v): v for v in capi.all_variants()}
    v = None if name is None else names[name]
    plan = capi.sgemm_tail_split(v if v is not None else names["lean_64x64x64_w4x1_splitk"], M, N, K)
    print(f"[tail] {M}x{N}x{K} {name} plan {plan}", flush=True)
    assert plan[0] > 1
    A, B, Cin = make_problem(M, N, K, 31, dist="normal", with_c=True)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    for alpha, beta in ((1.0, 0.0), (0.75, -1.25)):
        ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
        outs = []
        for _ in range(2):
            dC = to_dev(Cin, torch) if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
            sgemm(dA, dB, dC, alpha=alpha, beta=beta, variant=v)
            torch.cuda.synchronize()
            outs.append(dC.cpu().numpy())
        check_close(outs[0], ref, f"{M}x{N}x{K} {name} beta={beta}")
        assert np.array_equal(outs[0], outs[1])


SHORT_K_CASES = [(2944, 2944, 256), (2048, 2056, 132), (1536, 1540, 64)]


@pytest.mark.parametrize("M,N,K", SHORT_K_CASES, ids=[f"{m}x{n}x{k}" for m, n, k in SHORT_K_CASES])
def test_short_k_auto(M, N, K):
    """Short K on a full wave of 64x64 tiles: the automatic choice takes the
    32-deep K tile (a K remainder in the second case, one K tile in the
    third); every element against the oracle, beta = 0 over NaN C and
    beta != 0."""
    torch = torch_cuda()
    A, B, Cin = make_problem(M, N, K, seed=M + N + K, dist="normal", with_c=True)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    v = capi.sgemm_select_variant(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dA.data_ptr(), N)
    assert capi.sgemm_variant_name(v) == "lean_64x64x32_w4x1_splitk"
    for alpha, beta in ((1.0, 0.0), (-0.5, 1.5)):
        dC = to_dev(Cin, torch) if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
        sgemm(dA, dB, dC, alpha=alpha, beta=beta)
        torch.cuda.synchronize()
        check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta),
                    f"short K {M}x{N}x{K} beta={beta}")


def test_last_wave_split_128_tiles():
    """The automatic choice on 128x128 tiles splits a partly filled last wave
    too (6016^3: 2209 tiles, 161 in the last wave, split 3 ways): the seeded
    sample of 4096 entries plus the corners, and the full last 128 rows
    (the last tile row, where the raster order puts the second launch's
    tiles) and first 128 rows against the oracle, beta = 0 over NaN C and
    beta != 0."""
    torch = torch_cuda()
    M = N = K = 6016
    names = {capi.sgemm_variant_name(v): v for v in capi.all_variants()}
    probe = torch.empty(1, device="cuda")
    v = capi.sgemm_select_variant(M, N, K, probe.data_ptr(), K, probe.data_ptr(), N, 0.0, probe.data_ptr(), N)
    assert capi.sgemm_variant_name(v) == "lean_128x128x32_w2x2_splitk"
    assert capi.sgemm_tail_split(v, M, N, K) == (3, 161)
    A, B, Cin = make_problem(M, N, K, 41, with_c=True)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    I, J = sample_indices(M, N, 41)
    for alpha, beta in ((1.0, 0.0), (0.5, 2.0)):
        dC = to_dev(Cin, torch) if beta != 0.0 else torch.full((M, N), float("nan"), device="cuda")
        sgemm(dA, dB, dC, alpha=alpha, beta=beta)
        torch.cuda.synchronize()
        got = dC.cpu().numpy()
        cin = Cin if beta != 0.0 else None
        check_close(got[I, J], oracle.sgemm_ref_sampled(A, B, I, J, cin, alpha=alpha, beta=beta),
                    f"6016^3 sample beta={beta}")
        for r0 in (0, M - 128):
            slab_c = None if cin is None else np.ascontiguousarray(cin[r0:r0 + 128])
            ref = oracle.sgemm_ref(np.ascontiguousarray(A[r0:r0 + 128]), B, slab_c, alpha=alpha, beta=beta)
            check_close(got[r0:r0 + 128], ref, f"6016^3 rows {r0}.. beta={beta}")


def test_binding_uses_the_current_stream():
    """The binding passes the current stream's handle, also inside a
    torch.cuda.stream() block, and a given stream's handle otherwise."""
    torch = torch_cuda()
    import fp32_sgemm_tuning_amd as pkg
    dev = torch.device("cuda", torch.cuda.current_device())
    assert pkg._stream_handle(dev, None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert pkg._stream_handle(dev, None) == side.cuda_stream
    assert pkg._stream_handle(dev, side) == side.cuda_stream
    # a product enqueued on the side stream is ordered on it
    A, B, _ = make_problem(300, 200, 100, 5)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    dC = torch.full((300, 200), float("nan"), device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sgemm(dA, dB, dC)
    side.synchronize()
    check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B), "side stream")


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [(1024, 1024, 1023, 1024, 1024, 1024), (2048, 2046, 2048, 2048, 2048, 2048),
                                              (517, 301, 1001, 1004, 304, 308)])
def test_aligned_rows_ragged_k_or_n(M, N, K, lda, ldb, ldc):
    """Aligned, padded operands whose K or N is not a multiple of 4 (the
    4-byte kernels take them): parity with the oracle, NaN in the padding."""
    torch = torch_cuda()
    A, B, Cin = make_problem(M, N, K, seed=M + N + K, dist="normal", with_c=True)
    v = capi.sgemm_select_variant(M, N, K, 256, lda, 512, ldb, 0.0, 1024, ldc)
    assert capi.sgemm_variant_info(v)[4] == 0, capi.sgemm_variant_name(v)
    dA, _ = padded_device(A, lda, torch)
    dB, _ = padded_device(B, ldb, torch)
    dC, _ = padded_device(Cin, ldc, torch)
    sgemm(dA, dB, dC, alpha=1.25, beta=-0.5)
    torch.cuda.synchronize()
    check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=1.25, beta=-0.5), f"{M}x{N}x{K} ld {lda},{ldb},{ldc}")
