"""GPU parity of the transposed, column-major and strided-batched entry
points (sgemm_op, sgemm_cm, sgemm_strided_batched, sgemm_cm_strided_batched)
against the oracle.  The oracle takes op(A) and op(B) as plain row-major
arrays; the transposed and column-major storages are built from them on the
host, inside buffers whose padding holds NaN."""
import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import capi, sgemm_op
from fp32_sgemm_tuning_amd.inputs import make_problem
from gpu_util import check_close, torch_cuda

pytestmark = pytest.mark.gpu

N_, T_ = capi.SGEMM_OP_N, capi.SGEMM_OP_T
OPS = [(N_, N_), (T_, N_), (N_, T_), (T_, T_)]
OP_IDS = ["NN", "TN", "NT", "TT"]
SHAPES = [(1, 1, 1), (7, 5, 3), (64, 64, 64), (130, 67, 77), (256, 384, 96), (300, 260, 1028),
          (129, 131, 1001), (1024, 1024, 1024), (517, 999, 333)]


def _stored(x, transposed, pad, torch, offset=0):
    """Device buffer holding x (or x^T when transposed) row-major with `pad`
    extra NaN columns per row; returns (device view of the stored matrix, ld)."""
    s = np.ascontiguousarray(x.T if transposed else x)
    rows, cols = s.shape
    ld = cols + pad
    buf = torch.full((offset + rows * ld + 8,), float("nan"), dtype=torch.float32, device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(torch.from_numpy(s).to("cuda"))
    return view, max(ld, 1)


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (-0.75, 1.5)], ids=["b0", "b1"])
def test_row_major_ops(ops, shape, ab):
    torch = torch_cuda()
    op_a, op_b = ops
    M, N, K = shape
    alpha, beta = ab
    A, B, Cin = make_problem(M, N, K, seed=M + 2 * N + 3 * K + op_a + 2 * op_b, dist="normal", with_c=True)
    dA, lda = _stored(A, op_a == T_, 3, torch, offset=1)
    dB, ldb = _stored(B, op_b == T_, 5, torch, offset=2)
    dC, ldc = _stored(Cin, False, 4, torch)
    if beta == 0.0:
        dC.fill_(float("nan"))
    st = capi.sgemm_op(op_a, op_b, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta,
                       dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    torch.cuda.synchronize()
    check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=alpha, beta=beta),
                f"row-major op {ops} {shape}")


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", [(7, 5, 3), (130, 67, 77), (300, 260, 1028), (1024, 768, 512)],
                         ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_column_major_ops(ops, shape):
    """BLAS convention: X (r x c) stored column-major is X^T stored row-major."""
    torch = torch_cuda()
    op_a, op_b = ops
    M, N, K = shape
    A, B, Cin = make_problem(M, N, K, seed=7 * M + N + K, dist="normal", with_c=True)
    # column-major storage of op(A) = A:  A^T row-major; of op(A) = A^T (A
    # stored K x M column-major): A row-major.
    dA, lda = _stored(A, op_a == N_, 2, torch)
    dB, ldb = _stored(B, op_b == N_, 1, torch)
    dC, ldc = _stored(Cin, True, 3, torch)
    st = capi.sgemm_cm(op_a, op_b, M, N, K, 0.5, dA.data_ptr(), lda, dB.data_ptr(), ldb, -2.0,
                       dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    torch.cuda.synchronize()
    check_close(dC.cpu().numpy().T, oracle.sgemm_ref(A, B, Cin, alpha=0.5, beta=-2.0),
                f"column-major op {ops} {shape}")


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape,batch", [((64, 64, 64), 5), ((130, 67, 77), 3), ((256, 256, 512), 4),
                                         ((1, 1, 1), 2), ((33, 100, 200), 7)],
                         ids=["64x5", "130x67x77x3", "256x4", "1x2", "33x100x200x7"])
def test_strided_batched(ops, shape, batch):
    """Each problem of a strided batch equals the oracle on its own inputs;
    problem strides include padding between matrices."""
    torch = torch_cuda()
    op_a, op_b = ops
    M, N, K = shape
    probs = [make_problem(M, N, K, seed=100 + z, dist="normal", with_c=True) for z in range(batch)]
    sa = (K * M if op_a == T_ else M * K) + 17
    sb = (N * K if op_b == T_ else K * N) + 9
    sc = M * N + 5
    ra, ca = (K, M) if op_a == T_ else (M, K)
    rb, cb = (N, K) if op_b == T_ else (K, N)
    bufA = torch.full((batch * sa,), float("nan"), device="cuda")
    bufB = torch.full((batch * sb,), float("nan"), device="cuda")
    bufC = torch.full((batch * sc,), float("nan"), device="cuda")
    for z, (A, B, Cin) in enumerate(probs):
        bufA[z * sa:z * sa + ra * ca].copy_(torch.from_numpy(np.ascontiguousarray(A.T if op_a == T_ else A)).flatten())
        bufB[z * sb:z * sb + rb * cb].copy_(torch.from_numpy(np.ascontiguousarray(B.T if op_b == T_ else B)).flatten())
        bufC[z * sc:z * sc + M * N].copy_(torch.from_numpy(Cin).flatten())
    st = capi.sgemm_strided_batched(op_a, op_b, M, N, K, 1.25, bufA.data_ptr(), ca, sa, bufB.data_ptr(), cb, sb,
                                    0.5, bufC.data_ptr(), N, sc, batch, torch.cuda.current_stream().cuda_stream)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    torch.cuda.synchronize()
    host = bufC.cpu().numpy()
    for z, (A, B, Cin) in enumerate(probs):
        check_close(host[z * sc:z * sc + M * N].reshape(M, N), oracle.sgemm_ref(A, B, Cin, alpha=1.25, beta=0.5),
                    f"batch {ops} {shape} problem {z}")
        assert np.isnan(host[z * sc + M * N:(z + 1) * sc]).all(), "write between C problems"


def test_batched_shared_operand_and_column_major():
    """stride 0 shares B across the batch; the column-major batched entry
    equals the row-major one on transposed storage."""
    torch = torch_cuda()
    M, N, K, batch = 96, 80, 144, 6
    As = [make_problem(M, N, K, seed=300 + z, dist="normal")[0] for z in range(batch)]
    B = make_problem(M, N, K, seed=299, dist="normal")[1]
    dA = torch.from_numpy(np.stack(As)).cuda()
    dB = torch.from_numpy(B).cuda()[None]
    C = sgemm_op(dA, dB)                       # [batch, M, N], B shared (batch 1)
    # Row-major C is column-major C^T = B^T A^T (N x M), whose column-major
    # operands are B (stored as row-major B, ld N) and A (row-major, ld K).
    Ccm = torch.full((batch, M, N), float("nan"), device="cuda")
    st = capi.sgemm_cm_strided_batched(N_, N_, N, M, K, 1.0, dB.data_ptr(), N, 0, dA.data_ptr(), K, M * K,
                                       0.0, Ccm.data_ptr(), N, M * N, batch, torch.cuda.current_stream().cuda_stream)
    assert st == capi.SGEMM_STATUS_OK
    torch.cuda.synchronize()
    for z in range(batch):
        ref = oracle.sgemm_ref(As[z], B)
        check_close(C[z].cpu().numpy(), ref, f"shared B, problem {z}")
        check_close(Ccm[z].cpu().numpy(), ref, f"column-major batch, problem {z}")


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
def test_large_transposed_sampled(ops):
    """A 2048^3 product through each op pair (the 128x128 or 64x64 lean tile
    in 4-byte mode), compared on the 4096-entry sample and bit-identical on a
    repeat."""
    torch = torch_cuda()
    from fp32_sgemm_tuning_amd.inputs import sample_indices
    op_a, op_b = ops
    n = 2048
    A, B, _ = make_problem(n, n, n, 11)
    dA = torch.from_numpy(np.ascontiguousarray(A.T if op_a == T_ else A)).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B.T if op_b == T_ else B)).cuda()
    c1 = sgemm_op(dA, dB, trans_a=op_a == T_, trans_b=op_b == T_)
    c2 = sgemm_op(dA, dB, trans_a=op_a == T_, trans_b=op_b == T_)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    I, J = sample_indices(n, n, 11)
    got = c1.cpu().numpy()[I, J]
    check_close(got, oracle.sgemm_ref_sampled(A, B, I, J), f"2048^3 {ops}")


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", [(1940, 2044, 132), (2048, 2048, 96)], ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_transposed_16byte_stages(ops, shape):
    """Grids of 256 128x128 tiles take the 128x128x32 lean tile, where aligned
    transposed operands keep their stored orientation in LDS (16-byte loads,
    row-group and column-group fragment reads); edges in M, N and a K
    remainder, NaN padding, beta != 0."""
    torch = torch_cuda()
    op_a, op_b = ops
    M, N, K = shape
    A, B, Cin = make_problem(M, N, K, seed=M + N + K + 5 * op_a + 7 * op_b, dist="normal", with_c=True)
    dA, lda = _stored(A, op_a == T_, 4, torch)
    dB, ldb = _stored(B, op_b == T_, 8, torch)
    dC, ldc = _stored(Cin, False, 4, torch)
    st = capi.sgemm_op(op_a, op_b, M, N, K, 1.5, dA.data_ptr(), lda, dB.data_ptr(), ldb, -0.5,
                       dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    torch.cuda.synchronize()
    check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=1.5, beta=-0.5), f"16-byte op {ops} {shape}")


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (200, 300, 260), (64, 64, 64), (3072, 512, 128)],
                         ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_transposed_aligned_small(ops, shape):
    """Aligned operands (leading dimensions multiples of 4) on grids that
    pick the 64x64 tile: the 16-byte B^T stage there, the 4-byte gather for
    a transposed A (or the 128x128 tile when its grid is large enough)."""
    torch = torch_cuda()
    op_a, op_b = ops
    M, N, K = shape
    A, B, Cin = make_problem(M, N, K, seed=2 * M + N + K + op_a + op_b, dist="normal", with_c=True)
    dA, lda = _stored(A, op_a == T_, 4, torch)
    dB, ldb = _stored(B, op_b == T_, 4, torch)
    dC, ldc = _stored(Cin, False, 4, torch)
    st = capi.sgemm_op(op_a, op_b, M, N, K, 1.0, dA.data_ptr(), lda, dB.data_ptr(), ldb, 0.25,
                       dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    torch.cuda.synchronize()
    check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=1.0, beta=0.25), f"aligned op {ops} {shape}")


@pytest.mark.parametrize("ops", OPS[1:], ids=OP_IDS[1:])
@pytest.mark.parametrize("shape,pads", [((777, 333, 1501), (0, 0, 1)), ((1030, 1022, 515), (4, 4, 3)),
                                        ((640, 700, 900), (1, 3, 0))],
                         ids=["C-unaligned", "C-unaligned-padded", "operands-unaligned"])
def test_transposed_operands_copied(ops, shape, pads):
    """Problems without 16-byte loads for the whole product that are large
    enough to copy their transposed operands into row-major buffers first:
    parity with the oracle for beta = 0 (NaN C) and beta != 0, twice in a row
    (the second call reuses the copy buffer)."""
    torch = torch_cuda()
    op_a, op_b = ops
    M, N, K = shape
    pa, pb, pc = pads
    A, B, Cin = make_problem(M, N, K, seed=M + N + K + op_a + 2 * op_b, dist="normal", with_c=True)
    dA, lda = _stored(A, op_a == T_, pa, torch)
    dB, ldb = _stored(B, op_b == T_, pb, torch)
    for beta in (0.0, 0.75):
        for _ in range(2):
            dC, ldc = _stored(Cin, False, pc, torch, offset=1)
            if beta == 0.0:
                dC.fill_(float("nan"))
            st = capi.sgemm_op(op_a, op_b, M, N, K, 1.5, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta,
                               dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
            assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
            torch.cuda.synchronize()
            check_close(dC.cpu().numpy(), oracle.sgemm_ref(A, B, Cin, alpha=1.5, beta=beta),
                        f"copied op {ops} {shape} beta={beta}")


@pytest.mark.parametrize("ops", [(T_, N_), (N_, T_), (T_, T_)], ids=["TN", "NT", "TT"])
@pytest.mark.parametrize("shared", ["none", "A", "B"])
def test_batched_transposed_operands_copied(ops, shared):
    """Strided batches whose transposed operands lack 16-byte rows (odd
    strides and leading dimensions), large enough that they are copied into
    row-major buffers (per problem, or once for an operand of stride 0):
    every problem equals the oracle, NaN between the stored problems is
    never read and C between problems is never written."""
    torch = torch_cuda()
    op_a, op_b = ops
    M, N, K, batch = 700, 515, 611, 3
    probs = [make_problem(M, N, K, seed=700 + z, dist="normal", with_c=True) for z in range(batch)]
    if shared == "A":
        probs = [(probs[0][0], B, C) for (_, B, C) in probs]
    if shared == "B":
        probs = [(A, probs[0][1], C) for (A, _, C) in probs]
    ra, ca = (K, M) if op_a == T_ else (M, K)
    rb, cb = (N, K) if op_b == T_ else (K, N)
    lda, ldb = ca + 1, cb + 3
    sa = 0 if shared == "A" else ra * lda + 17
    sb = 0 if shared == "B" else rb * ldb + 9
    sc = M * N + 5
    bufA = torch.full((max(1, batch if sa else 1) * (ra * lda + 17),), float("nan"), device="cuda")
    bufB = torch.full((max(1, batch if sb else 1) * (rb * ldb + 9),), float("nan"), device="cuda")
    bufC = torch.full((batch * sc,), float("nan"), device="cuda")
    for z, (A, B, Cin) in enumerate(probs):
        sA_ = np.ascontiguousarray(A.T if op_a == T_ else A)
        sB_ = np.ascontiguousarray(B.T if op_b == T_ else B)
        bufA[z * sa:z * sa + ra * lda].view(ra, lda)[:, :ca].copy_(torch.from_numpy(sA_))
        bufB[z * sb:z * sb + rb * ldb].view(rb, ldb)[:, :cb].copy_(torch.from_numpy(sB_))
        bufC[z * sc:z * sc + M * N].copy_(torch.from_numpy(Cin).flatten())
    print(f"[batched copy] {ops} shared={shared}", flush=True)
    st = capi.sgemm_strided_batched(op_a, op_b, M, N, K, 1.25, bufA.data_ptr(), lda, sa, bufB.data_ptr(), ldb, sb,
                                    -0.5, bufC.data_ptr(), N, sc, batch, torch.cuda.current_stream().cuda_stream)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    torch.cuda.synchronize()
    host = bufC.cpu().numpy()
    for z, (A, B, Cin) in enumerate(probs):
        check_close(host[z * sc:z * sc + M * N].reshape(M, N), oracle.sgemm_ref(A, B, Cin, alpha=1.25, beta=-0.5),
                    f"batched copy {ops} shared={shared} problem {z}")
        assert np.isnan(host[z * sc + M * N:(z + 1) * sc]).all(), "write between C problems"


V64 = None


def _v64():
    global V64
    if V64 is None:
        V64 = {capi.sgemm_variant_name(v): v for v in capi.all_variants()}["lean_64x64x64_w4x1_splitk"]
    return V64


# One transposed problem with 16-byte loads on 64x64x64 tiles splits K as
# sgemm() does: over the whole grid (the split-K factor of the 64x64x64
# variant above 1) or over the last wave (its last-wave split above 1).
OP_SPLIT_CASES = [
    # (M, N, K, plan)
    (512, 512, 4096, "grid"),
    (384, 384, 384, "grid"),
    (516, 772, 4100, "grid"),       # edge tiles and a 4-deep K remainder
    (1536, 1536, 1536, "tail"),
    (1600, 1600, 1600, "tail"),
]


@pytest.mark.parametrize("ops", OPS[1:], ids=OP_IDS[1:])
@pytest.mark.parametrize("M,N,K,plan", OP_SPLIT_CASES, ids=[f"{m}x{n}x{k}" for m, n, k, _ in OP_SPLIT_CASES])
@pytest.mark.parametrize("ab", [(1.0, 0.0), (-0.75, 1.5)], ids=["b0", "b1"])
def test_transposed_split(ops, M, N, K, plan, ab):
    """Transposed operands on grids whose plan splits K: the result matches
    the oracle element by element (NaN in C's padding and, with beta = 0, in
    C itself) and repeats bit for bit."""
    torch = torch_cuda()
    op_a, op_b = ops
    alpha, beta = ab
    if plan == "grid":
        assert capi.sgemm_split_factor(_v64(), M, N, K) > 1
    else:
        assert capi.sgemm_split_factor(_v64(), M, N, K) == 1 and capi.sgemm_tail_split(_v64(), M, N, K)[0] > 1
    print(f"[op split] {OP_IDS[OPS.index(ops)]} {M}x{N}x{K} {plan} alpha {alpha} beta {beta}", flush=True)
    A, B, Cin = make_problem(M, N, K, seed=M + 3 * N + K + op_a + 2 * op_b, dist="normal", with_c=True)
    dA, lda = _stored(A, op_a == T_, 4, torch)
    dB, ldb = _stored(B, op_b == T_, 8, torch)
    ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
    outs = []
    for _ in range(2):
        dC, ldc = _stored(Cin, False, 4, torch)
        if beta == 0.0:
            dC.fill_(float("nan"))
        st = capi.sgemm_op(op_a, op_b, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta,
                           dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
        assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
        torch.cuda.synchronize()
        full = dC.cpu().numpy()
        outs.append(full)
    check_close(outs[0], ref, f"transposed split {ops} {M}x{N}x{K}")
    assert np.array_equal(outs[0], outs[1]), "split result changed between identical calls"


# Strided batches on 64x64x64 tiles with 16-byte loads split K over the
# tiles of all their problems together (the factor of the restated rule,
# splitk_fit.choose with the batch).
BATCH_SPLIT_CASES = [
    # (batch, M, N, K, shared): shared "A" / "B" = that operand's stride is 0
    (4, 256, 256, 4096, None),
    (3, 128, 192, 8192, "A"),
    (2, 260, 516, 4100, None),      # edge tiles and a 4-deep K remainder
    (6, 64, 64, 2048, "B"),
    (5, 320, 320, 1024, None),
]


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("case", BATCH_SPLIT_CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}")
def test_batched_split(ops, case):
    """A strided batch whose grid splits K: every problem matches the oracle
    element by element (beta != 0 and, in a second call, beta = 0 over NaN
    C), the gaps between the C problems stay NaN, and a repeat is bit for
    bit the same."""
    from fp32_sgemm_tuning_amd import splitk_fit
    torch = torch_cuda()
    op_a, op_b = ops
    batch, M, N, K, shared = case
    assert splitk_fit.choose(M, N, K, batch=batch) > 1
    print(f"[batch split] {OP_IDS[OPS.index(ops)]} {case}", flush=True)
    probs = [make_problem(M, N, K, seed=100 * batch + M + N + K + z, dist="normal", with_c=True) for z in range(batch)]
    if shared == "A":
        probs = [(probs[0][0], B, C) for _, B, C in probs]
    elif shared == "B":
        probs = [(A, probs[0][1], C) for A, _, C in probs]
    ta, tb = op_a == T_, op_b == T_
    ra, ca = (K, M) if ta else (M, K)
    rb, cb = (N, K) if tb else (K, N)
    lda, ldb, ldc = ca + 4, cb + 8, N + 4
    sa = 0 if shared == "A" else ra * lda + 8
    sb = 0 if shared == "B" else rb * ldb + 4
    sc = M * ldc + 12
    bufA = torch.full((max(batch * sa, ra * lda) + 8,), float("nan"), device="cuda")
    bufB = torch.full((max(batch * sb, rb * ldb) + 8,), float("nan"), device="cuda")

    def put(buf, off, x, ld):
        rows, cols = x.shape
        buf[off:off + rows * ld].view(rows, ld)[:, :cols].copy_(torch.from_numpy(np.ascontiguousarray(x)))

    for z, (A, B, _) in enumerate(probs):
        put(bufA, z * sa, A.T if ta else A, lda)
        put(bufB, z * sb, B.T if tb else B, ldb)
    h = torch.cuda.current_stream().cuda_stream
    for alpha, beta in ((-0.5, 1.25), (1.0, 0.0)):
        results = []
        for _ in range(2):
            bufC = torch.full((batch * sc + 8,), float("nan"), device="cuda")
            if beta != 0.0:
                for z, (_, _, Cin) in enumerate(probs):
                    put(bufC, z * sc, Cin, ldc)
            st = capi.sgemm_strided_batched(op_a, op_b, M, N, K, alpha, bufA.data_ptr(), lda, sa, bufB.data_ptr(),
                                            ldb, sb, beta, bufC.data_ptr(), ldc, sc, batch, h)
            assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
            torch.cuda.synchronize()
            results.append(bufC.cpu().numpy())
        host = results[0]
        for z, (A, B, Cin) in enumerate(probs):
            got = host[z * sc:z * sc + M * ldc].reshape(M, ldc)
            check_close(got[:, :N], oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta),
                        f"batched split {ops} {case} problem {z} beta={beta}")
            assert np.isnan(got[:, N:]).all(), "write into C's row padding"
            assert np.isnan(host[z * sc + M * ldc:(z + 1) * sc]).all(), "write between C problems"
        assert np.array_equal(results[0], results[1], equal_nan=True), "split result changed between calls"
