"""sgemm_noalloc, the entry point for callers that cannot allocate: its
split-K partials and counters live in the library's static device scratch.
Checked through the C ABI against sgemm() on the same inputs, two calls in a
row with the second smaller (the scratch keeps the first call's contents),
and against the fp64 oracle; the plan is sgemm()'s, so the bits agree too,
up to the largest plans, which the scratch holds.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import capi
from fp32_sgemm_tuning_amd.inputs import make_problem
from gpu_util import check_close, padded_device, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Pairs of problems, the second smaller; each splits K (the first of the
# last pair splits the last wave of tiles into a second launch).
PAIRS = [
    ((640, 640, 4096), (512, 512, 2048)),          # S = 5, then S = 4
    ((1536, 1532, 1000), (256, 256, 8192)),        # last-wave split, then S = 16
    ((767, 767, 4095), (509, 515, 1021)),          # 4-byte loads (K, N not multiples of 4)
]


def _run(entry, A, B, Cin, alpha, beta, torch, stream):
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = (K + 3) // 4 * 4, (N + 3) // 4 * 4, (N + 3) // 4 * 4
    dA, _ = padded_device(A, lda, torch)
    dB, _ = padded_device(B, ldb, torch)
    dC, _ = padded_device(Cin, ldc, torch)
    if beta == 0.0:
        dC.fill_(float("nan"))
    st = entry(M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta, dC.data_ptr(), ldc, stream)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    return dC


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}x{p[0][1]}x{p[0][2]}-then-{p[1][0]}x{p[1][1]}")
@pytest.mark.parametrize("ab", [(1.0, 0.0), (0.75, -1.5)], ids=["b0", "b1"])
def test_noalloc_matches_sgemm(pair, ab):
    torch = torch_cuda()
    alpha, beta = ab
    stream = torch.cuda.current_stream().cuda_stream
    names = {capi.sgemm_variant_name(v): v for v in capi.all_variants()}
    for i, (M, N, K) in enumerate(pair):
        A, B, Cin = make_problem(M, N, K, seed=M + N + K + i, dist="normal", with_c=True)
        v = capi.sgemm_select_variant(M, N, K, 256, (K + 3) // 4 * 4, 256, (N + 3) // 4 * 4, beta, 256,
                                      (N + 3) // 4 * 4)
        splits = capi.sgemm_split_factor(v, M, N, K)
        tail = capi.sgemm_tail_split(v, M, N, K)[0]
        print(f"[noalloc] {M}x{N}x{K} {capi.sgemm_variant_name(v)} S={splits} tail={tail} beta={beta}", flush=True)
        assert splits > 1 or tail > 1, "the case must use the scratch"
        got = _run(capi.sgemm_noalloc, A, B, Cin, alpha, beta, torch, stream)
        want = _run(capi.sgemm, A, B, Cin, alpha, beta, torch, stream)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want.cpu().numpy()
        ref = oracle.sgemm_ref(A, B, Cin if beta != 0.0 else None, alpha=alpha, beta=beta)
        check_close(g, ref, f"sgemm_noalloc {M}x{N}x{K}")
        check_close(g, w, f"sgemm_noalloc against sgemm {M}x{N}x{K}")
        assert np.array_equal(g, w), "same plan, different bits"
    assert "lean_64x64x64_w4x1_splitk" in names


def test_noalloc_repeats_and_streams():
    """Repeated calls reuse the scratch (its counters are cleared per call)
    and give identical bits; calls ordered on a side stream work too."""
    torch = torch_cuda()
    M, N, K = 512, 512, 4096
    A, B, _ = make_problem(M, N, K, 71)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    side = torch.cuda.Stream()
    outs = []
    for h in (torch.cuda.current_stream().cuda_stream, side.cuda_stream, side.cuda_stream):
        C = torch.full((M, N), float("nan"), device="cuda")
        torch.cuda.synchronize()
        st = capi.sgemm_noalloc(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(), N, h)
        assert st == capi.SGEMM_STATUS_OK
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy())
    check_close(outs[0], oracle.sgemm_ref(A, B), "sgemm_noalloc 512x512x4096")
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])


def test_noalloc_runs_the_largest_plans():
    """The scratch holds every plan sgemm() makes: the largest forced split
    (SGEMM_SPLITK = 16, read at load, on a 260-tile grid: about 61 MiB of
    partials) and the largest automatic one (6592x6592x8192: 144 tiles of
    128x128 in the last wave split 7 ways, 63 MiB) run through sgemm_noalloc with
    the bits of sgemm().  In a child process, since the setting is read
    once per process."""
    torch_cuda()
    code = f"""
import sys; sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
import torch
from fp32_sgemm_tuning_amd import capi
h = torch.cuda.current_stream().cuda_stream
def both(M, N, K, expect_sum):
    A = torch.rand((M, K), device='cuda') - 0.5; B = torch.rand((K, N), device='cuda') - 0.5
    C1 = torch.full((M, N), float('nan'), device='cuda'); C2 = torch.full((M, N), float('nan'), device='cuda')
    assert capi.sgemm_noalloc(M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C1.data_ptr(), N, h) == 0
    assert capi.sgemm(M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C2.data_ptr(), N, h) == 0
    torch.cuda.synchronize()
    assert bool(torch.equal(C1, C2)), (M, N, K)
    assert bool(torch.isfinite(C1).all())
    return expect_sum
M, N, K = 1280, 832, 16384
v = capi.sgemm_select_variant(M, N, K, 256, K, 256, N, 0.0, 256, N)
s = capi.sgemm_split_factor(v, M, N, K)
assert s * 260 * 64 * 64 * 4 > 48 << 20, s
both(M, N, K, None)
print('forced', s)
"""
    env = dict(os.environ, SGEMM_SPLITK="16")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240)
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "forced" in r.stdout
    torch = torch_cuda()
    M, N, K = 6592, 6592, 8192
    v = capi.sgemm_select_variant(M, N, K, 256, K, 256, N, 0.0, 256, N)
    plan = capi.sgemm_tail_split(v, M, N, K)
    assert capi.sgemm_variant_name(v) == "lean_128x128x32_w2x2_splitk" and plan == (7, 144), plan
    assert plan[0] * plan[1] * 128 * 128 * 4 > 60 << 20
    A, B, _ = make_problem(M, N, K, 72)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    h = torch.cuda.current_stream().cuda_stream
    outs = []
    for entry in (capi.sgemm_noalloc, capi.sgemm):
        C = torch.full((M, N), float("nan"), device="cuda")
        assert entry(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(), N, h) == 0
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]), "sgemm_noalloc and sgemm differ on 6592x6592x8192"
    I = np.array([0, M - 1, M - 1, M // 2, M - 64], dtype=np.int64)
    J = np.array([0, N - 1, 0, N // 3, N - 1], dtype=np.int64)
    check_close(outs[0][I, J], oracle.sgemm_ref_sampled(A, B, I, J), "6592x6592x8192 entries")
