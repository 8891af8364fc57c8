"""Calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Under capture the library neither allocates nor clears its split-K
workspace, so shapes that split K eagerly (a small grid, the last partial
wave, 16-bit inputs on a small grid) run unsplit inside the graph.  Each
graph is replayed three times with eager work and synchronisations between
the replays, and every replay is checked against the fp64 oracle (the eager
call is checked too; its summation order differs, so the two are not
compared bit for bit).
"""
import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import capi, sgemm, sgemm_lowp
from fp32_sgemm_tuning_amd.inputs import make_problem, make_problem_16bit
from gpu_util import check_close, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _replays(torch, run, out, ref, what):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        out.fill_(float("nan"))     # eager work between replays
        junk = torch.ones(1 << 20, device="cuda").cumsum(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), ref, f"{what}, replay {i}")
        del junk


@pytest.mark.parametrize("M,N,K", [(512, 512, 4096), (1536, 1536, 1536), (300, 200, 500)])
def test_fp32_graph_replay(M, N, K):
    torch = torch_cuda()
    print(f"[graph] fp32 {M}x{N}x{K}", flush=True)
    A, B, _ = make_problem(M, N, K, 41)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    dC = torch.empty((M, N), device="cuda")
    ref = oracle.sgemm_ref(A, B)
    sgemm(dA, dB, dC)
    torch.cuda.synchronize()
    check_close(dC.cpu().numpy(), ref, f"eager {M}x{N}x{K}")
    _replays(torch, lambda: sgemm(dA, dB, dC), dC, ref, f"fp32 {M}x{N}x{K}")


def test_lowp_graph_replay():
    torch = torch_cuda()
    M, N, K = 1024, 1024, 8192
    print(f"[graph] bf16 {M}x{N}x{K}", flush=True)
    names = {capi.sgemm_lowp_variant_name(v): v for v in capi.lowp_variants()}
    assert capi.sgemm_lowp_split_factor(names["lowp_128x128x64_s2"], M, N, K) > 1
    A, B, _ = make_problem_16bit(M, N, K, seed=43, dtype="bf16")
    dA = torch.from_numpy(A).to(torch.bfloat16).cuda()
    dB = torch.from_numpy(B).to(torch.bfloat16).cuda()
    dC = torch.empty((M, N), device="cuda")
    ref = oracle.sgemm_ref(A, B)
    sgemm_lowp(dA, dB, dC)
    torch.cuda.synchronize()
    check_close(dC.cpu().numpy(), ref, "eager bf16")
    _replays(torch, lambda: sgemm_lowp(dA, dB, dC), dC, ref, "bf16")
