"""GPU checks of the boundary's resource rules: the device memory the library
keeps stays bounded however many streams come and go, buffers are released
on request, and a HIP error the caller left pending is neither consumed nor
reported as the library's.

Streams are created and destroyed through the HIP runtime itself (the one
PyTorch loaded; PyTorch's own streams come from a fixed pool), so every
stream below is a distinct, short-lived hipStream_t.
"""
import ctypes

import numpy as np
import pytest

import oracle
from fp32_sgemm_tuning_amd import capi
from fp32_sgemm_tuning_amd.inputs import make_problem
from gpu_util import check_close, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

HIP_ERROR_INVALID_DEVICE = 101


def hip_runtime(torch):
    """The HIP runtime mapped in this process (PyTorch's), with the few
    entry points these tests call."""
    torch.cuda.init()
    paths = {line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line}
    assert len(paths) == 1, paths
    rt = ctypes.CDLL(paths.pop())
    vp = ctypes.c_void_p
    rt.hipStreamCreate.argtypes = [ctypes.POINTER(vp)]
    rt.hipStreamDestroy.argtypes = [vp]
    rt.hipStreamSynchronize.argtypes = [vp]
    rt.hipSetDevice.argtypes = [ctypes.c_int]
    rt.hipGetDevice.argtypes = [ctypes.POINTER(ctypes.c_int)]
    for f in (rt.hipStreamCreate, rt.hipStreamDestroy, rt.hipStreamSynchronize, rt.hipSetDevice, rt.hipGetDevice,
              rt.hipGetLastError, rt.hipPeekAtLastError):
        f.restype = ctypes.c_int
    return rt


def test_memory_bounded_over_stream_churn():
    """32 streams, each created, used for a split-K product and a product
    whose unaligned transposed operand is copied, then destroyed: the
    library never holds more than its per-device maximum of workspaces and
    copy buffers, the free device memory does not drift, and every stream's
    results are right (and identical)."""
    torch = torch_cuda()
    rt = hip_runtime(torch)
    M, N, K = 512, 512, 2048                     # 64 tiles of 64x64: K split
    A, B, _ = make_problem(M, N, K, 61)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    v = capi.sgemm_select_variant(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dA.data_ptr(), N)
    assert capi.sgemm_split_factor(v, M, N, K) > 1
    # op(A) = A^T stored K x M with an odd leading dimension: copied first
    At = torch.full((K, M + 1), float("nan"), device="cuda")
    At[:, :M] = dA.t()
    C = torch.empty((M, N), device="cuda")
    C2 = torch.empty((M, N), device="cuda")
    ref = oracle.sgemm_ref(A, B)
    torch.cuda.synchronize()
    copy_bytes = 4 * M * ((K + 3) // 4 * 4) + 256
    cap = (capi.SGEMM_MAX_STREAM_WORKSPACES * capi.SGEMM_WORKSPACE_BYTES
           + capi.SGEMM_MAX_COPY_BUFFERS * copy_bytes)
    held0 = capi.sgemm_workspace_bytes()
    free0 = torch.cuda.mem_get_info()[0]
    first = None
    for i in range(32):
        s = ctypes.c_void_p()
        assert rt.hipStreamCreate(ctypes.byref(s)) == 0
        st = capi.sgemm(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(), N, s.value)
        assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
        st = capi.sgemm_op(capi.SGEMM_OP_T, capi.SGEMM_OP_N, M, N, K, 1.0, At.data_ptr(), M + 1, dB.data_ptr(), N,
                           0.0, C2.data_ptr(), N, s.value)
        assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
        assert rt.hipStreamSynchronize(s) == 0
        assert rt.hipStreamDestroy(s) == 0
        held = capi.sgemm_workspace_bytes()
        assert 0 <= held <= max(cap, held0), (i, held, cap)
        got = C.cpu().numpy()
        if first is None:
            first = got
            check_close(got, ref, "split-K on a fresh stream")
            check_close(C2.cpu().numpy(), ref, "copied transposed operand on a fresh stream")
        else:
            assert np.array_equal(got, first), f"stream {i}: result differs"
            assert np.array_equal(C2.cpu().numpy(), first), f"stream {i}: transposed result differs"
    drift = free0 - torch.cuda.mem_get_info()[0]
    print(f"[boundary] library holds {capi.sgemm_workspace_bytes()} bytes; free memory drift {drift} bytes",
          flush=True)
    assert drift <= cap + (64 << 20), drift


def test_release_workspaces():
    """sgemm_release_workspaces frees what the library holds on the device
    once the kernels that use it are done; later calls allocate again."""
    torch = torch_cuda()
    M, N, K = 512, 512, 2048
    A, B, _ = make_problem(M, N, K, 62)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    C = torch.empty((M, N), device="cuda")
    h = torch.cuda.current_stream().cuda_stream
    assert capi.sgemm(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(), N, h) == 0
    assert capi.sgemm_workspace_bytes() >= capi.SGEMM_WORKSPACE_BYTES
    assert capi.sgemm_release_workspaces() == capi.SGEMM_STATUS_OK     # waits for the product first
    assert capi.sgemm_workspace_bytes() == 0
    check_close(C.cpu().numpy(), oracle.sgemm_ref(A, B), "before release")
    C.fill_(float("nan"))
    assert capi.sgemm(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(), N, h) == 0
    torch.cuda.synchronize()
    assert capi.sgemm_workspace_bytes() >= capi.SGEMM_WORKSPACE_BYTES
    check_close(C.cpu().numpy(), oracle.sgemm_ref(A, B), "after release")


def test_pending_hip_error_left_alone():
    """A HIP error the caller left pending (here: hipSetDevice on a device
    that does not exist) does not make the library's call fail, and the
    library does not consume it: if the runtime itself keeps a pending error
    across successful calls, the caller still reads it after the product."""
    torch = torch_cuda()
    rt = hip_runtime(torch)
    M, N, K = 512, 512, 2048
    A, B, _ = make_problem(M, N, K, 63)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    C = torch.empty((M, N), device="cuda")
    h = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    rt.hipGetLastError()                                        # start clean
    # how this runtime treats a pending error across a successful call
    assert rt.hipSetDevice(1 << 20) == HIP_ERROR_INVALID_DEVICE
    d = ctypes.c_int(-1)
    assert rt.hipGetDevice(ctypes.byref(d)) == 0
    keeps = rt.hipPeekAtLastError() == HIP_ERROR_INVALID_DEVICE
    rt.hipGetLastError()
    print(f"[boundary] runtime keeps a pending error across a successful call: {keeps}", flush=True)
    assert rt.hipSetDevice(1 << 20) == HIP_ERROR_INVALID_DEVICE
    st = capi.sgemm(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, C.data_ptr(), N, h)
    assert st == capi.SGEMM_STATUS_OK, capi.sgemm_strerror(st)
    after = rt.hipGetLastError()
    if keeps:
        assert after == HIP_ERROR_INVALID_DEVICE, after
    torch.cuda.synchronize()
    check_close(C.cpu().numpy(), oracle.sgemm_ref(A, B), "with a pending error")


def test_concurrent_streams_contend_for_workspaces():
    """Twelve host threads, each on a stream of its own (more streams than
    the library keeps workspaces), run split-K products concurrently: the
    workspaces are handed between streams (the first such hand-over drains
    the device once, later ones wait on the event recorded at the end of
    each call), the memory held stays within the maximum, and every result
    is bit for bit the single-stream split one, or, for a call that found
    every workspace held at that moment and ran K unsplit, the unsplit
    kernel's."""
    import threading
    torch = torch_cuda()
    M, N, K = 512, 512, 2048                     # 64 tiles of 64x64: K split
    A, B, _ = make_problem(M, N, K, 64)
    dA, dB = to_dev(A, torch), to_dev(B, torch)
    v = capi.sgemm_select_variant(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dA.data_ptr(), N)
    assert capi.sgemm_split_factor(v, M, N, K) > 1
    ref_c = torch.empty((M, N), device="cuda")
    h0 = torch.cuda.current_stream().cuda_stream
    assert capi.sgemm(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, ref_c.data_ptr(), N, h0) == 0
    names = {capi.sgemm_variant_name(x): x for x in capi.all_variants()}
    plain_c = torch.empty((M, N), device="cuda")
    assert capi.sgemm_ex(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, plain_c.data_ptr(), N, h0,
                         names["lean_64x64x64_w4x1"]) == 0
    torch.cuda.synchronize()
    expect, plain = ref_c.cpu().numpy(), plain_c.cpu().numpy()
    check_close(expect, oracle.sgemm_ref(A, B), "single stream")
    threads, calls = 12, 20
    streams = [torch.cuda.Stream() for _ in range(threads)]
    outs = [torch.full((calls, M, N), float("nan"), device="cuda") for _ in range(threads)]
    errors = []
    torch.cuda.synchronize()

    def work(t):
        try:
            h = streams[t].cuda_stream
            for i in range(calls):
                st = capi.sgemm(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, outs[t][i].data_ptr(), N, h)
                if st != capi.SGEMM_STATUS_OK:
                    errors.append((t, i, capi.sgemm_strerror(st)))
                    return
        except Exception as e:                   # reported below
            errors.append((t, repr(e)))

    pool = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
    for p in pool:
        p.start()
    for p in pool:
        p.join(timeout=120)
    assert not any(p.is_alive() for p in pool), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    cap = capi.SGEMM_MAX_STREAM_WORKSPACES * capi.SGEMM_WORKSPACE_BYTES + capi.SGEMM_MAX_COPY_BUFFERS * (4 << 30)
    assert capi.sgemm_workspace_bytes() <= cap
    unsplit = 0
    for t in range(threads):
        got = outs[t].cpu().numpy()
        for i in range(calls):
            if np.array_equal(got[i], expect):
                continue
            assert np.array_equal(got[i], plain), f"thread {t} call {i} matches neither plan"
            unsplit += 1
    print(f"[boundary] {threads * calls} concurrent calls, {unsplit} ran unsplit", flush=True)
