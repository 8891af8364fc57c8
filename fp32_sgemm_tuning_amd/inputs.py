"""Seeded synthetic inputs for the SGEMM workloads.

This module only draws random numbers; it holds none of the GEMM's
arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle receive
the arrays it returns.

Recipe (one numpy PCG64 generator per problem, ``default_rng(seed)``):
  * draw A [M,K], then B [K,N], then C_in [M,N] (only when beta != 0), each
    row-major float32;
  * "uniform[-1,1)" is ``rng.random(shape, float32) * 2 - 1`` (exact in
    float32: multiples of 2**-23 in [-1, 1));
  * "normal(0,1)" is ``rng.standard_normal(shape, float32)``.
The sampled check of a large product draws 4096 row indices, then 4096
column indices, from ``default_rng(seed + 10000)`` (uniform, with
replacement) and appends the four corners.

The workloads are the square FP32 SGEMMs the pages time (4096^3 on every
page, smaller N on the shared-memory tiling wiki) plus a ragged shape and a
beta != 0 run that exercise the edge tiles and the epilogue.
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    dist: str        # "uniform" or "normal"
    alpha: float
    beta: float
    sampled: bool    # check a 4096-entry sample instead of every entry

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def describe(self) -> str:
        d = "U[-1,1)" if self.dist == "uniform" else "N(0,1)"
        return (f"sgemm {self.M}x{self.N}x{self.K} fp32 row-major, {d} seed {self.seed}, "
                f"alpha={self.alpha:g} beta={self.beta:g}")


WORKLOADS = {
    w.name: w for w in [
        Workload("sq256", 256, 256, 256, 0, "uniform", 1.0, 0.0, False),
        Workload("sq1024", 1024, 1024, 1024, 1, "uniform", 1.0, 0.0, False),
        Workload("sq4096", 4096, 4096, 4096, 2, "uniform", 1.0, 0.0, False),
        Workload("sq4096_beta", 4096, 4096, 4096, 2, "uniform", 0.5, 2.0, False),
        Workload("ragged", 3001, 4999, 2047, 3, "normal", 1.5, -0.5, False),
        Workload("sq512", 512, 512, 512, 4, "uniform", 1.0, 0.0, False),
        Workload("sq2048", 2048, 2048, 2048, 5, "uniform", 1.0, 0.0, False),
        Workload("sq8192", 8192, 8192, 8192, 6, "uniform", 1.0, 0.0, True),
    ]
}


def _draw(rng, shape, dist):
    if dist == "uniform":
        x = rng.random(shape, dtype=np.float32)
        x *= np.float32(2.0)
        x -= np.float32(1.0)
        return x
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    raise ValueError(dist)


def make_problem(M, N, K, seed, dist="uniform", with_c=False):
    """Return (A, B, C_in or None) drawn in that order from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    A = _draw(rng, (M, K), dist)
    B = _draw(rng, (K, N), dist)
    C = _draw(rng, (M, N), dist) if with_c else None
    return A, B, C


def workload_inputs(w: Workload):
    return make_problem(w.M, w.N, w.K, w.seed, w.dist, with_c=(w.beta != 0.0))


def sample_indices(M, N, seed, n=4096):
    """Seeded sample of output positions (rows then columns), plus the corners."""
    rng = np.random.default_rng(seed + 10000)
    I = rng.integers(0, M, size=n, dtype=np.int64)
    J = rng.integers(0, N, size=n, dtype=np.int64)
    I = np.concatenate([I, np.array([0, 0, M - 1, M - 1], dtype=np.int64)])
    J = np.concatenate([J, np.array([0, N - 1, 0, N - 1], dtype=np.int64)])
    return I, J


def small_int_matrix(rng, shape, lo, hi):
    """Integers in [lo, hi] stored as float32 (exact)."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def to_16bit_values(x, dtype):
    """float32 array -> float32 array whose every entry is a value of the
    16-bit type `dtype` ("bf16": the low 16 bits of each float32 cleared;
    "f16": numpy's float16 conversion).  A choice of input values, not part of
    the GEMM: both sides then see the same 16-bit numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    raise ValueError(dtype)


def make_problem_16bit(M, N, K, seed, dtype, dist="uniform", with_c=False):
    """make_problem() with A and B made 16-bit values (to_16bit_values); C_in
    stays float32.  All three are float32 arrays."""
    A, B, C = make_problem(M, N, K, seed, dist, with_c)
    return to_16bit_values(A, dtype), to_16bit_values(B, dtype), C
