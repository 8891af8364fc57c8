"""Work and traffic model of SGEMM used for measurement and roofline figures.

  * FLOPs: each of the M*N outputs is a length-K dot product, 2*M*N*K FLOPs
    in total; TFLOP/s = 2MNK / t ("Matmul I: tiling and shared memory",
    section 1; the 4096^3 figure of 137.44 GFLOP in "2D Register Tiling:
    The Outer Product", Where We Are On The Roofline).  The alpha/beta
    epilogue is not counted.
  * Block-tile global traffic: a BM x BN tile walked over K loads
    K*(1/BM + 1/BN) elements per output; BK cancels ("2D Register Tiling",
    The Arithmetic).  The same form one level down gives the per-output
    on-chip loads of a TM x TN register tile.
  * Compulsory HBM bytes: A, B and C written once, plus C read when
    beta != 0 (skipped when beta == 0, "The Final Kernel", Skipping The
    Read Of C).
"""

FP32_BYTES = 4

# MI355X published peaks (AMD product specification).
MI355X_FP32_MATRIX_TFLOPS = 157.3      # dense FP32 MFMA, 256 CUs x 256 FLOP/clk x 2.4 GHz
MI355X_FP32_VECTOR_TFLOPS = 157.3
MI355X_HBM_GBPS = 8000.0
MI355X_CUS = 256
MI355X_SCLK_GHZ = 2.4


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    return flops(M, N, K) / seconds / 1e12


def min_hbm_bytes(M: int, N: int, K: int, beta_nonzero: bool) -> int:
    """Compulsory traffic: read A and B once, write C once, read C iff beta != 0."""
    c_passes = 2 if beta_nonzero else 1
    return FP32_BYTES * (M * K + K * N + c_passes * M * N)


def c_read_bytes(M: int, N: int) -> int:
    return FP32_BYTES * M * N


def tile_loads_per_output(K: int, BM: int, BN: int) -> float:
    """Elements fetched from global memory per output for a BM x BN block tile."""
    return K * (1.0 / BM + 1.0 / BN)


def tile_global_bytes(M: int, N: int, K: int, BM: int, BN: int) -> float:
    return FP32_BYTES * M * N * tile_loads_per_output(K, BM, BN)


def register_tile_loads_per_output(K: int, TM: int, TN: int) -> float:
    """On-chip (shared/LDS) element loads per output for a TM x TN register tile."""
    return K * (1.0 / TM + 1.0 / TN)


def arithmetic_intensity(flop: float, nbytes: float) -> float:
    return flop / nbytes
