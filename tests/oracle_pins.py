"""Pins that tie the CPU oracle to facts fixed outside itself.

Each pin takes an ``Oracle`` and raises AssertionError when the oracle
disagrees with a closed form, an exact integer or rational computation, a
special case that reduces to a known matrix (identity, permutation,
all-ones), an independent library routine, or an invariant of the
definition.  The pins are chosen so that a plausible slip anywhere in the
oracle (a dropped k term, a wrong sign, an ignored leading dimension, a
transposed operand, a read of C when beta == 0, float instead of double
accumulation) fails at least one of them; ``test_oracle_mutants.py`` checks
exactly that on deliberately broken copies of the oracle.

Definition pinned: C = alpha * A @ B + beta * C_in with row-major FP32
operands ("Matmul I: tiling and shared memory", section 1; epilogue of "2D
Register Tiling: The Outer Product", The Kernel), C_in unread when beta == 0
("The Final Kernel", Skipping The Read Of C).

Run as a script (``python tests/oracle_pins.py --lib PATH``) it applies every
pin to the oracle library at PATH and exits 1 if any fails.
"""
import itertools
import os
import sys
from fractions import Fraction

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

from fp32_sgemm_tuning_amd.inputs import make_problem, small_int_matrix, sample_indices  # noqa: E402

U = 2.0 ** -53  # unit roundoff of fp64


def _padded(x, ld, fill=np.nan):
    """Copy x into a row-major buffer with leading dimension ld; the padding
    columns hold `fill` so that reading them would show in the result."""
    rows, cols = x.shape
    buf = np.full((rows, ld), fill, dtype=np.float32)
    buf[:, :cols] = x
    return buf[:, :cols]


def _exact_gemm(A, B, C_in, alpha, beta):
    """Exact rational value of alpha*A@B + beta*C_in (pure Python)."""
    M, K = A.shape
    N = B.shape[1]
    a, b = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    out = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
            v = a * s
            if beta != 0:
                v += b * Fraction(float(C_in[i, j]))
            out[i][j] = v
    return out


def pin_identity(orc):
    """A = I_K: the product is B itself, bit for bit."""
    rng = np.random.default_rng(11)
    K, N = 33, 47
    A = np.eye(K, dtype=np.float32)
    B = rng.standard_normal((K, N), dtype=np.float32)
    C = orc.sgemm_ref(A, B)
    assert np.array_equal(C, B.astype(np.float64)), "I @ B != B"


def pin_row_permutation(orc):
    """A = P (row permutation matrix, K = M): row i of C is row perm[i] of B."""
    rng = np.random.default_rng(12)
    M = K = 41
    N = 23
    perm = rng.permutation(M)
    A = np.zeros((M, K), dtype=np.float32)
    A[np.arange(M), perm] = 1.0
    B = rng.standard_normal((K, N), dtype=np.float32)
    C = orc.sgemm_ref(A, B)
    assert np.array_equal(C, B[perm].astype(np.float64)), "P @ B != B[perm]"


def pin_column_permutation(orc):
    """B = Q with Q[k, perm[k]] = 1 (K = N): column perm[k] of C is column k of A."""
    rng = np.random.default_rng(13)
    M, K = 19, 31
    N = K
    perm = rng.permutation(K)
    A = rng.standard_normal((M, K), dtype=np.float32)
    B = np.zeros((K, N), dtype=np.float32)
    B[np.arange(K), perm] = 1.0
    C = orc.sgemm_ref(A, B)
    expect = np.empty((M, N), dtype=np.float64)
    expect[:, perm] = A.astype(np.float64)
    assert np.array_equal(C, expect), "A @ Q has the wrong columns"


def pin_all_ones(orc):
    """All-ones A [M,K] and B [K,N]: every entry of C is exactly K.  Padded
    rows hold NaN, so a read beyond column K-1 of A or N-1 of B shows."""
    for (M, N, K) in [(5, 7, 2047), (3, 4, 1), (6, 2, 2), (1, 1, 3)]:
        A = _padded(np.ones((M, K), dtype=np.float32), K + 5)
        B = _padded(np.ones((K, N), dtype=np.float32), N + 3)
        C = orc.sgemm_ref(A, B)
        assert np.array_equal(C, np.full((M, N), float(K))), f"all-ones {M}x{N}x{K}"


def pin_small_integers(orc):
    """Integer A, B in [-32, 32]: the exact product is an integer matrix that
    int64 arithmetic computes exactly (no rounding anywhere)."""
    rng = np.random.default_rng(14)
    for (M, N, K) in [(37, 29, 101), (16, 48, 8192), (1, 65, 7)]:
        A = small_int_matrix(rng, (M, K), -32, 32)
        B = small_int_matrix(rng, (K, N), -32, 32)
        S = A.astype(np.int64) @ B.astype(np.int64)
        C = orc.sgemm_ref(A, B)
        assert np.array_equal(C, S.astype(np.float64)), f"integer product {M}x{N}x{K}"


def pin_epilogue_exact(orc):
    """alpha = 1.5, beta = -0.5 on integer A, B, C_in: the exact value
    1.5*S - 0.5*C_in is a half-integer well inside fp64's exact range."""
    rng = np.random.default_rng(15)
    M, N, K = 23, 31, 257
    A = small_int_matrix(rng, (M, K), -16, 16)
    B = small_int_matrix(rng, (K, N), -16, 16)
    Cin = small_int_matrix(rng, (M, N), -1000, 1000)
    S = A.astype(np.int64) @ B.astype(np.int64)
    # 1.5*S - 0.5*C = (3*S - C) / 2 exactly
    expect = (3 * S - Cin.astype(np.int64)).astype(np.float64) / 2.0
    C = orc.sgemm_ref(A, B, Cin, alpha=1.5, beta=-0.5)
    assert np.array_equal(C, expect), "alpha*S + beta*C_in epilogue"
    # beta alone: alpha = 0 leaves exactly beta * C_in
    C0 = orc.sgemm_ref(A, B, Cin, alpha=0.0, beta=2.0)
    assert np.array_equal(C0, 2.0 * Cin.astype(np.float64)), "alpha = 0"


def pin_beta_zero_ignores_c(orc):
    """beta == 0: C_in is never read, so NaN/Inf in it cannot reach C."""
    rng = np.random.default_rng(16)
    A, B, _ = make_problem(9, 13, 17, 16)
    ref = orc.sgemm_ref(A, B)
    for fill in (np.nan, np.inf):
        Cin = np.full((9, 13), fill, dtype=np.float32)
        C = orc.sgemm_ref(A, B, Cin, alpha=1.0, beta=0.0)
        assert np.all(np.isfinite(C)), "C_in leaked into a beta == 0 result"
        assert np.array_equal(C, ref), "beta == 0 result changed with C_in"
    del rng


def pin_degenerate_sizes(orc):
    """K == 0 gives beta*C_in (zeros when beta == 0); M == 0 or N == 0 give
    empty results."""
    Cin = np.arange(12, dtype=np.float32).reshape(3, 4) - 5
    A = np.zeros((3, 0), dtype=np.float32)
    B = np.zeros((0, 4), dtype=np.float32)
    C = orc.sgemm_ref(A, B, Cin, alpha=1.0, beta=-2.0)
    assert np.array_equal(C, -2.0 * Cin.astype(np.float64)), "K == 0 with beta"
    C = orc.sgemm_ref(A, B)
    assert np.array_equal(C, np.zeros((3, 4))), "K == 0 with beta == 0"
    C = orc.sgemm_ref(np.zeros((0, 5), np.float32), np.ones((5, 4), np.float32))
    assert C.shape == (0, 4)
    C = orc.sgemm_ref(np.ones((3, 5), np.float32), np.zeros((5, 0), np.float32))
    assert C.shape == (3, 0)


def pin_rational_bruteforce(orc):
    """Tiny shapes against exact rational arithmetic: the fp64 result stays
    within the classical bound (K+2) * u * (|alpha| sum|a b| + |beta c|)."""
    rng = np.random.default_rng(17)
    sizes = [1, 2, 3, 5, 8, 17]
    for M, N, K in [(1, 1, 1), (2, 3, 5), (5, 2, 17), (3, 8, 2), (8, 5, 3), (17, 3, 8), (2, 17, 1)]:
        assert M in sizes and N in sizes and K in sizes
        A = rng.standard_normal((M, K), dtype=np.float32)
        B = rng.standard_normal((K, N), dtype=np.float32)
        Cin = rng.standard_normal((M, N), dtype=np.float32)
        alpha = float(np.float32(rng.uniform(-2, 2)))
        beta = float(np.float32(rng.uniform(-2, 2)))
        C = orc.sgemm_ref(A, B, Cin, alpha=alpha, beta=beta)
        exact = _exact_gemm(A, B, Cin, alpha, beta)
        absS = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        bound = (K + 2) * U * (abs(alpha) * absS + abs(beta) * np.abs(Cin.astype(np.float64)))
        for i in range(M):
            for j in range(N):
                err = abs(Fraction(C[i, j]) - exact[i][j])
                assert err <= Fraction(bound[i, j]) * 2, f"entry ({i},{j}) of {M}x{N}x{K}"


def pin_exhaustive_2x2x2(orc):
    """Every pair of 2x2 matrices with entries in {-1, 0, 1} (81 x 81 pairs)
    for alpha, beta in {0, 1, -0.5}, checked against exact integer sums.
    All 81 A's are stacked into one 162x2 matrix and all B's into one 2x162
    matrix, so block (a, b) of the product is A_a @ B_b."""
    vals = (-1.0, 0.0, 1.0)
    mats = [np.array(v, dtype=np.float32).reshape(2, 2) for v in itertools.product(vals, repeat=4)]
    A = np.concatenate(mats, axis=0)                 # [162, 2]
    B = np.concatenate(mats, axis=1)                 # [2, 162]
    Cin = np.tile(np.array([[3.0, -1.0], [0.5, -7.0]], dtype=np.float32), (81, 81))
    S = np.empty((162, 162), dtype=np.int64)
    for a, Am in enumerate(mats):
        for b, Bm in enumerate(mats):
            for i in range(2):
                for j in range(2):
                    S[2 * a + i, 2 * b + j] = sum(int(Am[i, k]) * int(Bm[k, j]) for k in range(2))
    for alpha in (0.0, 1.0, -0.5):
        for beta in (0.0, 1.0, -0.5):
            C = orc.sgemm_ref(A, B, Cin, alpha=alpha, beta=beta)
            expect = alpha * S.astype(np.float64)
            if beta != 0.0:
                expect = expect + beta * Cin.astype(np.float64)
            assert np.array_equal(C, expect), f"2x2x2 exhaustive alpha={alpha} beta={beta}"


def pin_library_crosscheck(orc):
    """Against numpy's fp64 matmul (an independent code path) at 256^3 and on
    a ragged shape: relative to sum|a b| the two agree to 1e-13."""
    for (M, N, K, seed) in [(256, 256, 256, 0), (97, 131, 389, 3)]:
        A, B, _ = make_problem(M, N, K, seed)
        C = orc.sgemm_ref(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        scale = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        assert np.all(np.abs(C - ref) <= 1e-13 * scale + 1e-300), f"numpy cross-check {M}x{N}x{K}"


def pin_linearity_and_transpose(orc):
    """alpha = 2 doubles every entry exactly; (A B)^T = B^T A^T bit for bit
    (same products, same k order)."""
    A, B, _ = make_problem(37, 53, 71, 18)
    C1 = orc.sgemm_ref(A, B, alpha=1.0)
    C2 = orc.sgemm_ref(A, B, alpha=2.0)
    assert np.array_equal(C2, 2.0 * C1), "alpha linearity"
    Ct = orc.sgemm_ref(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(Ct, C1.T), "transpose identity"


def pin_leading_dimensions(orc):
    """Padded leading dimensions (padding holds NaN) give the same result as
    packed operands, for A, B and C_in."""
    A, B, Cin = make_problem(29, 43, 61, 19, with_c=True)
    ref = orc.sgemm_ref(A, B, Cin, alpha=0.75, beta=1.25)
    C = orc.sgemm_ref(_padded(A, 64), _padded(B, 47), _padded(Cin, 50), alpha=0.75, beta=1.25)
    assert np.array_equal(C, ref), "leading dimensions"


def pin_sampled_matches_full(orc):
    """The sampled entry point returns the full product's entries bit for bit."""
    A, B, Cin = make_problem(300, 211, 150, 20, with_c=True)
    full = orc.sgemm_ref(A, B, Cin, alpha=1.5, beta=-0.5)
    I, J = sample_indices(300, 211, 20, n=500)
    s = orc.sgemm_ref_sampled(A, B, I, J, Cin, alpha=1.5, beta=-0.5)
    assert np.array_equal(s, full[I, J]), "sampled vs full"


def pin_thread_invariance(orc):
    """Rows are independent: one thread and many threads give identical bits."""
    A, B, _ = make_problem(128, 96, 333, 21)
    orc.set_threads(1)
    one = orc.sgemm_ref(A, B)
    orc.set_threads(4)
    many = orc.sgemm_ref(A, B)
    orc.set_threads(os.cpu_count() or 1)
    assert np.array_equal(one, many), "thread count changed the result"


ALL_PINS = [
    pin_identity, pin_row_permutation, pin_column_permutation, pin_all_ones,
    pin_small_integers, pin_epilogue_exact, pin_beta_zero_ignores_c,
    pin_degenerate_sizes, pin_rational_bruteforce, pin_exhaustive_2x2x2,
    pin_library_crosscheck, pin_linearity_and_transpose, pin_leading_dimensions,
    pin_sampled_matches_full, pin_thread_invariance,
]


def main(argv):
    from oracle import Oracle
    lib = argv[argv.index("--lib") + 1] if "--lib" in argv else None
    orc = Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            failed.append(pin.__name__)
            print(f"FAIL {pin.__name__}: {e}", flush=True)
        except Exception as e:  # an error inside the oracle counts as a failed pin
            failed.append(pin.__name__)
            print(f"ERROR {pin.__name__}: {type(e).__name__}: {e}", flush=True)
    print(f"{len(ALL_PINS) - len(failed)}/{len(ALL_PINS)} pins hold", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
