/*
 * sgemm.h - C ABI of the MI355X (gfx950) single-precision GEMM library
 * (libsgemm.so).
 *
 * Operation.  C = alpha * A * B + beta * C for row-major FP32 matrices
 * A [M,K], B [K,N] and C [M,N]; each output is a length-K dot product and the
 * whole product counts 2*M*N*K FLOPs ("Matmul I: tiling and shared memory",
 * section 1).  The epilogue has the form alpha*acc + beta*C ("2D Register
 * Tiling: The Outer Product", The Kernel) and, when beta == 0, C is never
 * read ("The Final Kernel: Retuning Against the Pipeline", Skipping The Read
 * Of C), so NaN or Inf already in C cannot reach the result.  Elements outside
 * the matrices contribute nothing and only in-range outputs are written
 * ("Matmul I", section 6).
 *
 * Layout.  Element (i,k) of A is A[i*lda + k], (k,j) of B is B[k*ldb + j],
 * (i,j) of C is C[i*ldc + j]; lda >= max(1,K), ldb >= max(1,N),
 * ldc >= max(1,N).  Columns j in [N, ldc) of C are never written.
 * Arithmetic is FP32 (v_mfma_f32_16x16x4_f32 matrix instructions, FP32
 * accumulate); no reduced-precision inputs are used.
 *
 * Pointers.  A, B and C are device pointers of the current HIP device.
 * C must not overlap A or B (not checked).  Any alignment is accepted: when
 * A, B and C are 16-byte aligned and lda, ldb, ldc are multiples of 4 the
 * library uses 128-bit loads and stores, otherwise 32-bit ones.
 *
 * Ownership and execution.  The caller owns A, B and C.  A call validates
 * its arguments, enqueues one kernel on `stream` (a hipStream_t; NULL is the
 * null stream; two kernels when the last wave of tiles is split, see
 * sgemm_tail_split) and returns without synchronising.  Calls are thread-safe
 * and deterministic: the same inputs and the same split of K (see
 * "Workspace") give the same bits.
 *
 * Workspace.  Small tile grids split K over several workgroups per output
 * tile (split-K).  Those calls use a workspace of SGEMM_WORKSPACE_BYTES
 * (64 MiB of partial tiles and 4096 tile counters) that the library
 * allocates with hipMalloc for a stream on its first such call.  A device
 * keeps at most SGEMM_MAX_STREAM_WORKSPACES of them, each bound to one stream
 * (the per-thread default stream counts once per host thread); when more
 * streams ask, the least recently used workspace that no call in progress
 * holds is handed to the new stream once the kernels queued on it have
 * finished, so device memory stays bounded however many streams a process
 * creates and destroys.  Until a stream first finds every workspace of its
 * device taken, calls record nothing at their end (each stream keeps its
 * workspace); that call waits once for the device to drain
 * (hipDeviceSynchronize) before it takes over an idle workspace, and from
 * then on every split call records an event at its end that marks the
 * workspace's last use.  The counters are cleared on the stream before a workspace's
 * first use and left cleared by every call.  Calls on one stream share its
 * workspace in stream order.  The partial tiles of a tile are added in a
 * fixed order, so split-K results are deterministic too.  A call that finds
 * no workspace free without waiting for another call (every one held at
 * that moment), and every call on a stream under graph capture, runs with K
 * unsplit: the same result within rounding, nothing allocated or waited
 * for.  No call waits while holding the library's lock, so calls on
 * different streams never block each other.  An allocation failure returns
 * SGEMM_STATUS_HIP_ERROR before anything is enqueued.  sgemm_op(), sgemm_cm()
 * and sgemm_lowp() keep copy buffers the same way (see sgemm_op).
 * sgemm_workspace_bytes() reports the device memory held and
 * sgemm_release_workspaces() frees it.
 *
 * HIP errors.  Every launch's status is taken from the launch call itself:
 * the library never calls hipGetLastError or hipPeekAtLastError, so it
 * neither consumes a HIP error the caller left pending nor reports such an
 * error as its own.
 *
 * Errors.  Arguments are checked before anything is enqueued, so a call that
 * returns an error has written nothing.  M == 0 or N == 0 returns
 * SGEMM_STATUS_OK without launching.  K == 0 writes alpha*0 + beta*C
 * (alpha*0 when beta == 0).
 */
#ifndef SGEMM_MI355X_H
#define SGEMM_MI355X_H

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_STATUS_OK 0
#define SGEMM_STATUS_INVALID_DIM (-1)       /* M, N, K < 0, or a leading dimension too small, or too many tiles */
#define SGEMM_STATUS_NULL_POINTER (-2)      /* NULL A, B or C with a non-empty extent */
#define SGEMM_STATUS_HIP_ERROR (-3)         /* the HIP runtime reported an error; see sgemm_last_hip_error() */
#define SGEMM_STATUS_INVALID_VARIANT (-4)   /* sgemm_ex: no such variant */
#define SGEMM_STATUS_UNSUPPORTED (-5)       /* sgemm_ex: variant needs 16-byte alignment the arguments lack */
#define SGEMM_STATUS_INVALID_OP (-6)        /* an operation code other than SGEMM_OP_N / SGEMM_OP_T */

#define SGEMM_STATUS_INVALID_DTYPE (-7)     /* sgemm_lowp: an input type other than SGEMM_DTYPE_BF16 / _F16 */
#define SGEMM_STATUS_SCRATCH_TOO_SMALL (-8) /* sgemm_noalloc: the split of K needs more than its scratch */

/* Device memory the library keeps between calls (see "Workspace" above). */
#define SGEMM_WORKSPACE_BYTES (64ll * 1024 * 1024 + 16 * 1024)  /* one split-K workspace */
#define SGEMM_MAX_STREAM_WORKSPACES 8       /* split-K workspaces kept per device */
#define SGEMM_MAX_COPY_BUFFERS 2            /* copy buffers kept per device */
#define SGEMM_MAX_COPY_BUFFER_BYTES (4ll << 30)  /* largest copy buffer; larger copies are not made */
#define SGEMM_NOALLOC_SCRATCH_BYTES (64ll * 1024 * 1024 + 16 * 1024)  /* sgemm_noalloc's static scratch, per device */

/* Input element types of sgemm_lowp. */
#define SGEMM_DTYPE_BF16 1                  /* bfloat16: 1 sign, 8 exponent, 7 fraction bits */
#define SGEMM_DTYPE_F16 2                   /* IEEE binary16 */

/* Operation codes of the sgemm_op family. */
#define SGEMM_OP_N 0                        /* use the stored matrix as is */
#define SGEMM_OP_T 1                        /* use the transpose of the stored matrix */

/* Variant ids for sgemm_ex(). */
#define SGEMM_VARIANT_AUTO (-1)             /* what sgemm() picks */
#define SGEMM_VARIANT_SIMPLE 0              /* 64x64 tile, single LDS buffer, 32-bit loads: the plain cross-check kernel */
#define SGEMM_VARIANT_DB128_VEC 1           /* 128x128x32 tile, double-buffered LDS, 128-bit loads/stores (needs alignment) */
#define SGEMM_VARIANT_DB128_SCALAR 2        /* the same tile with 32-bit loads/stores (any alignment) */
/* Ids 3 .. sgemm_num_variants()-1 are further kernels and tile shapes with
 * 128-bit access (double-buffered, section-pipelined, direct-to-LDS, lean
 * direct-to-LDS, and the split-K form of the lean 128x128x32 kernel), kept
 * for tile sweeps; sgemm_variant_name() and sgemm_variant_info() describe
 * them.  The direct-to-LDS kernels take the shapes they support (whole tiles,
 * or for the lean kernels K >= the K tile with K and N multiples of 4) and
 * use the guarded kernel of the same tile otherwise. */

/*
 * sgemm: C = alpha*A*B + beta*C (see above).  Picks the kernel variant from
 * the alignment class and the shape: the lean direct-to-LDS kernel with
 * 16-byte loads when the operands allow 128-bit access, else with 4-byte
 * loads (any alignment); on 64x64x64 block tiles when a 128x128 grid would
 * have at most 256 tiles or a less full last wave over the 256 compute
 * units, else on 128x128x32 tiles.  The 64x64x64 forms split K when their
 * own grid is under one wave of resident blocks (512 tiles) and splitting
 * saves time by the library's cost model (see sgemm_split_factor), and
 * split the last wave of a larger grid (see sgemm_tail_split).  Shapes a
 * lean kernel does not take go to a guarded kernel.  beta == 0 selects an
 * epilogue that never reads C.  Returns SGEMM_STATUS_*.
 */
int sgemm(int M, int N, int K, float alpha,
          const float *A, int lda,
          const float *B, int ldb,
          float beta, float *C, int ldc,
          void *stream);

/*
 * sgemm_ex: as sgemm() with the kernel variant forced (SGEMM_VARIANT_*; AUTO
 * behaves like sgemm()).  Intended for tests and tile sweeps.  Returns
 * SGEMM_STATUS_INVALID_VARIANT for an unknown id and SGEMM_STATUS_UNSUPPORTED
 * when a 128-bit variant is forced on arguments that lack its alignment.
 */
int sgemm_ex(int M, int N, int K, float alpha,
             const float *A, int lda,
             const float *B, int ldb,
             float beta, float *C, int ldc,
             void *stream, int variant);

/*
 * sgemm_noalloc: sgemm() for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, operation, variant choice and split of K as
 * sgemm(), so the same bits; it never calls hipMalloc or hipFree, on the
 * first call or later.  Its split-K partial tiles and tile counters live in
 * a static device array of SGEMM_NOALLOC_SCRATCH_BYTES that the library's
 * code holds on every device it is loaded on, until the process ends; the
 * first call on a device looks up that array's address there.  Each call
 * that splits K first clears the counters it uses with a small kernel on
 * `stream` (no memset, so the call can be captured into a graph; under
 * capture K is split as outside it).  Every call on a device shares that
 * device's array and the array keeps the last call's contents: calls that
 * overlap in time on one device (on different streams, or from different
 * host threads) race and must be ordered by the caller; calls in order on
 * one stream are safe.  The array holds 64 MiB of partial tiles, as much
 * as a split-K workspace, and sgemm() keeps every split within that (the
 * automatic choice reaches 63 MiB on large 128x128 grids whose last wave
 * splits; SGEMM_SPLITK is clamped to it), so every plan fits;
 * SGEMM_STATUS_SCRATCH_TOO_SMALL, with nothing enqueued, guards a plan that
 * would not.  Other statuses as for sgemm().
 */
int sgemm_noalloc(int M, int N, int K, float alpha,
                  const float *A, int lda,
                  const float *B, int ldb,
                  float beta, float *C, int ldc,
                  void *stream);

/*
 * sgemm_select_variant: the variant id sgemm() would run for these arguments
 * (no launch, no HIP call; pointers are only inspected for alignment).
 * Returns a negative status for invalid arguments.
 */
int sgemm_select_variant(int M, int N, int K,
                         const float *A, int lda,
                         const float *B, int ldb,
                         float beta, const float *C, int ldc);

/* Number of variant ids (valid ids are 0 .. n-1). */
int sgemm_num_variants(void);

/* Static name of a variant, or NULL for an unknown id. */
const char *sgemm_variant_name(int variant);

/*
 * sgemm_variant_info: block tile (bm x bn, K step bk) of a variant and whether
 * it needs 16-byte aligned operands (needs_vec = 1).  Any output pointer may
 * be NULL.  Returns SGEMM_STATUS_OK or SGEMM_STATUS_INVALID_VARIANT.
 */
int sgemm_variant_info(int variant, int *bm, int *bn, int *bk, int *needs_vec);

/*
 * sgemm_op: C = alpha * op(A) * op(B) + beta * C, row-major, with
 * op(X) = X (SGEMM_OP_N) or X^T (SGEMM_OP_T).  op(A) is M x K and op(B) is
 * K x N: with op_a = SGEMM_OP_T, A is stored K x M (element (i,k) of op(A)
 * at A[k*lda + i], lda >= max(1,M)); with op_b = SGEMM_OP_T, B is stored
 * N x K (element (k,j) of op(B) at B[j*ldb + k], ldb >= max(1,K)).  The
 * untransposed forms have the layout of sgemm().  The operation is the same
 * dot-product definition as sgemm() with the operands read through the
 * transpose ("Matmul I: tiling and shared memory", section 1); the pages
 * stop at packed untransposed operands and name the column-major BLAS
 * convention only in passing.  sgemm_op(N, N, ...) is sgemm().  A
 * transposed operand with 16-byte aligned rows (base, leading dimension and
 * its contiguous extent multiples of 4 floats) is read in its stored
 * orientation with 16-byte loads; such a product on 64x64 tiles splits K
 * (over the whole grid or over its last wave of tiles) by the rule and with
 * the workspaces of sgemm(), so the factor sgemm_split_factor() and
 * sgemm_tail_split() give for the variant lean_64x64x64_w4x1_splitk
 * applies.  One without is, for a problem large
 * enough that the copy takes less time than the product, first transposed
 * into a row-major copy in the stream's copy buffer (allocated with
 * hipMalloc on first need, grown once the kernels queued with it have
 * finished, at most SGEMM_MAX_COPY_BUFFERS per device, handed between
 * streams like the split-K workspaces), and the product then runs as sgemm()
 * on the copy; otherwise, always under graph capture, and when the stream's
 * buffer is held by a call in progress on another host thread, it is
 * gathered with 4-byte loads.  Environment variable SGEMM_PACK = 1 / -1
 * forces the copy on / off, for sweeps.  Returns SGEMM_STATUS_*; SGEMM_STATUS_INVALID_OP for
 * another op code; SGEMM_STATUS_HIP_ERROR if the buffer cannot be allocated
 * (nothing enqueued).
 */
int sgemm_op(int op_a, int op_b, int M, int N, int K, float alpha,
             const float *A, int lda,
             const float *B, int ldb,
             float beta, float *C, int ldc,
             void *stream);

/*
 * sgemm_strided_batched: `batch` independent sgemm_op problems of one shape;
 * problem z uses A + z*stride_a, B + z*stride_b and C + z*stride_c (in
 * elements).  0 <= batch <= 65535.  stride_a and stride_b may be 0 (one
 * operand shared by all problems); the C problems must not overlap:
 * stride_c >= (M-1)*ldc + N when batch > 1.  One kernel launch for the whole
 * batch.  On 64x64 tiles with 16-byte loads K is split as in sgemm() with
 * the tiles of all problems counted together (so a batch of small problems
 * with long K spreads over the chip), using the stream's split-K workspace;
 * other batches do not split.  Unaligned transposed operands are copied as in
 * sgemm_op(), for the whole batch in one launch per operand (an operand of
 * stride 0 once), when the copies' traffic takes less time than the product
 * and the copies fit in SGEMM_MAX_COPY_BUFFER_BYTES; the same buffer rules
 * apply.  batch == 0 is a no-op.  Returns SGEMM_STATUS_*.
 */
int sgemm_strided_batched(int op_a, int op_b, int M, int N, int K, float alpha,
                          const float *A, int lda, long long stride_a,
                          const float *B, int ldb, long long stride_b,
                          float beta, float *C, int ldc, long long stride_c,
                          int batch, void *stream);

/*
 * sgemm_cm, sgemm_cm_strided_batched: the same operations on column-major
 * matrices (the BLAS convention): element (i,j) of an r x c matrix X at
 * X[i + j*ld], ld >= max(1,r); op(A) is M x K, op(B) is K x N, C is M x N
 * with ldc >= max(1,M).  A column-major matrix is the row-major storage of
 * its transpose, so these run the row-major product C^T = op(B)^T op(A)^T.
 */
int sgemm_cm(int op_a, int op_b, int M, int N, int K, float alpha,
             const float *A, int lda,
             const float *B, int ldb,
             float beta, float *C, int ldc,
             void *stream);
int sgemm_cm_strided_batched(int op_a, int op_b, int M, int N, int K, float alpha,
                             const float *A, int lda, long long stride_a,
                             const float *B, int ldb, long long stride_b,
                             float beta, float *C, int ldc, long long stride_c,
                             int batch, void *stream);

/*
 * sgemm_lowp: C = alpha * A * B + beta * C with 16-bit inputs and FP32
 * accumulation and output.  A [M,K] and B [K,N] are row-major arrays of
 * `dtype` elements (SGEMM_DTYPE_BF16 or SGEMM_DTYPE_F16; lda and ldb count
 * elements), C [M,N] is row-major FP32.  The product of two 16-bit values is
 * exact in FP32, so the result is that of sgemm() on the inputs widened to
 * FP32, up to summation order.  The pages name 16-bit inputs on matrix
 * units with FP32 accumulation as the step past FP32 ("gpu_matmul",
 * Conclusion & Next Steps; "The Final Kernel: Retuning Against the
 * Pipeline", What Could Be Improved, And What It Would Take).
 *
 * Fast path: A and B 16-byte aligned, lda, ldb, N and K multiples of 8 and
 * K >= 32.  It runs the matrix instructions v_mfma_f32_16x16x32_bf16 / _f16
 * on 128x128, 256x128 or 256x256 block tiles, picked from the shape, with
 * 16-byte C access when C is 16-byte aligned and ldc a multiple of 4.  Other
 * operands (unaligned rows, K or N not multiples of 8) of a problem with
 * K >= 64, large enough that copying them takes less time than the plain
 * kernel would, are first copied into zero-padded aligned buffers (K and N
 * rounded up to multiples of 8; the stream's copy buffer, as for
 * sgemm_op; an operand the fast path takes as it is, with K a multiple of
 * 8, is used in place) and run on the fast path; the rest (and a call whose stream's
 * buffer is held by another call at that moment) runs a plain kernel that
 * widens each element on load.  SGEMM_PACK = 1 / -1 forces the copy on / off.  Small
 * tile grids split K and use the workspace described above (same rules:
 * allocated on first use per (device, stream), no split under graph
 * capture, deterministic).  Argument checks, layout rules and status codes
 * as for sgemm(), plus SGEMM_STATUS_INVALID_DTYPE, which is checked first.
 */
int sgemm_lowp(int dtype, int M, int N, int K, float alpha,
               const void *A, int lda,
               const void *B, int ldb,
               float beta, float *C, int ldc,
               void *stream);

/*
 * sgemm_lowp_ex: sgemm_lowp() with the kernel variant forced, for tests and
 * tile sweeps: SGEMM_VARIANT_AUTO (-1) behaves like sgemm_lowp(), 0 is the
 * plain kernel (any shape), 1 .. n-1 the matrix-instruction kernel on a block
 * tile and stage count that sgemm_lowp_variant_name() names.  Returns
 * SGEMM_STATUS_INVALID_VARIANT for an unknown id and SGEMM_STATUS_UNSUPPORTED
 * when a variant other than 0 is forced on operands outside its fast path.
 */
int sgemm_lowp_ex(int dtype, int M, int N, int K, float alpha,
                  const void *A, int lda,
                  const void *B, int ldb,
                  float beta, float *C, int ldc,
                  void *stream, int variant);

/*
 * sgemm_lowp_op: sgemm_lowp() with op(A) and op(B) as in sgemm_op(): with
 * op_a = SGEMM_OP_T, A is stored K x M (lda >= max(1,M)); with op_b =
 * SGEMM_OP_T, B is stored N x K (ldb >= max(1,K)); leading dimensions count
 * elements.  `variant` as in sgemm_lowp_ex() (SGEMM_VARIANT_AUTO for the
 * automatic choice); transposed operands run on the alternating-schedule
 * variants or the plain kernel, with each operand kept in LDS in its stored
 * orientation (16-byte chunks along its contiguous extent, which must be a
 * multiple of 8 elements for the fast path).  With transposed operands the
 * 128x128 alternating variant splits K on grids of few tiles, as the
 * 128x128 two-stage kernel does (same workspace
 * rules, deterministic; 512x512x8192 BF16 TN 69 -> 25 us; untransposed
 * operands split on it from 16 tiles up).  With
 * SGEMM_VARIANT_AUTO, operands the fast path cannot take are copied as in
 * sgemm_lowp(), transposed on the way into zero-padded row-major buffers,
 * and the product runs untransposed on the copies (where it may split K,
 * deterministically); an untransposed operand the fast path takes as it is
 * (K a multiple of 8) is used in place.  Returns SGEMM_STATUS_*;
 * SGEMM_STATUS_INVALID_OP for another op code.
 */
int sgemm_lowp_op(int dtype, int op_a, int op_b, int M, int N, int K, float alpha,
                  const void *A, int lda,
                  const void *B, int ldb,
                  float beta, float *C, int ldc,
                  void *stream, int variant);

/*
 * sgemm_lowp_strided_batched: `batch` independent sgemm_lowp_op() problems of
 * one shape, problem z on A + z*stride_a, B + z*stride_b (in 16-bit
 * elements) and C + z*stride_c (in floats); the rules of
 * sgemm_strided_batched() (0 <= batch <= 65535, strides of A and B may be 0,
 * C problems must not overlap, one launch) and the automatic variant choice
 * over batch x tiles; a batch on the 128x128 two-stage kernel or the 128x128
 * alternating kernel splits K over its problems' tiles together
 * (sgemm_lowp_split_factor for untransposed ones).  Batches the fast kernels cannot take
 * (unaligned rows, K or N not multiples of 8, or stride_a or stride_b not a
 * multiple of 8 elements, which leaves problems after the first unaligned)
 * are copied into zero-padded buffers as in sgemm_lowp(), one launch per
 * operand for the whole batch (an operand of stride 0 once), when that
 * takes less time than the plain kernel and the copies fit in
 * SGEMM_MAX_COPY_BUFFER_BYTES; the rest run on the plain kernel.  A
 * transposed batch on the 128x128 alternating kernel splits K as in
 * sgemm_lowp_op(), over its problems' tiles together.  Returns
 * SGEMM_STATUS_*.
 */
int sgemm_lowp_strided_batched(int dtype, int op_a, int op_b, int M, int N, int K, float alpha,
                               const void *A, int lda, long long stride_a,
                               const void *B, int ldb, long long stride_b,
                               float beta, float *C, int ldc, long long stride_c,
                               int batch, void *stream);

/* The variant sgemm_lowp() would run for these arguments (no launch; the
 * pointers are only inspected for alignment), or SGEMM_STATUS_INVALID_DIM.
 * 0 (the plain kernel) also where sgemm_lowp() copies the operands and runs
 * a fast kernel on the copies. */
int sgemm_lowp_select_variant(int M, int N, int K,
                              const void *A, int lda,
                              const void *B, int ldb);

/* Split-K factor (1 = no split) that sgemm_lowp_ex() with this variant would
 * use for an M x N x K problem outside graph capture; no HIP call.  (A strided
 * batch of untransposed problems counts its problems' tiles together; the
 * environment variable SGEMM_SPLITK = S caps the factor at S, for sweeps.)
 * Returns the factor, SGEMM_STATUS_INVALID_VARIANT or
 * SGEMM_STATUS_INVALID_DIM. */
int sgemm_lowp_split_factor(int variant, int M, int N, int K);

/* Static name of a sgemm_lowp_ex() variant, or NULL for an unknown id. */
const char *sgemm_lowp_variant_name(int variant);

/*
 * sgemm_split_factor: the number of workgroups per output tile along K
 * (1 = no split) that sgemm_ex() with this variant would use for an
 * M x N x K problem whose operands the variant's split-K kernel takes (see
 * "Workspace" above; environment variable SGEMM_SPLITK = S forces S for
 * sweeps).  Only grids of fewer than 512 tiles split; the factor (at most
 * 16, at least two K tiles per split) is the one of least modelled kernel
 * time: the busiest compute unit's share of K tiles plus a fixed cost per
 * pair of resident blocks, bounded below by the grid's operand traffic,
 * plus a fixed cost of splitting and one per split (the partials read
 * back); taken when that is at most 95% of the unsplit time.  The model's
 * constants are fitted to kernel-trace durations of 46 small grids at up
 * to 12 factors each.  Always 1 for variants
 * without split-K.  No HIP call.  Returns the factor,
 * SGEMM_STATUS_INVALID_VARIANT or SGEMM_STATUS_INVALID_DIM (negative sizes).
 */
int sgemm_split_factor(int variant, int M, int N, int K);

/*
 * sgemm_tail_split: the split of the last wave that sgemm_ex() with this
 * variant would make for an M x N x K problem with packed leading dimensions
 * outside graph capture (no HIP call).  A split-capable variant whose grid
 * is whole waves of tiles (two workgroups per compute unit) plus a partly
 * filled last wave, and that does not split K already, runs as two launches
 * on the stream when the same cost model as sgemm_split_factor (plus a fixed
 * cost for the second launch) says that saves at least 5%: the whole waves,
 * then the last wave's tiles with K split S ways.  Returns S (1: a single
 * launch) and, if tail_tiles is not
 * NULL, stores the number of tiles in the second launch (0 when S is 1);
 * SGEMM_STATUS_INVALID_VARIANT or SGEMM_STATUS_INVALID_DIM on bad arguments.
 */
int sgemm_tail_split(int variant, int M, int N, int K, int *tail_tiles);

/*
 * sgemm_workspace_bytes: device memory (bytes) the library holds on the
 * current device for split-K workspaces and copy buffers; at most
 * SGEMM_MAX_STREAM_WORKSPACES * SGEMM_WORKSPACE_BYTES + SGEMM_MAX_COPY_BUFFERS
 * * SGEMM_MAX_COPY_BUFFER_BYTES.  SGEMM_STATUS_HIP_ERROR if the current
 * device cannot be read.
 */
long long sgemm_workspace_bytes(void);

/*
 * sgemm_release_workspaces: free the workspaces and copy buffers the library
 * holds on the current device, each after the kernels queued with it have
 * finished (this call waits for them: on an event where one marks the last
 * use, else once for the whole device, hipDeviceSynchronize).  Buffers held by calls in progress on
 * other host threads at that moment are left alone.  Later calls allocate
 * again as needed.  Returns SGEMM_STATUS_OK or SGEMM_STATUS_HIP_ERROR (a
 * buffer whose wait or free failed is kept and never reused).
 */
int sgemm_release_workspaces(void);

/* Static text for a status code. */
const char *sgemm_strerror(int status);

/* Text of the last HIP error seen by this thread ("" if none). */
const char *sgemm_last_hip_error(void);

/* Library version (monotonic integer). */
int sgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_MI355X_H */
