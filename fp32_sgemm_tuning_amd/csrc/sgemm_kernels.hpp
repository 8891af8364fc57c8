// FP32 SGEMM kernels for gfx950 (CDNA4): C = alpha*A*B + beta*C, row-major.
//
// Every kernel multiplies on the matrix cores with v_mfma_f32_16x16x4_f32
// (true FP32 inputs, FP32 accumulate).  Lane layout of that instruction
// (wave of 64 lanes, l = lane id):
//   A operand  : lane l supplies A[row = l % 16][k = l / 16]       (16 x 4)
//   B operand  : lane l supplies B[k = l / 16][col = l % 16]       (4 x 16)
//   accumulator: lane l, register r holds D[row = 4*(l/16) + r][col = l % 16]
//
// The block-tile / register-tile / staged-K-loop structure follows the
// pages' ladder: shared tiles that every thread of the block reuses
// ("Matmul I: tiling and shared memory", sections 5-6), an outer-product
// register tile per thread ("2D Register Tiling: The Outer Product"), wide
// 128-bit loads ("gpu_matmul" blog, Kernel 6 & 7: Vectorization), a
// wave-contiguous footprint in the B tile (same blog, Kernel 8: Warptiling)
// and a K loop that loads the next tile while computing on the current one
// with one barrier per tile (same blog, Kernel 9 & 10: Staging; "The Final
// Kernel", What Pipelining Changed About Scarcity).  On gfx950 the register
// outer product is the MFMA itself, and the wave (64 lanes) is the unit that
// owns a register tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm_mi355x {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Args {
    const float *A;
    const float *B;
    float *C;
    long lda, ldb, ldc;     // leading dimensions in elements
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;   // block tiles along M and N
    int group_m;            // tile rows per raster group (>= 1)
    int xcd_remap;          // 1: give each XCD a contiguous run of tiles
};

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Map the launch index of a workgroup to its (tile_m, tile_n).
//
// Workgroups are handed to the 8 XCDs of the chip in round-robin order, and
// each XCD has its own L2.  With xcd_remap the launch index is first
// rearranged so that XCD x receives a contiguous run of logical tile ids;
// the logical ids are then walked in groups of `group_m` tile rows, column
// by column inside a group, so tiles that run together share rows of A and
// columns of B.
__device__ __forceinline__ void tile_coords(const Args &p, int &tm, int &tn) {
    int bid = blockIdx.x;
    const int nwg = gridDim.x;
    if (p.xcd_remap) {
        const int per = nwg >> 3;            // full rounds over the 8 XCDs
        if (bid < (per << 3)) bid = (bid & 7) * per + (bid >> 3);
    }
    const int gm = p.group_m;
    const int group_size = gm * p.tiles_n;
    const int g = bid / group_size;
    const int first_m = g * gm;
    const int rows = min(p.tiles_m - first_m, gm);
    const int in_group = bid - g * group_size;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// ---------------------------------------------------------------------------
// Plain cross-check kernel: 64x64 block tile, BK = 16, one LDS buffer, every
// global load a guarded 32-bit load with zero fill, every store guarded.  The
// shape of "Matmul I", section 6 (load, barrier, multiply, barrier), with the
// per-thread multiply-add replaced by MFMA.  Four waves in a 2x2 grid, each
// owning a 32x32 sub-tile (2x2 MFMA tiles).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sgemm_simple_kernel(Args p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BM][BK + 1];
    __shared__ float Bs[BK][BN + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    f32x4 acc[2][2];
    for (int mi = 0; mi < 2; ++mi)
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < p.K; k0 += BK) {
        for (int e = tid; e < BM * BK; e += 256) {
            const int r = e / BK, c = e % BK;
            const int gi = m0 + r, gk = k0 + c;
            As[r][c] = (gi < p.M && gk < p.K) ? p.A[(long)gi * p.lda + gk] : 0.0f;
        }
        for (int e = tid; e < BK * BN; e += 256) {
            const int r = e / BN, c = e % BN;
            const int gk = k0 + r, gj = n0 + c;
            Bs[r][c] = (gk < p.K && gj < p.N) ? p.B[(long)gk * p.ldb + gj] : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < BK; kk += 4) {
            for (int mi = 0; mi < 2; ++mi) {
                const float a = As[wm * 32 + mi * 16 + (lane & 15)][kk + (lane >> 4)];
                for (int ni = 0; ni < 2; ++ni) {
                    const float b = Bs[kk + (lane >> 4)][wn * 32 + ni * 16 + (lane & 15)];
                    acc[mi][ni] = mfma_16x16x4(a, b, acc[mi][ni]);
                }
            }
        }
        __syncthreads();
    }

    for (int mi = 0; mi < 2; ++mi)
        for (int ni = 0; ni < 2; ++ni)
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 32 + mi * 16 + 4 * (lane >> 4) + r;
                const int col = n0 + wn * 32 + ni * 16 + (lane & 15);
                if (row < p.M && col < p.N) {
                    float v = p.alpha * acc[mi][ni][r];
                    float *c = p.C + (long)row * p.ldc + col;
                    if (p.beta != 0.0f) v += p.beta * *c;
                    *c = v;
                }
            }
}

// ---------------------------------------------------------------------------
// Double-buffered kernel.
//
// Block tile BM x BN, K step BK (a multiple of 16), WAVES_M x WAVES_N waves;
// each wave owns a WM x WN register tile (WM a multiple of 16, WN a multiple
// of 64) held in (WM/16) x (WN/16) MFMA accumulators.
//
// LDS layout (two stages, no padding, every access 16-byte aligned):
//   A stage: BM x BK floats, k-contiguous 16-byte chunks in the permuted
//            order of ALayout<BK>, so that the fragment reads below touch
//            distinct banks.
//   B stage: [BK][BN] n-contiguous, natural order.
//
// Fragment reads use one ds_read_b128 per lane and rely on two freedoms of
// the contraction (the sum over k does not care how k is numbered, and the
// columns inside a wave tile may be renumbered if the epilogue undoes it):
//   A: lane l reads row (l % 16) of a 16-row slab, chunk (4h + l / 16): four
//      consecutive k.  Element j of that read feeds MFMA step j, so the
//      instruction's k index q = l / 16 stands for the real k = 16h + 4q + j.
//   B: for step j, lane l reads row k = 16h + 4(l/16) + j, columns
//      4(l % 16) .. +3 of a 64-column slab.  Element i feeds column group i:
//      the instruction's column c stands for the real column 4c + i.
// After the four column groups each lane holds four consecutive real
// columns of one row, which the epilogue writes with one 128-bit store.
//
// K loop: prologue stages tile 0; then, per tile t, issue the global loads
// of tile t+1 into registers, run the MFMAs of tile t from LDS stage t%2,
// write the registers into stage (t+1)%2, one barrier.
//
// VEC   : 128-bit global loads and stores (A, B, C 16-byte aligned, lda,
//         ldb, ldc multiples of 4); otherwise 32-bit ones.
// GUARD : some tile crosses M, N or K; out-of-range loads read 0 and
//         out-of-range outputs are not stored.
// BETA0 : beta == 0; C is never read.
// ---------------------------------------------------------------------------
// Bank behaviour of 128-bit LDS accesses on gfx950, as measured with
// SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE on single-wave access patterns:
//   ds_write_b128: 8 consecutive lanes per pass over 32 banks (128 bytes).
//   ds_read_b128 : 16 lanes per pass, the passes pairing lanes {0-7, 24-31},
//                  {8-15, 16-23}, {32-39, 56-63} and {40-47, 48-55}; a pass
//                  whose lanes hit distinct 16-byte bank slots takes one
//                  cycle, so a conflict-free read costs 4 cycles per wave.
//                  The slot is address bits 4..7 with some higher address
//                  bits folded in: 16 rows of 64 bytes always collide
//                  pairwise, 16 rows of 128 bytes with the swizzle below do
//                  not.
// Hence every A stage is stored as rows of 128 bytes (8 chunks of 4 k):
//   BK = 32: one logical row per LDS row, chunk c at c ^ s(row).
//   BK = 16: two logical rows per LDS row: rows 32g + r and 32g + 16 + r
//            (r < 16) share LDS row 16g + r, in chunks 0..3 and 4..7, XOR
//            s(r).  A fragment read of a 16-row slab then has exactly the
//            access pattern of the BK = 32 layout.
//   BK = 64: rows of 256 bytes, chunk c at c ^ (row % 16).
// with s(r) = (r / 2) % 8.  Fragment reads (lane l on row l % 16 of a slab,
// chunk l / 16) are then conflict-free, and so are the stage writes, since
// each 8-lane write pass covers one whole 128-byte LDS row.  The B tile needs
// no swizzle: 16 lanes read 256 contiguous bytes of one row.
template <int BK>
struct ALayout;

template <>
struct ALayout<32> {
    // float offset of (row m, chunk c) inside the A stage
    static __host__ __device__ __forceinline__ int offset(int m, int c) { return m * 32 + 4 * (c ^ ((m >> 1) & 7)); }
    // global-load assignment: 8 consecutive loaders share one row
    static __host__ __device__ __forceinline__ void coords(int e, int &m, int &c) { m = e >> 3; c = e & 7; }
};

template <>
struct ALayout<16> {
    static __host__ __device__ __forceinline__ int offset(int m, int c) {
        const int r = m & 15;
        const int lds_row = ((m >> 5) << 4) + r;
        const int chunk = ((((m >> 4) & 1) << 2) | c) ^ ((r >> 1) & 7);
        return lds_row * 32 + 4 * chunk;
    }
    // 8 consecutive loaders fill one LDS row: 4 chunks of row 32g + r and
    // 4 chunks of row 32g + 16 + r.
    static __host__ __device__ __forceinline__ void coords(int e, int &m, int &c) {
        c = e & 3;
        const int q = e >> 2;
        m = ((q >> 5) << 5) + ((q & 1) << 4) + ((q & 31) >> 1);
    }
};

template <>
struct ALayout<64> {
    static __host__ __device__ __forceinline__ int offset(int m, int c) { return m * 64 + 4 * (c ^ (m & 15)); }
    static __host__ __device__ __forceinline__ void coords(int e, int &m, int &c) { m = e >> 4; c = e & 15; }
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool VEC, bool GUARD, bool BETA0>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
sgemm_db_kernel(Args p) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int MI = WM / 16;          // 16-row MFMA tiles per wave
    constexpr int NJ = WN / 64;          // 64-column slabs per wave
    constexpr int KH = BK / 16;          // 16-deep halves of a K step
    constexpr int A_CHUNKS = BM * BK / 4;
    constexpr int B_CHUNKS = BK * BN / 4;
    constexpr int A_PER = A_CHUNKS / NT;
    constexpr int B_PER = B_CHUNKS / NT;
    constexpr int B_CPR = BN / 4;        // chunks per B row
    constexpr int STAGE = BM * BK + BK * BN;
    static_assert(BM % (16 * WAVES_M) == 0 && BN % (64 * WAVES_N) == 0, "wave tile");
    static_assert(BK == 16 || BK == 32 || BK == 64, "BK");
    static_assert(BM % 32 == 0, "A layout pairs 16-row slabs");
    static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "load split");

    __shared__ __attribute__((aligned(16))) float lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    // ---- global -> registers ------------------------------------------------
    f32x4 ra[A_PER], rb[B_PER];

    auto load_a = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int e = tid + NT * i;
            int r, c;
            ALayout<BK>::coords(e, r, c);
            const int gi = m0 + r, gk = k0 + 4 * c;
            const float *src = p.A + (long)gi * p.lda + gk;
            if (!GUARD) {
                if (VEC) ra[i] = *reinterpret_cast<const f32x4 *>(src);
                else ra[i] = f32x4{src[0], src[1], src[2], src[3]};
            } else if (gi < M && gk + 3 < K) {
                if (VEC) ra[i] = *reinterpret_cast<const f32x4 *>(src);
                else ra[i] = f32x4{src[0], src[1], src[2], src[3]};
            } else {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (gi < M) {
                    if (gk + 0 < K) v[0] = src[0];
                    if (gk + 1 < K) v[1] = src[1];
                    if (gk + 2 < K) v[2] = src[2];
                }
                ra[i] = v;
            }
        }
    };
    auto load_b = [&](int k0) {
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int e = tid + NT * i;
            const int r = e / B_CPR, c = e % B_CPR;
            const int gk = k0 + r, gj = n0 + 4 * c;
            const float *src = p.B + (long)gk * p.ldb + gj;
            if (!GUARD) {
                if (VEC) rb[i] = *reinterpret_cast<const f32x4 *>(src);
                else rb[i] = f32x4{src[0], src[1], src[2], src[3]};
            } else if (gk < K && gj + 3 < N) {
                if (VEC) rb[i] = *reinterpret_cast<const f32x4 *>(src);
                else rb[i] = f32x4{src[0], src[1], src[2], src[3]};
            } else {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (gk < K) {
                    if (gj + 0 < N) v[0] = src[0];
                    if (gj + 1 < N) v[1] = src[1];
                    if (gj + 2 < N) v[2] = src[2];
                }
                rb[i] = v;
            }
        }
    };
    // ---- registers -> LDS stage ---------------------------------------------
    auto store_stage = [&](int s) {
        float *As = lds + s * STAGE;
        float *Bs = As + BM * BK;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int e = tid + NT * i;
            int r, c;
            ALayout<BK>::coords(e, r, c);
            *reinterpret_cast<f32x4 *>(As + ALayout<BK>::offset(r, c)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int e = tid + NT * i;
            const int r = e / B_CPR, c = e % B_CPR;
            *reinterpret_cast<f32x4 *>(Bs + r * BN + 4 * c) = rb[i];
        }
    };

    f32x4 acc[MI][NJ][4];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mi][nj][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- MFMAs of one LDS stage -----------------------------------------------
    auto compute_stage = [&](int s) {
        const float *As = lds + s * STAGE;
        const float *Bs = As + BM * BK;
        const int lrow = lane & 15;
        const int lq = lane >> 4;
#pragma unroll
        for (int h = 0; h < KH; ++h) {
            f32x4 a[MI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = wm * WM + mi * 16 + lrow;
                a[mi] = *reinterpret_cast<const f32x4 *>(As + ALayout<BK>::offset(r, 4 * h + lq));
            }
            f32x4 b[4][NJ];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj) {
                    const int k = 16 * h + 4 * lq + j;
                    const int c = wn * WN + nj * 64 + 4 * lrow;
                    b[j][nj] = *reinterpret_cast<const f32x4 *>(Bs + k * BN + c);
                }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[mi][nj][i] = mfma_16x16x4(a[mi][j], b[j][nj][i], acc[mi][nj][i]);
        }
    };

    const int T = (K + BK - 1) / BK;
    if (T > 0) {
        load_a(0);
        load_b(0);
        store_stage(0);
        __syncthreads();
        for (int t = 0; t < T; ++t) {
            const bool more = (t + 1 < T);
            if (more) {
                load_a((t + 1) * BK);
                load_b((t + 1) * BK);
            }
            compute_stage(t & 1);
            if (more) store_stage((t + 1) & 1);
            __syncthreads();
        }
    }

    // ---- epilogue: C = alpha*acc (+ beta*C) -----------------------------------
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WM + mi * 16 + 4 * (lane >> 4) + r;
                const int col = n0 + wn * WN + nj * 64 + 4 * (lane & 15);
                f32x4 v = {acc[mi][nj][0][r], acc[mi][nj][1][r], acc[mi][nj][2][r], acc[mi][nj][3][r]};
                v *= alpha;
                float *dst = p.C + (long)row * p.ldc + col;
                const bool full = !GUARD || (row < M && col + 3 < N);
                if (full) {
                    if (VEC) {
                        if (!BETA0) v += beta * *reinterpret_cast<const f32x4 *>(dst);
                        *reinterpret_cast<f32x4 *>(dst) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float o = v[e];
                            if (!BETA0) o += beta * dst[e];
                            dst[e] = o;
                        }
                    }
                } else if (row < M) {
#pragma unroll
                    for (int e = 0; e < 3; ++e) {
                        if (col + e < N) {
                            float o = v[e];
                            if (!BETA0) o += beta * dst[e];
                            dst[e] = o;
                        }
                    }
                }
            }
}

}  // namespace sgemm_mi355x
