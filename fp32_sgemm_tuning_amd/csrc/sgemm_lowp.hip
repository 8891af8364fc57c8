// GEMM with BF16 or FP16 inputs and FP32 accumulation and output:
// C = alpha * A * B + beta * C, A [M,K] and B [K,N] row-major 16-bit, C
// [M,N] row-major FP32.  (Built with MFMA results in VGPRs; see
// sgemm_lean.hpp.)
//
// The kernel is the lean direct-to-LDS design on 16-bit data, with
// v_mfma_f32_16x16x32_{bf16,f16} (16x16 outputs, 32 k per instruction).
// Lane layout of that instruction (checked on gfx950 with a probe): lane l
// supplies A[l%16][8*(l/16) + e] and B[8*(l/16) + e][l%16], e = 0..7, and
// receives D[4*(l/16) + r][l%16], r = 0..3.
//
//   - A stage: rows of the K tile.  BK = 64 gives 128-byte rows in the
//     swizzled layout of the FP32 kernels (16-byte chunk c of row m at
//     c ^ ((m/2) % 8)); BK = 32 gives 64-byte rows, two 16-row slabs per
//     128-byte LDS row (the FP32 kernels' BK = 16 layout).  One ds_read_b128
//     at chunk 4s + l/16 of row m is the A fragment of k step s.
//   - B stays in its stored orientation, [k][n] with n contiguous, and is
//     read with the LDS transpose read ds_read_b64_tr_b16.  Within each group
//     of 16 lanes it hands lane i element e of the 8-byte row that source lane
//     4e + i/4 points at, taken at element i%4.  So when the 16 lanes of group
//     g point at rows k0 + 8g + {0..3} and column runs n0 + 4*{0..3}, lane i
//     receives B[k0 + 8g + e][n0 + i], e = 0..3: two such reads (rows +0 and
//     +4) make the B fragment of one 16-column block.  The 32-byte units of a
//     B row are XOR-swizzled (lowp_b_slot) so that the reads are free of bank
//     conflicts.
//   - The product is formed transposed (B fragment first), so each lane holds
//     four consecutive columns of one C row: 16-byte C stores.
//   - NSTAGE LDS stages: the loads of K tile t + NSTAGE are issued while tile
//     t is multiplied, so NSTAGE - 1 tiles are in flight; one barrier per
//     tile, placed behind the first MFMAs of a step.
//   - PP (alternating schedule, eight waves): the waves split into two groups
//     of four, one wave of each per SIMD, that alternate fragment reads and
//     MFMAs half a tile apart, so that on every SIMD one wave multiplies
//     while the other reads.
//   - Loads, edges, K remainder and per-tile descriptors as in the lean FP32
//     kernel, on 16-byte chunks of 8 elements: N and K must be multiples of 8
//     and the operands' rows 16-byte aligned; other shapes take the plain
//     kernel with 16-bit loads.
//   - SPLIT (the 128x128 two-stage and alternating kernels): blockIdx.y
//     takes its share of the K tiles and the split-K hand-off of the FP32
//     kernels adds the partial tiles in a fixed order.
#include "sgemm_lean.hpp"

namespace sgemm_mi355x {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 *lds_i16x4_ptr;

// f(IntC<I>{}) for I = 0 .. N-1, unrolled at compile time.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(IntC<I>{});
        static_for<I + 1, N>(f);
    }
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma_16x16x32(i32x4 a, i32x4 b, f32x4 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

// Slot of 16-byte chunk c in row k of a [k][x] stage (B, or A stored
// transposed): the 32-byte units of a row are XORed with (k % 4) +
// 4 * ((k / 8) % 2).  A transposed read takes
// four rows k..k+3 per group of 16 lanes, and the hardware pairs the groups
// {0,1} and {2,3} of a wave, whose rows differ by 8: measured free of bank
// conflicts on gfx950 (the XOR with k % 4 alone measured two-way conflicts).
__host__ __device__ constexpr int lowp_b_slot(int c, int k) {
    return 2 * ((c >> 1) ^ ((k & 3) | (((k >> 3) & 1) << 2))) + (c & 1);
}

// 16-byte direct load of one chunk per lane into LDS at lds_base + 16 *
// lane, through the buffer descriptor {base, range} (raw, stride 0: an
// offset at or past `range` loads zeros and touches no memory).  Written as
// inline assembly on purpose: the compiler's wait insertion treats every
// LDS transpose read issued after a direct-to-LDS load it knows of as a
// possible reader of that load and waits for all loads in flight first,
// which would serialise the K pipeline.  Ordering is explicit instead: the
// stage a load writes is read only after a wait on vmcnt and a barrier.
__device__ __forceinline__ void dma16_lowp(const char *base, int range, unsigned lds_base, int voffset) {
    // every operand but the lane offset is wave-uniform; readfirstlane keeps
    // it in scalar registers where the compiler cannot prove that by itself
    const unsigned long b = reinterpret_cast<unsigned long>(base);
    const i32x4 rsrc = {__builtin_amdgcn_readfirstlane((int)(unsigned)b),
                        __builtin_amdgcn_readfirstlane((int)((unsigned)(b >> 32) & 0xffffu)),
                        __builtin_amdgcn_readfirstlane(range), 0x00020000};
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane((int)lds_base))
                 : "memory", "m0");
}

// Number of N items placed at or before slot q when spread evenly over the
// SPAN slots from FIRST on (all of them from the last slot on).
constexpr int spread_upto(int q, int N, int FIRST, int SPAN) {
    return q < FIRST ? 0 : (q >= FIRST + SPAN - 1 || (q - FIRST) * N / SPAN + 1 > N ? N : (q - FIRST) * N / SPAN + 1);
}

// s_waitcnt with vmcnt <= N, lgkmcnt 0 and expcnt at its maximum (gfx9
// encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}

// BM x BN block tile, WAVES_M x WAVES_N waves, NSTAGE LDS stages of one
// BK-deep K tile each (BK = 64: two k steps per tile, A rows of 128 bytes;
// BK = 32: one k step, A rows of 64 bytes in the paired-slab layout).
// SPLIT: split-K, gridDim.y blocks per output tile, each on a contiguous
// share of the K tiles (the remainder tile with the first), combined by
// split_reduce_n as in the FP32 lean kernel.
// TA / TB: A stored as A^T ([K][M], element (i,k) at A[k*lda + i]) / B as
// B^T ([N][K], element (k,j) at B[j*ldb + k]).  Each operand keeps its
// stored orientation in LDS: an operand stored k-contiguous (A, or B^T) sits
// in the A-stage layout and is read with ds_read_b128; one stored
// m- or n-contiguous (B, or A^T) sits in the swizzled [k][x] layout and is
// read with the transpose read.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int NSTAGE, bool PP, bool BETA0, bool EDGE, bool F16,
          bool SPLIT, bool TA = false, bool TB = false>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
sgemm_lowp_kernel(Args p) {
    static_assert(BK == 32 || BK == 64, "K tile");
    static_assert(!PP || WAVES_M * WAVES_N == 8, "the alternating schedule runs 8 waves");
    using AL = ALayout<BK / 2>;                             // A stage layout (its unit is 4 bytes)
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int MI = WM / 16, NB = WN / 16;               // 16x16 blocks per wave
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2, STAGE = A_BYTES + B_BYTES;
    constexpr int NA = A_BYTES / 16 / NT, NBL = B_BYTES / 16 / NT;
    constexpr int L = NA + NBL;                             // 16-byte loads per lane per K tile
    constexpr int AROW = BM * 2, ACH = BM / 8;              // [k][m] A stage (TA): bytes, chunks per row
    constexpr int BROW = BN * 2, BCH = BN / 8;              // [k][n] B stage (!TB): bytes, chunks per row
    constexpr int NRB = TB ? NB : 2 * NB;                   // B fragment reads per k step
    constexpr int NM = MI * NB;                             // MFMAs per k step
    constexpr int QSYNC = NM / 4 > NB ? NM / 4 : NB;        // MFMAs of a step ahead of the barrier
    static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "wave tile");
    static_assert(A_BYTES % (16 * NT) == 0 && B_BYTES % (16 * NT) == 0, "load split");
    static_assert((TB || BN % 128 == 0) && (!TA || BM % 128 == 0),
                  "the [k][x] swizzle needs eight 32-byte units per row");
    static_assert(NSTAGE >= 2 && NSTAGE * STAGE <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) char lds[NSTAGE * STAGE];

    batch_offset<2>(p);                                     // problem blockIdx.z of a strided batch
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    const int slot = tile_coords(p, tm, tn);          // split-K workspace slot
    const int m0 = tm * BM, n0 = tn * BN;
    const char *Ab = reinterpret_cast<const char *>(p.A);
    const char *Bb = reinterpret_cast<const char *>(p.B);

    // Direct-load coordinates of load i of this lane, 16-byte chunk u of the
    // operand's stage: a k-contiguous stage gives (row x, chunk c = 8
    // elements of k), a [k][x] stage (row k, chunk c = 8 elements of x).
    // k8: the chunk's first k (compared with kr for the K remainder tile).
    auto coords = [&](bool kcontig, int xch, int i, int &x, int &c, int &k8) {
        const int u = (i * NWAVES + wave) * 64 + lane;
        if (kcontig) {
            AL::inverse(u, x, c);
            k8 = 8 * c;                                     // first k of the chunk
        } else {
            const int k = u / xch;
            c = lowp_b_slot(u % xch, k);                    // the swizzle is its own inverse
            x = 8 * c;                                      // first x of the chunk
            k8 = k;
        }
    };
    unsigned offA[NA], offB[NBL];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        int x, c, k;
        coords(!TA, ACH, i, x, c, k);
        const bool out = EDGE && m0 + x >= p.M;
        offA[i] = out ? kOutOfRange : 2u * (unsigned)(TA ? k * (int)p.lda + 8 * c : x * (int)p.lda + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
        int x, c, k;
        coords(TB, BCH, i, x, c, k);
        const bool out = EDGE && n0 + x >= p.N;
        offB[i] = out ? kOutOfRange : 2u * (unsigned)(TB ? x * (int)p.ldb + 8 * c : k * (int)p.ldb + 8 * c);
    }

    // K remainder: k in [K - kr, K), taken first; full tiles from k = 0, on
    // the operands' own alignment (as in the lean FP32 kernel)
    const int kr = EDGE ? p.K % BK : 0;
    const int tail = kr != 0;
    const long kfull = (long)p.K - kr;
    // K tiles of this block: all of them, or this split's share; ntiles
    // counts this block's tiles, t_first is the first one's index
    int t_first = 0, ntiles = p.K / BK + tail;
    if constexpr (SPLIT) {
        const int S = gridDim.y, y = blockIdx.y, total = ntiles;
        t_first = (int)((long)total * y / S);
        ntiles = (int)((long)total * (y + 1) / S) - t_first;
    }
    const bool remainder_first = tail && t_first == 0;
    // Per-tile descriptors: the block's part of one K tile of each stored
    // operand (rows up to M or N, BK deep), based at that tile.
    // (untransposed B is read in whole 8-element chunks: its range covers N
    // rounded up to a chunk, which the library's padded copies hold)
    const long rowsA = min(BM, p.M - m0), colsB = TB ? min(BN, p.N - n0) : min(BN, (p.N - n0 + 7) & ~7);
    const int rangeA = (int)(TA ? 2L * ((long)(BK - 1) * p.lda + rowsA) : 2L * ((rowsA - 1) * p.lda + BK));
    const int rangeB = (int)(TB ? 2L * ((colsB - 1) * p.ldb + BK) : 2L * ((long)(BK - 1) * p.ldb + colsB));
    const char *cornerA = TA ? Ab + 2L * m0 : Ab + 2L * m0 * p.lda;
    const char *cornerB = TB ? Bb + 2L * n0 * p.ldb : Bb + 2L * n0;
    const long kstrideA = TA ? p.lda : 1, kstrideB = TB ? 1 : p.ldb;
    // LDS byte address of a point in the stages (wave-uniform)
    const unsigned lds0 = (unsigned)reinterpret_cast<uintptr_t>((lds_addr_t)lds);
    // LDS address of this wave's 1 KiB of load g in stage `st` (A loads
    // first, then B)
    auto dst = [&](int st, int g) {
        return lds0 + (unsigned)(st * STAGE + (g < NA ? 0 : A_BYTES) + ((g < NA ? g : g - NA) * NWAVES + wave) * 1024);
    };
    // load g of K tile t into stage `st`.  Tiles past the last get an empty
    // range: their loads touch no memory and write zeros, so every tile
    // issues the same number of loads and the vmcnt waits stay constant.
    auto issue_one = [&](int t, int st, int g) {
        const bool live = t < ntiles;
        const long kfirst = (long)max(t_first + t - tail, 0) * BK;
        if (g < NA)
            dma16_lowp(cornerA + 2 * kfirst * kstrideA, live ? rangeA : 0, dst(st, g), (int)offA[g]);
        else
            dma16_lowp(cornerB + 2 * kfirst * kstrideB, live ? rangeB : 0, dst(st, g), (int)offB[g - NA]);
    };
    auto issue_remainder = [&]() {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            int x, c, k;
            coords(!TA, ACH, i, x, c, k);
            dma16_lowp(cornerA + 2 * kfull * kstrideA, rangeA, dst(0, i), (int)(k < kr ? offA[i] : kOutOfRange));
        }
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            int x, c, k;
            coords(TB, BCH, i, x, c, k);
            dma16_lowp(cornerB + 2 * kfull * kstrideB, rangeB, dst(0, NA + i), (int)(k < kr ? offB[i] : kOutOfRange));
        }
    };

    // Fragments of one k step (32 k): A per 16-row slab, B per 16-column
    // block.  The B fragments are double-buffered (every MFMA of a step uses
    // all of them).  The A fragments are not: the MFMAs run slab by slab and
    // slab mi's fragment for the next step is read right after its last
    // MFMA of this step, which keeps the 256x256 tile within 256 VGPRs.
    const int lrow = lane & 15, lg = lane >> 4;
    i32x4 fa[MI];
    i32x4 fb[2][NB];
    // the two transposed 8-byte reads of one 16-wide block of a [k][x] stage
    // (row length ROW bytes) at x0: lane l gets x0 + l%16, k = 32s + 8(l/16) + e
    auto read_tr = [&](const char *base, int rowbytes, int x0, int s, i32x4 &f) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int k = 32 * s + 8 * lg + 4 * half + (lrow >> 2);
            const int x = x0 + 4 * (lrow & 3);
            const char *addr = base + k * rowbytes + 16 * lowp_b_slot(x >> 3, k) + 8 * ((x >> 2) & 1);
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(addr));
            const i32x2 w = __builtin_bit_cast(i32x2, v);
            f[2 * half] = w[0];
            f[2 * half + 1] = w[1];
        }
    };
    auto read_a_into = [&](int mi, const char *stage, int s, i32x4 *f) {
        if constexpr (TA) {
            read_tr(stage, AROW, wm * WM + mi * 16, s, f[mi]);
        } else {
            const int m = wm * WM + mi * 16 + lrow;
            f[mi] = *reinterpret_cast<const i32x4 *>(stage + 4 * AL::offset(m, 4 * s + lg));
        }
    };
    auto read_a = [&](int mi, const char *stage, int s) { read_a_into(mi, stage, s, fa); };
    // B read r of k step s: from a [k][n] stage, block r/2 and its
    // transposed 8-byte read r%2; from an [n][k] stage (TB), block r
    auto read_b = [&](int r, const char *stage, int s, i32x4 *f) {
        if constexpr (TB) {
            const int n = wn * WN + 16 * r + lrow;
            f[r] = *reinterpret_cast<const i32x4 *>(stage + A_BYTES + 4 * AL::offset(n, 4 * s + lg));
        } else {
            const int nb = r / 2, half = r % 2;
            const int k = 32 * s + 8 * lg + 4 * half + (lrow >> 2);
            const int n = wn * WN + 16 * nb + 4 * (lrow & 3);
            const int c = n >> 3;
            const char *addr = stage + A_BYTES + k * BROW + 16 * lowp_b_slot(c, k) + 8 * ((n >> 2) & 1);
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(addr));
            const i32x2 w = __builtin_bit_cast(i32x2, v);
            f[nb][2 * half] = w[0];
            f[nb][2 * half + 1] = w[1];
        }
    };

    // The product is formed transposed: the B fragment is the instruction's
    // first operand and the A fragment its second, so block (mi, nb) holds
    // C^T and lane l receives C[row l%16][columns 4*(l/16) .. +3].
    f32x4 acc[MI][NB];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mi][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One k step: MFMA q = (slab q / NB, block q % NB) from fa and fb[BC].
    // After MFMA QB-1 (QB a multiple of NB; before MFMA 0 when QB is 0) the
    // `sync` hook runs; every read of the step comes after it.  After a
    // slab's last MFMA (and the hook) its A fragment of step `s` of stage
    // `rs` is read; the B reads of that step
    // go into fb[1 - BC], spread from the hook to 3/4 of the step; the G
    // direct loads are spread from the hook to the end.
    auto step = [&](auto bc, const char *rs, int s, auto qb, auto gcount, auto &&sync, auto &&issue) {
        constexpr int BC = decltype(bc)::value;
        constexpr int QB = decltype(qb)::value;
        constexpr int G = decltype(gcount)::value;
        constexpr int FIRST = QB > 0 ? QB - 1 : 0;
        constexpr int RSPAN = NM * 3 / 4 - FIRST, GSPAN = NM - FIRST;
        static_assert(QB <= NM && RSPAN > 0, "the reads need MFMAs after the hook");
        if constexpr (QB == 0) {
            sync();
            __builtin_amdgcn_sched_barrier(0);
        }
        static_for<0, NM>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            acc[q / NB][q % NB] = mfma_16x16x32<F16>(fb[BC][q % NB], fa[q / NB], acc[q / NB][q % NB]);
            if constexpr (q == QB - 1) {
                __builtin_amdgcn_sched_barrier(0);
                sync();
                __builtin_amdgcn_sched_barrier(0);
            }
            // slab mi is read after its last MFMA, and not before the hook
            if constexpr (q == QB - 1)
                static_for<0, QB / NB>([&](auto mc) { read_a(decltype(mc)::value, rs, s); });
            if constexpr (q % NB == NB - 1 && q >= QB) read_a(q / NB, rs, s);
            static_for<spread_upto(q - 1, NRB, FIRST, RSPAN), spread_upto(q, NRB, FIRST, RSPAN)>(
                [&](auto r) { read_b(decltype(r)::value, rs, s, fb[1 - BC]); });
            static_for<spread_upto(q - 1, G, FIRST, GSPAN), spread_upto(q, G, FIRST, GSPAN)>(
                [&](auto g) { issue(decltype(g)::value); });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Wait until tile t+1 has landed (the loads of the NSTAGE-2 tiles after
    // it may stay in flight) and this wave's reads are done, then the
    // barrier: every wave's part of tile t+1 is in LDS and no wave still
    // reads the stage the next loads overwrite.
    auto sync_tile = [&]() {
        wait_vm_lgkm0<(NSTAGE - 2) * L>();
        __builtin_amdgcn_s_barrier();
    };
    // Race-check build (SGEMM_LDS_POISON, see sgemm_lean.hpp): NaN bits into
    // the LDS units this lane's loads of stage `st` fill, landed before those
    // loads are issued.
    auto poison = [&](int st) {
        if constexpr (SGEMM_LDS_POISON) {
#pragma unroll
            for (int g = 0; g < L; ++g)
                *reinterpret_cast<i32x4 *>(lds + (dst(st, g) - lds0) + 16 * lane) = i32x4{-1, -1, -1, -1};
            wait_lgkmcnt0();
        }
    };
    // BK = 64: one K tile in stage SC.  Step 0 reads step 1 of the same
    // stage.  Step 1 runs its first MFMAs, syncs, then reads step 0 of tile
    // t+1 and loads tile t+NSTAGE into SC.  BK = 32: the one step of tile t
    // (B fragments in fb[P]) runs its first MFMAs, syncs, loads tile
    // t+NSTAGE into SC and reads tile t+1.  The MFMAs before the barrier
    // keep the matrix unit busy while the waves meet.
    auto tile = [&](int t, auto sc, auto pc) {
        constexpr int SC = decltype(sc)::value;
        constexpr int SN = (SC + 1) % NSTAGE;
        const char *cs = lds + SC * STAGE;
        const char *ns = lds + SN * STAGE;
        auto none = [&](int) {};
        if constexpr (BK == 64) {
            step(IntC<0>{}, cs, 1, IntC<0>{}, IntC<0>{}, [&]() {}, none);
            step(IntC<1>{}, ns, 0, IntC<QSYNC>{}, IntC<L>{},
                 [&]() {
                     sync_tile();
                     poison(SC);     // every wave's reads of SC are done
                 },
                 [&](int g) { issue_one(t + NSTAGE, SC, g); });
        } else {
            step(pc, ns, 0, IntC<QSYNC>{}, IntC<0>{},
                 [&]() {
                     sync_tile();
                     poison(SC);
#pragma unroll
                     for (int g = 0; g < L; ++g) issue_one(t + NSTAGE, SC, g);
                 },
                 none);
        }
    };

    if constexpr (PP) {
        if (ntiles > 0) {
            // Alternating schedule: waves 0-3 and 4-7 share the four SIMDs,
            // one of each per SIMD.  Each wave alternates a memory phase
            // (fragment reads of tile t from LDS, the loads of tile
            // t+NSTAGE-1) and a compute phase (the MFMAs of tile t), and the
            // second group runs one phase behind the first, so that on every
            // SIMD one wave multiplies while the other reads.  Every phase
            // ends with a barrier of all eight waves.
            const int group = wave >> 2;
            static_for<0, NSTAGE>([&](auto sc) { poison(decltype(sc)::value); });
            if (remainder_first) {
                issue_remainder();
            } else {
#pragma unroll
                for (int g = 0; g < L; ++g) issue_one(0, 0, g);
            }
            static_for<1, NSTAGE - 1>([&](auto sc) {
#pragma unroll
                for (int g = 0; g < L; ++g) issue_one(decltype(sc)::value, decltype(sc)::value, g);
            });
            wait_vm_lgkm0<(NSTAGE - 2) * L>();
            __builtin_amdgcn_s_barrier();
            if (group) __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            constexpr int KS = BK / 32;                     // k steps per tile
            i32x4 pa[KS][MI], pb[KS][NB];
            auto pp_tile = [&](int t, auto sc) {
                constexpr int SC = decltype(sc)::value;
                const char *cs = lds + SC * STAGE;
                // memory phase: fragments of tile t, loads of tile
                // t+NSTAGE-1 into the stage tile t-1 had (free: both groups
                // read it before the last barrier and waited for the reads)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) read_a_into(mi, cs, ks, pa[ks]);
#pragma unroll
                    for (int r = 0; r < NRB; ++r) read_b(r, cs, ks, pb[ks]);
                }
                poison((SC + NSTAGE - 1) % NSTAGE);
#pragma unroll
                for (int g = 0; g < L; ++g) issue_one(t + NSTAGE - 1, (SC + NSTAGE - 1) % NSTAGE, g);
                __builtin_amdgcn_sched_barrier(0);
                // the next phase of the other group reads tile t (group 0)
                // or tile t+1 (group 1): this wave's loads of it have landed
                if (group) wait_vm_lgkm0<(NSTAGE - 2) * L>();
                else wait_vm_lgkm0<(NSTAGE - 1) * L>();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                // compute phase
                static_for<0, KS * NM>([&](auto qc) {
                    constexpr int ks = decltype(qc)::value / NM, q = decltype(qc)::value % NM;
                    acc[q / NB][q % NB] = mfma_16x16x32<F16>(pb[ks][q % NB], pa[ks][q / NB], acc[q / NB][q % NB]);
                });
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_lgkm0<(NSTAGE - 2) * L>();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            };
            for (int t0 = 0; t0 < ntiles; t0 += NSTAGE) {
                static_for<0, NSTAGE>([&](auto uc) {
                    const int t = t0 + decltype(uc)::value;
                    if (t < ntiles) pp_tile(t, uc);
                });
            }
            if (!group) __builtin_amdgcn_s_barrier();
            wait_vmcnt0();
        }
    } else if (ntiles > 0) {
        static_for<0, NSTAGE>([&](auto sc) { poison(decltype(sc)::value); });
        if (remainder_first) {
            issue_remainder();
        } else {
#pragma unroll
            for (int g = 0; g < L; ++g) issue_one(0, 0, g);
        }
        static_for<1, NSTAGE>([&](auto sc) {
#pragma unroll
            for (int g = 0; g < L; ++g) issue_one(decltype(sc)::value, decltype(sc)::value, g);
        });
        wait_vm_lgkm0<(NSTAGE - 1) * L>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) read_a(mi, lds, 0);
#pragma unroll
        for (int r = 0; r < NRB; ++r) read_b(r, lds, 0, fb[0]);
        // unrolled so that the stage (and for BK = 32 the B buffer) of
        // every tile is a compile-time constant
        constexpr int U = (BK == 32 && NSTAGE % 2) ? 2 * NSTAGE : NSTAGE;
        for (int t0 = 0; t0 < ntiles; t0 += U) {
            static_for<0, U>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                const int t = t0 + u;
                if (t < ntiles) tile(t, IntC<u % NSTAGE>{}, IntC<u % 2>{});
            });
        }
        // drain: the loads of the tiles past the last write zeros into LDS
        // and must land before the workgroup ends
        wait_vmcnt0();
    }

    if constexpr (SPLIT) {
        if (!split_reduce_n<NT, MI * NB>(p, slot, tid, reinterpret_cast<unsigned *>(lds),
                                         [&](int c) -> f32x4 & { return acc[c / NB][c % NB]; }))
            return;
    }

    // C = alpha * acc (+ beta * C): block (mi, nb) holds row l%16 and
    // columns 4*(l/16) .. +3 of its 16x16 output block; 16-byte accesses
    // when C's rows are 16-byte aligned and the four columns lie below N.
    // (N need not be a multiple of 4: the product on the library's padded
    // copies runs with the true N, so the last vector of a row may straddle
    // N; its columns are then stored one by one.)
    const float alpha = p.alpha, beta = p.beta;
    const bool vecc = (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && (p.ldc & 3) == 0;
    if constexpr (BETA0 || EDGE) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = m0 + wm * WM + mi * 16 + lrow;
                const int col = n0 + wn * WN + nb * 16 + 4 * lg;
                if (EDGE && row >= p.M) continue;
                float *dst = p.C + (long)row * p.ldc + col;
                if (vecc && (!EDGE || col + 3 < p.N)) {
                    f32x4 o = acc[mi][nb] * alpha;
                    if (!BETA0) o += *reinterpret_cast<const f32x4 *>(dst) * beta;
                    *reinterpret_cast<f32x4 *>(dst) = o;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (EDGE && col + r >= p.N) continue;
                        float o = alpha * acc[mi][nb][r];
                        if (!BETA0) o += beta * dst[r];
                        dst[r] = o;
                    }
                }
            }
        return;
    }
    // Whole tiles with beta != 0: the C values of a row group's NB blocks
    // are loaded before the first of their stores.  Each is read and written
    // by this lane alone and the rows of C are disjoint (ldc >= N), so the
    // order is free, and the loads wait for memory once per row group
    // instead of once per block (a compiler cannot move a load above a store
    // it cannot prove disjoint).  The 16-byte test of C is taken once,
    // outside the loops, so that no branch splits a row group's loads from
    // its stores.  (4096^3 BF16, alpha = beta = 1: 117.7 -> 112.3 us.  Edge
    // tiles keep the per-block order: their guarded loads, made branch-free,
    // ran slower than the waits they saved.)
    auto write = [&](auto vec_c) __attribute__((always_inline)) {
        constexpr bool VC = decltype(vec_c)::value;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int row = m0 + wm * WM + mi * 16 + lrow;
            f32x4 cin[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float *src = p.C + (long)row * p.ldc + n0 + wn * WN + nb * 16 + 4 * lg;
                if constexpr (VC) {
                    cin[nb] = *reinterpret_cast<const f32x4 *>(src);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) cin[nb][r] = src[r];
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float *dst = p.C + (long)row * p.ldc + n0 + wn * WN + nb * 16 + 4 * lg;
                if constexpr (VC) {
                    *reinterpret_cast<f32x4 *>(dst) = acc[mi][nb] * alpha + cin[nb] * beta;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[r] = alpha * acc[mi][nb][r] + beta * cin[nb][r];
                }
            }
        }
    };
    if (vecc) write(std::true_type{});
    else write(std::false_type{});
}

template <int BM, int BN, int BK, int WM, int WN, int NSTAGE, bool F16, bool PP, bool SPLIT, bool TA = false,
          bool TB = false>
hipError_t launch_lowp(const Args &a0, hipStream_t stream, int batch = 1) {
    const Args a = tiled(a0, BM, BN);
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)(SPLIT ? a.splits : 1), (unsigned)batch);
    const dim3 block(64 * WM * WN);
    const bool edge = (a.M % BM) || (a.N % BN) || (a.K % BK);
#define SGEMM_LAUNCH(Z, E) \
    launch_k(sgemm_lowp_kernel<BM, BN, BK, WM, WN, NSTAGE, PP, Z, E, F16, SPLIT, TA, TB>, grid, block, stream, a)
    if (edge) {
        if (a.beta == 0.0f) return SGEMM_LAUNCH(true, true);
        return SGEMM_LAUNCH(false, true);
    }
    if (a.beta == 0.0f) return SGEMM_LAUNCH(true, false);
    return SGEMM_LAUNCH(false, false);
#undef SGEMM_LAUNCH
}

// One alternating kernel with each of the four operand orientations (SP:
// its split-K form).
template <int BM, int BN, int BK, int NS, bool SP>
hipError_t launch_lowp_alt_op(const Args &a, bool f16, bool ta, bool tb, int batch, hipStream_t s) {
#define SGEMM_O(F, A, B) launch_lowp<BM, BN, BK, 2, 4, NS, F, true, SP, A, B>(a, s, batch)
    if (f16) {
        if (ta && tb) return SGEMM_O(true, true, true);
        if (ta) return SGEMM_O(true, true, false);
        if (tb) return SGEMM_O(true, false, true);
        return SGEMM_O(true, false, false);
    }
    if (ta && tb) return SGEMM_O(false, true, true);
    if (ta) return SGEMM_O(false, true, false);
    if (tb) return SGEMM_O(false, false, true);
    return SGEMM_O(false, false, false);
#undef SGEMM_O
}

// Launcher called from the C ABI's translation unit; `tile` picks the block
// tile, K tile, waves and number of stages (the table of variants in the C
// ABI's translation unit lists them in this order).  a.splits > 1 runs the
// split-K form (built for the 128x128 two-stage kernel and the 128x128
// alternating kernel); ta / tb (transposed operands) are built for the two
// alternating kernels; batch problems on gridDim.z.  Returns the launch's
// status.
hipError_t launch_lowp_tile(const Args &a, bool f16, int tile, bool ta, bool tb, int batch, hipStream_t s) {
#define SGEMM_T(BM, BN, BK, WM, WN, NS, PP, SP)                                          \
    (f16 ? launch_lowp<BM, BN, BK, WM, WN, NS, true, PP, SP>(a, s, batch)                \
         : launch_lowp<BM, BN, BK, WM, WN, NS, false, PP, SP>(a, s, batch))
    const bool split = a.splits > 1;
    switch (tile) {
        case 1: return SGEMM_T(256, 128, 64, 2, 4, 3, false, false);
        case 2: return SGEMM_T(256, 256, 32, 2, 4, 4, false, false);
        case 3: return launch_lowp_alt_op<256, 256, 32, 4, false>(a, f16, ta, tb, batch, s);
        case 4:
            if (split) return launch_lowp_alt_op<128, 128, 64, 4, true>(a, f16, ta, tb, batch, s);
            return launch_lowp_alt_op<128, 128, 64, 4, false>(a, f16, ta, tb, batch, s);
        default:
            if (split) return SGEMM_T(128, 128, 64, 2, 2, 2, false, true);
            return SGEMM_T(128, 128, 64, 2, 2, 2, false, false);
    }
#undef SGEMM_T
}

}  // namespace sgemm_mi355x
