// Lean direct-to-LDS SGEMM kernel and its launch template.
//
// Included only by the translation units sgemm_lean*.hip, which are compiled
// with MFMA results kept in ordinary VGPRs (-mllvm -amdgpu-mfma-vgpr-form).
// With the default accumulation registers the two-stage unrolled loop below
// gets accumulator copies between the unrolled halves and fragment round
// trips through the accumulation file, one VALU copy for every five MFMAs;
// in VGPR form the K loop is MFMAs, LDS reads, direct loads and a few scalar
// instructions only.  The flag applies to a whole translation unit, and
// kernels of the shared header that hold 256 accumulators per lane do not
// fit 256 VGPRs, hence the separate files.  Only wave tiles of up to 64x128
// outputs are instantiated from here.  The instantiations are spread over
// three translation units so that they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "sgemm_kernels.hpp"

namespace sgemm_mi355x {

// A buffer offset past every descriptor's range (ranges are below 2^31).
constexpr unsigned kOutOfRange = 0x80000000u;

// Race-check build.  With SGEMM_LDS_POISON set to 1 (a separate build of
// these kernels, libsgemm_poison.so), every LDS stage is filled with NaN
// bits (0xFFFFFFFF: NaN as FP32, BF16 and FP16) as soon as its last reader
// has passed the barrier that frees it, and before the direct loads that
// refill it are issued; the split-K ticket word holds the same bits between
// its two barriers.  A barrier missing or misplaced then lets a wave read
// NaN, or an invalid ticket, and the result goes wrong whatever the timing,
// where the plain build would read stale or half-written values that happen
// to be right most of the time.  The counterpart of running each thread as
// far as it can go before switching, which makes a missing barrier give a
// wrong answer every time ("Matmul I: tiling and shared memory", section 6,
// note 3).
#ifndef SGEMM_LDS_POISON
#define SGEMM_LDS_POISON 0
#endif
constexpr unsigned kPoisonBits = 0xFFFFFFFFu;

// s_waitcnt with lgkmcnt 0 and the other counters at their maximum: the
// wave's LDS writes have landed (gfx9 encoding, as wait_vmcnt0 below).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// One direct load per lane into LDS: 16 or 4 bytes from the buffer at
// voffset + soffset to the LDS address of `dst` plus 16 or 4 bytes per lane.
// (The size must be a literal at the call, hence one function per size.)
typedef __attribute__((address_space(3))) void *lds_addr_t;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_addr_t dst, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voffset, soffset, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, lds_addr_t dst, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voffset, soffset, 0, 0);
}
template <bool DW>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, lds_addr_t dst, int voffset, int soffset) {
    if constexpr (DW)
        dma4(r, dst, voffset, soffset);
    else
        dma16(r, dst, voffset, soffset);
}

// s_waitcnt with vmcnt 0 and the other counters at their maximum
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Split-K hand-off of one output tile.  Every block stores its partial
// accumulators (NACC 16-byte chunks per thread, acc(c) for chunk c) to
// workspace slot blockIdx.y of the tile (chunk-major: chunk c of thread t at
// c * NT + t, so each store and load instruction covers one contiguous run)
// and takes a ticket from the tile's counter.  The tiles of problem
// blockIdx.z of a strided batch follow those of the problems before it, in
// the partials and in the counters.  Returns false
// for all blocks but the last; the last one reads all partials back, leaves
// their sum in split order in acc and resets the counter for the next call.
// The ticket is shared through word 0 of the kernel's own LDS buffer
// (`ticket`), free by then: the barrier below follows every wave's last LDS
// read and its last direct-to-LDS load.  A second LDS object would cost the
// whole K loop: the compiler then no longer tells the direct-to-LDS writes
// apart from the fragment reads and waits for every load to land before the
// next LDS read.
//
// Every XCD has its own L2, so the partials move at device scope: the
// stores and loads carry the device-scope cache policy (sc1, the encoding
// the compiler uses for relaxed agent-scope atomics), each block waits for
// its stores to complete before the barrier that precedes its ticket, and
// the ticket is a device-scope atomic.  No cache-wide write-back or
// invalidate is needed, so other blocks keep their cached A and B.
template <int NT, int NACC, class Ref>
__device__ __forceinline__ bool split_reduce_n(const Args &p, int tile_id, int tid, unsigned *ticket, Ref &&acc) {
    constexpr int TILE = NT * NACC * 4;                 // floats per partial tile
    constexpr int kDeviceScope = 16;                    // cache policy bits: sc1
    const int S = gridDim.y, y = blockIdx.y;
    const long tile = (long)blockIdx.z * gridDim.x + tile_id;
    const __amdgpu_buffer_rsrc_t slab = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.ws + tile * S * TILE), (short)0, S * TILE * 4, 0x00020000);
#pragma unroll
    for (int c = 0; c < NACC; ++c)
        __builtin_amdgcn_raw_buffer_store_b128(acc(c), slab, (c * NT + tid) * 16, y * TILE * 4, kDeviceScope);
    wait_vmcnt0();
    __syncthreads();
    if (tid == 0) {
        if constexpr (SGEMM_LDS_POISON) *reinterpret_cast<volatile unsigned *>(ticket) = kPoisonBits;
        *ticket = atomicAdd(p.counters + tile, 1u);
    }
    __syncthreads();
    if (*ticket != (unsigned)(S - 1)) return false;
    // every partial, this block's own included, is read back in split
    // order, so the sum needs no registers beyond the accumulators
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int c = 0; c < NACC; ++c) {
            const f32x4 x =
                __builtin_amdgcn_raw_buffer_load_b128(slab, (c * NT + tid) * 16, s * TILE * 4, kDeviceScope);
            acc(c) = s == 0 ? x : acc(c) + x;
        }
    }
    if (tid == 0) atomicExch(p.counters + tile, 0u);
    return true;
}

// The same for the FP32 lean kernels' accumulator layout.
template <class T>
__device__ __forceinline__ bool split_reduce(const Args &p, int tile_id, int tid, unsigned *ticket,
                                             f32x4 (&acc)[T::MI][T::NJ][4]) {
    return split_reduce_n<T::NT, T::MI * T::NJ * 4>(
        p, tile_id, tid, ticket, [&](int c) -> f32x4 & { return acc[c / (T::NJ * 4)][(c / 4) % T::NJ][c % 4]; });
}

// ---------------------------------------------------------------------------
// Lean direct-to-LDS kernel: the section schedule of sgemm_dtl_kernel with
// the per-tile address arithmetic taken out of the K loop.
//
// In the K loop of the direct-to-LDS kernel about a quarter of the issued
// instructions besides the MFMAs were address arithmetic: reading the wave
// index back into a scalar for M0, 64-bit adds advancing every load address
// per tile, and ORs placing the runtime stage base into every LDS read
// address.  Here
//   - the wave index is wave-uniform (a scalar), so M0 is scalar arithmetic;
//   - the direct loads are buffer loads (buffer_load_dwordx4 ... lds): a
//     wave-uniform descriptor, a loop-invariant 32-bit per-lane byte offset
//     and a scalar offset that advances one tile per iteration;
//   - the tile loop is unrolled by the two LDS stages, so every fragment read
//     address is a loop-invariant register plus an immediate.
// The byte offsets within one K tile of the block's part of A and B must
// fit the 31-bit buffer range (BM * lda and BK * ldb, or for transposed
// operands BK * lda and BN * ldb, below 2^29 elements); the operands
// themselves may be of any size.
//
// DW = false: 16-byte loads (A, B, C 16-byte aligned, leading dimensions
// multiples of 4).  DW = true: 4-byte loads of single floats into the same
// LDS layout and 32-bit C access, for any alignment; four times the load
// instructions, and every edge below is exact to the element, so N and K
// need not be multiples of 4.
//
// TA / TB: A stored transposed ([K][M], element (m, k) at k * lda + m) / B
// stored transposed ([N][K], element (k, n) at n * ldb + k).  With 16-byte
// loads the operand keeps its stored orientation in LDS (TileOps describes
// the fragment reads; TA needs 64-row wave tiles, M a multiple of 4 for A's
// edge chunks, TB needs K a multiple of 4).  With 4-byte loads each lane
// picks the element that the untransposed LDS layout keeps at its position,
// so fragments, MFMAs and epilogue stay untransposed; the loads of one
// instruction then come from up to 32 rows of the stored operand.
//
// EDGE = false: M, N and K are whole numbers of tiles.  EDGE = true: any M
// and N, and any K of at least BK, with K and N multiples of 4 unless DW.
// The hardware range check of buffer loads does the edges without a branch
// in the K loop (it compares the per-lane offset with the descriptor's
// range):
//   - each descriptor covers the block's part of one K tile, which lies
//     inside its operand;
//   - elements of rows past M or columns past N get an offset beyond every
//     range (set once, before the K loop);
//   - a K remainder kr = K % BK is the last kr columns of A and rows of B,
//     k in [K - kr, K), taken as the first tile, whose elements past K get
//     that offset too; the full tiles follow, from k = 0, so they keep the
//     operands' own alignment (from k = kr every row segment of A would
//     start kr floats off a 16-byte boundary).
// Out-of-range loads access no memory and deposit zeros, which is what the
// K remainder needs (A's padding past column K may hold anything).  Rows past
// M and columns past N only reach accumulators that the guarded epilogue
// does not store.
//
// Strided batches: problem blockIdx.z, on pointers moved by the strides.
//
// SPLIT = true: split-K.  gridDim.y = S blocks share each output tile; block
// y takes K tiles [y * T / S, (y + 1) * T / S) of the T tiles (the remainder
// tile, if any, goes to y = 0), writes its partial tile to the workspace and
// counts itself in on the tile's counter.  The block that arrives last adds
// the S partials in the fixed order y = 0 .. S-1 (so the result does not
// depend on arrival order), resets the counter and runs the epilogue.  No
// block waits for another.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool BETA0, bool EDGE, bool SPLIT, bool DW, bool TA,
          bool TB>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
sgemm_lean_kernel(Args p) {
    batch_offset(p);
    // Transposed operands with 16-byte loads keep their stored orientation in
    // LDS (see TileOps); with 4-byte loads they are gathered into the
    // untransposed layout.
    constexpr bool LTA = TA && !DW, LTB = TB && !DW;
    // DW: 4-byte loads and 32-bit C access (any alignment), else 16-byte ones
    using T = TileOps<BM, BN, BK, WAVES_M, WAVES_N, !DW, EDGE, LTA, LTB>;
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int KH = T::KH;
    static_assert(KH == 2 || KH == 4, "BK must be 32 or 64");
    constexpr int EW = DW ? 1 : 4;                          // floats per lane per load
    constexpr int LSTEP = 64 * EW;                          // floats of LDS per load instruction
    constexpr int NA = BM * BK / EW / T::NT;
    constexpr int NB = BK * BN / EW / T::NT;
    constexpr int NM = T::MI * T::NJ * 16;
    constexpr int NR = T::NREAD;
    constexpr int LS = KH == 4 ? 2 : 1;                     // sections carrying the loads
    constexpr int PER = (NA + NB + LS - 1) / LS;
    __shared__ __attribute__((aligned(16))) float lds[2 * T::STAGE];
    typedef __attribute__((address_space(3))) void *lds_ptr;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    const int slot = tile_coords(p, tm, tn);          // split-K workspace slot
    const int m0 = tm * BM, n0 = tn * BN;

    // Loop-invariant per-lane byte offsets of the direct loads.  Load i of a
    // lane fills LDS unit u = (i * NWAVES + wave) * 64 + lane of the stage (a
    // 16-byte chunk, or with DW one float of chunk u / 4); the A offset is
    // that of the logical (row, k) the swizzled layout keeps there.
    auto a_coords = [&](int i, int &m, int &k) {
        const int u = (i * NWAVES + wave) * 64 + lane;
        if constexpr (LTA) {            // [BK][BM] stage (chunks swizzled for word reads)
            k = u / (BM / 4);
            const int slot = u % (BM / 4);
            m = 4 * (T::TA_W ? slot ^ T::ta_swz(k) : slot);
        } else {
            int c;
            ALayout<BK>::inverse(DW ? u / 4 : u, m, c);
            k = 4 * c + (DW ? u % 4 : 0);
        }
    };
    auto b_coords = [&](int i, int &r, int &col) {
        const int u = (i * NWAVES + wave) * 64 + lane;
        if constexpr (LTB) {            // [BN][BK] stage in the swizzled layout
            int c;
            ALayout<BK>::inverse(u, col, c);
            r = 4 * c;
        } else {
            const int g = u * EW;       // float index in the B stage
            r = g / BN;
            col = g % BN;
        }
    };
    // Element (m, k) of the A tile is at m * lda + k from the tile's corner,
    // or k * lda + m when A is stored transposed (TA); likewise (k, n) of B at
    // k * ldb + n, or n * ldb + k (TB).  Rows past M and columns past N get
    // an offset beyond every range (EDGE).
    unsigned offA[NA], offB[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        int m, k;
        a_coords(i, m, k);
        const int e = TA ? k * (int)p.lda + m : m * (int)p.lda + k;
        offA[i] = (EDGE && m0 + m >= p.M) ? kOutOfRange : 4u * (unsigned)e;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        int r, col;
        b_coords(i, r, col);
        const int e = TB ? col * (int)p.ldb + r : r * (int)p.ldb + col;
        offB[i] = (EDGE && n0 + col >= p.N) ? kOutOfRange : 4u * (unsigned)e;
    }
    // K remainder taken first (EDGE only): tile 0 covers k in [K - kr, K),
    // full tiles t >= 1 cover k from (t - 1) * BK.
    const int kr = EDGE ? p.K % BK : 0;
    const int tail = kr != 0;
    const long kfull = (long)p.K - kr;
    const int ntiles = p.K / BK + tail;
    // K tiles of this block: all of them, or this split's share
    int t_begin = 0, t_end = ntiles;
    if constexpr (SPLIT) {
        const int S = gridDim.y, y = blockIdx.y;
        t_begin = (int)((long)ntiles * y / S);
        t_end = (int)((long)ntiles * (y + 1) / S);
    }

    // Buffer descriptors.  Block corner at k = 0 in each stored operand and
    // its k stride.  Every K tile is loaded through descriptors based at that
    // tile (a 64-bit scalar base, a few scalar instructions per tile), so only
    // the offsets within one tile need to fit the 31-bit range and the
    // operands may be of any size.  The range of each descriptor is the extent
    // of the block's part of one tile (rows up to M, columns up to N, BK deep),
    // so every in-range load stays inside the operand, and the out-of-range
    // offset lies beyond it.
    const float *cornerA = TA ? p.A + m0 : p.A + (long)m0 * p.lda;
    const float *cornerB = TB ? p.B + (long)n0 * p.ldb : p.B + n0;
    const long kstrideA = TA ? p.lda : 1, kstrideB = TB ? 1 : p.ldb;
    const long rowsA = min(BM, p.M - m0), colsB = min(BN, p.N - n0);
    const int rangeA = (int)(TA ? 4L * ((long)(BK - 1) * p.lda + rowsA) : 4L * ((rowsA - 1) * p.lda + BK));
    const int rangeB = (int)(TB ? 4L * ((colsB - 1) * p.ldb + BK) : 4L * ((long)(BK - 1) * p.ldb + colsB));
    auto tile_rsrc = [](const float *corner, long kstride, long kfirst, int range) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)(corner + kfirst * kstride), (short)0, range, 0x00020000);
    };

    // Loads of tile t >= tail (a full tile, k from (t - tail) * BK).
    // (The explicit int conversions matter: with the array element passed as
    // is, the host pass drops the kernel and its launch stub.)
    auto issue_one = [&](int t, float *stage, int i) {
        const long kfirst = (long)max(t - tail, 0) * BK;
        if (i < NA)
            dma<DW>(tile_rsrc(cornerA, kstrideA, kfirst, rangeA), (lds_ptr)(stage + (i * NWAVES + wave) * LSTEP),
                    (int)offA[i], 0);
        else
            dma<DW>(tile_rsrc(cornerB, kstrideB, kfirst, rangeB),
                    (lds_ptr)(stage + BM * BK + ((i - NA) * NWAVES + wave) * LSTEP), (int)offB[i - NA], 0);
    };
    // Loads of the K remainder tile, on descriptors based at k = K - kr
    // (the ranges reach past K, where every offset is out of range).
    auto issue_remainder = [&](float *stage) {
        const __amdgpu_buffer_rsrc_t rA0 = tile_rsrc(cornerA, kstrideA, kfull, rangeA);
        const __amdgpu_buffer_rsrc_t rB0 = tile_rsrc(cornerB, kstrideB, kfull, rangeB);
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            int m, k;
            a_coords(i, m, k);
            const unsigned off = k < kr ? offA[i] : kOutOfRange;
            dma<DW>(rA0, (lds_ptr)(stage + (i * NWAVES + wave) * LSTEP), (int)off, 0);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            int r, col;
            b_coords(i, r, col);
            const unsigned off = r < kr ? offB[i] : kOutOfRange;
            dma<DW>(rB0, (lds_ptr)(stage + BM * BK + (i * NWAVES + wave) * LSTEP), (int)off, 0);
        }
    };

    f32x4 acc[T::MI][T::NJ][4];
#pragma unroll
    for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < T::NJ; ++nj)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mi][nj][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    typename T::Frags F[2];

    // Race-check build: NaN bits into the LDS units this lane's direct loads
    // of `stage` fill, landed before those loads are issued.
    auto poison = [&](float *stage) {
        if constexpr (SGEMM_LDS_POISON) {
            const float nan = __uint_as_float(kPoisonBits);
#pragma unroll
            for (int i = 0; i < NA + NB; ++i) {
                float *u = i < NA ? stage + (i * NWAVES + wave) * LSTEP
                                  : stage + BM * BK + ((i - NA) * NWAVES + wave) * LSTEP;
                if constexpr (DW)
                    u[lane] = nan;
                else
                    *reinterpret_cast<f32x4 *>(u + 4 * lane) = f32x4{nan, nan, nan, nan};
            }
            wait_lgkmcnt0();
        }
    };

    // one K tile held in stage SC (compile time); loads of tile t+1 go to
    // the other stage
    auto tile = [&](int t, auto sc) {
        constexpr int SC = decltype(sc)::value;
        constexpr int SN = 1 - SC;
        const float *cs = lds + SC * T::STAGE;
        float *ns = lds + SN * T::STAGE;
        const int t_next = min(t + 1, t_end - 1);
        poison(ns);     // its last reads were before the barrier that ended the previous tile
        auto section = [&](auto hc) {
            constexpr int h = decltype(hc)::value;
            constexpr int g_lo = h * PER < NA + NB ? h * PER : NA + NB;
            constexpr int g_hi = (h + 1) * PER < NA + NB ? (h + 1) * PER : NA + NB;
            emit_spread<NM, NR, NM * 3 / 4, (h < LS) ? g_hi - g_lo : 0>(
                [&](auto q) { T::template mma_one<decltype(q)::value>(acc, F[h & 1]); },
                [&](auto r) { T::template read_one<decltype(r)::value>(cs, wm, wn, lane, h + 1, F[(h + 1) & 1]); },
                [&](auto g) { issue_one(t_next, ns, g_lo + decltype(g)::value); });
            __builtin_amdgcn_sched_barrier(0);
        };
        section(IntC<0>{});
        if constexpr (KH == 4) {
            section(IntC<1>{});
            section(IntC<2>{});
        }
        wait_vmcnt0();
        __syncthreads();
        emit_spread<NM, NR, NR, 0>(
            [&](auto q) { T::template mma_one<decltype(q)::value>(acc, F[(KH - 1) & 1]); },
            [&](auto r) { T::template read_one<decltype(r)::value>(ns, wm, wn, lane, 0, F[0]); },
            [&](auto) {});
        __builtin_amdgcn_sched_barrier(0);
    };

    if (t_end > t_begin) {
        poison(lds);
        poison(lds + T::STAGE);
        if (tail && t_begin == 0) {
            issue_remainder(lds);
        } else {
#pragma unroll
            for (int i = 0; i < NA + NB; ++i) issue_one(t_begin, lds, i);
        }
        wait_vmcnt0();
        __syncthreads();
        T::read_frags(lds, wm, wn, lane, 0, F[0]);
        int t = t_begin;
        for (; t + 1 < t_end; t += 2) {
            tile(t, IntC<0>{});
            tile(t + 1, IntC<1>{});
        }
        if (t < t_end) tile(t, IntC<0>{});
    }
    if constexpr (SPLIT) {
        if (!split_reduce<T>(p, slot, tid, reinterpret_cast<unsigned *>(lds), acc)) return;
    }
    T::template epilogue<BETA0>(p, m0, n0, wm, wn, lane, acc);
}


template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool SPLIT, bool DW = false, bool TA = false,
          bool TB = false>
hipError_t launch_lean(const Args &a0, int splits, hipStream_t stream, int batch = 1) {
    const Args a = tiled(a0, BM, BN);
    // a.tile_count > 0: this launch covers tiles a.tile_base .. + tile_count - 1
    const int tiles = a0.tile_count > 0 ? a0.tile_count : a.tiles_m * a.tiles_n;
    const dim3 grid((unsigned)tiles, (unsigned)splits, (unsigned)batch);
    const dim3 block(64 * WAVES_M * WAVES_N);
    const bool edge = (a.M % BM) || (a.N % BN) || (a.K % BK);
#define SGEMM_LAUNCH(Z, E) \
    launch_k(sgemm_lean_kernel<BM, BN, BK, WAVES_M, WAVES_N, Z, E, SPLIT, DW, TA, TB>, grid, block, stream, a)
    if (edge) {
        if (a.beta == 0.0f) return SGEMM_LAUNCH(true, true);
        return SGEMM_LAUNCH(false, true);
    }
    if (a.beta == 0.0f) return SGEMM_LAUNCH(true, false);
    return SGEMM_LAUNCH(false, false);
#undef SGEMM_LAUNCH
}

}  // namespace sgemm_mi355x
