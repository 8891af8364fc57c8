// Lean direct-to-LDS SGEMM kernel, in a translation unit of its own.
//
// This file is compiled with MFMA results kept in ordinary VGPRs
// (-mllvm -amdgpu-mfma-vgpr-form).  With the default accumulation registers
// the two-stage unrolled loop below gets accumulator copies between the
// unrolled halves and fragment round trips through the accumulation file,
// one VALU copy for every five MFMAs; in VGPR form the K loop is MFMAs, LDS
// reads, direct loads and a few scalar instructions only.  The flag applies
// to a whole translation unit, and kernels of the shared header that hold
// 256 accumulators per lane do not fit 256 VGPRs, hence the separate file.
// Only wave tiles of 64x64 or 64x128 outputs are instantiated here.
#include <hip/hip_runtime.h>

#include "sgemm_kernels.hpp"

namespace sgemm_mi355x {

// s_waitcnt with vmcnt 0 and the other counters at their maximum
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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
// Whole tiles only, and every byte offset inside A's row block and B's
// column block must fit the 31-bit buffer range (BM * lda + K and K * ldb
// below 2^29 elements); other cases take the guarded kernels.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool BETA0>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
sgemm_lean_kernel(Args p) {
    using T = TileOps<BM, BN, BK, WAVES_M, WAVES_N, true, false>;
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int KH = T::KH;
    static_assert(KH == 2 || KH == 4, "BK must be 32 or 64");
    constexpr int NA = BM * BK / 4 / T::NT;
    constexpr int NB = BK * BN / 4 / T::NT;
    constexpr int NM = T::MI * T::NJ * 16;
    constexpr int NR = T::MI + 4 * T::NJ;
    constexpr int LS = KH == 4 ? 2 : 1;                     // sections carrying the loads
    constexpr int PER = (NA + NB + LS - 1) / LS;
    __shared__ __attribute__((aligned(16))) float lds[2 * T::STAGE];
    typedef __attribute__((address_space(3))) void *lds_ptr;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // loop-invariant per-lane byte offsets of the direct loads
    unsigned offA[NA], offB[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        int m, c;
        ALayout<BK>::inverse((i * NWAVES + wave) * 64 + lane, m, c);
        offA[i] = 4u * (unsigned)(m * (int)p.lda + 4 * c);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int q = (i * NWAVES + wave) * 64 + lane;
        offB[i] = 4u * (unsigned)((q / T::B_CPR) * (int)p.ldb + 4 * (q % T::B_CPR));
    }
    // Buffer descriptors at the block's first row of A and first column of
    // B; the per-tile advance goes in the scalar offset of each load.
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.A + (long)m0 * p.lda), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.B + n0), (short)0, 0x7fffffff, 0x00020000);
    const unsigned stepA = 4u * BK, stepB = 4u * BK * (unsigned)p.ldb;

    // (The explicit int conversions matter: with the array element passed
    // as is, the host pass drops the kernel and its launch stub.)
    auto issue_one = [&](int t, float *stage, int i) {
        if (i < NA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr)(stage + (i * NWAVES + wave) * 256), 16,
                                                     (int)offA[i], (int)(t * stepA), 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_ptr)(stage + BM * BK + ((i - NA) * NWAVES + wave) * 256),
                                                     16, (int)offB[i - NA], (int)(t * stepB), 0, 0);
    };

    f32x4 acc[T::MI][T::NJ][4];
#pragma unroll
    for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < T::NJ; ++nj)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mi][nj][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = p.K / BK;
    typename T::Frags F[2];

    // one K tile held in stage SC (compile time); loads of tile t+1 go to
    // the other stage
    auto tile = [&](int t, auto sc) {
        constexpr int SC = decltype(sc)::value;
        constexpr int SN = 1 - SC;
        const float *cs = lds + SC * T::STAGE;
        float *ns = lds + SN * T::STAGE;
        const int t_next = min(t + 1, ntiles - 1);
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

    if (ntiles > 0) {
#pragma unroll
        for (int i = 0; i < NA + NB; ++i) issue_one(0, lds, i);
        wait_vmcnt0();
        __syncthreads();
        T::read_frags(lds, wm, wn, lane, 0, F[0]);
        int t = 0;
        for (; t + 1 < ntiles; t += 2) {
            tile(t, IntC<0>{});
            tile(t + 1, IntC<1>{});
        }
        if (t < ntiles) tile(t, IntC<0>{});
    }
    T::template epilogue<BETA0>(p, m0, n0, wm, wn, lane, acc);
}


template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
void launch_lean(const Args &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(64 * WAVES_M * WAVES_N);
    if (a.beta == 0.0f)
        hipLaunchKernelGGL((sgemm_lean_kernel<BM, BN, BK, WAVES_M, WAVES_N, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((sgemm_lean_kernel<BM, BN, BK, WAVES_M, WAVES_N, false>), grid, block, 0, stream, a);
}

// Launchers called from the C ABI's translation unit.
void launch_lean_128x128x64_w2x2(const Args &a, hipStream_t s) { launch_lean<128, 128, 64, 2, 2>(a, s); }
void launch_lean_128x128x32_w2x2(const Args &a, hipStream_t s) { launch_lean<128, 128, 32, 2, 2>(a, s); }
void launch_lean_256x128x32_w4x2(const Args &a, hipStream_t s) { launch_lean<256, 128, 32, 4, 2>(a, s); }
void launch_lean_128x256x32_w2x4(const Args &a, hipStream_t s) { launch_lean<128, 256, 32, 2, 4>(a, s); }
void launch_lean_256x256x32_w4x2(const Args &a, hipStream_t s) { launch_lean<256, 256, 32, 4, 2>(a, s); }

}  // namespace sgemm_mi355x
