// Lean kernels: transposed operands and strided batches.
// (Built with MFMA results in VGPRs; see sgemm_lean.hpp.)
#include "sgemm_lean.hpp"

namespace sgemm_mi355x {

// Transposed operands and strided batches: the 16-byte form when the caller
// has checked the operands' alignment (dw false), else the 4-byte form, on
// 64x64x64 tiles (tile64) or 128x128x32 tiles.
template <int BM, int BN, int BK, int WM, int WN>
hipError_t launch_lean_ops(const Args &a, bool dw, bool ta, bool tb, int batch, hipStream_t s) {
    if (!dw) {
        if (ta && tb)
            return launch_lean<BM, BN, BK, WM, WN, false, false, true, true>(a, 1, s, batch);
        if (ta)
            return launch_lean<BM, BN, BK, WM, WN, false, false, true, false>(a, 1, s, batch);
        if (tb)
            return launch_lean<BM, BN, BK, WM, WN, false, false, false, true>(a, 1, s, batch);
        return launch_lean<BM, BN, BK, WM, WN, false, false, false, false>(a, 1, s, batch);
    }
    if (ta && tb)
        return launch_lean<BM, BN, BK, WM, WN, false, true, true, true>(a, 1, s, batch);
    if (ta)
        return launch_lean<BM, BN, BK, WM, WN, false, true, true, false>(a, 1, s, batch);
    if (tb)
        return launch_lean<BM, BN, BK, WM, WN, false, true, false, true>(a, 1, s, batch);
    return launch_lean<BM, BN, BK, WM, WN, false, true, false, false>(a, 1, s, batch);
}
hipError_t launch_lean_general(const Args &a, bool tile64, bool dw, bool ta, bool tb, int batch, hipStream_t s) {
    if (tile64)
        return launch_lean_ops<64, 64, 64, 4, 1>(a, dw, ta, tb, batch, s);
    return launch_lean_ops<128, 128, 32, 2, 2>(a, dw, ta, tb, batch, s);
}

}  // namespace sgemm_mi355x
