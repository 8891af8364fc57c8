// Lean kernels: split-K through sgemm_op and the strided batches (16-byte
// loads, 64x64x64 tiles, any operand orientation, one or more problems).
// (Built with MFMA results in VGPRs; see sgemm_lean.hpp.)
#include "sgemm_lean.hpp"

namespace sgemm_mi355x {

// a.ws and a.counters hold splits * batch * tiles partial tiles and batch *
// tiles zeroed counters (as for launch_lean_splitk_64x64x64_w4x1, per
// problem of the batch).
hipError_t launch_lean_splitk_g_64x64x64_w4x1(const Args &a, int splits, bool ta, bool tb, int batch,
                                              hipStream_t s) {
    if (ta && tb)
        return launch_lean<64, 64, 64, 4, 1, true, false, true, true>(a, splits, s, batch);
    if (ta)
        return launch_lean<64, 64, 64, 4, 1, true, false, true, false>(a, splits, s, batch);
    if (tb)
        return launch_lean<64, 64, 64, 4, 1, true, false, false, true>(a, splits, s, batch);
    return launch_lean<64, 64, 64, 4, 1, true, false, false, false>(a, splits, s, batch);
}

}  // namespace sgemm_mi355x
