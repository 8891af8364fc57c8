// Lean kernels: split-K with transposed operands (16-byte loads, 64x64x64
// tiles), for one transposed problem whose grid or last wave splits K.
// (Built with MFMA results in VGPRs; see sgemm_lean.hpp.)
#include "sgemm_lean.hpp"

namespace sgemm_mi355x {

// a.ws and a.counters as for launch_lean_splitk_64x64x64_w4x1; ta or tb set.
hipError_t launch_lean_splitk_t_64x64x64_w4x1(const Args &a, int splits, bool ta, bool tb, hipStream_t s) {
    if (ta && tb)
        return launch_lean<64, 64, 64, 4, 1, true, false, true, true>(a, splits, s);
    if (ta)
        return launch_lean<64, 64, 64, 4, 1, true, false, true, false>(a, splits, s);
    return launch_lean<64, 64, 64, 4, 1, true, false, false, true>(a, splits, s);
}

}  // namespace sgemm_mi355x
