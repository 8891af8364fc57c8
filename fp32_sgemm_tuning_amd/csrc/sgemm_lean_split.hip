// Lean kernels: split-K.
// (Built with MFMA results in VGPRs; see sgemm_lean.hpp.)
#include "sgemm_lean.hpp"

namespace sgemm_mi355x {

// Split-K over `splits` >= 2 blocks per tile; a.ws and a.counters must hold
// splits * tiles * BM * BN floats and `tiles` zeroed counters.  Each returns
// its launch's status.
hipError_t launch_lean_splitk_128x128x32_w2x2(const Args &a, int splits, hipStream_t s) {
    return launch_lean<128, 128, 32, 2, 2, true>(a, splits, s);
}
hipError_t launch_lean_splitk_64x64x32_w4x1(const Args &a, int splits, hipStream_t s) {
    return launch_lean<64, 64, 32, 4, 1, true>(a, splits, s);
}
hipError_t launch_lean_splitk_64x64x64_w4x1(const Args &a, int splits, hipStream_t s) {
    return launch_lean<64, 64, 64, 4, 1, true>(a, splits, s);
}
hipError_t launch_lean_splitk_64x128x32_w2x2(const Args &a, int splits, hipStream_t s) {
    return launch_lean<64, 128, 32, 2, 2, true>(a, splits, s);
}
hipError_t launch_lean_splitk_128x64x32_w4x1(const Args &a, int splits, hipStream_t s) {
    return launch_lean<128, 64, 32, 4, 1, true>(a, splits, s);
}
// 4-byte loads (any alignment)
hipError_t launch_lean_splitk_dw_64x64x64_w4x1(const Args &a, int splits, hipStream_t s) {
    return launch_lean<64, 64, 64, 4, 1, true, true>(a, splits, s);
}

}  // namespace sgemm_mi355x
