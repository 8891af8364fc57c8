// Lean kernels: untransposed single problems (16-byte and 4-byte loads).
// (Built with MFMA results in VGPRs; see sgemm_lean.hpp.)
#include "sgemm_lean.hpp"

namespace sgemm_mi355x {

// Launchers called from the C ABI's translation unit; each returns its
// launch's status.
hipError_t launch_lean_128x128x64_w2x2(const Args &a, hipStream_t s) {
    return launch_lean<128, 128, 64, 2, 2, false>(a, 1, s);
}
hipError_t launch_lean_128x128x32_w2x2(const Args &a, hipStream_t s) {
    return launch_lean<128, 128, 32, 2, 2, false>(a, 1, s);
}
hipError_t launch_lean_256x128x32_w4x2(const Args &a, hipStream_t s) {
    return launch_lean<256, 128, 32, 4, 2, false>(a, 1, s);
}
hipError_t launch_lean_128x256x32_w2x4(const Args &a, hipStream_t s) {
    return launch_lean<128, 256, 32, 2, 4, false>(a, 1, s);
}
hipError_t launch_lean_64x64x32_w4x1(const Args &a, hipStream_t s) {
    return launch_lean<64, 64, 32, 4, 1, false>(a, 1, s);
}
hipError_t launch_lean_64x64x64_w4x1(const Args &a, hipStream_t s) {
    return launch_lean<64, 64, 64, 4, 1, false>(a, 1, s);
}
hipError_t launch_lean_64x128x32_w2x2(const Args &a, hipStream_t s) {
    return launch_lean<64, 128, 32, 2, 2, false>(a, 1, s);
}
hipError_t launch_lean_128x64x32_w4x1(const Args &a, hipStream_t s) {
    return launch_lean<128, 64, 32, 4, 1, false>(a, 1, s);
}
// 4-byte loads, 32-bit C access: any alignment and leading dimensions
hipError_t launch_lean_dw_128x128x32_w2x2(const Args &a, hipStream_t s) {
    return launch_lean<128, 128, 32, 2, 2, false, true>(a, 1, s);
}
hipError_t launch_lean_dw_64x64x64_w4x1(const Args &a, hipStream_t s) {
    return launch_lean<64, 64, 64, 4, 1, false, true>(a, 1, s);
}

}  // namespace sgemm_mi355x
