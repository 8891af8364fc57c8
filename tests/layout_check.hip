// Host-side check of the LDS A-stage layouts of the double-buffered kernel
// (ALayout<BK> in sgemm_kernels.hpp), run on the CPU:
//   - the loader assignment e -> (row, chunk) is a bijection onto the tile;
//   - offsets are a bijection onto the stage, 16-byte aligned, and inverse()
//     maps each 16-byte LDS position back to its (row, chunk);
//   - each group of 8 consecutive loaders writes 128 contiguous bytes
//     (one ds_write_b128 pass without bank conflicts);
//   - for every 16-row slab and k-chunk group, the 16 lanes of each
//     ds_read_b128 pass ({0-7,24-31}, {8-15,16-23}, ...) hit 16 distinct
//     16-byte slots of the bank window.
#include <cstdio>
#include <set>
#include <vector>
#include "sgemm_kernels.hpp"

using namespace sgemm_mi355x;

template <int BK, int BM>
static int check() {
    int bad = 0;
    constexpr int CPR = BK / 4;
    std::set<std::pair<int, int>> rc;
    std::set<int> offs;
    std::vector<int> off_of_e(BM * CPR);
    for (int e = 0; e < BM * CPR; ++e) {
        int m, c;
        ALayout<BK>::coords(e, m, c);
        if (m < 0 || m >= BM || c < 0 || c >= CPR) { ++bad; continue; }
        rc.insert({m, c});
        const int o = ALayout<BK>::offset(m, c);
        int mi, ci;                                      // the direct-load inverse
        ALayout<BK>::inverse(o / 4, mi, ci);
        if (mi != m || ci != c) ++bad;
        if (o % 4 || o < 0 || o >= BM * BK) ++bad;
        offs.insert(o);
        off_of_e[e] = o;
    }
    if ((int)rc.size() != BM * CPR || (int)offs.size() != BM * CPR) ++bad;
    for (int e0 = 0; e0 < BM * CPR; e0 += 8) {          // write passes
        int lo = 1 << 30, hi = -1;
        for (int e = e0; e < e0 + 8; ++e) { lo = lo < off_of_e[e] ? lo : off_of_e[e]; hi = hi > off_of_e[e] ? hi : off_of_e[e]; }
        if (hi - lo != 28 || lo % 32) ++bad;             // 8 chunks = 32 floats = 128 bytes
    }
    static const int pass_lanes[4][16] = {
        {0, 1, 2, 3, 4, 5, 6, 7, 24, 25, 26, 27, 28, 29, 30, 31},
        {8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21, 22, 23},
        {32, 33, 34, 35, 36, 37, 38, 39, 56, 57, 58, 59, 60, 61, 62, 63},
        {40, 41, 42, 43, 44, 45, 46, 47, 48, 49, 50, 51, 52, 53, 54, 55}};
    for (int slab = 0; slab < BM / 16; ++slab)
        for (int h = 0; h < BK / 16; ++h)
            for (int p = 0; p < 4; ++p) {
                std::set<int> slots;
                for (int i = 0; i < 16; ++i) {
                    const int l = pass_lanes[p][i];
                    const int byte = 4 * ALayout<BK>::offset(slab * 16 + (l & 15), 4 * h + (l >> 4));
                    slots.insert((byte >> 4) & 15);
                }
                if (slots.size() != 16) ++bad;
            }
    printf("BK=%d BM=%d: %s\n", BK, BM, bad ? "FAIL" : "ok");
    return bad;
}

int main() {
    int bad = 0;
    bad += check<16, 128>();
    bad += check<16, 256>();
    bad += check<32, 128>();
    bad += check<32, 256>();
    bad += check<64, 128>();
    return bad ? 1 : 0;
}
