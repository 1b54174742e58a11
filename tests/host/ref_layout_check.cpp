// Host-side check of the tiled layout of the searches' fp32 reference
// output (ref_offset and friends in awq_internal.h): over the padded domain
// of several shapes, every (row, column) maps to a distinct offset inside
// ref_tiled_floats, and the 16 values a lane holds for one 32 x 32 sub-tile
// (accumulator element e of v_mfma_f32_32x32x16: row 8 (e / 4) + 4 (lane / 32)
// + e % 4, column lane % 32) are contiguous at ref_subtile_base + 16 lane.
// Prints "ok" and exits 0, or names the first failure and exits 1.
#include <cstdio>
#include <vector>

#include "../../weight_only_int4_quantize_amd/csrc/awq_internal.h"

using awq::kRefTileM;
using awq::kRefTileN;
using awq::ref_offset;
using awq::ref_subtile_base;
using awq::ref_tiled_floats;

static bool check(int64_t M, int64_t N) {
    const int64_t tiles_n = (N + kRefTileN - 1) / kRefTileN;
    const int64_t Mp = (M + kRefTileM - 1) / kRefTileM * kRefTileM;
    const int64_t Np = tiles_n * kRefTileN;
    const int64_t total = ref_tiled_floats(M, N);
    if (total != Mp * Np) {
        std::printf("M=%lld N=%lld: %lld floats, expected %lld\n", (long long)M, (long long)N, (long long)total,
                    (long long)(Mp * Np));
        return false;
    }
    std::vector<unsigned char> seen(static_cast<size_t>(total), 0);
    for (int64_t m = 0; m < Mp; ++m)
        for (int64_t n = 0; n < Np; ++n) {
            const int64_t o = ref_offset(m, n, tiles_n);
            if (o < 0 || o >= total || seen[o]) {
                std::printf("M=%lld N=%lld: (%lld, %lld) -> %lld out of range or taken\n", (long long)M,
                            (long long)N, (long long)m, (long long)n, (long long)o);
                return false;
            }
            seen[o] = 1;
        }
    for (int64_t m0 = 0; m0 < Mp; m0 += 32)
        for (int64_t n0 = 0; n0 < Np; n0 += 32)
            for (int lane = 0; lane < 64; ++lane)
                for (int e = 0; e < 16; ++e) {
                    const int64_t m = m0 + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
                    const int64_t n = n0 + lane % 32;
                    if (ref_offset(m, n, tiles_n) != ref_subtile_base(m0, n0, tiles_n) + 16 * lane + e) {
                        std::printf("M=%lld N=%lld: sub-tile (%lld, %lld) lane %d element %d misplaced\n",
                                    (long long)M, (long long)N, (long long)m0, (long long)n0, lane, e);
                        return false;
                    }
                }
    return true;
}

int main() {
    const int64_t shapes[][2] = {{1, 1}, {32, 32}, {256, 128}, {257, 129}, {1000, 700}, {77, 4096}, {512, 384}};
    for (const auto& s : shapes)
        if (!check(s[0], s[1])) return 1;
    std::printf("ok\n");
    return 0;
}
