// Exhaustive check of the binade search grid built by the library's host code (build_fq_grid):
// for every fp32 pattern u in [2, 4) and every codebook with b <= 4 at d in {64, 128, 256}, the top
// b bits of w = bits(u) + E[cell(u)] must equal #{k : thr_u[k] <= u}, and the top byte of w must
// be idx * 2^(8-b) or idx * 2^(8-b) + 2^(8-b) - 1 (the two centroid rows of idx).  Prints one line
// per codebook and exits non-zero on any mismatch.
#include "tables.hpp"

#include <cstdio>
#include <cstring>
#include <vector>

int main() {
    int fails = 0;
    for (int d : {64, 128, 256})
        for (int b = 1; b <= 4; ++b) {
            std::vector<double> t, c;
            if (tq::lloyd_max(d, b, t, c) != 0) { std::printf("d=%d b=%d: codebook failed\n", d, b); ++fails; continue; }
            std::vector<uint32_t> E;
            if (!tq::build_fq_grid(t, b, E)) { std::printf("d=%d b=%d: no binade grid\n", d, b); continue; }
            std::vector<uint32_t> T;
            for (double x : t) {
                const float f = (float)(3.0 + tq::kFqKappa * x);
                uint32_t u;
                std::memcpy(&u, &f, 4);
                T.push_back(u);
            }
            const uint32_t R = 1u << (8 - b);
            long bad_idx = 0, bad_row = 0;
            for (uint32_t u = 0x40000000u; u < 0x40800000u; ++u) {
                const uint32_t w = u + E[(u >> 16) & 0x7fu];
                uint32_t want = 0;
                for (uint32_t x : T) want += (x <= u);
                if ((w >> (32 - b)) != want) ++bad_idx;
                const uint32_t top = w >> 24;
                if (top != want * R && top != want * R + R - 1) ++bad_row;
            }
            std::printf("d=%d b=%d: index mismatches %ld, centroid-row mismatches %ld\n", d, b, bad_idx, bad_row);
            if (bad_idx || bad_row) ++fails;
        }
    return fails ? 1 : 0;
}
