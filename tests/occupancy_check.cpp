// Checks gcq::lds_reservation (gradient_compression_quantize_amd/csrc/occupancy.h)
// on the host: whenever it returns a reservation, a workgroup's LDS (its own
// plus the reservation), rounded up to any allocation unit of 256, 512, 1280
// or 2560 bytes, lets exactly the requested number of workgroups share a CU,
// and stays within the per-workgroup limit. Prints OK and exits 0, or names
// the failing case.
#include <cstdio>
#include <cstdlib>

#include "occupancy.h"

using gcq::lds_reservation;

// the CU of gfx950: 160 KB of LDS, all of it available to one workgroup
static_assert(lds_reservation(163840, 163840, 3, 0) == 53760 - 256, "3 per CU");
static_assert(lds_reservation(163840, 163840, 4, 0) == 40960 - 256, "4 per CU");
static_assert(lds_reservation(163840, 163840, 5, 0) == 30720 - 256, "5 per CU");
static_assert(lds_reservation(163840, 163840, 6, 0) == 25600 - 256, "6 per CU");
static_assert(lds_reservation(163840, 163840, 6, 21504) == 25600 - 256 - 21504, "own LDS");
static_assert(lds_reservation(163840, 163840, 0, 0) == 0, "no cap");
static_assert(lds_reservation(163840, 163840, 6, 29696) == 0, "own LDS already holds it to 5");
static_assert(lds_reservation(163840, 65536, 1, 0) == 0, "more than one workgroup may take");

int main()
{
    const size_t cus[] = {65536, 98304, 163840};
    const size_t blocks[] = {65536, 163840};
    const size_t owns[] = {0, 16, 256, 1000, 5120, 8192, 16384, 21504, 24576, 29696};
    const size_t units[] = {256, 512, 1280, 2560};
    long checked = 0;
    for (size_t L : cus)
        for (size_t B : blocks) {
            if (B > L)
                continue;
            for (int per_cu = 0; per_cu <= 24; ++per_cu)
                for (size_t own : owns) {
                    const size_t r = lds_reservation(L, B, per_cu, own);
                    if (r == 0)
                        continue;
                    for (size_t g : units) {
                        const size_t alloc = (own + r + g - 1) / g * g;
                        const bool fits = size_t(per_cu) * alloc <= L;
                        const bool one_more = size_t(per_cu + 1) * alloc <= L;
                        if (!fits || one_more || own + r > B) {
                            std::printf("FAIL L=%zu B=%zu per_cu=%d own=%zu unit=%zu r=%zu\n", L, B,
                                        per_cu, own, g, r);
                            return 1;
                        }
                        ++checked;
                    }
                }
        }
    // every cap the library uses is expressible on gfx950 for the kernels'
    // own LDS (0 to 16 bytes, the staged kernels' 16 KB, the ternary 21.5 KB)
    for (int per_cu = 3; per_cu <= 6; ++per_cu)
        for (size_t own : {size_t(0), size_t(16), size_t(16384)})
            if (lds_reservation(163840, 163840, per_cu, own) == 0) {
                std::printf("FAIL: no reservation for %d per CU, own %zu\n", per_cu, own);
                return 1;
            }
    std::printf("checked %ld reservations\nOK\n", checked);
    return 0;
}
