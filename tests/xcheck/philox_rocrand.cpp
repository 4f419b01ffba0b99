// Third-party cross-check for the oracle's Philox4x32-10: rocRAND's
// open-source header (rocrand/rocrand_philox4x32_10.h), host side only.
// Test-only. Reads "c0 c1 c2 c3 k0 k1" and prints the ten-round output.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct Exposed : rocrand_device::philox4x32_10_engine {
    using philox4x32_10_engine::ten_rounds;
};

int main()
{
    unsigned c0, c1, c2, c3, k0, k1;
    Exposed e;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = e.ten_rounds(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
