// Third-party cross-check for the oracle's Philox4x32-10: PyTorch's
// open-source header-only engine (ATen/core/PhiloxRNGEngine.h). Test-only.
// Reads "seed subsequence offset" triples; prints the four 32-bit outputs of
// the block the engine starts at. The engine's key is the seed, and its
// counter is (offset lo, offset hi, subsequence lo, subsequence hi).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>

int main()
{
    unsigned long long seed, sub, off;
    while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
        at::philox_engine e(seed, sub, off);
        unsigned a = e(), b = e(), c = e(), d = e();
        std::printf("%u %u %u %u\n", a, b, c, d);
    }
    return 0;
}
