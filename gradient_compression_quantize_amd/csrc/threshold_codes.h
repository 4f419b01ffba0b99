// threshold_codes.h -- pieces shared by the two packings of the threshold
// quantizer's codes (16 per word in twobit.hip, 5 per byte in ternary.hip).
//
// apache/incubator-mxnet PR #8342 "[WIP] 2bit gradient compression",
// "Two bit quantization": a value at or above the positive threshold is
// sent as code 1 (read back as the positive threshold), one at or below the
// negative threshold as code 2 (the negative threshold), anything else as
// code 0 (zero). "Format of compressed gradient": every block opens with
// the negative threshold, the positive threshold and the size as floats.
#pragma once

#include "gcq_internal.h"

#include <cmath>

namespace gcq {
namespace {

// Value a code stands for; code 3 is never written and reads as zero.
__device__ __forceinline__ float code_value(uint32_t c, float neg, float pos)
{
    return c == 1u ? pos : (c == 2u ? neg : 0.0f);
}

__device__ __forceinline__ void write_header(uint32_t* blk, float neg, float pos, float n_f)
{
    blk[0] = f2u(neg);
    blk[1] = f2u(pos);
    blk[2] = f2u(n_f);
}

// Dequantization table in LDS: for worker w and a 4-bit nibble v (two codes,
// the earlier value in the high pair), entry 16w + v holds the two values.
// One worker's 16 entries span 128 bytes -- every LDS bank once -- so a
// wave's lookups into it never conflict. Ends with a block barrier.
__device__ __forceinline__ void build_nibble_table(float2* lut, const PtrTable<uint32_t>& tab,
                                                   int W)
{
    for (int w = 0; w < W; ++w) {
        if (threadIdx.x < 16) {
            const uint32_t* b = tab.p[w];
            const float neg = u2f(b[0]);
            const float pos = u2f(b[1]);
            const uint32_t v = threadIdx.x;
            lut[16 * w + v] = make_float2(code_value(v >> 2, neg, pos), code_value(v & 3u, neg, pos));
        }
    }
    __syncthreads();
}

// Host: thresholds must satisfy neg < 0 < pos (so 0 is always code 0).
inline int check_thresholds(float neg, float pos)
{
    if (!(std::isfinite(neg) && std::isfinite(pos) && neg < 0.0f && pos > 0.0f))
        return fail(GC_EINVAL, "thresholds must be finite with neg_threshold < 0 < pos_threshold");
    return GC_OK;
}

}  // namespace
}  // namespace gcq
