// gcq_internal.h -- shared pieces of libgcq.so (not installed, not part of
// the ABI): error state, launch checks, and CDNA4 wavefront helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "gcq.h"
#include "occupancy.h"

#define GCQ_API extern "C" __attribute__((visibility("default")))

namespace gcq {

// Wavefront size of CDNA (gfx9 family, gfx950 included).
constexpr int kWave = 64;

// ---- error state ---------------------------------------------------------
void set_error(const std::string& msg);
void clear_error();
int fail(gc_status code, const std::string& msg);
// Checks the launch that was just enqueued on this thread.
int check_launch(const char* what);
const char* last_error();

// ---- host helpers ----------------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

// Cap on the workgroups of one launch: larger problems make the kernels
// stride. 2^20 workgroups keep launches far below the 2^32 work-item limit.
// The environment variable GCQ_MAX_GRID_BLOCKS, read once per process, can
// lower it (tests use it to reach the striding paths at small sizes).
size_t max_grid_blocks();

// W device pointers passed by value in the kernel argument segment.
template <typename T>
struct PtrTable {
    const T* p[GC_MAX_WORKERS];
};

// ---- device helpers --------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// CDNA4 dispatches the workgroups of a launch round-robin over its 8 XCDs,
// each with its own L2: workgroup i runs on XCD i % 8. This bijection of
// [0, B) gives each XCD one contiguous range of logical workgroup indices,
// so that neighbouring tiles (which share the cache lines at their edges)
// meet in the same L2.
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t i, uint32_t B)
{
    const uint32_t q = B / kXcds, r = B % kXcds, x = i % kXcds, k = i / kXcds;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// OR of a 32-bit value over the 4 lanes of a DPP quad (lanes 4k..4k+3);
// every lane of the quad gets the result. Two quad_perm moves, no LDS.
// quad_perm selectors: [1,0,3,2] = 0xB1 (xor 1), [2,3,0,1] = 0x4E (xor 2).
__device__ __forceinline__ uint32_t quad_or(uint32_t x)
{
    x |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(x), 0xB1, 0xF, 0xF, true));
    x |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(x), 0x4E, 0xF, 0xF, true));
    return x;
}

// Orders this wave's LDS accesses across its lanes: LDS operations of one
// wave complete in issue order, so it suffices that the compiler moves no
// LDS access across this point.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace gcq
