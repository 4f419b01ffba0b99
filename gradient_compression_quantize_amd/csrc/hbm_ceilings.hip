// hbm_ceilings.hip -- plain streaming kernels that measure what this part's
// HBM gives each access mix of the hot path (libgcq_ceilings.so, used by the
// benchmark only; not part of libgcq.so).
//
// Each kernel moves exactly the bytes of one hot-path kernel, with the same
// tile shapes, alignments and non-temporal hints, but with trivial arithmetic
// in place of the quantization (XORs, ORs and adds that keep every load live):
//   read      n fp32 per buffer read, as the max-norm reads: chunked (one
//             contiguous chunk per workgroup, two loads in flight per lane)
//             or one 4 KB tile per wave
//   write     n fp32 written: one 4 KB tile per wave, or a grid-stride fill
//   compress  8 B read + 4 B written per value, and one 4-byte word per 16
//             values 12 bytes into a block (the 2-bit compress)
//   dequant   one 4-byte word per 16 values from each of W blocks, 12 bytes
//             into each, and 4 B written per value (the W-block
//             dequantize-sum), in three patterns: the kernel's (one tile per
//             wave, one 256 B word load per block), wide reads (two tiles per
//             wave, one 512 B load per block) and workgroup bursts (a
//             1024-thread workgroup stages 16 tiles' words of every block in
//             LDS with 16-byte loads, then writes 64 KB)
//   ternary   the same for the ternary dequantize-sum: one 4-byte element per
//             20 values from each of W blocks, 4 B written per value
//   quantize  4 B read + 1 B written per value
//   levelsum  W B read + 8 B written per value (an int32 sum and an fp32)
// A hot-path kernel's rate over its mix's rate here is how close it runs to
// what the memory system gives that access mix.
//
// Sizes: n must be a multiple of gcq_ceiling_quantum() (16384 values), so
// every tile is whole and no access is conditional.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <string>

#include "gcq_ceilings.h"
#include "occupancy.h"

#define GCQ_CEIL_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxBufs = 64;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr size_t kTileF4 = 256;     // float4 slots per wave tile
constexpr size_t kTileVals = 1024;  // values per wave tile
constexpr int kBurstThreads = 1024;
constexpr int kBurstTiles = kBurstThreads / kWave;  // 16 tiles per burst workgroup
constexpr int kBurstWords = kBurstTiles * kWave;    // 1024 words of each block
constexpr size_t kQuantum = size_t(kBurstTiles) * kTileVals;  // 16384 values

template <typename T>
struct Ptrs {
    const T* p[kMaxBufs];
};

thread_local std::string g_err;

// Workgroups per CU the 256-thread kernels are held to (0: what their
// registers allow), through an LDS reservation they never touch.
std::atomic<int> g_wg_per_cu{0};

size_t cap_lds() { return gcq::lds_for_wg_per_cu(g_wg_per_cu.load(std::memory_order_relaxed)); }

int fail(const std::string& m)
{
    g_err = m;
    return -1;
}

int launched(const char* what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(std::string(what) + ": " + hipGetErrorString(e));
    return 0;
}

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }

__device__ __forceinline__ f32x4 spread(uint32_t x, int u)
{
    return f32x4{float(x & 255u), float((x >> 8) & 255u), float((x >> 16) & 255u),
                 float(x >> (24 + u))};
}

// ---- read -------------------------------------------------------------------

// Workgroup x of buffer blockIdx.y reads float4 slots [x chunk4, min((x+1)
// chunk4, n4)) with two non-temporal loads in flight per lane (chunk4 and n4
// are multiples of 512, so pairs never straddle the end) and writes the OR
// of the bits it read to sink.
__global__ __launch_bounds__(kThreads) void ceil_read_chunked_kernel(Ptrs<float> bufs, size_t n4,
                                                                     size_t chunk4,
                                                                     uint32_t* __restrict__ sink)
{
    const f32x4* g = reinterpret_cast<const f32x4*>(bufs.p[blockIdx.y]);
    const size_t lo = size_t(blockIdx.x) * chunk4;
    const size_t hi = lo + chunk4 < n4 ? lo + chunk4 : n4;
    uint32_t acc = 0;
    for (size_t q = lo + threadIdx.x; q < hi; q += 2 * kThreads) {
        const f32x4 a = __builtin_nontemporal_load(g + q);
        const f32x4 b = __builtin_nontemporal_load(g + q + kThreads);
        acc |= fbits(a.x) | fbits(a.y) | fbits(a.z) | fbits(a.w) | fbits(b.x) | fbits(b.y) |
               fbits(b.z) | fbits(b.w);
    }
    __shared__ uint32_t red[kWaves];
    for (int off = kWave / 2; off > 0; off >>= 1)
        acc |= __shfl_xor(acc, off);
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[size_t(blockIdx.y) * gridDim.x + blockIdx.x] = red[0] | red[1] | red[2] | red[3];
}

// One tile of 4 float4 slots per lane per wave; one word per tile to sink.
__global__ __launch_bounds__(kThreads) void ceil_read_tile_kernel(const float* __restrict__ src,
                                                                  uint32_t* __restrict__ sink)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const f32x4* g = reinterpret_cast<const f32x4*>(src) + tile * kTileF4 + lane;
    f32x4 a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        a[u] = __builtin_nontemporal_load(g + u * kWave);
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        acc |= fbits(a[u].x) | fbits(a[u].y) | fbits(a[u].z) | fbits(a[u].w);
    for (int off = kWave / 2; off > 0; off >>= 1)
        acc |= __shfl_xor(acc, off);
    if (lane == 0)
        sink[tile] = acc;
}

// ---- write ------------------------------------------------------------------

// One 4 KB tile per wave: 4 lane-contiguous non-temporal float4 stores.
__global__ __launch_bounds__(kThreads) void ceil_write_tile_kernel(float* __restrict__ dst, float v)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    f32x4* o = reinterpret_cast<f32x4*>(dst) + tile * kTileF4 + lane;
    const f32x4 x = {v, v + 1.0f, v + 2.0f, float(lane)};
#pragma unroll
    for (int u = 0; u < 4; ++u)
        __builtin_nontemporal_store(x, o + u * kWave);
}

// Grid-stride fill in passes of 4 x 256 float4 per workgroup (n4 is a
// multiple of 1024, so passes are whole).
__global__ __launch_bounds__(kThreads) void ceil_write_stride_kernel(float* __restrict__ dst,
                                                                     size_t n4, float v)
{
    f32x4* o = reinterpret_cast<f32x4*>(dst);
    const f32x4 x = {v, v, v, v};
    constexpr size_t per = 4 * kThreads;
    for (size_t c = size_t(blockIdx.x) * per; c < n4; c += size_t(gridDim.x) * per) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            __builtin_nontemporal_store(x, o + c + u * kThreads + threadIdx.x);
    }
}

// ---- the compress mix --------------------------------------------------------

// Per wave tile: 4 float4 of a and of b read, a + b written over b, and one
// word per lane to words[3 + 64 tile + lane] (12 bytes into the block, as
// the 2-bit payload).
__global__ __launch_bounds__(kThreads) void ceil_compress_mix_kernel(const float* __restrict__ a,
                                                                     float* __restrict__ b,
                                                                     uint32_t* __restrict__ words)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const f32x4* a4 = reinterpret_cast<const f32x4*>(a) + tile * kTileF4 + lane;
    f32x4* b4 = reinterpret_cast<f32x4*>(b) + tile * kTileF4 + lane;
    f32x4 x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        x[u] = __builtin_nontemporal_load(a4 + u * kWave);
        y[u] = __builtin_nontemporal_load(b4 + u * kWave);
    }
    uint32_t w = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const f32x4 s = x[u] + y[u];
        __builtin_nontemporal_store(s, b4 + u * kWave);
        w ^= fbits(s.x) ^ fbits(s.y) ^ fbits(s.z) ^ fbits(s.w);
    }
    __builtin_nontemporal_store(w, words + 3 + tile * kWave + lane);
}

// ---- the dequantize-sum mix ----------------------------------------------------

constexpr int kDeqW = 8;

// The kernel's pattern: lane L loads word L of the tile from each block (one
// 256 B load per block, 12 bytes off the line grid), then writes the tile's
// 4 KB as 4 lane-contiguous float4 stores.
__global__ __launch_bounds__(kThreads) void ceil_dequant_tile_kernel(Ptrs<uint32_t> blk,
                                                                     float* __restrict__ out)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t w[kDeqW];
#pragma unroll
    for (int k = 0; k < kDeqW; ++k)
        w[k] = __builtin_nontemporal_load(blk.p[k] + 3 + tile * kWave + lane);
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < kDeqW; ++k)
        x ^= w[k];
    f32x4* o = reinterpret_cast<f32x4*>(out) + tile * kTileF4 + lane;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        __builtin_nontemporal_store(spread(x, u), o + u * kWave);
}

// Wide reads: each wave covers two tiles; lane L loads 8 bytes of each block
// (512 B per load instruction), then writes 8 KB. The loads start 16 bytes
// into the block (8-byte aligned) rather than 12: same byte count, one
// word's shift.
__global__ __launch_bounds__(kThreads) void ceil_dequant_wide_kernel(Ptrs<uint32_t> blk,
                                                                     float* __restrict__ out)
{
    const size_t pair = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    u32x2 v[kDeqW];
#pragma unroll
    for (int k = 0; k < kDeqW; ++k)
        v[k] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(blk.p[k] + 4 + pair * 2 * kWave) + lane);
    uint32_t x = 0, y = 0;
#pragma unroll
    for (int k = 0; k < kDeqW; ++k) {
        x ^= v[k].x;
        y ^= v[k].y;
    }
    f32x4* o = reinterpret_cast<f32x4*>(out) + pair * 2 * kTileF4 + lane;
#pragma unroll
    for (int u = 0; u < 8; ++u)
        __builtin_nontemporal_store(spread((u & 1) ? y : x, u & 3), o + u * kWave);
}

// Workgroup bursts: workgroup g covers tiles 16 g .. 16 g + 15. Phase 1
// stages words [1024 g, 1024 g + 1028) of every block -- the 16 tiles' words
// 3 + 1024 g .. 3 + 1024 g + 1023 and the first three of the float4 below
// them -- with 16-byte loads into LDS (257 float4 per block, 32.9 KB at
// W = 8); after one barrier, each wave writes its tile's 4 KB.
__global__ __launch_bounds__(kBurstThreads) void ceil_dequant_burst_kernel(Ptrs<uint32_t> blk,
                                                                           float* __restrict__ out)
{
    constexpr int kRow = kBurstWords / 4 + 1;  // float4 per block
    __shared__ u32x4 st[kDeqW][kRow];
    const size_t g = blockIdx.x;
    for (int e = threadIdx.x; e < kDeqW * kRow; e += kBurstThreads) {
        const int k = e / kRow, j = e % kRow;
        st[k][j] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(blk.p[k] + g * kBurstWords) + j);
    }
    __syncthreads();
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(st);
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < kDeqW; ++k)
        x ^= sw[k * 4 * kRow + 3 + wave * kWave + lane];
    f32x4* o = reinterpret_cast<f32x4*>(out) + (g * kBurstTiles + wave) * kTileF4 + lane;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        __builtin_nontemporal_store(spread(x, u), o + u * kWave);
}

// The ternary dequantize-sum's pattern: a wave tile is 64 elements (1280
// values); lane L loads element L of the tile from each block (256 B per
// load, 12 bytes into the block), then writes the tile's 5 KB as 5
// lane-contiguous float4 stores.
constexpr size_t kTernTileVals = 1280;

__global__ __launch_bounds__(kThreads) void ceil_dequant_ternary_kernel(Ptrs<uint32_t> blk,
                                                                        float* __restrict__ out)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t w[kDeqW];
#pragma unroll
    for (int k = 0; k < kDeqW; ++k)
        w[k] = __builtin_nontemporal_load(blk.p[k] + 3 + tile * kWave + lane);
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < kDeqW; ++k)
        x ^= w[k];
    f32x4* o = reinterpret_cast<f32x4*>(out) + tile * (kTernTileVals / 4) + lane;
#pragma unroll
    for (int u = 0; u < 5; ++u)
        __builtin_nontemporal_store(spread(x, u & 3), o + u * kWave);
}

// ---- the quantize mix --------------------------------------------------------

// Per wave tile: 4 float4 read per lane, one 4-byte word per float4 written
// (lane-contiguous, 256 B per store instruction), as the quantize's levels.
__global__ __launch_bounds__(kThreads) void ceil_quantize_mix_kernel(const float* __restrict__ src,
                                                                     uint32_t* __restrict__ dst)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const f32x4* g = reinterpret_cast<const f32x4*>(src) + tile * kTileF4 + lane;
    f32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        x[u] = __builtin_nontemporal_load(g + u * kWave);
#pragma unroll
    for (int u = 0; u < 4; ++u)
        __builtin_nontemporal_store(fbits(x[u].x) ^ fbits(x[u].y) ^ fbits(x[u].z) ^ fbits(x[u].w),
                                    dst + tile * kTileF4 + u * kWave + lane);
}

// ---- the level-sum mix --------------------------------------------------------

// Per wave tile of 2 x 64 slots of 4 values: one word (4 int8) per slot from
// each of the W level buffers, then an int4 and a float4 written per slot.
__global__ __launch_bounds__(kThreads) void ceil_levelsum_mix_kernel(Ptrs<uint32_t> lv,
                                                                     int32_t* __restrict__ sums,
                                                                     float* __restrict__ out)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t w[kDeqW][2];
#pragma unroll
    for (int k = 0; k < kDeqW; ++k)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            w[k][u] = __builtin_nontemporal_load(lv.p[k] + tile * 2 * kWave + u * kWave + lane);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < kDeqW; ++k)
            x += w[k][u];
        const size_t q = tile * 2 * kWave + u * kWave + lane;
        const i32x4 S = {int(x & 255u), int((x >> 8) & 255u), int((x >> 16) & 255u), int(x >> 24)};
        __builtin_nontemporal_store(S, reinterpret_cast<i32x4*>(sums) + q);
        const f32x4 v = {float(S.x), float(S.y), float(S.z), float(S.w)};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out) + q);
    }
}

// ---- the fused quantize-sum mix -------------------------------------------------

// Per wave tile of 4 x 64 slots of 4 values: the workers in turn, each one's
// 4 float4 per lane loaded together (the fused kernel's worker loop), then an
// int4 and a float4 written per slot.
__global__ __launch_bounds__(kThreads) void ceil_quantize_sum_mix_kernel(Ptrs<float> g,
                                                                         int32_t* __restrict__ sums,
                                                                         float* __restrict__ out)
{
    const size_t tile = size_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const size_t q0 = tile * kTileF4 + lane;
    i32x4 S[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        S[u] = i32x4{0, 0, 0, 0};
#pragma unroll 1
    for (int k = 0; k < kDeqW; ++k) {
        const f32x4* src = reinterpret_cast<const f32x4*>(g.p[k]) + q0;
        f32x4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            x[u] = __builtin_nontemporal_load(src + u * kWave);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            S[u] += i32x4{int(fbits(x[u].x) & 1u), int(fbits(x[u].y) & 1u),
                          int(fbits(x[u].z) & 1u), int(fbits(x[u].w) & 1u)};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        __builtin_nontemporal_store(S[u], reinterpret_cast<i32x4*>(sums) + q0 + u * kWave);
        const f32x4 v = {float(S[u].x), float(S[u].y), float(S[u].z), float(S[u].w)};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out) + q0 + u * kWave);
    }
}

bool whole(size_t n) { return n > 0 && n % kQuantum == 0; }

}  // namespace

GCQ_CEIL_API const char* gcq_ceiling_last_error(void) { return g_err.c_str(); }

GCQ_CEIL_API size_t gcq_ceiling_quantum(void) { return kQuantum; }

GCQ_CEIL_API int gcq_ceiling_set_wg_per_cu(int per_cu)
{
    if (per_cu < 0)
        return fail("gcq_ceiling_set_wg_per_cu: per_cu must be >= 0");
    g_wg_per_cu.store(per_cu, std::memory_order_relaxed);
    return 0;
}

GCQ_CEIL_API size_t gcq_ceiling_block_words(size_t n) { return 3 + n / 16 + 4; }

GCQ_CEIL_API size_t gcq_ceiling_ternary_quantum(void) { return 81920; }

GCQ_CEIL_API int gcq_ceiling_dequant_ternary(const uint32_t* const* blocks, int W, size_t n,
                                             size_t block_cap_words, float* out,
                                             hipStream_t stream)
{
    // whole workgroups of 4 tiles of 1280 values; n / 20 elements per block
    if (n == 0 || n % gcq_ceiling_ternary_quantum() || W != kDeqW || !blocks || !aligned16(out) ||
        block_cap_words < 3 + n / 20)
        return fail("gcq_ceiling_dequant_ternary: bad arguments (W must be 8)");
    Ptrs<uint32_t> tab{};
    for (int k = 0; k < W; ++k) {
        if (!aligned16(blocks[k]))
            return fail("gcq_ceiling_dequant_ternary: blocks must be 16-byte aligned");
        tab.p[k] = blocks[k];
    }
    hipLaunchKernelGGL(ceil_dequant_ternary_kernel, dim3(unsigned(n / kTernTileVals / kWaves)),
                       dim3(kThreads), cap_lds(), stream, tab, out);
    return launched("gcq_ceiling_dequant_ternary");
}

GCQ_CEIL_API size_t gcq_ceiling_read_sink_words(int nbufs, size_t n)
{
    return size_t(nbufs) * (n / kTileVals);
}

GCQ_CEIL_API int gcq_ceiling_read(const float* const* bufs, int nbufs, size_t n, int pattern,
                                  uint32_t* sink, size_t sink_words, hipStream_t stream)
{
    if (!whole(n) || nbufs < 1 || nbufs > kMaxBufs || !bufs || !sink ||
        sink_words < gcq_ceiling_read_sink_words(nbufs, n))
        return fail("gcq_ceiling_read: bad arguments");
    Ptrs<float> tab{};
    for (int k = 0; k < nbufs; ++k) {
        if (!aligned16(bufs[k]))
            return fail("gcq_ceiling_read: buffers must be 16-byte aligned");
        tab.p[k] = bufs[k];
    }
    const size_t n4 = n / 4;
    if (pattern == GCQ_CEIL_READ_CHUNKED) {
        // the max-norm's grid: about 4096 chunks per buffer, here multiples
        // of 512 slots (n4 is a multiple of 4096)
        const size_t chunk4 = ((n4 + 4095) / 4096 + 511) / 512 * 512;
        const size_t gx = (n4 + chunk4 - 1) / chunk4;
        hipLaunchKernelGGL(ceil_read_chunked_kernel, dim3(unsigned(gx), unsigned(nbufs)),
                           dim3(kThreads), cap_lds(), stream, tab, n4, chunk4, sink);
        return launched("gcq_ceiling_read (chunked)");
    }
    if (pattern == GCQ_CEIL_READ_TILE) {
        const size_t tiles = n / kTileVals;
        for (int k = 0; k < nbufs; ++k) {
            hipLaunchKernelGGL(ceil_read_tile_kernel, dim3(unsigned(tiles / kWaves)),
                               dim3(kThreads), cap_lds(), stream, bufs[k],
                               sink + size_t(k) * tiles);
            if (int rc = launched("gcq_ceiling_read (tile)"))
                return rc;
        }
        return 0;
    }
    return fail("gcq_ceiling_read: unknown pattern");
}

GCQ_CEIL_API int gcq_ceiling_write(float* dst, size_t n, int pattern, hipStream_t stream)
{
    if (!whole(n) || !aligned16(dst))
        return fail("gcq_ceiling_write: bad arguments");
    if (pattern == GCQ_CEIL_WRITE_TILE) {
        hipLaunchKernelGGL(ceil_write_tile_kernel, dim3(unsigned(n / kTileVals / kWaves)),
                           dim3(kThreads), cap_lds(), stream, dst, 1.0f);
        return launched("gcq_ceiling_write (tile)");
    }
    if (pattern == GCQ_CEIL_WRITE_STRIDE) {
        hipLaunchKernelGGL(ceil_write_stride_kernel, dim3(2048), dim3(kThreads), cap_lds(), stream,
                           dst, n / 4, 1.0f);
        return launched("gcq_ceiling_write (stride)");
    }
    return fail("gcq_ceiling_write: unknown pattern");
}

GCQ_CEIL_API int gcq_ceiling_compress(const float* a, float* b, size_t n, uint32_t* words,
                                      size_t words_cap, hipStream_t stream)
{
    if (!whole(n) || !aligned16(a) || !aligned16(b) || !words ||
        words_cap < gcq_ceiling_block_words(n))
        return fail("gcq_ceiling_compress: bad arguments");
    hipLaunchKernelGGL(ceil_compress_mix_kernel, dim3(unsigned(n / kTileVals / kWaves)),
                       dim3(kThreads), cap_lds(), stream, a, b, words);
    return launched("gcq_ceiling_compress");
}

GCQ_CEIL_API int gcq_ceiling_dequant(const uint32_t* const* blocks, int W, size_t n,
                                     size_t block_cap_words, int pattern, float* out,
                                     hipStream_t stream)
{
    if (!whole(n) || W != kDeqW || !blocks || !aligned16(out) ||
        block_cap_words < gcq_ceiling_block_words(n))
        return fail("gcq_ceiling_dequant: bad arguments (W must be 8)");
    Ptrs<uint32_t> tab{};
    for (int k = 0; k < W; ++k) {
        if (!aligned16(blocks[k]))
            return fail("gcq_ceiling_dequant: blocks must be 16-byte aligned");
        tab.p[k] = blocks[k];
    }
    const size_t tiles = n / kTileVals;
    switch (pattern) {
    case GCQ_CEIL_DEQ_TILE:
        hipLaunchKernelGGL(ceil_dequant_tile_kernel, dim3(unsigned(tiles / kWaves)),
                           dim3(kThreads), cap_lds(), stream, tab, out);
        return launched("gcq_ceiling_dequant (tile)");
    case GCQ_CEIL_DEQ_WIDE:
        hipLaunchKernelGGL(ceil_dequant_wide_kernel, dim3(unsigned(tiles / 2 / kWaves)),
                           dim3(kThreads), cap_lds(), stream, tab, out);
        return launched("gcq_ceiling_dequant (wide)");
    case GCQ_CEIL_DEQ_BURST:
        hipLaunchKernelGGL(ceil_dequant_burst_kernel, dim3(unsigned(tiles / kBurstTiles)),
                           dim3(kBurstThreads), 0, stream, tab, out);
        return launched("gcq_ceiling_dequant (burst)");
    default:
        return fail("gcq_ceiling_dequant: unknown pattern");
    }
}

GCQ_CEIL_API int gcq_ceiling_quantize(const float* src, size_t n, uint32_t* dst,
                                      hipStream_t stream)
{
    if (!whole(n) || !aligned16(src) || !aligned16(dst))
        return fail("gcq_ceiling_quantize: bad arguments");
    hipLaunchKernelGGL(ceil_quantize_mix_kernel, dim3(unsigned(n / kTileVals / kWaves)),
                       dim3(kThreads), cap_lds(), stream, src, dst);
    return launched("gcq_ceiling_quantize");
}

GCQ_CEIL_API int gcq_ceiling_levelsum(const uint32_t* const* levels, int W, size_t n,
                                      int32_t* sums, float* out, hipStream_t stream)
{
    if (!whole(n) || W != kDeqW || !levels || !aligned16(sums) || !aligned16(out))
        return fail("gcq_ceiling_levelsum: bad arguments (W must be 8)");
    Ptrs<uint32_t> tab{};
    for (int k = 0; k < W; ++k) {
        if (!aligned16(levels[k]))
            return fail("gcq_ceiling_levelsum: level buffers must be 16-byte aligned");
        tab.p[k] = levels[k];
    }
    hipLaunchKernelGGL(ceil_levelsum_mix_kernel, dim3(unsigned(n / 512 / kWaves)),
                       dim3(kThreads), cap_lds(), stream, tab, sums, out);
    return launched("gcq_ceiling_levelsum");
}

GCQ_CEIL_API int gcq_ceiling_quantize_sum(const float* const* grads, int W, size_t n,
                                          int32_t* sums, float* out, hipStream_t stream)
{
    if (!whole(n) || W != kDeqW || !grads || !aligned16(sums) || !aligned16(out))
        return fail("gcq_ceiling_quantize_sum: bad arguments (W must be 8)");
    Ptrs<float> tab{};
    for (int k = 0; k < W; ++k) {
        if (!aligned16(grads[k]))
            return fail("gcq_ceiling_quantize_sum: gradients must be 16-byte aligned");
        tab.p[k] = grads[k];
    }
    hipLaunchKernelGGL(ceil_quantize_sum_mix_kernel, dim3(unsigned(n / kTileVals / kWaves)),
                       dim3(kThreads), cap_lds(), stream, tab, sums, out);
    return launched("gcq_ceiling_quantize_sum");
}
