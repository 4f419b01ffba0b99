// qsgd.hip -- QSGDMaxNorm stochastic quantization, the simulated all-reduce
// of its integer levels, and the GlobalRandK sparsified variant.
//
// Method: vineeths96 "Gradient-Compression" page ("Quantization for
// Distributed Optimization"). "About The Project": the QSGDMaxNorm family is
// all-reduce compatible -- every worker scales by the same max-norm, so the
// integer levels of all workers can be summed and dequantized once.
// "Results": GRandK-MN sparsifies to K = 10000 indices shared by all workers
// before quantizing.
//
// Per element: level = sign(g) * floor(|g| / norm * s + u), u uniform from a
// counter-based Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), so every
// element's random number is a pure function of (seed, worker, index).
#include "gcq_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <string>

namespace gcq {
namespace {

constexpr int kThreads = 256;

// ---- Philox4x32-10 ---------------------------------------------------------
// Round: two 32x32->64 products (counter words 0 and 2 with the Philox-4x32
// multipliers); new words (hi_b ^ c1 ^ k0, lo_b, hi_a ^ c3 ^ k1, lo_a); the
// key advances by the two Weyl increments between rounds.
struct U4 {
    uint32_t x, y, z, w;
};

// Three-input XOR in one CDNA4 instruction (v_bitop3_b32, truth table 0x96:
// the parity of the three input bits). The quantize kernels are bound by
// VALU issue, and this halves the XORs of every Philox round.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t pa = uint64_t(0xD2511F53u) * c.x;
        const uint64_t pb = uint64_t(0xCD9E8D57u) * c.z;
        c = U4{xor3(uint32_t(pb >> 32), c.y, k0), uint32_t(pb), xor3(uint32_t(pa >> 32), c.w, k1),
               uint32_t(pa)};
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// ---- max |g| ---------------------------------------------------------------

__device__ __forceinline__ float wave_max(float m)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        m = fmaxf(m, __shfl_xor(m, off));
    return m;
}

// Workgroup max of m; valid in thread 0.
template <int NT>
__device__ __forceinline__ float block_max(float m)
{
    __shared__ float lds[NT / kWave];
    m = wave_max(m);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0)
        lds[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < NT / kWave; ++k)
            m = fmaxf(m, lds[k]);
    }
    return m;
}

// Each workgroup reduces one contiguous chunk of a worker's float4 slots,
// two non-temporal loads in flight per lane. Measured over 8 x 138M values:
// 512-byte-aligned chunks for ~4096 workgroups per worker read at ~88% of
// peak HBM bandwidth, against ~73% for 512 strided workgroups with four
// loads in flight each.
constexpr unsigned kMaxPartialsPerWorker = 4096;
constexpr int kMaxAbsUnroll = 2;
constexpr size_t kMaxAbsMinChunk = 2048;  // float4 slots per workgroup, at least
constexpr size_t kMaxAbsChunkAlign = 32;  // float4 slots: chunks start on 512 B
// At most 3 workgroups per CU (an LDS reservation; the registers allow 8):
// 647 against 658 us for 8 x 138M values; 4 per CU gave 653.
constexpr int kMaxAbsWgPerCu = 3;

struct MaxNormGrid {
    unsigned gx;    // workgroups per worker = partial maxima per worker
    size_t chunk4;  // float4 slots per workgroup
};

MaxNormGrid maxnorm_grid(size_t n)
{
    const size_t n4 = n >> 2;
    const size_t gx0 = std::max<size_t>(
        1, std::min<size_t>(ceil_div(n4, kMaxAbsMinChunk), kMaxPartialsPerWorker));
    const size_t chunk4 =
        ceil_div(ceil_div(n4, gx0), kMaxAbsChunkAlign) * kMaxAbsChunkAlign;
    const size_t gx = chunk4 ? std::max<size_t>(1, ceil_div(n4, chunk4)) : 1;
    return MaxNormGrid{unsigned(gx), chunk4};
}

// blockIdx.y = worker. The max is order-free, so a buffer off 16-byte
// alignment splits into a head of at most 3 values and a 16-byte-aligned
// rest. Workgroup x takes float4 slots [x chunk4, (x+1) chunk4) of the rest
// and writes their max |g|; workgroup 0 also takes the head and the scalar
// tail of the rest.
__global__ __launch_bounds__(kThreads) void maxabs_partial_kernel(PtrTable<float> tab, size_t n,
                                                                  size_t chunk4,
                                                                  float* __restrict__ partials)
{
    const float* __restrict__ g = tab.p[blockIdx.y];
    const size_t head =
        std::min<size_t>(((16u - (reinterpret_cast<uintptr_t>(g) & 15u)) & 15u) / 4u, n);
    const float* __restrict__ ga = g + head;
    const size_t na = n - head;
    float m = 0.0f;
    const f32x4* g4 = reinterpret_cast<const f32x4*>(ga);
    const size_t nfull = na >> 2;
    const size_t lo = size_t(blockIdx.x) * chunk4;
    const size_t hi = std::min(lo + chunk4, nfull);
    size_t q = lo + threadIdx.x;
    for (; q + (kMaxAbsUnroll - 1) * kThreads < hi; q += kMaxAbsUnroll * kThreads) {
        f32x4 v[kMaxAbsUnroll];
#pragma unroll
        for (int u = 0; u < kMaxAbsUnroll; ++u)
            v[u] = __builtin_nontemporal_load(g4 + q + u * kThreads);
#pragma unroll
        for (int u = 0; u < kMaxAbsUnroll; ++u)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)),
                               fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
    for (; q < hi; q += kThreads) {
        const f32x4 v = __builtin_nontemporal_load(g4 + q);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    if (blockIdx.x == 0) {
        for (size_t i = nfull * 4 + threadIdx.x; i < na; i += kThreads)
            m = fmaxf(m, fabsf(ga[i]));
        if (threadIdx.x < head)
            m = fmaxf(m, fabsf(g[threadIdx.x]));
    }
    m = block_max<kThreads>(m);
    if (threadIdx.x == 0)
        partials[size_t(blockIdx.y) * gridDim.x + blockIdx.x] = m;
}

constexpr int kFinalThreads = 1024;

constexpr int kFinalUnroll = 8;

// Eight independent loads in flight per lane: the partials are tens of
// thousands of floats, and one dependent load at a time made this
// latency-bound.
__global__ __launch_bounds__(kFinalThreads) void max_final_kernel(const float* __restrict__ partials,
                                                                  unsigned count,
                                                                  float* __restrict__ norm)
{
    float mu[kFinalUnroll];
#pragma unroll
    for (int u = 0; u < kFinalUnroll; ++u)
        mu[u] = 0.0f;
    unsigned i = threadIdx.x;
    for (; i + (kFinalUnroll - 1) * kFinalThreads < count; i += kFinalUnroll * kFinalThreads) {
#pragma unroll
        for (int u = 0; u < kFinalUnroll; ++u)
            mu[u] = fmaxf(mu[u], partials[i + u * kFinalThreads]);
    }
    for (; i < count; i += kFinalThreads)
        mu[0] = fmaxf(mu[0], partials[i]);
    float m = mu[0];
#pragma unroll
    for (int u = 1; u < kFinalUnroll; ++u)
        m = fmaxf(m, mu[u]);
    m = block_max<kFinalThreads>(m);
    if (threadIdx.x == 0)
        *norm = m;
}

// ---- quantize --------------------------------------------------------------

// floor(x + u) exactly, for x = (|g| / norm) * s (two fp32 roundings) and
// u = k * 2^-24 with k = r >> 8, in integer arithmetic:
//   x * 2^24 is exact (a power-of-two scaling of a value at most 127), and
//   floor(x + u) = floor((x * 2^24 + k) / 2^24) = (floor(x * 2^24) + k) >> 24,
// where floor(x * 2^24) < 2^31 and k < 2^24, so the sum fits in 32 bits.
// s24 = s * 2^24 is exact, and fl(q * s24) = fl(q * s) * 2^24 whenever
// fl(q * s) is a normal number; below that x < 2^-126 and every path gives
// level 0.
//
// The sign goes into the same integer. Scaling g itself (not |g|) gives
// X = sign(g) * |X| exactly (every step is sign-symmetric), and the
// truncating conversion gives F = sign(g) * floor(|X|). A value with its sign
// bit set adds k' = (~r) >> 8 = 2^24 - 1 - k instead of k: for an integer
// A = floor(|X|) + k >= 0, floor((2^24 - 1 - A) / 2^24) = -floor(A / 2^24),
// so the arithmetic shift of the "slot" F + k' by 24 is the signed level
// -floor(x + u). Either way the level is the slot's top byte read as int8
// (|level| <= 127), which is the two's-complement byte the wire carries.
//
// The quotient: the exact path divides (IEEE, correctly rounded) and then
// scales by s24. The fast path multiplies once, by c = fl(fl(1 / norm) * s24).
// Each side takes rounded steps (fl(1/norm), fl(inv * s24), fl(g * c); and
// fl(g / norm), fl(q * s24)), every one within 2^-24 relative of its real
// value while its result is a normal number -- which holds wherever the
// level can be nonzero (|X| >= 1 needs |g| / norm >= 2^-31). So for
// |g| <= norm the two values of |X| differ by at most 5 * 2^-24 * |X| <
// 5 * 127 = 635, and so do the two slots. The fast slot carries a bias of
// kSlack = 2048: when it lies at least 2 kSlack above a multiple of 2^24, the
// exact (unbiased) slot lies in [fast - 2 kSlack, fast] and so in the same
// 2^24 bucket, and the fast level is the exact level. Otherwise (about one
// value in 4000) the four values of the float4 are recomputed through the
// division. `fast` is false when norm is so small that c could overflow
// (norm < 2^-96; c <= 2^96 * 127 * 2^24 stays finite): then every value
// divides.
constexpr uint32_t kSlack = 2048;

// Smallest norm for which the fast path's multiplier stays finite.
constexpr float kFastNormMin = 0x1p-96f;

// Level slots of four values (one float4 slot and its four Philox words):
// the level of value k is t[k] >> 24 (arithmetic), and byte 3 of t[k].
// c = fl(fl(1 / norm) * s24) when fast. `fast` is uniform across the launch,
// so its test is a scalar branch; the exact branch is taken per lane.
__device__ __forceinline__ void qsgd_slots4(f32x4 g, U4 r, float norm, float c, float s24,
                                            bool fast, int32_t t[4])
{
    const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
    uint32_t k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // 0x00FFFFFF when g has its sign bit set, else 0: v_perm's byte
        // selector 9 replicates bit 31 of its low operand, 12 gives 0x00
        const uint32_t flip = __builtin_amdgcn_perm(0u, __float_as_uint(g[j]), 0x0C090909u);
        k[j] = (rr[j] >> 8) ^ flip;
    }
    bool exact = true;
    if (fast) {
        uint32_t low[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t tj = uint32_t(static_cast<int32_t>(g[j] * c)) + k[j] + kSlack;
            t[j] = int32_t(tj);
            low[j] = tj & 0x00FFFFFFu;
        }
        exact = min(min(low[0], low[1]), min(low[2], low[3])) < 2 * kSlack;
    }
    if (exact) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            t[j] = int32_t(uint32_t(static_cast<int32_t>((g[j] / norm) * s24)) + k[j]);
    }
}

__device__ __forceinline__ int level_of(int32_t slot) { return slot >> 24; }

// The four levels as the little-endian int8 bytes of one word: byte 3 of
// each slot, gathered by two byte permutes (selector 3 / 7: byte 3 of the
// low / high operand; 12: 0x00).
__device__ __forceinline__ uint32_t pack_levels4(const int32_t t[4])
{
    const uint32_t lo = __builtin_amdgcn_perm(uint32_t(t[1]), uint32_t(t[0]), 0x0C0C0703u);
    const uint32_t hi = __builtin_amdgcn_perm(uint32_t(t[3]), uint32_t(t[2]), 0x07030C0Cu);
    return lo | hi;
}

// Each wave takes tiles of kQTile float4 slots, kQUnroll per lane: the
// Philox counter (q lo, q hi, worker, 0) of slot q gives the four words of
// elements 4q .. 4q+3, and a lane's kQUnroll independent Philox chains
// interleave to fill the VALU pipeline (8 quantizes of 138M values took
// 0.96 / 0.93 / 0.96 ms with 2 / 4 / 8 chains; the kernel sits at its HBM
// ceiling with the Philox rounds close behind). Full tiles take a
// branch-free vector path, through load_slots' LDS stage when the gradient
// is only 4-byte aligned; the one partial tile, and levels without 4-byte
// alignment, take a checked element path. kLoop = false: one tile per wave
// (the usual case).
constexpr int kQUnroll = 4;
constexpr size_t kQTile = size_t(kWave) * kQUnroll;
// The aligned quantize runs at most 5 workgroups per CU, held there by an
// LDS reservation: 106 against 116 us per 138M values with the 8 its
// registers allow (7 and 6 per CU: 115-116 us; 4: 107 us; 3: 121 us).
constexpr int kQuantizeWgPerCu = 5;
// Levels 1-3 bytes off 4-byte alignment: 6 per CU, 112-113 against 115-116
// us (5 per CU: 112-114; 3 and 4: 118-133). The kernels for gradients only
// 4-byte aligned gained nothing from a cap and keep what their own LDS
// allows.
constexpr int kQuantizeBytesWgPerCu = 6;

// Float4 slots tb + u kWave + lane (u < U) of g, one per lane per u. kDword:
// g is only 4-byte aligned, so the tile's 4 U kWave values come in as
// lane-contiguous 4-byte loads (256 bytes per instruction) and are regrouped
// into the lanes' float4 slots through the wave's LDS stage (4 U kWave
// floats).
template <int U, bool kDword>
__device__ __forceinline__ void load_slots(const float* __restrict__ g, size_t tb, int lane,
                                           f32x4 (&v)[U], float* stage)
{
    if (!kDword) {
        const size_t q0 = tb + lane;
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g) + q0 +
                                              size_t(u) * kWave);
        return;
    }
    const float* base = g + tb * 4;
    float x[4 * U];
#pragma unroll
    for (int j = 0; j < 4 * U; ++j)
        x[j] = __builtin_nontemporal_load(base + j * kWave + lane);
#pragma unroll
    for (int j = 0; j < 4 * U; ++j)
        stage[j * kWave + lane] = x[j];
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = reinterpret_cast<const f32x4*>(stage)[u * kWave + lane];
    wave_lds_sync();  // these reads precede the next tile's writes
}

// Stores a full tile's packed level words when the levels sit sh = 1..3
// bytes past a 4-byte boundary. Slot q's four levels (packed[u] of the lane
// holding q) start at byte sh of aligned word q (counted from levels - sh),
// so aligned word q holds the last sh levels of slot q - 1 and the first
// 4 - sh of slot q: v_alignbyte of the two packed words, the previous slot's
// coming from the lane before (lane 63 of the previous u for lane 0). Inside
// the tile every such word is stored whole; the tile's first aligned word
// and the word after its last (shared with the neighbouring tiles) get only
// this tile's bytes, as byte stores.
template <int U>
__device__ __forceinline__ void store_levels_shifted(int8_t* __restrict__ levels, uint32_t sh,
                                                     size_t q0, int lane, const uint32_t (&packed)[U])
{
    uint32_t* a = reinterpret_cast<uint32_t*>(levels - sh);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t prev = static_cast<uint32_t>(__shfl_up(static_cast<int>(packed[u]), 1));
        if (u > 0) {
            const uint32_t last = __builtin_amdgcn_readlane(packed[u - 1], kWave - 1);
            if (lane == 0)
                prev = last;
        }
        const uint32_t word = __builtin_amdgcn_alignbyte(packed[u], prev, 4u - sh);
        if (u > 0 || lane > 0)
            __builtin_nontemporal_store(word, a + q0 + size_t(u) * kWave);
    }
    if (lane == 0) {
        // the first 4 - sh levels of the tile's first slot
        for (uint32_t k = 0; k < 4u - sh; ++k)
            levels[q0 * 4 + k] = int8_t(packed[0] >> (8 * k));
    }
    if (lane == kWave - 1) {
        // the last sh levels of the tile's last slot
        const size_t ql = q0 + size_t(U - 1) * kWave;
        for (uint32_t k = 4u - sh; k < 4u; ++k)
            levels[ql * 4 + k] = int8_t(packed[U - 1] >> (8 * k));
    }
}

// kDword: grad 4- but not 16-byte aligned (loads through load_slots).
// kLvShift: levels 1-3 bytes past a 4-byte boundary (lv_shift bytes); full
// tiles store words through store_levels_shifted.
template <bool kLoop, bool kDword, bool kLvShift>
__device__ __forceinline__ void qsgd_quantize_body(const float* __restrict__ grad, size_t n,
                                                   const float* __restrict__ norm_ptr, float s24,
                                                   uint32_t k0, uint32_t k1, uint32_t worker,
                                                   int8_t* __restrict__ levels, int vec,
                                                   uint32_t lv_shift)
{
    __shared__ float stage[kDword ? kThreads / kWave : 1][kDword ? 4 * kQTile : 1];
    const bool gvec = vec && !kDword;  // grad itself 16-byte aligned
    const float norm = *norm_ptr;
    const bool fast = norm >= kFastNormMin;
    const float c = fast ? (1.0f / norm) * s24 : 0.0f;
    const size_t nslots = (n + 3) >> 2;
    const size_t nfull = n >> 2;
    const size_t ntiles = (nslots + kQTile - 1) / kQTile;
    const int lane = threadIdx.x & (kWave - 1);
    const size_t stride = size_t(gridDim.x) * (kThreads / kWave);
    for (size_t t = size_t(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave; t < ntiles;
         t += stride) {
        const size_t q0 = t * kQTile + lane;
        if (vec && (t + 1) * kQTile <= nfull) {
            f32x4 g[kQUnroll];
            load_slots<kQUnroll, kDword>(grad, t * kQTile, lane, g,
                                         stage[kDword ? threadIdx.x / kWave : 0]);
            uint32_t packed[kQUnroll] = {};
            if (norm != 0.0f) {
                U4 r[kQUnroll];
#pragma unroll
                for (int u = 0; u < kQUnroll; ++u) {
                    const size_t q = q0 + size_t(u) * kWave;
                    r[u] = philox4x32_10(U4{uint32_t(q), uint32_t(q >> 32), worker, 0u}, k0, k1);
                }
#pragma unroll
                for (int u = 0; u < kQUnroll; ++u) {
                    int32_t t[4];
                    qsgd_slots4(g[u], r[u], norm, c, s24, fast, t);
                    packed[u] = pack_levels4(t);
                }
            }
            if (kLvShift) {
                store_levels_shifted<kQUnroll>(levels, lv_shift, q0, lane, packed);
            } else {
#pragma unroll
                for (int u = 0; u < kQUnroll; ++u)
                    __builtin_nontemporal_store(packed[u], reinterpret_cast<uint32_t*>(levels) +
                                                               q0 + size_t(u) * kWave);
            }
        } else {
            // the partial tile, or levels without 4-byte alignment. Whole
            // float4 slots are still one load (16-byte-aligned gradient)
            // and one word (4-byte-aligned levels), and every slot's load
            // goes out before any math (the registers are zeroed first, so
            // that no branch rewrites a register with a load in flight); the
            // one slot that straddles n, and other alignments, go element by
            // element.
            f32x4 g[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u)
                g[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (gvec) {
#pragma unroll
                for (int u = 0; u < kQUnroll; ++u) {
                    const size_t q = q0 + size_t(u) * kWave;
                    if (q < nfull)
                        g[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(grad) + q);
                }
            }
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const size_t q = q0 + size_t(u) * kWave;
                if (q >= nslots)
                    continue;
                // the slot's levels as one word (levels 4-byte aligned)
                const bool whole = !kLvShift && vec && q < nfull;
                if (!(gvec && q < nfull)) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        g[u][k] = (q * 4 + k < n) ? grad[q * 4 + k] : 0.0f;
                }
                int32_t t[4] = {0, 0, 0, 0};
                if (norm != 0.0f) {
                    const U4 r =
                        philox4x32_10(U4{uint32_t(q), uint32_t(q >> 32), worker, 0u}, k0, k1);
                    qsgd_slots4(g[u], r, norm, c, s24, fast, t);
                }
                if (whole) {
                    __builtin_nontemporal_store(pack_levels4(t),
                                                reinterpret_cast<uint32_t*>(levels) + q);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (q * 4 + k < n)
                            levels[q * 4 + k] = int8_t(level_of(t[k]));
                }
            }
        }
        if (!kLoop)
            break;
    }
}

// Entry kernels of the body above, named apart so that profiles keep the
// aligned and the 4-byte-aligned gradients, and levels at byte offsets,
// separate.
template <bool kLoop>
__global__ __launch_bounds__(kThreads) void qsgd_quantize_kernel(
    const float* __restrict__ grad, size_t n, const float* __restrict__ norm_ptr, float s24,
    uint32_t k0, uint32_t k1, uint32_t worker, int8_t* __restrict__ levels, int vec)
{
    qsgd_quantize_body<kLoop, false, false>(grad, n, norm_ptr, s24, k0, k1, worker, levels, vec,
                                            0u);
}

template <bool kLoop>
__global__ __launch_bounds__(kThreads) void qsgd_quantize_dword_kernel(
    const float* __restrict__ grad, size_t n, const float* __restrict__ norm_ptr, float s24,
    uint32_t k0, uint32_t k1, uint32_t worker, int8_t* __restrict__ levels, int vec)
{
    qsgd_quantize_body<kLoop, true, false>(grad, n, norm_ptr, s24, k0, k1, worker, levels, vec,
                                           0u);
}

// Levels 1-3 bytes past a 4-byte boundary (lv_shift); kDword: the gradient
// 4- but not 16-byte aligned.
template <bool kLoop, bool kDword>
__global__ __launch_bounds__(kThreads) void qsgd_quantize_bytes_kernel(
    const float* __restrict__ grad, size_t n, const float* __restrict__ norm_ptr, float s24,
    uint32_t k0, uint32_t k1, uint32_t worker, int8_t* __restrict__ levels, uint32_t lv_shift)
{
    qsgd_quantize_body<kLoop, kDword, true>(grad, n, norm_ptr, s24, k0, k1, worker, levels, 1,
                                            lv_shift);
}

// ---- level sum + dequantize ------------------------------------------------

__device__ __forceinline__ float dequant(float norm, int S, float s_f)
{
    const float t = norm * float(S);
    return t / s_f;
}

__device__ __forceinline__ int sbyte(uint32_t w, int k)
{
    return int32_t(w << (24 - 8 * k)) >> 24;
}

// Dense form. vec: every level pointer 4-byte aligned, out 16-byte aligned,
// sums NULL or 16-byte aligned. Each wave takes tiles of kDqTile float4 slots
// (kDqUnroll per lane); WC > 0: W == WC at compile time, so every worker's
// level words are in flight together (WC == 0: W read at run time, in groups
// of four).
constexpr int kDqUnroll = 2;
constexpr size_t kDqTile = size_t(kWave) * kDqUnroll;
// At most 5 workgroups per CU (an LDS reservation; the registers allow 8).
// Over 138M values: W = 8, 359-360 against 366 us (4 per CU: 358; 3: 359-363);
// W = 2, 219-220 against 224-228 us (4 per CU: 227; 3: 257).
constexpr int kLevelSumWgPerCu = 5;
// Sums and outputs only 4-byte aligned (their tiles staged through LDS): 3
// per CU, 399-400 against 424-429 us at W = 8. Levels at byte offsets
// 1-3 keep what their registers allow: a cap made them up to 60% slower.
constexpr int kLevelSumDwordWgPerCu = 3;

__device__ __forceinline__ void dequant_store(float norm, float s_f, i32x4 S, int32_t* sums,
                                              float* out, size_t q)
{
    if (sums)
        __builtin_nontemporal_store(S, reinterpret_cast<i32x4*>(sums) + q);
    const f32x4 o = {dequant(norm, S.x, s_f), dequant(norm, S.y, s_f), dequant(norm, S.z, s_f),
                     dequant(norm, S.w, s_f)};
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(out) + q);
}

// Byte offset (0..3) of each worker's levels past the 4-byte-aligned address
// the kernel is given for them, two bits per worker.
struct LevelShifts {
    uint32_t s[GC_MAX_WORKERS / 16];
};

__device__ __forceinline__ uint32_t level_shift(const LevelShifts& ls, int w)
{
    return (ls.s[w >> 4] >> (2 * (w & 15))) & 3u;
}

// Levels of worker w at byte offset sh (1..3) past the aligned word array a:
// the four int8 levels of slot q are bytes sh .. sh+3 of the word pair
// (a[q], a[q+1]), i.e. v_alignbyte of the two. words[u] holds a[q + 64 u]
// for this lane's slots q; a[q + 1 + 64 u] is the next lane's word, lane 0's
// word of the next u for lane 63, and for lane 63 at the last u one more
// load. That word holds the tile's last level bytes, so it lies inside the
// buffer (a word holding at least one of its bytes).
template <int U>
__device__ __forceinline__ void align_level_words(const uint32_t* __restrict__ a, size_t q,
                                                  uint32_t sh, int lane, uint32_t (&words)[U])
{
    uint32_t hi[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        hi[u] = static_cast<uint32_t>(__shfl_down(static_cast<int>(words[u]), 1));
#pragma unroll
    for (int u = 0; u + 1 < U; ++u) {
        const uint32_t next0 = __builtin_amdgcn_readfirstlane(words[u + 1]);
        if (lane == kWave - 1)
            hi[u] = next0;
    }
    if (lane == kWave - 1)
        hi[U - 1] = a[q + size_t(U - 1) * kWave + 1];
#pragma unroll
    for (int u = 0; u < U; ++u)
        words[u] = __builtin_amdgcn_alignbyte(hi[u], words[u], sh);
}

// kDword: sums and out 4- but not 16-byte aligned: a full tile's sums and
// values pass through the wave's LDS stage and leave as lane-contiguous
// 4-byte stores. kLvAny: tab holds each worker's levels rounded down to 4-byte
// alignment, `shifts` the byte offsets past them; full tiles still load
// words (align_level_words), and the partial tile reads bytes at the offset.
template <int WC, bool kDword, bool kLvAny>
__device__ __forceinline__ void qsgd_dequant_sum_body(const PtrTable<int8_t>& tab,
                                                      const LevelShifts& shifts, int W_rt,
                                                      size_t n, const float* __restrict__ norm_ptr,
                                                      float s_f, int32_t* __restrict__ sums,
                                                      float* __restrict__ out, int vec)
{
    __shared__ i32x4 st_s[kDword ? kThreads / kWave : 1][kDword ? kDqTile : 1];
    __shared__ f32x4 st_o[kDword ? kThreads / kWave : 1][kDword ? kDqTile : 1];
    const int W = WC > 0 ? WC : W_rt;
    const float norm = *norm_ptr;
    const size_t nslots = (n + 3) >> 2;
    const size_t nfull = n >> 2;
    const size_t ntiles = (nslots + kDqTile - 1) / kDqTile;
    const int lane = threadIdx.x & (kWave - 1);
    const size_t stride = size_t(gridDim.x) * (kThreads / kWave);
    for (size_t t = size_t(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave; t < ntiles;
         t += stride) {
        const size_t q0 = t * kDqTile + lane;
        if (vec && (t + 1) * kDqTile <= nfull) {
            i32x4 S[kDqUnroll];
#pragma unroll
            for (int u = 0; u < kDqUnroll; ++u)
                S[u] = i32x4{0, 0, 0, 0};
            // WC > 0: every worker's words in flight together. W at run
            // time: groups of eight, the next group's words loaded before
            // this group is summed.
            constexpr int kGroup = WC > 0 ? WC : 8;
            auto load_group = [&](uint32_t(&dst)[kGroup][kDqUnroll], int w0) {
#pragma unroll
                for (int dw = 0; dw < kGroup; ++dw)
#pragma unroll
                    for (int u = 0; u < kDqUnroll; ++u)
                        dst[dw][u] = (WC == 0 && w0 + dw >= W)
                                         ? 0u
                                         : __builtin_nontemporal_load(
                                               reinterpret_cast<const uint32_t*>(tab.p[w0 + dw]) +
                                               q0 + size_t(u) * kWave);
            };
            uint32_t words[kGroup][kDqUnroll], ahead[WC > 0 ? 1 : kGroup][kDqUnroll];
            load_group(words, 0);
            for (int w0 = 0; w0 < W; w0 += kGroup) {
                if constexpr (WC == 0) {
                    if (w0 + kGroup < W)
                        load_group(ahead, w0 + kGroup);
                }
                if (kLvAny) {
#pragma unroll
                    for (int dw = 0; dw < kGroup; ++dw) {
                        if (WC == 0 && w0 + dw >= W)
                            break;
                        const uint32_t sh = level_shift(shifts, w0 + dw);  // uniform
                        if (sh)
                            align_level_words<kDqUnroll>(
                                reinterpret_cast<const uint32_t*>(tab.p[w0 + dw]), q0, sh, lane,
                                words[dw]);
                    }
                }
#pragma unroll
                for (int dw = 0; dw < kGroup; ++dw)
#pragma unroll
                    for (int u = 0; u < kDqUnroll; ++u) {
                        S[u].x += sbyte(words[dw][u], 0);
                        S[u].y += sbyte(words[dw][u], 1);
                        S[u].z += sbyte(words[dw][u], 2);
                        S[u].w += sbyte(words[dw][u], 3);
                    }
                if constexpr (WC == 0) {
#pragma unroll
                    for (int dw = 0; dw < kGroup; ++dw)
#pragma unroll
                        for (int u = 0; u < kDqUnroll; ++u)
                            words[dw][u] = ahead[dw][u];
                }
            }
            if (kDword) {
                const int wave = threadIdx.x / kWave;
#pragma unroll
                for (int u = 0; u < kDqUnroll; ++u) {
                    st_s[wave][u * kWave + lane] = S[u];
                    st_o[wave][u * kWave + lane] =
                        f32x4{dequant(norm, S[u].x, s_f), dequant(norm, S[u].y, s_f),
                              dequant(norm, S[u].z, s_f), dequant(norm, S[u].w, s_f)};
                }
                wave_lds_sync();
                const int32_t* ss = reinterpret_cast<const int32_t*>(st_s[wave]);
                const float* so = reinterpret_cast<const float*>(st_o[wave]);
                const size_t i0 = t * kDqTile * 4;
#pragma unroll
                for (int j = 0; j < int(kDqTile) * 4 / kWave; ++j) {
                    const int e = j * kWave + lane;
                    if (sums)
                        __builtin_nontemporal_store(ss[e], sums + i0 + e);
                    __builtin_nontemporal_store(so[e], out + i0 + e);
                }
                wave_lds_sync();  // these reads precede the next tile's writes
            } else {
#pragma unroll
                for (int u = 0; u < kDqUnroll; ++u)
                    dequant_store(norm, s_f, S[u], sums, out, q0 + size_t(u) * kWave);
            }
        } else {
            // the partial tile, or levels without 4-byte alignment
#pragma unroll 1
            for (int u = 0; u < kDqUnroll; ++u) {
                const size_t q = q0 + size_t(u) * kWave;
#pragma unroll 1
                for (size_t i = q * 4; i < q * 4 + 4 && i < n; ++i) {
                    int S = 0;
#pragma unroll 1
                    for (int w = 0; w < W; ++w)
                        S += int(tab.p[w][i + (kLvAny ? level_shift(shifts, w) : 0u)]);
                    if (sums)
                        sums[i] = S;
                    out[i] = dequant(norm, S, s_f);
                }
            }
        }
    }
}

// Entry kernels of the body above, named apart so that profiles keep the
// aligned and the 4-byte-aligned outputs, and the levels at byte offsets,
// separate.
template <int WC>
__global__ __launch_bounds__(kThreads) void qsgd_dequant_sum_kernel(
    PtrTable<int8_t> tab, int W, size_t n, const float* __restrict__ norm_ptr, float s_f,
    int32_t* __restrict__ sums, float* __restrict__ out, int vec)
{
    qsgd_dequant_sum_body<WC, false, false>(tab, LevelShifts{}, W, n, norm_ptr, s_f, sums, out,
                                            vec);
}

template <int WC>
__global__ __launch_bounds__(kThreads) void qsgd_dequant_sum_dword_kernel(
    PtrTable<int8_t> tab, int W, size_t n, const float* __restrict__ norm_ptr, float s_f,
    int32_t* __restrict__ sums, float* __restrict__ out, int vec)
{
    qsgd_dequant_sum_body<WC, true, false>(tab, LevelShifts{}, W, n, norm_ptr, s_f, sums, out,
                                           vec);
}

// Levels of some worker 1-3 bytes off 4-byte alignment; kDword as above.
template <int WC, bool kDword>
__global__ __launch_bounds__(kThreads) void qsgd_dequant_sum_bytes_kernel(
    PtrTable<int8_t> tab, LevelShifts shifts, int W, size_t n, const float* __restrict__ norm_ptr,
    float s_f, int32_t* __restrict__ sums, float* __restrict__ out)
{
    qsgd_dequant_sum_body<WC, kDword, true>(tab, shifts, W, n, norm_ptr, s_f, sums, out, 1);
}

// ---- fused quantize + level sum + dequantize --------------------------------
//
// The W quantizes and the dense level sum of one simulated step in a single
// pass: for each float4 slot, every worker's four Philox words (counter
// (q lo, q hi, w, 0), as in the quantize kernel) and four levels, with the
// same arithmetic, added into int32 sums, then dequantized. The int8 levels
// -- what each worker would put on the wire -- are never written: a step
// reads 4 W n bytes and writes 8 n (4 n without the sums) instead of
// 5 W n + W n + 8 n. Each wave takes a tile of kFUnroll float4 slots per
// lane, lane-contiguous, and runs through the workers one after another:
// every worker's 4 KB of the tile is one contiguous stream of loads, with
// the lane's kFUnroll Philox chains interleaved. At W = 8 over 138M values
// this measured 4-5% faster than one slot per thread with the workers'
// loads grouped by four. Full tiles take a branch-free vector path (staged
// through LDS for buffers only 4-byte aligned); the one partial tile goes
// slot by slot. kLoop = false: one tile per wave (the usual case).
constexpr int kFUnroll = 4;
constexpr size_t kFTile = size_t(kWave) * kFUnroll;

// kDword: some gradient, or out or sums, is 4- but not 16-byte aligned. Each
// worker's tile comes in through load_slots' LDS stage, and the same stage
// then regroups the sums and the values for lane-contiguous 4-byte stores.
template <int WC, bool kLoop, bool kDword>
__device__ __forceinline__ void qsgd_quantize_sum_body(const PtrTable<float>& tab, int W_rt,
                                                       size_t n,
                                                       const float* __restrict__ norm_ptr,
                                                       float s24, float s_f, uint32_t k0,
                                                       uint32_t k1, int32_t* __restrict__ sums,
                                                       float* __restrict__ out, int vec)
{
    __shared__ float stage_all[kDword ? kThreads / kWave : 1][kDword ? 4 * kFTile : 1];
    float* stage = stage_all[kDword ? threadIdx.x / kWave : 0];
    const int W = WC > 0 ? WC : W_rt;
    const float norm = *norm_ptr;
    const bool fast = norm >= kFastNormMin;
    const float c = fast ? (1.0f / norm) * s24 : 0.0f;
    const size_t nslots = (n + 3) >> 2;
    const size_t nfull = n >> 2;
    const size_t ntiles = (nslots + kFTile - 1) / kFTile;
    const int lane = threadIdx.x & (kWave - 1);
    const size_t stride = size_t(gridDim.x) * (kThreads / kWave);
    for (size_t t = size_t(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave; t < ntiles;
         t += stride) {
        const size_t q0 = t * kFTile + lane;
        if (vec && (t + 1) * kFTile <= nfull) {
            i32x4 S[kFUnroll];
#pragma unroll
            for (int u = 0; u < kFUnroll; ++u)
                S[u] = i32x4{0, 0, 0, 0};
            if (norm != 0.0f) {
#pragma unroll 1
                for (int w = 0; w < W; ++w) {
                    f32x4 g[kFUnroll];
                    load_slots<kFUnroll, kDword>(tab.p[w], t * kFTile, lane, g, stage);
                    U4 r[kFUnroll];
#pragma unroll
                    for (int u = 0; u < kFUnroll; ++u) {
                        const size_t q = q0 + size_t(u) * kWave;
                        r[u] = philox4x32_10(U4{uint32_t(q), uint32_t(q >> 32), uint32_t(w), 0u},
                                             k0, k1);
                    }
#pragma unroll
                    for (int u = 0; u < kFUnroll; ++u) {
                        int32_t tt[4];
                        qsgd_slots4(g[u], r[u], norm, c, s24, fast, tt);
                        S[u] += i32x4{level_of(tt[0]), level_of(tt[1]), level_of(tt[2]),
                                      level_of(tt[3])};
                    }
                }
            }
            if (kDword) {
                const size_t i0 = t * kFTile * 4;
                if (sums) {
#pragma unroll
                    for (int u = 0; u < kFUnroll; ++u)
                        reinterpret_cast<i32x4*>(stage)[u * kWave + lane] = S[u];
                    wave_lds_sync();
#pragma unroll
                    for (int j = 0; j < 4 * kFUnroll; ++j) {
                        const int e = j * kWave + lane;
                        __builtin_nontemporal_store(reinterpret_cast<const int32_t*>(stage)[e],
                                                    sums + i0 + e);
                    }
                    wave_lds_sync();
                }
#pragma unroll
                for (int u = 0; u < kFUnroll; ++u)
                    reinterpret_cast<f32x4*>(stage)[u * kWave + lane] =
                        f32x4{dequant(norm, S[u].x, s_f), dequant(norm, S[u].y, s_f),
                              dequant(norm, S[u].z, s_f), dequant(norm, S[u].w, s_f)};
                wave_lds_sync();
#pragma unroll
                for (int j = 0; j < 4 * kFUnroll; ++j) {
                    const int e = j * kWave + lane;
                    __builtin_nontemporal_store(stage[e], out + i0 + e);
                }
                wave_lds_sync();  // these reads precede the next tile's writes
            } else {
#pragma unroll
                for (int u = 0; u < kFUnroll; ++u)
                    dequant_store(norm, s_f, S[u], sums, out, q0 + size_t(u) * kWave);
            }
        } else {
            // the partial tile
#pragma unroll 1
            for (int u = 0; u < kFUnroll; ++u) {
                const size_t q = q0 + size_t(u) * kWave;
                if (q >= nslots)
                    break;
                i32x4 S = {0, 0, 0, 0};
#pragma unroll 1
                for (int w = 0; w < W; ++w) {
                    f32x4 g;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        g[k] = (q * 4 + k < n) ? tab.p[w][q * 4 + k] : 0.0f;
                    if (norm != 0.0f) {
                        int32_t tt[4];
                        qsgd_slots4(
                            g, philox4x32_10(U4{uint32_t(q), uint32_t(q >> 32), uint32_t(w), 0u},
                                             k0, k1),
                            norm, c, s24, fast, tt);
                        S += i32x4{level_of(tt[0]), level_of(tt[1]), level_of(tt[2]),
                                   level_of(tt[3])};
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const size_t i = q * 4 + k;
                    if (i < n) {
                        if (sums)
                            sums[i] = S[k];
                        out[i] = dequant(norm, S[k], s_f);
                    }
                }
            }
        }
        if (!kLoop)
            break;
    }
}

// Entry kernels of the body above, named apart so that profiles keep the
// aligned and the 4-byte-aligned buffers separate.
template <int WC, bool kLoop>
__global__ __launch_bounds__(kThreads) void qsgd_quantize_sum_kernel(
    PtrTable<float> tab, int W, size_t n, const float* __restrict__ norm_ptr, float s24,
    float s_f, uint32_t k0, uint32_t k1, int32_t* __restrict__ sums, float* __restrict__ out,
    int vec)
{
    qsgd_quantize_sum_body<WC, kLoop, false>(tab, W, n, norm_ptr, s24, s_f, k0, k1, sums, out,
                                             vec);
}

template <int WC, bool kLoop>
__global__ __launch_bounds__(kThreads) void qsgd_quantize_sum_dword_kernel(
    PtrTable<float> tab, int W, size_t n, const float* __restrict__ norm_ptr, float s24,
    float s_f, uint32_t k0, uint32_t k1, int32_t* __restrict__ sums, float* __restrict__ out,
    int vec)
{
    qsgd_quantize_sum_body<WC, kLoop, true>(tab, W, n, norm_ptr, s24, s_f, k0, k1, sums, out,
                                            vec);
}

constexpr int kFillUnroll = 4;

// Zero out[0, n) (out 4-byte aligned) with workgroups b = 0 .. nb-1 (of NT
// threads) of a launch: lane-contiguous non-temporal float4 stores. A buffer
// off 16-byte alignment has its head of at most 3 values zeroed by
// workgroup 0 and the 16-byte-aligned rest filled the same way (a fill does
// not care in which order the values are written).
template <int NT = kThreads>
__device__ __forceinline__ void fill_zero_range(float* __restrict__ out, size_t n, size_t b,
                                                size_t nb)
{
    const size_t head =
        std::min<size_t>(((16u - (reinterpret_cast<uintptr_t>(out) & 15u)) & 15u) / 4u, n);
    if (b == 0 && threadIdx.x < head)
        out[threadIdx.x] = 0.0f;
    out += head;
    n -= head;
    const size_t stride = nb * NT;
    const size_t tid = b * NT + threadIdx.x;
    const size_t nfull = n >> 2;
    f32x4* o4 = reinterpret_cast<f32x4*>(out);
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    // blocks of kFillUnroll * NT float4, lane-contiguous
    const size_t per = size_t(kFillUnroll) * NT;
    for (size_t c = b * per; c < nfull; c += nb * per) {
#pragma unroll
        for (int u = 0; u < kFillUnroll; ++u) {
            const size_t q = c + size_t(u) * NT + threadIdx.x;
            if (q < nfull)
                __builtin_nontemporal_store(z, o4 + q);
        }
    }
    for (size_t i = nfull * 4 + tid; i < n; i += stride)
        out[i] = 0.0f;
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* __restrict__ out, size_t n)
{
    fill_zero_range(out, n, blockIdx.x, gridDim.x);
}

// Sparse form: value k lands at out[idx[k]] (out already zeroed).
__global__ __launch_bounds__(kThreads) void qsgd_dequant_scatter_kernel(
    PtrTable<int8_t> tab, int W, size_t K, const float* __restrict__ norm_ptr, float s_f,
    int32_t* __restrict__ sums, float* __restrict__ out, const uint32_t* __restrict__ idx)
{
    const float norm = *norm_ptr;
    const size_t stride = size_t(gridDim.x) * kThreads;
    for (size_t k = size_t(blockIdx.x) * kThreads + threadIdx.x; k < K; k += stride) {
        int S = 0;
        for (int w = 0; w < W; ++w)
            S += int(tab.p[w][k]);
        if (sums)
            sums[k] = S;
        out[idx[k]] = dequant(norm, S, s_f);
    }
}

// ---- GlobalRandK index draw -------------------------------------------------
//
// The draw is a partial Fisher-Yates shuffle of 0..n-1: step t swaps
// positions t and j[t] >= t, and the index taken at step t is the value at
// position j[t] just before step t. Position p >= T is changed before step T
// only by earlier steps that targeted it, so its value before step T is:
//   the value position t' held before step t', for the last t' < T with
//   j[t'] == p; or p itself if no earlier step targeted it.
// Following that rule from (p, T) = (j[t], t) down to a position nobody
// targeted gives the index of step t, for every t in parallel. Draws are
// hashed by target position (chained buckets) to find "the last t' < T".
// One workgroup does it all: in LDS for K <= kRandKLdsMax (each chain step
// is an LDS access, not a round trip to L2), in the caller's workspace above.
constexpr int kRandKThreads = 1024;

__device__ __forceinline__ uint32_t slot_of(uint32_t p, int hbits)
{
    return (p * 0x9E3779B1u) >> (32 - hbits);
}

__global__ __launch_bounds__(kRandKThreads) void grandk_indices_kernel(
    size_t n, uint32_t K, uint32_t k0, uint32_t k1, uint32_t* __restrict__ idx,
    uint32_t* __restrict__ target, int32_t* __restrict__ next, int32_t* __restrict__ heads,
    int hbits)
{
    const uint32_t nheads = 1u << hbits;
    // draws; clear the buckets
    for (uint32_t t = threadIdx.x; t < K; t += kRandKThreads) {
        const U4 r = philox4x32_10(U4{t, 0u, 0u, 1u}, k0, k1);
        const uint64_t R = (uint64_t(r.y) << 32) | r.x;
        const uint64_t span = uint64_t(n) - t;
        target[t] = t + uint32_t(__umul64hi(R, span));
    }
    for (uint32_t h = threadIdx.x; h < nheads; h += kRandKThreads)
        heads[h] = -1;
    __threadfence();
    __syncthreads();
    __threadfence();
    // bucket every step by its target position
    for (uint32_t t = threadIdx.x; t < K; t += kRandKThreads)
        next[t] = atomicExch(&heads[slot_of(target[t], hbits)], int32_t(t));
    __threadfence();
    __syncthreads();
    __threadfence();
    // resolve
    for (uint32_t t = threadIdx.x; t < K; t += kRandKThreads) {
        uint32_t p = target[t];
        int32_t T = int32_t(t);
        for (;;) {
            int32_t best = -1;
            for (int32_t e = heads[slot_of(p, hbits)]; e >= 0; e = next[e])
                if (target[e] == p && e < T && e > best)
                    best = e;
            if (best < 0)
                break;
            p = uint32_t(best);
            T = best;
        }
        idx[t] = p;
    }
}

// K up to kRandKLdsMax: the whole structure lives in LDS (128 KB): targets,
// 16-bit chain links, and at most 2^13 bucket heads (load factor <= 2).
constexpr uint32_t kRandKLdsMax = 16384;
constexpr int kRandKLdsHeadBits = 13;

// The LDS draw by one workgroup of kRandKThreads threads.
__device__ __forceinline__ void grandk_draw_lds(size_t n, uint32_t K, uint32_t k0, uint32_t k1,
                                                uint32_t* __restrict__ idx, int hbits)
{
    __shared__ uint32_t target[kRandKLdsMax];
    __shared__ int16_t next[kRandKLdsMax];
    __shared__ int32_t heads[1 << kRandKLdsHeadBits];
    const uint32_t nheads = 1u << hbits;
    for (uint32_t t = threadIdx.x; t < K; t += kRandKThreads) {
        const U4 r = philox4x32_10(U4{t, 0u, 0u, 1u}, k0, k1);
        const uint64_t R = (uint64_t(r.y) << 32) | r.x;
        target[t] = t + uint32_t(__umul64hi(R, uint64_t(n) - t));
    }
    for (uint32_t h = threadIdx.x; h < nheads; h += kRandKThreads)
        heads[h] = -1;
    __syncthreads();
    for (uint32_t t = threadIdx.x; t < K; t += kRandKThreads)
        next[t] = int16_t(atomicExch(&heads[slot_of(target[t], hbits)], int32_t(t)));
    __syncthreads();
    for (uint32_t t = threadIdx.x; t < K; t += kRandKThreads) {
        uint32_t p = target[t];
        int32_t T = int32_t(t);
        for (;;) {
            int32_t best = -1;
            for (int32_t e = heads[slot_of(p, hbits)]; e >= 0; e = next[e])
                if (target[e] == p && e < T && e > best)
                    best = e;
            if (best < 0)
                break;
            p = uint32_t(best);
            T = best;
        }
        idx[t] = p;
    }
}

__global__ __launch_bounds__(kRandKThreads) void grandk_indices_lds_kernel(
    size_t n, uint32_t K, uint32_t k0, uint32_t k1, uint32_t* __restrict__ idx, int hbits)
{
    grandk_draw_lds(n, K, k0, k1, idx, hbits);
}

int randk_lds_hash_bits(uint32_t K)
{
    int b = 6;
    while (b < kRandKLdsHeadBits && (uint64_t(1) << b) < uint64_t(K))
        ++b;
    return b;
}

int randk_hash_bits(uint32_t K)
{
    int b = 6;
    while ((uint64_t(1) << b) < 2 * uint64_t(K))
        ++b;
    return b;
}

size_t randk_ws_bytes(uint32_t K)
{
    return 4 * ((size_t(1) << randk_hash_bits(K)) + 2 * size_t(K));
}

__global__ __launch_bounds__(kThreads) void gather_kernel(const float* __restrict__ x,
                                                          const uint32_t* __restrict__ idx,
                                                          size_t K, float* __restrict__ out)
{
    const size_t stride = size_t(gridDim.x) * kThreads;
    for (size_t k = size_t(blockIdx.x) * kThreads + threadIdx.x; k < K; k += stride)
        out[k] = x[idx[k]];
}

// ---- the whole GlobalRandK-MN step ------------------------------------------
//
// Three launches instead of one per worker per stage. Launch 1 is the index
// draw above, with the dense zero fill beside it when the draw runs in LDS.
// Launch 2: its first workgroups gather g_w[idx[k]] of every worker into the
// workspace (worker w at offset w * Kp, Kp = K rounded up to a multiple of 4)
// and write one partial max |g| each; any remaining workgroups zero the
// dense output (when launch 1 could not). Launch 3: every workgroup reduces the
// same partials to the shared norm (the max is exact and order-free), then
// takes float4 slots of the gathered values: for each worker the Philox
// words of (slot, worker, 0) and the levels, exactly as
// qsgd_maxnorm_quantize computes them on the gathered array; the int32 sum
// of the W levels; its dequantized value, scattered to dense[idx[k]].
constexpr unsigned kGkMaxGatherBlocks = 1024;
constexpr int kGkQThreads = 256;

// Launch 1 when K <= kRandKLdsMax: workgroup 0 draws the indices in LDS
// while the others zero dense[0, fill_n). The draw's 128 KB of LDS holds
// every workgroup of the launch to one per CU, which at 1024 threads still
// gives the fill 16 waves per CU.
__global__ __launch_bounds__(kRandKThreads) void grandk_draw_fill_kernel(
    size_t n, uint32_t K, uint32_t k0, uint32_t k1, uint32_t* __restrict__ idx, int hbits,
    float* __restrict__ dense, size_t fill_n)
{
    if (blockIdx.x == 0) {
        if (K > 0)
            grandk_draw_lds(n, K, k0, k1, idx, hbits);
        return;
    }
    fill_zero_range<kRandKThreads>(dense, fill_n, blockIdx.x - 1, gridDim.x - 1);
}

// Share of the dense fill that runs beside the LDS draw in launch 1; the
// rest runs beside the gathers in launch 2 (the scatter in launch 3 comes
// after both). Launch 1 lasts about max(draw, its fill), launch 2 about
// max(gathers, the rest of the fill), so the split puts about as much fill
// beside the draw as the draw takes. The draw is bound by one CU's ALU, so
// its time follows the device's core clock: measured on MI355X, about 2980
// cycles per index (1.24 ns at 2.4 GHz). The fill zeroes about 1.43 values
// per ns at this part's write rate. The split takes their product for the
// device's reported clock, 6% over, so that the fill (the longer job) stays
// on the critical path. Only the speed depends on it, never the results.
// Returns n, or a multiple of 4 below n, so that launch 2's part keeps
// dense's float4 alignment.
constexpr double kDrawCyclesPerIndex = 2980.0;
constexpr double kFillValuesPerNs = 1.43;
constexpr double kFillSplitMargin = 1.06;

// Core clock of the current device in GHz (2.4 if the runtime cannot say),
// queried once per device.
double core_clock_ghz()
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> khz[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 2.4;
    int v = dev >= 0 && dev < kMaxDevices ? khz[dev].load(std::memory_order_relaxed) : 0;
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate, dev) != hipSuccess || v <= 0)
            v = 2400000;
        if (dev >= 0 && dev < kMaxDevices)
            khz[dev].store(v, std::memory_order_relaxed);
    }
    return double(v) * 1e-6;
}

size_t grandk_fill_split(size_t n, uint32_t K)
{
    const double draw_ns = kDrawCyclesPerIndex / core_clock_ghz() * double(K);
    const double share = kFillSplitMargin * kFillValuesPerNs * draw_ns / double(n);
    if (share >= 1.0)
        return n;
    return size_t(share * double(n)) & ~size_t(3);
}

__global__ __launch_bounds__(kThreads) void grandk_gather_fill_kernel(
    PtrTable<float> tab, int W, uint32_t K, size_t Kp, const uint32_t* __restrict__ idx,
    float* __restrict__ gathered, float* __restrict__ partials, unsigned gather_blocks,
    float* __restrict__ dense, size_t n)
{
    if (blockIdx.x >= gather_blocks) {
        fill_zero_range(dense, n, blockIdx.x - gather_blocks,
                        gridDim.x - gather_blocks);
        return;
    }
    const size_t total = size_t(W) * K;
    float m = 0.0f;
    for (size_t e = size_t(blockIdx.x) * kThreads + threadIdx.x; e < total;
         e += size_t(gather_blocks) * kThreads) {
        const size_t w = e / K, k = e % K;
        const float v = tab.p[w][idx[k]];
        gathered[w * Kp + k] = v;
        m = fmaxf(m, fabsf(v));
    }
    m = block_max<kThreads>(m);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = m;
}

// One thread per (slot, worker): a workgroup takes kGkQThreads / W slots,
// each thread draws one worker's Philox words for its slot and adds the four
// levels into the slot's int32 sums in LDS (integer adds: exact in any
// order), then the slots are dequantized and scattered.
__global__ __launch_bounds__(kGkQThreads) void grandk_quantize_scatter_kernel(
    int W, uint32_t K, size_t Kp, const float* __restrict__ gathered,
    const float* __restrict__ partials, unsigned nparts, float s24, float s_f, uint32_t k0,
    uint32_t k1, const uint32_t* __restrict__ idx, int32_t* __restrict__ sums,
    float* __restrict__ dense, float* __restrict__ norm_out)
{
    __shared__ float norm_sh;
    __shared__ int32_t lsum[kGkQThreads][4];
    float m = 0.0f;
    for (unsigned i = threadIdx.x; i < nparts; i += kGkQThreads)
        m = fmaxf(m, partials[i]);
    m = block_max<kGkQThreads>(m);
    if (threadIdx.x == 0) {
        norm_sh = m;
        if (blockIdx.x == 0 && norm_out)
            *norm_out = m;
    }
    for (int e = threadIdx.x; e < kGkQThreads * 4; e += kGkQThreads)
        lsum[e >> 2][e & 3] = 0;
    __syncthreads();
    const float norm = norm_sh;
    const bool fast = norm >= kFastNormMin;
    const float c = fast ? (1.0f / norm) * s24 : 0.0f;
    const int spb = kGkQThreads / W;  // slots per workgroup pass (W <= 64: at least 4)
    const int ls = int(threadIdx.x) / W, w = int(threadIdx.x) % W;
    const size_t nslots = (size_t(K) + 3) >> 2;
    for (size_t base = size_t(blockIdx.x) * spb; base < nslots; base += size_t(gridDim.x) * spb) {
        const size_t q = base + size_t(ls);
        if (ls < spb && q < nslots && norm != 0.0f) {
            f32x4 g = reinterpret_cast<const f32x4*>(gathered + size_t(w) * Kp)[q];
            // the padding past K holds no value: level 0, as in the quantize
            // kernel's partial slot
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (q * 4 + k >= K)
                    g[k] = 0.0f;
            int32_t t[4];
            qsgd_slots4(g, philox4x32_10(U4{uint32_t(q), uint32_t(q >> 32), uint32_t(w), 0u}, k0, k1),
                        norm, c, s24, fast, t);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                atomicAdd(&lsum[ls][k], level_of(t[k]));
        }
        __syncthreads();
        for (int e = threadIdx.x; e < spb * 4; e += kGkQThreads) {
            const size_t i = (base + size_t(e >> 2)) * 4 + (e & 3);
            const int32_t S = lsum[e >> 2][e & 3];
            lsum[e >> 2][e & 3] = 0;
            if (i < K) {
                if (sums)
                    sums[i] = S;
                dense[idx[i]] = dequant(norm, S, s_f);
            }
        }
        __syncthreads();
    }
}

struct GrandkStepLayout {
    size_t Kp, gathered_off, partials_off, draw_off, total;
    unsigned gather_blocks;
};

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

GrandkStepLayout grandk_step_layout(int W, uint32_t K)
{
    GrandkStepLayout L{};
    L.Kp = (size_t(K) + 3) & ~size_t(3);
    const size_t total = size_t(W) * K;
    // at most half of the launch cap, so that the fill keeps workgroups too
    L.gather_blocks = unsigned(std::max<size_t>(
        1, std::min<size_t>({ceil_div(total, kThreads), size_t(kGkMaxGatherBlocks),
                             max_grid_blocks() / 2})));
    L.gathered_off = 0;
    L.partials_off = align256(size_t(W) * L.Kp * 4);
    L.draw_off = L.partials_off + align256(size_t(L.gather_blocks) * 4);
    L.total = L.draw_off + (K > kRandKLdsMax ? align256(randk_ws_bytes(K)) : 0);
    return L;
}

size_t grid_for(size_t items)
{
    return std::max<size_t>(1, std::min(ceil_div(items, kThreads), max_grid_blocks()));
}

}  // namespace
}  // namespace gcq

using namespace gcq;

namespace gcq {
namespace {

// The two launches of the max-norm, with the partial maxima in `partials`
// (mg.gx * W floats of device memory). Arguments are validated by the caller.
int launch_maxnorm(const PtrTable<float>& tab, int W, size_t n, const MaxNormGrid& mg,
                   float* partials, float* norm, hipStream_t stream)
{
    hipLaunchKernelGGL(maxabs_partial_kernel, dim3(mg.gx, unsigned(W)), dim3(kThreads),
                       lds_cap(maxabs_partial_kernel, kMaxAbsWgPerCu), stream, tab, n, mg.chunk4,
                       partials);
    if (int rc = check_launch("qsgd_global_maxnorm (partials)"))
        return rc;
    hipLaunchKernelGGL(max_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream, partials,
                       mg.gx * unsigned(W), norm);
    return check_launch("qsgd_global_maxnorm (final)");
}

// Validates the gradient pointers and the output of a max-norm call.
int maxnorm_table(const char* what, const float* const* grads, int W, size_t n, float* norm,
                  PtrTable<float>& tab)
{
    if (!grads || !norm || !aligned4(norm))
        return fail(GC_EINVAL, std::string(what) + ": NULL or misaligned pointer");
    for (int w = 0; w < W; ++w) {
        if ((n > 0 && !grads[w]) || !aligned4(grads[w]))
            return fail(GC_EINVAL, std::string(what) + ": a gradient pointer is NULL or misaligned");
        tab.p[w] = grads[w];
    }
    return GC_OK;
}

}  // namespace
}  // namespace gcq

GCQ_API int qsgd_global_maxnorm(const float* const* grads, int W, size_t n, float* norm, void* ws,
                                size_t* ws_bytes, hipStream_t stream)
{
    clear_error();
    if (W < 1 || W > GC_MAX_WORKERS)
        return fail(GC_EINVAL, "qsgd_global_maxnorm: W must be in [1, 64]");
    if (!ws_bytes)
        return fail(GC_EINVAL, "qsgd_global_maxnorm: ws_bytes is NULL");
    const MaxNormGrid mg = maxnorm_grid(n);
    const size_t need = size_t(mg.gx) * size_t(W) * sizeof(float);
    if (!ws) {
        *ws_bytes = need;
        return GC_OK;
    }
    if (*ws_bytes < need || !aligned4(ws))
        return fail(GC_EINVAL, "qsgd_global_maxnorm: workspace too small or misaligned");
    PtrTable<float> tab{};
    if (int rc = maxnorm_table("qsgd_global_maxnorm", grads, W, n, norm, tab))
        return rc;
    return launch_maxnorm(tab, W, n, mg, static_cast<float*>(ws), norm, stream);
}

// ---- the max-norm without a workspace ---------------------------------------
//
// For callers that cannot allocate (code under HIP graph capture, tight
// loops): the partial maxima go to this file-scope device array instead of a
// caller workspace. It holds the most partials any valid call makes:
// kMaxPartialsPerWorker workgroups for each of GC_MAX_WORKERS workers, 1 MiB;
// each device the library runs on keeps its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on each device comes from hipGetSymbolAddress, once per
// device, and only that address is passed to the kernels.
constexpr size_t kScratchFloats = size_t(gcq::kMaxPartialsPerWorker) * GC_MAX_WORKERS;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace gcq {
namespace {

constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kScratchMaxDevices] = {};

// Device address of `scratch` on the current device: looked up on the first
// call on that device (with that device current), then remembered.
int scratch_on_current_device(float** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(GC_EHIP, std::string("qsgd_global_maxnorm_noalloc: hipGetDevice: ") +
                                 hipGetErrorString(e));
    if (dev < 0 || dev >= kScratchMaxDevices)
        return fail(GC_EUNSUPPORTED, "qsgd_global_maxnorm_noalloc: device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GC_EHIP, std::string("qsgd_global_maxnorm_noalloc: hipGetSymbolAddress: ") +
                                     hipGetErrorString(e));
        g_scratch_dev[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_dev[dev];
    return GC_OK;
}

}  // namespace
}  // namespace gcq

GCQ_API int qsgd_global_maxnorm_noalloc(const float* const* grads, int W, size_t n, float* norm,
                                        hipStream_t stream)
{
    clear_error();
    if (W < 1 || W > GC_MAX_WORKERS)
        return fail(GC_EINVAL, "qsgd_global_maxnorm_noalloc: W must be in [1, 64]");
    const MaxNormGrid mg = maxnorm_grid(n);
    if (size_t(mg.gx) * size_t(W) > kScratchFloats)
        return fail(GC_EUNSUPPORTED, "qsgd_global_maxnorm_noalloc: the partial maxima exceed "
                                     "the fixed 1 MiB device array");
    PtrTable<float> tab{};
    if (int rc = maxnorm_table("qsgd_global_maxnorm_noalloc", grads, W, n, norm, tab))
        return rc;
    float* partials = nullptr;
    if (int rc = scratch_on_current_device(&partials))
        return rc;
    return launch_maxnorm(tab, W, n, mg, partials, norm, stream);
}

GCQ_API int qsgd_maxnorm_quantize(const float* grad, size_t n, const float* norm, int s,
                                  uint64_t seed, uint32_t worker, int8_t* levels,
                                  hipStream_t stream)
{
    clear_error();
    if (s < 1 || s > 127)
        return fail(GC_EINVAL, "qsgd_maxnorm_quantize: s must be in [1, 127]");
    if (!norm || !aligned4(norm))
        return fail(GC_EINVAL, "qsgd_maxnorm_quantize: norm is NULL or misaligned");
    if (n > 0 && (!grad || !levels))
        return fail(GC_EINVAL, "qsgd_maxnorm_quantize: grad or levels is NULL with n > 0");
    if (!aligned4(grad))
        return fail(GC_EINVAL, "qsgd_maxnorm_quantize: grad must be 4-byte aligned");
    if (n == 0)
        return GC_OK;
    const size_t ntiles = ceil_div(ceil_div(n, 4), kQTile);
    const size_t want = ceil_div(ntiles, kThreads / kWave);
    const dim3 grid(std::min(want, max_grid_blocks())), block(kThreads);
    const float s24 = float(s) * 16777216.0f;  // exact: s <= 127
    const bool loop = want > max_grid_blocks();
    if (!aligned4(levels)) {
        // levels 1-3 bytes past a 4-byte boundary: full tiles still store
        // words (realigned in registers), the gradient float4 or staged
        const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(levels) & 3u);
        const bool g16 = aligned16(grad);
#define GCQ_QB_LAUNCH(L, D)                                                                     \
    hipLaunchKernelGGL((qsgd_quantize_bytes_kernel<L, D>), grid, block,                           \
                       lds_cap((qsgd_quantize_bytes_kernel<L, D>), kQuantizeBytesWgPerCu),        \
                       stream, grad, n, norm, s24, uint32_t(seed), uint32_t(seed >> 32), worker,  \
                       levels, sh)
        if (loop && g16)
            GCQ_QB_LAUNCH(true, false);
        else if (loop)
            GCQ_QB_LAUNCH(true, true);
        else if (g16)
            GCQ_QB_LAUNCH(false, false);
        else
            GCQ_QB_LAUNCH(false, true);
#undef GCQ_QB_LAUNCH
        return check_launch("qsgd_maxnorm_quantize");
    }
    // levels 4-byte aligned: whole slots of levels as words; the gradient's
    // loads are float4 when it is 16-byte aligned, else staged
    const int vec = 1;
    const bool dword = !aligned16(grad);
    const int vec_kernel = aligned16(grad) ? 1 : 0;
#define GCQ_Q_LAUNCH(K, L, V, LDS)                                                            \
    hipLaunchKernelGGL((K<L>), grid, block, LDS, stream, grad, n, norm, s24, uint32_t(seed), \
                       uint32_t(seed >> 32), worker, levels, V)
    if (dword && loop)
        GCQ_Q_LAUNCH(qsgd_quantize_dword_kernel, true, vec, 0);
    else if (dword)
        GCQ_Q_LAUNCH(qsgd_quantize_dword_kernel, false, vec, 0);
    else if (loop)
        GCQ_Q_LAUNCH(qsgd_quantize_kernel, true, vec_kernel,
                     lds_cap(qsgd_quantize_kernel<true>, kQuantizeWgPerCu));
    else
        GCQ_Q_LAUNCH(qsgd_quantize_kernel, false, vec_kernel,
                     lds_cap(qsgd_quantize_kernel<false>, kQuantizeWgPerCu));
#undef GCQ_Q_LAUNCH
    return check_launch("qsgd_maxnorm_quantize");
}

GCQ_API int qsgd_dequant_sum(const int8_t* const* levels, int W, size_t n, const float* norm,
                             int s, int32_t* sums, float* out, const uint32_t* scatter_idx,
                             size_t dense_n, hipStream_t stream)
{
    clear_error();
    if (W < 1 || W > GC_MAX_WORKERS)
        return fail(GC_EINVAL, "qsgd_dequant_sum: W must be in [1, 64]");
    if (s < 1 || s > 127)
        return fail(GC_EINVAL, "qsgd_dequant_sum: s must be in [1, 127]");
    if (!levels || !norm || !aligned4(norm))
        return fail(GC_EINVAL, "qsgd_dequant_sum: NULL or misaligned pointer");
    if (!aligned4(out) || !aligned4(sums) || !aligned4(scatter_idx))
        return fail(GC_EINVAL, "qsgd_dequant_sum: out, sums and scatter_idx must be 4-byte aligned");
    const size_t out_n = scatter_idx ? dense_n : n;
    if (out_n > 0 && !out)
        return fail(GC_EINVAL, "qsgd_dequant_sum: out is NULL");
    if (scatter_idx && n > dense_n)
        return fail(GC_EINVAL, "qsgd_dequant_sum: more scattered values than dense_n");
    PtrTable<int8_t> tab{};
    bool lv_aligned = true;
    for (int w = 0; w < W; ++w) {
        if (n > 0 && !levels[w])
            return fail(GC_EINVAL, "qsgd_dequant_sum: a level pointer is NULL");
        tab.p[w] = levels[w];
        lv_aligned = lv_aligned && aligned4(levels[w]);
    }
    const float s_f = float(s);
    if (!scatter_idx) {
        if (n == 0)
            return GC_OK;
        const bool out_aligned = aligned16(out) && (!sums || aligned16(sums));
        if (!lv_aligned) {
            // levels 1-3 bytes off 4-byte alignment: word loads from each
            // worker's levels rounded down to 4 bytes, realigned in registers
            PtrTable<int8_t> base{};
            LevelShifts sh{};
            for (int w = 0; w < W; ++w) {
                const uint32_t b = uint32_t(reinterpret_cast<uintptr_t>(levels[w]) & 3u);
                base.p[w] = levels[w] - b;
                sh.s[w >> 4] |= b << (2 * (w & 15));
            }
            const size_t ntiles = ceil_div(ceil_div(n, 4), kDqTile);
            const dim3 grid(std::max<size_t>(1, std::min(ceil_div(ntiles, kThreads / kWave),
                                                         max_grid_blocks()))),
                block(kThreads);
#define GCQ_DQB_LAUNCH(k)                                                                      \
    do {                                                                                       \
        if (out_aligned)                                                                       \
            hipLaunchKernelGGL((qsgd_dequant_sum_bytes_kernel<k, false>), grid, block, 0,      \
                               stream, base, sh, W, n, norm, s_f, sums, out);                  \
        else                                                                                   \
            hipLaunchKernelGGL((qsgd_dequant_sum_bytes_kernel<k, true>), grid, block, 0,       \
                               stream, base, sh, W, n, norm, s_f, sums, out);                  \
    } while (0)
            if (W == 8)
                GCQ_DQB_LAUNCH(8);
            else
                GCQ_DQB_LAUNCH(0);
#undef GCQ_DQB_LAUNCH
            return check_launch("qsgd_dequant_sum");
        }
        // levels 4-byte aligned: word loads; outputs staged when not 16-byte aligned
        const bool dword = lv_aligned && !out_aligned;
        const int vec = lv_aligned ? 1 : 0;
        const size_t ntiles = ceil_div(ceil_div(n, 4), kDqTile);
        const dim3 grid(std::max<size_t>(1, std::min(ceil_div(ntiles, kThreads / kWave),
                                                     max_grid_blocks()))),
            block(kThreads);
        switch (W) {
#define GCQ_DQ_CASE(k)                                                                      \
    case k:                                                                                 \
        if (dword)                                                                          \
            hipLaunchKernelGGL((qsgd_dequant_sum_dword_kernel<k>), grid, block,             \
                               lds_cap(qsgd_dequant_sum_dword_kernel<k>,                    \
                                       kLevelSumDwordWgPerCu),                              \
                               stream, tab, W, n, norm, s_f, sums, out, vec);               \
        else                                                                                \
            hipLaunchKernelGGL((qsgd_dequant_sum_kernel<k>), grid, block,                   \
                               lds_cap(qsgd_dequant_sum_kernel<k>, kLevelSumWgPerCu),       \
                               stream, tab, W, n, norm, s_f, sums, out,                     \
                               out_aligned ? vec : 0);                                      \
        break;
            GCQ_DQ_CASE(1)
            GCQ_DQ_CASE(2)
            GCQ_DQ_CASE(3)
            GCQ_DQ_CASE(4)
            GCQ_DQ_CASE(5)
            GCQ_DQ_CASE(6)
            GCQ_DQ_CASE(7)
            GCQ_DQ_CASE(8)
#undef GCQ_DQ_CASE
        default:
            if (dword)
                hipLaunchKernelGGL((qsgd_dequant_sum_dword_kernel<0>), grid, block,
                                   lds_cap(qsgd_dequant_sum_dword_kernel<0>,
                                           kLevelSumDwordWgPerCu),
                                   stream, tab, W, n, norm, s_f, sums, out, vec);
            else
                hipLaunchKernelGGL((qsgd_dequant_sum_kernel<0>), grid, block,
                                   lds_cap(qsgd_dequant_sum_kernel<0>, kLevelSumWgPerCu),
                                   stream, tab, W, n, norm, s_f, sums, out,
                                   out_aligned ? vec : 0);
        }
        return check_launch("qsgd_dequant_sum");
    }
    if (dense_n > 0) {
        hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(ceil_div(dense_n, 4 * kFillUnroll))),
                           dim3(kThreads), 0, stream, out, dense_n);
        if (int rc = check_launch("qsgd_dequant_sum (fill)"))
            return rc;
    }
    if (n == 0)
        return GC_OK;
    hipLaunchKernelGGL(qsgd_dequant_scatter_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream,
                       tab, W, n, norm, s_f, sums, out, scatter_idx);
    return check_launch("qsgd_dequant_sum (scatter)");
}

GCQ_API int qsgd_quantize_sum(const float* const* grads, int W, size_t n, const float* norm,
                              int s, uint64_t seed, int32_t* sums, float* out,
                              hipStream_t stream)
{
    clear_error();
    if (W < 1 || W > GC_MAX_WORKERS)
        return fail(GC_EINVAL, "qsgd_quantize_sum: W must be in [1, 64]");
    if (s < 1 || s > 127)
        return fail(GC_EINVAL, "qsgd_quantize_sum: s must be in [1, 127]");
    if (!grads || !norm || !aligned4(norm))
        return fail(GC_EINVAL, "qsgd_quantize_sum: NULL or misaligned pointer");
    if (n > 0 && !out)
        return fail(GC_EINVAL, "qsgd_quantize_sum: out is NULL with n > 0");
    if (!aligned4(out) || !aligned4(sums))
        return fail(GC_EINVAL, "qsgd_quantize_sum: out and sums must be 4-byte aligned");
    PtrTable<float> tab{};
    bool g_aligned = true;
    for (int w = 0; w < W; ++w) {
        if (n > 0 && !grads[w])
            return fail(GC_EINVAL, "qsgd_quantize_sum: a gradient pointer is NULL");
        if (!aligned4(grads[w]))
            return fail(GC_EINVAL, "qsgd_quantize_sum: gradients must be 4-byte aligned");
        tab.p[w] = grads[w];
        g_aligned = g_aligned && aligned16(grads[w]);
    }
    if (n == 0)
        return GC_OK;
    const int vec = (g_aligned && aligned16(out) && (!sums || aligned16(sums))) ? 1 : 0;
    const size_t ntiles = ceil_div(ceil_div(n, 4), kFTile);
    const size_t want = ceil_div(ntiles, kThreads / kWave);
    const dim3 grid(unsigned(std::min(want, max_grid_blocks()))), block(kThreads);
    const bool loop = want > max_grid_blocks();
    const float s24 = float(s) * 16777216.0f;  // exact: s <= 127
    const float s_f = float(s);
    const uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
    // every buffer is 4-byte aligned here; without 16-byte alignment
    // everywhere, the staged kernel keeps whole tiles on the vector path
#define GCQ_QS_LAUNCH(k)                                                                       \
    do {                                                                                       \
        if (!vec && loop)                                                                      \
            hipLaunchKernelGGL((qsgd_quantize_sum_dword_kernel<k, true>), grid, block, 0,     \
                               stream, tab, W, n, norm, s24, s_f, k0, k1, sums, out, 1);      \
        else if (!vec)                                                                         \
            hipLaunchKernelGGL((qsgd_quantize_sum_dword_kernel<k, false>), grid, block, 0,    \
                               stream, tab, W, n, norm, s24, s_f, k0, k1, sums, out, 1);      \
        else if (loop)                                                                         \
            hipLaunchKernelGGL((qsgd_quantize_sum_kernel<k, true>), grid, block, 0, stream,   \
                               tab, W, n, norm, s24, s_f, k0, k1, sums, out, vec);            \
        else                                                                                   \
            hipLaunchKernelGGL((qsgd_quantize_sum_kernel<k, false>), grid, block, 0, stream,  \
                               tab, W, n, norm, s24, s_f, k0, k1, sums, out, vec);            \
    } while (0)
    switch (W) {
    case 1: GCQ_QS_LAUNCH(1); break;
    case 2: GCQ_QS_LAUNCH(2); break;
    case 4: GCQ_QS_LAUNCH(4); break;
    case 8: GCQ_QS_LAUNCH(8); break;
    default: GCQ_QS_LAUNCH(0);
    }
#undef GCQ_QS_LAUNCH
    return check_launch("qsgd_quantize_sum");
}

GCQ_API int grandk_indices(size_t n, uint32_t K, uint64_t seed, uint32_t* idx, void* ws,
                           size_t* ws_bytes, hipStream_t stream)
{
    clear_error();
    if (!ws_bytes)
        return fail(GC_EINVAL, "grandk_indices: ws_bytes is NULL");
    if (n < 1 || n > (size_t(1) << 32) || size_t(K) > n)
        return fail(GC_EINVAL, "grandk_indices: need 1 <= n <= 2^32 and K <= n");
    if (K > (1u << 30))
        return fail(GC_EUNSUPPORTED, "grandk_indices: K above 2^30");
    const size_t need = randk_ws_bytes(K);
    if (!ws) {
        *ws_bytes = need;
        return GC_OK;
    }
    if (*ws_bytes < need || !aligned4(ws))
        return fail(GC_EINVAL, "grandk_indices: workspace too small or misaligned");
    if (K > 0 && (!idx || !aligned4(idx)))
        return fail(GC_EINVAL, "grandk_indices: idx is NULL or misaligned");
    if (K == 0)
        return GC_OK;
    if (K <= kRandKLdsMax) {
        hipLaunchKernelGGL(grandk_indices_lds_kernel, dim3(1), dim3(kRandKThreads), 0, stream, n,
                           K, uint32_t(seed), uint32_t(seed >> 32), idx, randk_lds_hash_bits(K));
        return check_launch("grandk_indices");
    }
    const int hbits = randk_hash_bits(K);
    int32_t* heads = static_cast<int32_t*>(ws);
    uint32_t* target = reinterpret_cast<uint32_t*>(heads + (size_t(1) << hbits));
    int32_t* next = reinterpret_cast<int32_t*>(target + K);
    hipLaunchKernelGGL(grandk_indices_kernel, dim3(1), dim3(kRandKThreads), 0, stream, n, K,
                       uint32_t(seed), uint32_t(seed >> 32), idx, target, next, heads, hbits);
    return check_launch("grandk_indices");
}

GCQ_API int gather_f32(const float* x, const uint32_t* idx, size_t K, float* out,
                       hipStream_t stream)
{
    clear_error();
    if (K > 0 && (!x || !idx || !out))
        return fail(GC_EINVAL, "gather_f32: NULL pointer with K > 0");
    if (!aligned4(x) || !aligned4(idx) || !aligned4(out))
        return fail(GC_EINVAL, "gather_f32: buffers must be 4-byte aligned");
    if (K == 0)
        return GC_OK;
    hipLaunchKernelGGL(gather_kernel, dim3(grid_for(K)), dim3(kThreads), 0, stream, x, idx, K,
                       out);
    return check_launch("gather_f32");
}

GCQ_API int grandk_mn_step(const float* const* grads, int W, size_t n, uint32_t K,
                           uint64_t seed, int s, uint32_t* idx, int32_t* sums, float* dense,
                           float* norm, void* ws, size_t* ws_bytes, hipStream_t stream)
{
    clear_error();
    if (!ws_bytes)
        return fail(GC_EINVAL, "grandk_mn_step: ws_bytes is NULL");
    if (W < 1 || W > GC_MAX_WORKERS)
        return fail(GC_EINVAL, "grandk_mn_step: W must be in [1, 64]");
    if (s < 1 || s > 127)
        return fail(GC_EINVAL, "grandk_mn_step: s must be in [1, 127]");
    if (n < 1 || n > (size_t(1) << 32) || size_t(K) > n)
        return fail(GC_EINVAL, "grandk_mn_step: need 1 <= n <= 2^32 and K <= n");
    if (K > (1u << 30))
        return fail(GC_EUNSUPPORTED, "grandk_mn_step: K above 2^30");
    const GrandkStepLayout L = grandk_step_layout(W, K);
    if (!ws) {
        *ws_bytes = L.total;
        return GC_OK;
    }
    if (*ws_bytes < L.total || !aligned16(ws))
        return fail(GC_EINVAL, "grandk_mn_step: workspace too small or not 16-byte aligned");
    if (!grads || !dense || !aligned4(dense) || !aligned4(sums) || !aligned4(norm))
        return fail(GC_EINVAL, "grandk_mn_step: NULL or misaligned pointer");
    if (K > 0 && (!idx || !aligned4(idx)))
        return fail(GC_EINVAL, "grandk_mn_step: idx is NULL or misaligned");
    PtrTable<float> tab{};
    for (int w = 0; w < W; ++w) {
        if (!grads[w] || !aligned4(grads[w]))
            return fail(GC_EINVAL, "grandk_mn_step: a gradient pointer is NULL or misaligned");
        tab.p[w] = grads[w];
    }
    char* base = static_cast<char*>(ws);
    float* gathered = reinterpret_cast<float*>(base + L.gathered_off);
    float* partials = reinterpret_cast<float*>(base + L.partials_off);
    const uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
    const size_t cap = max_grid_blocks();
    // launch 1: the shared index draw; with the draw in LDS, the dense zero
    // fill runs beside it in the same launch
    size_t split = 0;  // dense[0, split) is zeroed in launch 1, the rest in launch 2
    if (K <= kRandKLdsMax) {
        split = grandk_fill_split(n, K);
        const size_t fb = std::max<size_t>(
            1, std::min(ceil_div(ceil_div(split, 4 * kFillUnroll), kRandKThreads),
                        cap > 1 ? cap - 1 : 1));
        hipLaunchKernelGGL(grandk_draw_fill_kernel, dim3(unsigned(1 + fb)), dim3(kRandKThreads),
                           0, stream, n, K, k0, k1, idx, randk_lds_hash_bits(K), dense, split);
    } else {
        const int hbits = randk_hash_bits(K);
        int32_t* heads = reinterpret_cast<int32_t*>(base + L.draw_off);
        uint32_t* target = reinterpret_cast<uint32_t*>(heads + (size_t(1) << hbits));
        int32_t* next = reinterpret_cast<int32_t*>(target + K);
        hipLaunchKernelGGL(grandk_indices_kernel, dim3(1), dim3(kRandKThreads), 0, stream, n, K,
                           k0, k1, idx, target, next, heads, hbits);
    }
    if (int rc = check_launch("grandk_mn_step (draw)"))
        return rc;
    // launch 2: gathers and partial maxima, and the fill of dense[split, n)
    const size_t rest = n - split;
    const size_t fill_blocks =
        rest == 0 ? 0
                  : std::max<size_t>(1, std::min(ceil_div(ceil_div(rest, 4 * kFillUnroll), kThreads),
                                                 cap > L.gather_blocks ? cap - L.gather_blocks : 1));
    hipLaunchKernelGGL(grandk_gather_fill_kernel, dim3(unsigned(L.gather_blocks + fill_blocks)),
                       dim3(kThreads), 0, stream, tab, W, K, L.Kp, idx, gathered, partials,
                       L.gather_blocks, dense + split, rest);
    if (int rc = check_launch("grandk_mn_step (gather, fill)"))
        return rc;
    // launch 3: norm, levels, sum, dequantize, scatter
    const size_t spb = size_t(kGkQThreads / W);
    const size_t qblocks = std::max<size_t>(
        1, std::min(ceil_div(ceil_div(size_t(K), 4), spb), max_grid_blocks()));
    const float s24 = float(s) * 16777216.0f;  // exact: s <= 127
    hipLaunchKernelGGL(grandk_quantize_scatter_kernel, dim3(unsigned(qblocks)), dim3(kGkQThreads),
                       0, stream, W, K, L.Kp, gathered, partials, L.gather_blocks, s24, float(s),
                       k0, k1, idx, sums, dense, norm);
    return check_launch("grandk_mn_step (quantize, scatter)");
}
