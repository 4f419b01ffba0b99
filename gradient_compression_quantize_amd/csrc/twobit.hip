// twobit.hip -- 2-bit threshold quantization with residual error feedback,
// its dequantization / W-worker sum, and the many-tensor launcher.
//
// Method: apache/incubator-mxnet PR #8342 "[WIP] 2bit gradient compression",
// sections "Approach" (quantize before sending, keep the error as a
// residual added to the next gradient), "Two bit quantization" (inclusive
// thresholds, codes 01 / 10 / 00), "Format of compressed gradient" (header
// of neg threshold, pos threshold, size; 16 codes per 32-bit element, first
// value in the most significant pair), "Local kvstore" (every worker's
// buffer is dequantized and summed on the reducing device).
//
// Layout and mapping (HBM-bound, ~12.25 bytes moved per element):
//  - one wave owns a tile of kUnroll float4 slots per lane, lane-contiguous,
//    so each load/store instruction moves 1 KiB of grad / residual;
//  - the 4 codes of a lane's float4 form one byte; a DPP quad-OR joins the
//    4 bytes of lanes 4k..4k+3 into the 32-bit word of 16 codes, and one
//    ds_bpermute lines the tile's 64 words up so that lane L stores word L:
//    every payload word is written exactly once, in one coalesced store per
//    tile, with no atomics and no pre-zeroing of the output;
//  - the last tile of a tensor runs the same packing with the slots past n
//    read as zeros (code 00, never read or written) and the one float4 slot
//    that straddles n read and written element by element.
#include "gcq_internal.h"
#include "threshold_codes.h"

#include <algorithm>
#include <cmath>
#include <vector>

namespace gcq {
namespace {

constexpr int kThreads = 256;                          // 4 waves
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kUnroll = 4;                             // float4 per lane per tile
constexpr size_t kTileF4 = size_t(kWave) * kUnroll;    // 256 float4 slots
constexpr size_t kTileElems = kTileF4 * 4;             // 1024 values
constexpr size_t kBlockElems = kTileElems * kWavesPerBlock;  // 4096 values
// The compress runs at most 3 workgroups (12 waves) per CU, held there by
// an LDS reservation: measured ~1.4% faster over 8 x 25.6M values than the
// 8 its registers allow (49.5 against 50.2 us per launch); 4 per CU gained
// ~0.9%, 2 per CU nothing. Buffers only 4-byte aligned: 54.8-54.9 against
// 55.3-55.6 us.
constexpr int kCompressWgPerCu = 3;
// The many-tensor compress likewise, at 3 per CU: 213 against 219 us over
// the BERT-Base list (4 per CU: 215 us). The dequantize-sum keeps the 8 its
// registers allow: every cap from 3 to 6 per CU made it 2-20% slower, its
// LDS decode needing the waves to hide latency.
constexpr int kMultiWgPerCu = 3;
constexpr int kDequantWgPerCu = 0;
// A tile is 64 words of codes, one per lane: the cross-lane moves that
// gather and scatter words rely on it.
static_assert(kUnroll == 4 && kTileF4 == 256, "one tile = 64 words of codes");

// Code and residual of four values. Thresholds satisfy neg < 0 < pos, so at
// most one of the two comparisons holds and value 0 is always code 00.
__device__ __forceinline__ void classify4(f32x4 g, f32x4 r, float neg, float pos,
                                          f32x4& rn, uint32_t& byte)
{
    byte = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float v = g[k] + r[k];
        bool up = v >= pos;
        bool dn = v <= neg;
        float d = up ? pos : (dn ? neg : 0.0f);
        rn[k] = v - d;
        uint32_t c = up ? 1u : (dn ? 2u : 0u);
        byte |= c << (6 - 2 * k);
    }
}

// OR over the 16 lanes of each DPP row; every lane of the row gets the
// result. A quad OR, then rotations by 4 and 8 lanes within the row
// (row_ror:4 = 0x124, row_ror:8 = 0x128).
__device__ __forceinline__ uint32_t row_or(uint32_t x)
{
    x = quad_or(x);
    x |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(x), 0x124, 0xF, 0xF, true));
    x |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(x), 0x128, 0xF, 0xF, true));
    return x;
}

// One wave tile of kTileElems values starting at element e0 (a multiple of
// 16), for grad and residual of any 4-byte alignment: lane-contiguous 4-byte
// accesses, one value per lane in each of 16 steps (each load and store
// instruction moves 256 contiguous bytes). In step j, row r of the wave
// holds values e0 + 64 j + 16 r .. + 15, i.e. word 4 j + r of the tile; a
// row OR forms it and lane 4 j + r keeps it, so the tile's 64 words still
// leave in one coalesced store. kFull: the whole tile is below n; otherwise
// values at or past n are neither read nor written (code 00) and only words
// below ceil(n / 16) are stored.
template <bool kFull>
__device__ __forceinline__ void compress_dword_tile(const float* __restrict__ grad,
                                                    float* __restrict__ residual, size_t n,
                                                    float neg, float pos,
                                                    uint32_t* __restrict__ payload, size_t e0,
                                                    int lane)
{
    constexpr int kSteps = int(kTileElems) / kWave;
    float g[kSteps], r[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
        const size_t e = e0 + size_t(j) * kWave + lane;
        g[j] = 0.0f;
        r[j] = 0.0f;
        if (kFull || e < n) {
            g[j] = __builtin_nontemporal_load(grad + e);
            r[j] = __builtin_nontemporal_load(residual + e);
        }
    }
    const uint32_t shift = 30u - 2u * uint32_t(lane & 15);
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
        const size_t e = e0 + size_t(j) * kWave + lane;
        const float v = g[j] + r[j];
        const bool up = v >= pos;
        const bool dn = v <= neg;
        const float d = up ? pos : (dn ? neg : 0.0f);
        if (kFull || e < n)
            __builtin_nontemporal_store(v - d, residual + e);
        const uint32_t c = up ? 1u : (dn ? 2u : 0u);
        const uint32_t word = row_or(c << shift);
        // lane 4 j + r takes row r's word (row r starts at lane 16 r)
        const uint32_t w = static_cast<uint32_t>(
            __builtin_amdgcn_ds_bpermute(64 * (lane & 3), static_cast<int>(word)));
        if ((lane >> 2) == j)
            mine = w;
    }
    const size_t jw = (e0 >> 4) + lane;
    if (kFull || jw < ((n + 15) >> 4))
        __builtin_nontemporal_store(mine, payload + jw);
}

// Tile e0 for grad or residual without 16-byte alignment.
__device__ __forceinline__ void compress_dword_tile_any(const float* __restrict__ grad,
                                                        float* __restrict__ residual, size_t n,
                                                        float neg, float pos,
                                                        uint32_t* __restrict__ payload,
                                                        size_t e0, int lane)
{
    if (e0 + kTileElems <= n)
        compress_dword_tile<true>(grad, residual, n, neg, pos, payload, e0, lane);
    else
        compress_dword_tile<false>(grad, residual, n, neg, pos, payload, e0, lane);
}

// One full wave tile: float4 slots q0 .. q0 + kTileF4 - 1, all below n / 4.
// `payload` is the block's element 3 (first word of codes).
__device__ __forceinline__ void compress_full_tile(const float* __restrict__ grad,
                                                   float* __restrict__ residual, float neg,
                                                   float pos, uint32_t* __restrict__ payload,
                                                   size_t q0, int lane)
{
    const f32x4* g4 = reinterpret_cast<const f32x4*>(grad);
    f32x4* r4 = reinterpret_cast<f32x4*>(residual);
    f32x4 g[kUnroll], r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const size_t q = q0 + size_t(u) * kWave + lane;
        // both streams are touched once: non-temporal loads keep them from
        // displacing each other in the caches
        g[u] = __builtin_nontemporal_load(g4 + q);
        r[u] = __builtin_nontemporal_load(r4 + q);
    }
    const uint32_t shift = 24u - 8u * uint32_t(lane & 3);
    uint32_t kept = 0;  // lane 4k + m keeps its quad's word of slot m
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const size_t q = q0 + size_t(u) * kWave + lane;
        f32x4 rn;
        uint32_t byte;
        classify4(g[u], r[u], neg, pos, rn, byte);
        __builtin_nontemporal_store(rn, r4 + q);
        const uint32_t word = quad_or(byte << shift);
        if ((lane & 3) == u)
            kept = word;
    }
    // The tile's 64 words leave in one coalesced 256-byte store: word L
    // covers slots 4L..4L+3, i.e. quad L % 16 of slot u = L / 16, which lane
    // 4 (L % 16) + L / 16 kept.
    const uint32_t mine = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(
        (4 * (lane & 15) + (lane >> 4)) * 4, static_cast<int>(kept)));
    __builtin_nontemporal_store(mine, payload + (q0 >> 2) + lane);
}

// The last tile of a tensor, partly below n: the full tile's arithmetic and
// cross-lane packing, with float4 slots at or past n / 4 read as zeros (code
// 00; nothing read or written there) and the one slot that straddles n read
// and written element by element. Every lane takes part in the DPP and
// ds_bpermute steps; only words below ceil(n / 16) are stored.
__device__ __forceinline__ void compress_partial_tile(const float* __restrict__ grad,
                                                      float* __restrict__ residual, size_t n,
                                                      float neg, float pos,
                                                      uint32_t* __restrict__ payload, size_t q0,
                                                      int lane)
{
    const f32x4* g4 = reinterpret_cast<const f32x4*>(grad);
    f32x4* r4 = reinterpret_cast<f32x4*>(residual);
    const size_t nq = n >> 2;  // float4 slots wholly below n
    const uint32_t rem = uint32_t(n & 3);
    const uint32_t shift = 24u - 8u * uint32_t(lane & 3);
    uint32_t kept = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const size_t q = q0 + size_t(u) * kWave + lane;
        f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f}, r = {0.0f, 0.0f, 0.0f, 0.0f};
        if (q < nq) {
            g = __builtin_nontemporal_load(g4 + q);
            r = __builtin_nontemporal_load(r4 + q);
        } else if (q == nq) {
            for (uint32_t k = 0; k < rem; ++k) {
                g[k] = grad[q * 4 + k];
                r[k] = residual[q * 4 + k];
            }
        }
        f32x4 rn;
        uint32_t byte;
        classify4(g, r, neg, pos, rn, byte);
        if (q < nq) {
            __builtin_nontemporal_store(rn, r4 + q);
        } else if (q == nq) {
            for (uint32_t k = 0; k < rem; ++k)
                residual[q * 4 + k] = rn[k];
        }
        const uint32_t word = quad_or(byte << shift);
        if ((lane & 3) == u)
            kept = word;
    }
    const uint32_t mine = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(
        (4 * (lane & 15) + (lane >> 4)) * 4, static_cast<int>(kept)));
    const size_t j = (q0 >> 2) + lane;
    if (j < ((n + 15) >> 4))
        payload[j] = mine;
}

// Tile q0 of a tensor of n values (grad and residual 16-byte aligned).
__device__ __forceinline__ void compress_tile(const float* __restrict__ grad,
                                              float* __restrict__ residual, size_t n, float neg,
                                              float pos, uint32_t* __restrict__ payload,
                                              size_t q0, int lane)
{
    if (q0 + kTileF4 <= (n >> 2))
        compress_full_tile(grad, residual, neg, pos, payload, q0, lane);
    else
        compress_partial_tile(grad, residual, n, neg, pos, payload, q0, lane);
}

// 16-byte-aligned grad and residual. kLoop = false: the grid has one wave
// per tile (the usual case); true: a capped grid strides over the tiles.
template <bool kLoop>
__global__ __launch_bounds__(kThreads) void compress_2bit_vec_kernel(
    const float* __restrict__ grad, float* __restrict__ residual, size_t n, float neg,
    float pos, float n_f, uint32_t* __restrict__ compr, size_t ntiles)
{
    if (blockIdx.x == 0 && threadIdx.x == 0)
        write_header(compr, neg, pos, n_f);
    const int lane = threadIdx.x & (kWave - 1);
    const size_t stride = size_t(gridDim.x) * kWavesPerBlock;
    // Tiles in dispatch order. (Measured: an XCD-contiguous mapping is ~5%
    // slower here -- eight separate streaming windows cost more in DRAM
    // locality than the few shared edge lines of the code words save -- and
    // taking the partial tile first is ~1% slower while hiding nothing
    // measurable.)
    for (size_t t = size_t(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; t < ntiles;
         t += stride) {
        compress_tile(grad, residual, n, neg, pos, compr + 3, t * kTileF4, lane);
        if (!kLoop)
            break;
    }
}

// Any 4-byte alignment of grad and residual: the same wave tiles through
// lane-contiguous 4-byte accesses (compress_dword_tile).
template <bool kLoop>
__global__ __launch_bounds__(kThreads) void compress_2bit_dword_kernel(
    const float* __restrict__ grad, float* __restrict__ residual, size_t n, float neg,
    float pos, float n_f, uint32_t* __restrict__ compr, size_t ntiles)
{
    if (blockIdx.x == 0 && threadIdx.x == 0)
        write_header(compr, neg, pos, n_f);
    const int lane = threadIdx.x & (kWave - 1);
    const size_t stride = size_t(gridDim.x) * kWavesPerBlock;
    for (size_t t = size_t(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; t < ntiles;
         t += stride) {
        compress_dword_tile_any(grad, residual, n, neg, pos, compr + 3, t * kTileElems, lane);
        if (!kLoop)
            break;
    }
}

// One wave tile of the W-block dequantize-and-sum (see compress_wave_tile).
// The tile's 1024 values are 64 words of each block: lane L loads word L
// (one coalesced 256-byte load per worker), and a ds_bpermute hands each
// lane the word of its float4 slot (word 16u + L/4 for slot u), so no word
// is fetched from memory twice. Decoding goes through the LDS nibble table.
// WC > 0: W == WC is known at compile time, so every worker's word is loaded
// before any is decoded; WC == 0: W read at run time, each lane decoding its
// own word (see the branch below).
// kDword: out without 16-byte alignment. The tile's float4 slots go to the
// wave's LDS stage and leave as lane-contiguous 4-byte stores.
// pre: this lane's W words, already loaded (WC > 0), or NULL to load them here.
template <int WC, bool kAcc, bool kDword>
__device__ __forceinline__ void decompress_full_tile(const PtrTable<uint32_t>& tab, int W_rt,
                                                     const float2* lut,
                                                     float* __restrict__ out, size_t q0,
                                                     int lane, f32x4* stage,
                                                     const uint32_t* pre = nullptr)
{
    const int W = WC > 0 ? WC : W_rt;
    const size_t jmine = (q0 >> 2) + lane;  // the word this lane fetches
    const uint32_t shift = 24u - 8u * uint32_t(lane & 3);
    f32x4* o4 = reinterpret_cast<f32x4*>(out);
    f32x4 acc[kUnroll];
    // Adds workers w0 .. w0 + G - 1 (those below W) of `words` into acc.
    auto decode = [&](const uint32_t* words, int w0, int G) {
#pragma unroll
        for (int dw = 0; dw < G; ++dw) {
            const int w = w0 + dw;
            if (WC == 0 && w >= W)
                break;
            const float2* t = lut + 16 * w;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                // all 64 lanes take part: lane 16u + L/4 holds this slot's word
                const uint32_t word = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(
                    (16 * u + (lane >> 2)) * 4, static_cast<int>(words[dw])));
                const uint32_t byte = (word >> shift) & 0xFFu;
                const float2 hi = t[byte >> 4];
                const float2 lo = t[byte & 15u];
                const f32x4 d = {hi.x, hi.y, lo.x, lo.y};
                acc[u] = (w == 0) ? d : acc[u] + d;
            }
        }
    };
    if constexpr (WC > 0) {
        // every worker's word in flight together
        uint32_t mine[WC];
#pragma unroll
        for (int w = 0; w < WC; ++w)
            mine[w] = pre ? pre[w] : __builtin_nontemporal_load(tab.p[w] + 3 + jmine);
        decode(mine, 0, WC);
    } else {
        // W at run time. Every lane decodes its own word of each worker (16
        // values, float4 slots 4L .. 4L+3 of the tile): no ds_bpermute per
        // worker, which at large W costs more than the table reads. Workers
        // go in groups of kGroup, the next group's words loaded before this
        // group is decoded; the tile then leaves through the wave's LDS
        // stage as lane-contiguous stores.
        constexpr int kGroup = 8;
        auto load = [&](uint32_t(&dst)[kGroup], int w0) {
#pragma unroll
            for (int dw = 0; dw < kGroup; ++dw)
                dst[dw] = w0 + dw < W ? __builtin_nontemporal_load(tab.p[w0 + dw] + 3 + jmine) : 0u;
        };
        float v16[16];
        uint32_t cur[kGroup], nxt[kGroup];
        load(cur, 0);
        for (int w0 = 0; w0 < W; w0 += kGroup) {
            if (w0 + kGroup < W)
                load(nxt, w0 + kGroup);
#pragma unroll
            for (int dw = 0; dw < kGroup; ++dw) {
                const int w = w0 + dw;
                if (w >= W)
                    break;
                const float2* t = lut + 16 * w;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t byte = (cur[dw] >> (24 - 8 * b)) & 0xFFu;
                    const float2 hi = t[byte >> 4];
                    const float2 lo = t[byte & 15u];
                    const float d[4] = {hi.x, hi.y, lo.x, lo.y};
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        v16[4 * b + k] = (w == 0) ? d[k] : v16[4 * b + k] + d[k];
                }
            }
#pragma unroll
            for (int dw = 0; dw < kGroup; ++dw)
                cur[dw] = nxt[dw];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            stage[4 * lane + k] = f32x4{v16[4 * k], v16[4 * k + 1], v16[4 * k + 2], v16[4 * k + 3]};
        wave_lds_sync();
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc[u] = stage[u * kWave + lane];
        if (kDword)
            wave_lds_sync();  // the staged reads below start from these same slots
    }
    if (kDword) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            stage[u * kWave + lane] = acc[u];
        wave_lds_sync();
        const float* sf = reinterpret_cast<const float*>(stage);
        float* o = out + q0 * 4;
#pragma unroll
        for (int j = 0; j < int(kTileElems) / kWave; ++j) {
            const int e = j * kWave + lane;
            float v = sf[e];
            if (kAcc)
                v = o[e] + v;
            __builtin_nontemporal_store(v, o + e);
        }
        wave_lds_sync();  // these reads precede the next tile's writes
        return;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const size_t q = q0 + size_t(u) * kWave + lane;
        f32x4 v = acc[u];
        if (kAcc)
            v = o4[q] + v;
        __builtin_nontemporal_store(v, o4 + q);
    }
}

// The last, partial tile: lane L decodes word q0/4 + L through the nibble
// table, one word load per worker, and writes the values below n.
__device__ __forceinline__ void decompress_tail_tile(const PtrTable<uint32_t>& tab, int W,
                                                     const float2* lut, size_t n,
                                                     float* __restrict__ out, int accumulate,
                                                     size_t q0, int lane)
{
    const size_t j = (q0 >> 2) + lane;
    if (j >= ((n + 15) >> 4))
        return;
    float acc[16];
#pragma unroll 1
    for (int w = 0; w < W; ++w) {
        const uint32_t word = tab.p[w][3 + j];
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
            const float2 v = lut[16 * w + ((word >> (28 - 2 * k)) & 15u)];
            acc[k] = (w == 0) ? v.x : acc[k] + v.x;
            acc[k + 1] = (w == 0) ? v.y : acc[k + 1] + v.y;
        }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const size_t i = j * 16 + k;
        if (i < n)
            out[i] = accumulate ? out[i] + acc[k] : acc[k];
    }
}

// Dequantize-and-sum of W blocks into out (kAcc: added to what out holds);
// kDword: out is 4- but not 16-byte aligned.
template <int WC, bool kAcc, bool kLoop, bool kDword>
__device__ __forceinline__ void decompress_2bit_body(const PtrTable<uint32_t>& tab, int W, size_t n,
                                                     float* __restrict__ out, size_t ntiles)
{
    __shared__ float2 lut[16 * GC_MAX_WORKERS];
    // the wave's stage: output transposes for 4-byte-aligned out, and the
    // run-time-W decode's hand-over from word order to store order
    constexpr bool kStage = kDword || WC == 0;
    __shared__ f32x4 stage[kStage ? kWavesPerBlock : 1][kStage ? kTileF4 : 1];
    const int lane = threadIdx.x & (kWave - 1);
    if (!kLoop && WC > 0) {
        // One tile per wave, W known: the tile's word loads go out before
        // the table is built, so they are in flight during the header loads
        // and the barrier (measured ~2% faster at W = 8 than loading after).
        const size_t t = xcd_contiguous(blockIdx.x, gridDim.x) * kWavesPerBlock + threadIdx.x / kWave;
        const size_t q0 = t < ntiles ? (ntiles - 1 - t) * kTileF4 : 0;
        const bool full = t < ntiles && q0 + kTileF4 <= (n >> 2);
        uint32_t pre[WC > 0 ? WC : 1];
        if (full) {
#pragma unroll
            for (int w = 0; w < (WC > 0 ? WC : 1); ++w)
                pre[w] = __builtin_nontemporal_load(tab.p[w] + 3 + (q0 >> 2) + lane);
        }
        build_nibble_table(lut, tab, WC);
        if (full)
            decompress_full_tile<WC, kAcc, kDword>(tab, W, lut, out, q0, lane,
                                                   stage[kStage ? threadIdx.x / kWave : 0], pre);
        else if (t < ntiles)
            decompress_tail_tile(tab, WC, lut, n, out, kAcc ? 1 : 0, q0, lane);
        return;
    }
    build_nibble_table(lut, tab, WC > 0 ? WC : W);
    const size_t stride = size_t(gridDim.x) * kWavesPerBlock;
    // Last tile first: the partial tile's scalar path reads all W blocks
    // word by word, so it starts with the first wave. XCD-contiguous: a
    // tile's 64 words of a block start 12 bytes into a cache line, so each
    // tile edge shares a line with the next tile; keeping neighbouring tiles
    // on one XCD fetches that line into one L2 instead of two (~10% fewer
    // bytes read from HBM).
    const size_t blk = kLoop ? blockIdx.x : xcd_contiguous(blockIdx.x, gridDim.x);
    for (size_t t = blk * kWavesPerBlock + threadIdx.x / kWave; t < ntiles; t += stride) {
        const size_t q0 = (ntiles - 1 - t) * kTileF4;
        if (q0 + kTileF4 <= (n >> 2))
            decompress_full_tile<WC, kAcc, kDword>(tab, W, lut, out, q0, lane,
                                                   stage[kStage ? threadIdx.x / kWave : 0]);
        else
            decompress_tail_tile(tab, WC > 0 ? WC : W, lut, n, out, kAcc ? 1 : 0, q0, lane);
        if (!kLoop)
            break;
    }
}

// The two entry kernels of the body above, named apart so that profiles
// keep the aligned and the 4-byte-aligned paths separate.
template <int WC, bool kAcc, bool kLoop>
__global__ __launch_bounds__(kThreads) void decompress_2bit_vec_kernel(
    PtrTable<uint32_t> tab, int W, size_t n, float* __restrict__ out, size_t ntiles)
{
    decompress_2bit_body<WC, kAcc, kLoop, false>(tab, W, n, out, ntiles);
}

template <int WC, bool kAcc, bool kLoop>
__global__ __launch_bounds__(kThreads) void decompress_2bit_dword_kernel(
    PtrTable<uint32_t> tab, int W, size_t n, float* __restrict__ out, size_t ntiles)
{
    decompress_2bit_body<WC, kAcc, kLoop, true>(tab, W, n, out, ntiles);
}

// ---- many tensors ----------------------------------------------------------

// One workgroup's share: kBlockElems values of one tensor, with everything
// the workgroup needs about that tensor in the same 48 bytes, so that it
// starts streaming after a single (scalar) descriptor load.
struct alignas(16) ChunkDesc {
    const float* grad;
    float* residual;
    uint64_t n;
    uint64_t word_off;  // first uint32 element of this tensor's block
    float n_f;          // (float)n, converted on the host
    uint32_t chunk;     // index of the kBlockElems-sized chunk inside the tensor
    uint32_t vec_ok;    // grad and residual both 16-byte aligned
    uint32_t pad;
};
static_assert(sizeof(ChunkDesc) == 48, "one 48-byte descriptor per chunk");

template <bool kLoop>
__global__ __launch_bounds__(kThreads) void compress_2bit_multi_kernel(
    const ChunkDesc* __restrict__ chunks, size_t nchunks, float neg, float pos,
    uint32_t* __restrict__ compr_base)
{
    const int lane = threadIdx.x & (kWave - 1);
    for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const ChunkDesc cd = chunks[c];
        uint32_t* blk = compr_base + cd.word_off;
        if (cd.chunk == 0 && threadIdx.x == 0)
            write_header(blk, neg, pos, cd.n_f);
        if (cd.vec_ok) {
            const size_t q0 = size_t(cd.chunk) * (kBlockElems / 4) +
                              size_t(threadIdx.x / kWave) * kTileF4;
            compress_tile(cd.grad, cd.residual, cd.n, neg, pos, blk + 3, q0, lane);
        } else {
            const size_t e0 = size_t(cd.chunk) * kBlockElems +
                              size_t(threadIdx.x / kWave) * kTileElems;
            if (e0 < cd.n)
                compress_dword_tile_any(cd.grad, cd.residual, cd.n, neg, pos, blk + 3, e0, lane);
        }
        if (!kLoop)
            break;
    }
}


size_t grid_for_tiles(size_t ntiles)
{
    return std::max<size_t>(1, std::min(ceil_div(ntiles, kWavesPerBlock), max_grid_blocks()));
}

// Whether a grid_for_tiles grid must stride (more tiles than waves).
bool tiles_need_loop(size_t ntiles)
{
    return ceil_div(ntiles, kWavesPerBlock) > max_grid_blocks();
}

}  // namespace
}  // namespace gcq

struct gc_plan {
    int device = 0;
    int T = 0;
    size_t nchunks = 0;
    size_t total_words = 0;
    std::vector<size_t> offsets;
    gcq::ChunkDesc* d_chunks = nullptr;
};

using namespace gcq;

GCQ_API size_t gc_compressed_2bit_words(size_t n) { return 3 + n / 16 + (n % 16 != 0 ? 1 : 0); }

GCQ_API int compress_2bit(const float* grad, float* residual, size_t n, float neg_threshold,
                          float pos_threshold, uint32_t* compr, hipStream_t stream)
{
    clear_error();
    if (!compr)
        return fail(GC_EINVAL, "compress_2bit: compr is NULL");
    if (n > 0 && (!grad || !residual))
        return fail(GC_EINVAL, "compress_2bit: grad or residual is NULL with n > 0");
    if (int rc = check_thresholds(neg_threshold, pos_threshold))
        return rc;
    if (!aligned4(compr) || !aligned4(grad) || !aligned4(residual))
        return fail(GC_EINVAL, "compress_2bit: buffers must be 4-byte aligned");
    const float n_f = static_cast<float>(n);
    if (n == 0 || (aligned16(grad) && aligned16(residual))) {
        const size_t ntiles = ceil_div(n, kTileElems);
        const dim3 grid(grid_for_tiles(ntiles)), block(kThreads);
        if (tiles_need_loop(ntiles))
            hipLaunchKernelGGL(compress_2bit_vec_kernel<true>, grid, block,
                               lds_cap(compress_2bit_vec_kernel<true>, kCompressWgPerCu),
                               stream, grad, residual, n, neg_threshold, pos_threshold, n_f,
                               compr, ntiles);
        else
            hipLaunchKernelGGL(compress_2bit_vec_kernel<false>, grid, block,
                               lds_cap(compress_2bit_vec_kernel<false>, kCompressWgPerCu),
                               stream, grad, residual, n, neg_threshold, pos_threshold, n_f,
                               compr, ntiles);
    } else {
        const size_t ntiles = ceil_div(n, kTileElems);
        const dim3 grid(grid_for_tiles(ntiles)), block(kThreads);
        if (tiles_need_loop(ntiles))
            hipLaunchKernelGGL(compress_2bit_dword_kernel<true>, grid, block,
                               lds_cap(compress_2bit_dword_kernel<true>, kCompressWgPerCu),
                               stream, grad, residual, n, neg_threshold, pos_threshold, n_f,
                               compr, ntiles);
        else
            hipLaunchKernelGGL(compress_2bit_dword_kernel<false>, grid, block,
                               lds_cap(compress_2bit_dword_kernel<false>, kCompressWgPerCu),
                               stream, grad, residual, n, neg_threshold, pos_threshold, n_f,
                               compr, ntiles);
    }
    return check_launch("compress_2bit");
}

template <bool kLoop, bool kDword>
static void launch_decompress_vec(const PtrTable<uint32_t>& tab, int W, size_t n, float* out,
                                  int accumulate, size_t ntiles, dim3 grid, dim3 block,
                                  hipStream_t stream)
{
    if (accumulate) {
        // only decompress_2bit accumulates (W == 1)
        if (kDword)
            hipLaunchKernelGGL((decompress_2bit_dword_kernel<1, true, kLoop>), grid, block, 0,
                               stream, tab, W, n, out, ntiles);
        else
            hipLaunchKernelGGL((decompress_2bit_vec_kernel<1, true, kLoop>), grid, block, 0,
                               stream, tab, W, n, out, ntiles);
        return;
    }
    switch (W) {
#define GCQ_DEC_CASE(k)                                                                    \
    case k:                                                                                \
        if (kDword)                                                                        \
            hipLaunchKernelGGL((decompress_2bit_dword_kernel<k, false, kLoop>), grid,      \
                               block, 0, stream, tab, W, n, out, ntiles);                  \
        else                                                                               \
            hipLaunchKernelGGL((decompress_2bit_vec_kernel<k, false, kLoop>), grid, block, \
                               lds_cap((decompress_2bit_vec_kernel<k, false, kLoop>),      \
                                       kDequantWgPerCu),                                   \
                               stream, tab, W, n, out, ntiles);                            \
        break;
        GCQ_DEC_CASE(1)
        GCQ_DEC_CASE(2)
        GCQ_DEC_CASE(3)
        GCQ_DEC_CASE(4)
        GCQ_DEC_CASE(5)
        GCQ_DEC_CASE(6)
        GCQ_DEC_CASE(7)
        GCQ_DEC_CASE(8)
#undef GCQ_DEC_CASE
    default:
        if (kDword)
            hipLaunchKernelGGL((decompress_2bit_dword_kernel<0, false, kLoop>), grid, block, 0,
                               stream, tab, W, n, out, ntiles);
        else
            hipLaunchKernelGGL((decompress_2bit_vec_kernel<0, false, kLoop>), grid, block,
                               lds_cap((decompress_2bit_vec_kernel<0, false, kLoop>),
                                       kDequantWgPerCu),
                               stream, tab, W, n, out, ntiles);
    }
}

static int launch_decompress(const PtrTable<uint32_t>& tab, int W, size_t n, float* out,
                             int accumulate, hipStream_t stream, const char* what)
{
    if (n == 0)
        return GC_OK;
    const size_t ntiles = ceil_div(n, kTileElems);
    const dim3 grid(grid_for_tiles(ntiles)), block(kThreads);
    const bool loop = tiles_need_loop(ntiles);
    if (aligned16(out)) {
        if (loop)
            launch_decompress_vec<true, false>(tab, W, n, out, accumulate, ntiles, grid, block, stream);
        else
            launch_decompress_vec<false, false>(tab, W, n, out, accumulate, ntiles, grid, block, stream);
    } else {
        if (loop)
            launch_decompress_vec<true, true>(tab, W, n, out, accumulate, ntiles, grid, block, stream);
        else
            launch_decompress_vec<false, true>(tab, W, n, out, accumulate, ntiles, grid, block, stream);
    }
    return check_launch(what);
}

GCQ_API int decompress_2bit(const uint32_t* compr, size_t n, float* out, int accumulate,
                            hipStream_t stream)
{
    clear_error();
    if (!compr)
        return fail(GC_EINVAL, "decompress_2bit: compr is NULL");
    if (n > 0 && !out)
        return fail(GC_EINVAL, "decompress_2bit: out is NULL with n > 0");
    if (accumulate != 0 && accumulate != 1)
        return fail(GC_EINVAL, "decompress_2bit: accumulate must be 0 or 1");
    if (!aligned4(compr) || !aligned4(out))
        return fail(GC_EINVAL, "decompress_2bit: buffers must be 4-byte aligned");
    PtrTable<uint32_t> tab{};
    tab.p[0] = compr;
    return launch_decompress(tab, 1, n, out, accumulate, stream, "decompress_2bit");
}

GCQ_API int decompress_2bit_sum(const uint32_t* const* compr, int W, size_t n, float* out,
                                hipStream_t stream)
{
    clear_error();
    if (!compr)
        return fail(GC_EINVAL, "decompress_2bit_sum: compr is NULL");
    if (W < 1 || W > GC_MAX_WORKERS)
        return fail(GC_EINVAL, "decompress_2bit_sum: W must be in [1, 64]");
    if (n > 0 && !out)
        return fail(GC_EINVAL, "decompress_2bit_sum: out is NULL with n > 0");
    if (!aligned4(out))
        return fail(GC_EINVAL, "decompress_2bit_sum: out must be 4-byte aligned");
    PtrTable<uint32_t> tab{};
    for (int w = 0; w < W; ++w) {
        if (!compr[w] || !aligned4(compr[w]))
            return fail(GC_EINVAL, "decompress_2bit_sum: a block pointer is NULL or misaligned");
        tab.p[w] = compr[w];
    }
    return launch_decompress(tab, W, n, out, 0, stream, "decompress_2bit_sum");
}

GCQ_API int gc_plan_2bit_multi_create(const float* const* grads, float* const* residuals,
                                      const size_t* ns, int T, gc_plan** plan)
{
    clear_error();
    if (!plan)
        return fail(GC_EINVAL, "gc_plan_2bit_multi_create: plan is NULL");
    *plan = nullptr;
    if (T < 1 || !grads || !residuals || !ns)
        return fail(GC_EINVAL, "gc_plan_2bit_multi_create: need T >= 1 and host arrays");

    std::vector<ChunkDesc> chunks;
    std::vector<size_t> offsets(static_cast<size_t>(T));
    size_t off = 0;
    for (int t = 0; t < T; ++t) {
        const size_t n = ns[t];
        if (n > 0 && (!grads[t] || !residuals[t]))
            return fail(GC_EINVAL, "gc_plan_2bit_multi_create: NULL tensor with n > 0");
        if (!aligned4(grads[t]) || !aligned4(residuals[t]))
            return fail(GC_EINVAL, "gc_plan_2bit_multi_create: tensors must be 4-byte aligned");
        const size_t nch = std::max<size_t>(1, ceil_div(n, kBlockElems));
        if (nch > 0xFFFFFFFFull)
            return fail(GC_EUNSUPPORTED, "gc_plan_2bit_multi_create: tensor too large");
        ChunkDesc d{};
        d.grad = grads[t];
        d.residual = residuals[t];
        d.n = n;
        d.word_off = off;
        d.n_f = static_cast<float>(n);
        d.vec_ok = (aligned16(grads[t]) && aligned16(residuals[t])) ? 1u : 0u;
        offsets[static_cast<size_t>(t)] = off;
        off += gc_compressed_2bit_words(n);
        // chunks in tensor order, each tensor's in address order (putting the
        // chunks that hold a partial tile first measured ~1.5% slower)
        for (size_t c = 0; c < nch; ++c) {
            d.chunk = static_cast<uint32_t>(c);
            chunks.push_back(d);
        }
    }

    gc_plan* p = new gc_plan();
    p->T = T;
    p->nchunks = chunks.size();
    p->total_words = off;
    p->offsets = std::move(offsets);
    if (hipGetDevice(&p->device) != hipSuccess ||
        hipMalloc(&p->d_chunks, chunks.size() * sizeof(ChunkDesc)) != hipSuccess ||
        hipMemcpy(p->d_chunks, chunks.data(), chunks.size() * sizeof(ChunkDesc),
                  hipMemcpyHostToDevice) != hipSuccess) {
        const hipError_t e = hipGetLastError();
        gc_plan_destroy(p);
        return fail(GC_EHIP, std::string("gc_plan_2bit_multi_create: ") + hipGetErrorString(e));
    }
    *plan = p;
    return GC_OK;
}

GCQ_API size_t gc_plan_compressed_words(const gc_plan* plan)
{
    return plan ? plan->total_words : 0;
}

GCQ_API int gc_plan_block_offsets(const gc_plan* plan, size_t* offsets)
{
    clear_error();
    if (!plan || !offsets)
        return fail(GC_EINVAL, "gc_plan_block_offsets: NULL argument");
    std::copy(plan->offsets.begin(), plan->offsets.end(), offsets);
    return GC_OK;
}

GCQ_API int compress_2bit_multi(gc_plan* plan, float neg_threshold, float pos_threshold,
                                uint32_t* compr_base, hipStream_t stream)
{
    clear_error();
    if (!plan || !compr_base)
        return fail(GC_EINVAL, "compress_2bit_multi: NULL plan or compr_base");
    if (int rc = check_thresholds(neg_threshold, pos_threshold))
        return rc;
    if (!aligned4(compr_base))
        return fail(GC_EINVAL, "compress_2bit_multi: compr_base must be 4-byte aligned");
    // the descriptor table and the tensors it points to live on the plan's
    // device: launching on another would read them from the wrong GPU
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return fail(GC_EHIP, "compress_2bit_multi: hipGetDevice failed");
    if (cur != plan->device)
        return fail(GC_EINVAL, "compress_2bit_multi: the plan was created on device " +
                                   std::to_string(plan->device) + ", the current device is " +
                                   std::to_string(cur));
    const size_t blocks = std::min(plan->nchunks, max_grid_blocks());
    if (blocks < plan->nchunks)
        hipLaunchKernelGGL(compress_2bit_multi_kernel<true>, dim3(blocks), dim3(kThreads),
                           lds_cap(compress_2bit_multi_kernel<true>, kMultiWgPerCu), stream,
                           plan->d_chunks, plan->nchunks, neg_threshold, pos_threshold,
                           compr_base);
    else
        hipLaunchKernelGGL(compress_2bit_multi_kernel<false>, dim3(blocks), dim3(kThreads),
                           lds_cap(compress_2bit_multi_kernel<false>, kMultiWgPerCu), stream,
                           plan->d_chunks, plan->nchunks, neg_threshold, pos_threshold,
                           compr_base);
    return check_launch("compress_2bit_multi");
}

GCQ_API void gc_plan_destroy(gc_plan* plan)
{
    if (!plan)
        return;
    if (plan->d_chunks) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(plan->device);
        (void)hipDeviceSynchronize();
        (void)hipFree(plan->d_chunks);
        (void)hipSetDevice(cur);
    }
    delete plan;
}
