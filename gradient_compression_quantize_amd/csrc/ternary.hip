// ternary.hip -- dense packing of the threshold quantizer's codes: five
// codes per byte as base-3 digits, 1.6 bits per value instead of 2.
//
// Method: apache/incubator-mxnet PR #8342 "[WIP] 2bit gradient compression".
// "Two bit quantization" notes that three codes leave one of the four 2-bit
// patterns unused and puts a denser packing off for later; this is that
// packing, with the same thresholds, codes and error feedback ("Approach")
// and the same 3-element header ("Format of compressed gradient"). Byte j of
// the payload (from element 3 on, bytes in memory order) holds values
// 5j .. 5j+4 as c0*81 + c1*27 + c2*9 + c3*3 + c4, the first value most
// significant; zero bytes pad the payload to whole 32-bit elements, so a
// block of n values takes 3 + ceil(n / 20) elements. Bytes 243..255 are
// never written; decoded, their leading digit 3 reads as zero.
//
// Layout and mapping (HBM-bound: ~12.2 bytes moved per value to compress,
// 4 + 0.2 W to dequantize-and-sum W blocks):
//  - one 32-bit element holds 20 values = 5 float4 slots, so a wave tile is
//    5 float4 slots per lane (1280 values, 64 elements): grad / residual /
//    out move lane-contiguous, 1 KiB per instruction;
//  - compress: each lane writes its slots' codes, one per byte, to a
//    wave-private LDS buffer; lane L reads back the 20 codes of element L
//    (5 consecutive dwords: distinct banks) and folds them into 4 base-3
//    bytes with byte dot products; one coalesced 256-byte store per tile;
//  - dequantize: lane L loads element L of each block (one 256-byte load per
//    worker), splits each byte into digits with multiply-shifts, reads the
//    values from a per-worker LDS table of digit pairs and sums them in
//    worker order; a wave-private LDS transpose turns each lane's 20
//    consecutive values into lane-contiguous float4 stores (storing them
//    directly, 80 bytes apart per lane, measured three times slower).
#include "gcq_internal.h"
#include "threshold_codes.h"

#include <algorithm>

namespace gcq {
namespace {

constexpr int kThreads = 256;                          // 4 waves
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kSlots = 5;                              // float4 slots per lane per tile
constexpr int kWordValues = 20;                        // values per 32-bit element
constexpr size_t kTileF4 = size_t(kWave) * kSlots;     // 320 float4 slots
constexpr size_t kTileElems = kTileF4 * 4;             // 1280 values
// Resident workgroups per CU, held by an LDS reservation the kernels never
// touch (0: what their registers and own LDS allow). The aligned compress
// measured the same at 3 to 6 per CU (51.0-51.4 us), so it keeps its 8. The
// dequantize-sum, which its own LDS holds to 7 per CU at W <= 8, runs at 6:
// 28.5 against 29.3 us at W = 8 (21.9 against 21.6 at W = 2; 3 and 4 per CU
// were slower).
constexpr int kCompressWgPerCu = 0;
constexpr int kDequantWgPerCu = 6;
static_assert(kTileElems == size_t(kWave) * kWordValues, "one tile = one element per lane");

__host__ __device__ inline size_t payload_words(size_t n)
{
    return n / kWordValues + (n % kWordValues != 0 ? 1 : 0);
}

// Code of one value (0 zero, 1 pos, 2 neg) and its new residual.
__device__ __forceinline__ uint32_t code_and_residual(float v, float neg, float pos, float& rn)
{
    const bool up = v >= pos;
    const bool dn = v <= neg;
    const float d = up ? pos : (dn ? neg : 0.0f);
    rn = v - d;
    return up ? 1u : (dn ? 2u : 0u);
}

// Codes of a float4 slot, value k in byte k, and the slot's new residual.
__device__ __forceinline__ uint32_t classify4_bytes(f32x4 g, f32x4 r, float neg, float pos,
                                                    f32x4& rn)
{
    uint32_t codes = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float rk;
        codes |= code_and_residual(g[k] + r[k], neg, pos, rk) << (8 * k);
        rn[k] = rk;
    }
    return codes;
}

constexpr uint32_t bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return a | b << 8 | c << 16 | d << 24;
}

__device__ __forceinline__ uint32_t dot4(uint32_t a, uint32_t b, uint32_t acc)
{
    return __builtin_amdgcn_udot4(a, b, acc, false);
}

// The element of 20 codes held one per byte (value 4k + i in byte i of
// c[k]): payload byte b is the base-3 number of values 5b .. 5b+4, first
// value most significant, each a sum of byte products.
__device__ __forceinline__ uint32_t fold_base3(const uint32_t (&c)[kSlots])
{
    const uint32_t b0 = dot4(c[0], bytes4(81, 27, 9, 3), dot4(c[1], bytes4(1, 0, 0, 0), 0u));
    const uint32_t b1 = dot4(c[1], bytes4(0, 81, 27, 9), dot4(c[2], bytes4(3, 1, 0, 0), 0u));
    const uint32_t b2 = dot4(c[2], bytes4(0, 0, 81, 27), dot4(c[3], bytes4(9, 3, 1, 0), 0u));
    const uint32_t b3 = dot4(c[3], bytes4(0, 0, 0, 81), dot4(c[4], bytes4(27, 9, 3, 1), 0u));
    return b0 | b1 << 8 | b2 << 16 | b3 << 24;
}

// Element j (values 20j .. 20j+19) by one thread, scalar accesses; values at
// or past n are digit 0 and are neither read nor written.
__device__ __forceinline__ uint32_t compress_word_scalar(const float* __restrict__ grad,
                                                         float* __restrict__ residual, size_t n,
                                                         float neg, float pos, size_t j)
{
    uint32_t word = 0;
    // rolled: this path serves misaligned buffers and the one partial tile
#pragma unroll 1
    for (int b = 0; b < 4; ++b) {
        uint32_t byte = 0;
#pragma unroll 1
        for (int k = 0; k < 5; ++k) {
            const size_t i = j * kWordValues + size_t(5 * b + k);
            uint32_t c = 0;
            if (i < n) {
                float rn;
                c = code_and_residual(grad[i] + residual[i], neg, pos, rn);
                residual[i] = rn;
            }
            byte = byte * 3u + c;
        }
        word |= byte << (8 * b);
    }
    return word;
}

// One full wave tile: float4 slots q0 .. q0 + kTileF4 - 1, all below n / 4.
// `codes` is this wave's kTileF4-dword LDS buffer.
__device__ __forceinline__ void compress_full_tile(const float* __restrict__ grad,
                                                   float* __restrict__ residual, float neg,
                                                   float pos, uint32_t* __restrict__ payload,
                                                   size_t q0, int lane, uint32_t* codes)
{
    const f32x4* g4 = reinterpret_cast<const f32x4*>(grad);
    f32x4* r4 = reinterpret_cast<f32x4*>(residual);
    f32x4 g[kSlots], r[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        const size_t q = q0 + size_t(u) * kWave + lane;
        g[u] = __builtin_nontemporal_load(g4 + q);
        r[u] = __builtin_nontemporal_load(r4 + q);
    }
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
        const size_t q = q0 + size_t(u) * kWave + lane;
        f32x4 rn;
        codes[u * kWave + lane] = classify4_bytes(g[u], r[u], neg, pos, rn);
        __builtin_nontemporal_store(rn, r4 + q);
    }
    wave_lds_sync();
    uint32_t c[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k)
        c[k] = codes[kSlots * lane + k];
    wave_lds_sync();  // these reads precede the next tile's writes
    __builtin_nontemporal_store(fold_base3(c), payload + q0 / kSlots + lane);
}

// The same full tile for grad and residual of any 4-byte alignment:
// lane-contiguous 4-byte accesses, one value per lane in each of 20 steps
// (256 bytes per load and store instruction). A quad OR gathers the codes
// of 4 consecutive values into the dword the vector path writes for their
// float4 slot; the fold and the store are the vector path's.
__device__ __forceinline__ void compress_dword_full_tile(const float* __restrict__ grad,
                                                         float* __restrict__ residual, float neg,
                                                         float pos,
                                                         uint32_t* __restrict__ payload,
                                                         size_t q0, int lane, uint32_t* codes)
{
    constexpr int kSteps = int(kTileF4) * 4 / kWave;
    const size_t e0 = q0 * 4;
    float g[kSteps], r[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
        const size_t e = e0 + size_t(j) * kWave + lane;
        g[j] = __builtin_nontemporal_load(grad + e);
        r[j] = __builtin_nontemporal_load(residual + e);
    }
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
        const size_t e = e0 + size_t(j) * kWave + lane;
        float rn;
        const uint32_t c = code_and_residual(g[j] + r[j], neg, pos, rn);
        __builtin_nontemporal_store(rn, residual + e);
        // value 64 j + lane of the tile: byte lane % 4 of dword 16 j + lane / 4
        const uint32_t four = quad_or(c << (8 * (lane & 3)));
        if ((lane & 3) == 0)
            codes[16 * j + (lane >> 2)] = four;
    }
    wave_lds_sync();
    uint32_t c[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k)
        c[k] = codes[kSlots * lane + k];
    wave_lds_sync();  // these reads precede the next tile's writes
    __builtin_nontemporal_store(fold_base3(c), payload + q0 / kSlots + lane);
}

// kDword: grad or residual without 16-byte alignment.
template <bool kDword>
__device__ __forceinline__ void compress_tile(const float* __restrict__ grad,
                                              float* __restrict__ residual, size_t n, float neg,
                                              float pos, uint32_t* __restrict__ payload,
                                              size_t q0, int lane, uint32_t* codes)
{
    if (q0 + kTileF4 <= (n >> 2)) {
        if (kDword)
            compress_dword_full_tile(grad, residual, neg, pos, payload, q0, lane, codes);
        else
            compress_full_tile(grad, residual, neg, pos, payload, q0, lane, codes);
    } else {
        const size_t j = q0 / kSlots + lane;
        if (j < payload_words(n))
            payload[j] = compress_word_scalar(grad, residual, n, neg, pos, j);
    }
}

// kLoop: a capped grid strides over tiles. kDword: grad or residual is 4-
// but not 16-byte aligned.
template <bool kLoop, bool kDword>
__device__ __forceinline__ void compress_ternary_body(const float* __restrict__ grad,
                                                      float* __restrict__ residual, size_t n,
                                                      float neg, float pos, float n_f,
                                                      uint32_t* __restrict__ compr, size_t ntiles)
{
    __shared__ uint32_t codes[kWavesPerBlock][kTileF4];
    if (blockIdx.x == 0 && threadIdx.x == 0)
        write_header(compr, neg, pos, n_f);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const size_t stride = size_t(gridDim.x) * kWavesPerBlock;
    for (size_t t = size_t(blockIdx.x) * kWavesPerBlock + wave; t < ntiles; t += stride) {
        compress_tile<kDword>(grad, residual, n, neg, pos, compr + 3, t * kTileF4, lane,
                              codes[wave]);
        if (!kLoop)
            break;
    }
}

// Entry kernels of the body above, named apart so that profiles keep the
// aligned and the 4-byte-aligned paths separate.
template <bool kLoop>
__global__ __launch_bounds__(kThreads) void compress_ternary_vec_kernel(
    const float* __restrict__ grad, float* __restrict__ residual, size_t n, float neg,
    float pos, float n_f, uint32_t* __restrict__ compr, size_t ntiles)
{
    compress_ternary_body<kLoop, false>(grad, residual, n, neg, pos, n_f, compr, ntiles);
}

template <bool kLoop>
__global__ __launch_bounds__(kThreads) void compress_ternary_dword_kernel(
    const float* __restrict__ grad, float* __restrict__ residual, size_t n, float neg,
    float pos, float n_f, uint32_t* __restrict__ compr, size_t ntiles)
{
    compress_ternary_body<kLoop, true>(grad, residual, n, neg, pos, n_f, compr, ntiles);
}

// Pair table in LDS: for worker w, entry 16w + p (p = 3a + b < 16) holds
// the values of the digit pair (a, b); a >= 3 -- only the leading digit of
// the never-written bytes 243..255 -- reads as zero. One worker's entries
// span 128 bytes, so a wave's lookups into it never conflict. Ends with a
// block barrier.
__device__ __forceinline__ void build_pair_table(float2* lut, const PtrTable<uint32_t>& tab,
                                                 int W)
{
    for (int w = 0; w < W; ++w) {
        if (threadIdx.x < 16) {
            const uint32_t* b = tab.p[w];
            const float neg = u2f(b[0]);
            const float pos = u2f(b[1]);
            const uint32_t p = threadIdx.x;
            lut[16 * w + p] = make_float2(code_value(p / 3u, neg, pos), code_value(p % 3u, neg, pos));
        }
    }
    __syncthreads();
}

// Digits of a payload byte x without a division: x = 27 p0 + 3 p1 + c4 with
// p0 = 3 c0 + c1 (the leading pair; 9 for x >= 243) and p1 = 3 c2 + c3.
// (2428 x) >> 16 is floor(x / 27) for every x < 256 and (11 r) >> 5 is
// floor(r / 3) for every r < 27 (checked at compile time below).
struct Digits {
    uint32_t p0, p1, c4;
};

__host__ __device__ constexpr Digits split_byte(uint32_t x)
{
    const uint32_t p0 = (x * 2428u) >> 16;
    const uint32_t r = x - 27u * p0;
    const uint32_t p1 = (r * 11u) >> 5;
    return Digits{p0, p1, r - 3u * p1};
}

constexpr bool split_byte_exact()
{
    for (uint32_t x = 0; x < 256u; ++x) {
        const Digits d = split_byte(x);
        if (d.p0 != x / 27u || d.p1 != x % 27u / 3u || d.c4 != x % 3u)
            return false;
    }
    return true;
}
static_assert(split_byte_exact(), "multiply-shift digit split must be exact for every byte");

// Adds (or, for the first worker, sets) the 20 values of one element into
// acc through worker pair table t: per byte two pairs and one single digit
// (entry 3 c4 holds (c4, 0)).
__device__ __forceinline__ void decode_element(uint32_t word, const float2* t,
                                               float (&acc)[kWordValues], bool first)
{
    const char* tb = reinterpret_cast<const char*>(t);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const Digits d = split_byte((word >> (8 * b)) & 0xFFu);
        const float2 q0 = *reinterpret_cast<const float2*>(tb + 8u * d.p0);
        const float2 q1 = *reinterpret_cast<const float2*>(tb + 8u * d.p1);
        const float s = *reinterpret_cast<const float*>(tb + 24u * d.c4);
        const float v[5] = {q0.x, q0.y, q1.x, q1.y, s};
#pragma unroll
        for (int k = 0; k < 5; ++k)
            acc[5 * b + k] = first ? v[k] : acc[5 * b + k] + v[k];
    }
}

// Byte offsets into a worker's pair table of the byte's two pairs and its
// single digit, packed (8 p0 | 8 p1 << 8 | 24 c4 << 16): the digit split of
// decode_element done once per byte value instead of once per byte read.
__host__ __device__ constexpr uint32_t packed_digit_offsets(uint32_t x)
{
    const Digits d = split_byte(x);
    return (8u * d.p0) | ((8u * d.p1) << 8) | ((24u * d.c4) << 16);
}

__device__ __forceinline__ void build_digit_table(uint32_t* offs)
{
    for (uint32_t x = threadIdx.x; x < 256u; x += blockDim.x)
        offs[x] = packed_digit_offsets(x);
}

// decode_element with the digit split read from the table of
// packed_digit_offsets.
__device__ __forceinline__ void decode_element_tab(uint32_t word, const float2* t,
                                                   const uint32_t* offs,
                                                   float (&acc)[kWordValues], bool first)
{
    const char* tb = reinterpret_cast<const char*>(t);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t o = offs[(word >> (8 * b)) & 0xFFu];
        const float2 q0 = *reinterpret_cast<const float2*>(tb + (o & 0xFFu));
        const float2 q1 = *reinterpret_cast<const float2*>(tb + ((o >> 8) & 0xFFu));
        const float s = *reinterpret_cast<const float*>(tb + (o >> 16));
        const float v[5] = {q0.x, q0.y, q1.x, q1.y, s};
#pragma unroll
        for (int k = 0; k < 5; ++k)
            acc[5 * b + k] = first ? v[k] : acc[5 * b + k] + v[k];
    }
}

// One full wave tile of the W-block dequantize-and-sum. WC > 0: W == WC at
// compile time, every worker's element in flight at once; WC == 0: W read at
// run time, in groups of eight, the next group's loads ahead of this one's
// decode. `stage` is this wave's kTileF4-float4 buffer.
// kDword: out without 16-byte alignment; the staged tile leaves as
// lane-contiguous 4-byte stores.
// pre: this lane's W elements, already loaded (WC > 0), or NULL to load them
// here.
template <int WC, bool kAcc, bool kDword>
__device__ __forceinline__ void decompress_full_tile(const PtrTable<uint32_t>& tab, int W_rt,
                                                     const float2* lut, float* __restrict__ out,
                                                     size_t q0, int lane, f32x4* stage,
                                                     const uint32_t* pre = nullptr,
                                                     const uint32_t* offs = nullptr)
{
    const int W = WC > 0 ? WC : W_rt;
    const size_t j = q0 / kSlots + lane;
    float acc[kWordValues];
    if constexpr (WC > 0) {
        // every worker's element in flight together
        uint32_t mine[WC];
#pragma unroll
        for (int w = 0; w < WC; ++w)
            mine[w] = pre ? pre[w] : __builtin_nontemporal_load(tab.p[w] + 3 + j);
#pragma unroll
        for (int w = 0; w < WC; ++w)
            decode_element(mine[w], lut + 16 * w, acc, w == 0);
    } else {
        // W at run time: groups of kGroup workers, the next group's elements
        // loaded before this group is decoded (two groups in flight)
        constexpr int kGroup = 8;
        auto load = [&](uint32_t(&dst)[kGroup], int w0) {
#pragma unroll
            for (int dw = 0; dw < kGroup; ++dw)
                dst[dw] = w0 + dw < W ? __builtin_nontemporal_load(tab.p[w0 + dw] + 3 + j) : 0u;
        };
        uint32_t cur[kGroup], nxt[kGroup];
        load(cur, 0);
        for (int w0 = 0; w0 < W; w0 += kGroup) {
            if (w0 + kGroup < W)
                load(nxt, w0 + kGroup);
#pragma unroll
            for (int dw = 0; dw < kGroup; ++dw) {
                if (w0 + dw >= W)
                    break;
                decode_element_tab(cur[dw], lut + 16 * (w0 + dw), offs, acc, w0 + dw == 0);
            }
#pragma unroll
            for (int dw = 0; dw < kGroup; ++dw)
                cur[dw] = nxt[dw];
        }
    }
    // lane L holds values 20L .. 20L+19 of the tile = float4 slots 5L .. 5L+4
#pragma unroll
    for (int k = 0; k < kSlots; ++k)
        stage[kSlots * lane + k] =
            f32x4{acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]};
    wave_lds_sync();
    if (kDword) {
        const float* sf = reinterpret_cast<const float*>(stage);
        float* o = out + q0 * 4;
#pragma unroll
        for (int k = 0; k < kSlots * 4; ++k) {
            const int e = k * kWave + lane;
            float v = sf[e];
            if (kAcc)
                v = o[e] + v;
            __builtin_nontemporal_store(v, o + e);
        }
    } else {
        f32x4* o4 = reinterpret_cast<f32x4*>(out);
#pragma unroll
        for (int u = 0; u < kSlots; ++u) {
            const size_t q = q0 + size_t(u) * kWave + lane;
            f32x4 v = stage[u * kWave + lane];
            if (kAcc)
                v = o4[q] + v;
            __builtin_nontemporal_store(v, o4 + q);
        }
    }
    wave_lds_sync();  // these reads precede the next tile's writes
}

// The last, partial tile: lane L decodes element q0/5 + L for every worker
// and writes the values below n.
__device__ __forceinline__ void decompress_tail_tile(const PtrTable<uint32_t>& tab, int W,
                                                     const float2* lut, size_t n,
                                                     float* __restrict__ out, int accumulate,
                                                     size_t q0, int lane)
{
    const size_t j = q0 / kSlots + lane;
    if (j >= payload_words(n))
        return;
    float acc[kWordValues];
#pragma unroll 1
    for (int w = 0; w < W; ++w)
        decode_element(tab.p[w][3 + j], lut + 16 * w, acc, w == 0);
#pragma unroll
    for (int k = 0; k < kWordValues; ++k) {
        const size_t i = j * kWordValues + k;
        if (i < n)
            out[i] = accumulate ? out[i] + acc[k] : acc[k];
    }
}

// Dequantize-and-sum of W blocks into out (kAcc: added to what out holds;
// kDword: out 4- but not 16-byte aligned). Last tile first, XCD-contiguous,
// as in the 2-bit kernel:
// the partial tile's scalar path starts with the first wave, and tiles whose
// 256-byte element runs share edge cache lines meet in one L2. The pair
// table holds WC workers when W is known at compile time (less LDS per
// workgroup, more workgroups per CU).
template <int WC, bool kAcc, bool kLoop, bool kDword>
__device__ __forceinline__ void decompress_ternary_body(const PtrTable<uint32_t>& tab, int W,
                                                        size_t n, float* __restrict__ out,
                                                        size_t ntiles)
{
    __shared__ float2 lut[16 * (WC > 0 ? WC : GC_MAX_WORKERS)];
    __shared__ f32x4 stage[kWavesPerBlock][kTileF4];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (!kLoop && WC > 0) {
        // One tile per wave, W known: the tile's element loads go out before
        // the table is built, as in the 2-bit kernel.
        const size_t t = xcd_contiguous(blockIdx.x, gridDim.x) * kWavesPerBlock + wave;
        const size_t q0 = t < ntiles ? (ntiles - 1 - t) * kTileF4 : 0;
        const bool full = t < ntiles && q0 + kTileF4 <= (n >> 2);
        uint32_t pre[WC > 0 ? WC : 1];
        if (full) {
#pragma unroll
            for (int w = 0; w < (WC > 0 ? WC : 1); ++w)
                pre[w] = __builtin_nontemporal_load(tab.p[w] + 3 + q0 / kSlots + lane);
        }
        build_pair_table(lut, tab, WC);
        if (full)
            decompress_full_tile<WC, kAcc, kDword>(tab, W, lut, out, q0, lane, stage[wave], pre);
        else if (t < ntiles)
            decompress_tail_tile(tab, WC, lut, n, out, kAcc ? 1 : 0, q0, lane);
        return;
    }
    __shared__ uint32_t offs[WC == 0 ? 256 : 1];
    if (WC == 0)
        build_digit_table(offs);  // the barrier in build_pair_table covers it
    build_pair_table(lut, tab, WC > 0 ? WC : W);
    const size_t stride = size_t(gridDim.x) * kWavesPerBlock;
    const size_t blk = kLoop ? blockIdx.x : xcd_contiguous(blockIdx.x, gridDim.x);
    for (size_t t = blk * kWavesPerBlock + wave; t < ntiles; t += stride) {
        const size_t q0 = (ntiles - 1 - t) * kTileF4;
        if (q0 + kTileF4 <= (n >> 2))
            decompress_full_tile<WC, kAcc, kDword>(tab, W, lut, out, q0, lane, stage[wave],
                                                   nullptr, offs);
        else
            decompress_tail_tile(tab, WC > 0 ? WC : W, lut, n, out, kAcc ? 1 : 0, q0, lane);
        if (!kLoop)
            break;
    }
}

template <int WC, bool kAcc, bool kLoop>
__global__ __launch_bounds__(kThreads) void decompress_ternary_vec_kernel(
    PtrTable<uint32_t> tab, int W, size_t n, float* __restrict__ out, size_t ntiles)
{
    decompress_ternary_body<WC, kAcc, kLoop, false>(tab, W, n, out, ntiles);
}

template <int WC, bool kAcc, bool kLoop>
__global__ __launch_bounds__(kThreads) void decompress_ternary_dword_kernel(
    PtrTable<uint32_t> tab, int W, size_t n, float* __restrict__ out, size_t ntiles)
{
    decompress_ternary_body<WC, kAcc, kLoop, true>(tab, W, n, out, ntiles);
}

size_t grid_for_tiles(size_t ntiles)
{
    return std::max<size_t>(1, std::min(ceil_div(ntiles, kWavesPerBlock), max_grid_blocks()));
}

bool tiles_need_loop(size_t ntiles)
{
    return ceil_div(ntiles, kWavesPerBlock) > max_grid_blocks();
}

template <bool kLoop, bool kDword>
void launch_decompress_vec(const PtrTable<uint32_t>& tab, int W, size_t n, float* out,
                           int accumulate, size_t ntiles, dim3 grid, dim3 block,
                           hipStream_t stream)
{
    if (accumulate) {
        // only decompress_ternary accumulates (W == 1)
        if (kDword)
            hipLaunchKernelGGL((decompress_ternary_dword_kernel<1, true, kLoop>), grid, block, 0,
                               stream, tab, W, n, out, ntiles);
        else
            hipLaunchKernelGGL((decompress_ternary_vec_kernel<1, true, kLoop>), grid, block, 0,
                               stream, tab, W, n, out, ntiles);
        return;
    }
    switch (W) {
#define GCQ_TDEC_CASE(k)                                                                    \
    case k:                                                                                 \
        if (kDword)                                                                         \
            hipLaunchKernelGGL((decompress_ternary_dword_kernel<k, false, kLoop>), grid,    \
                               block, 0, stream, tab, W, n, out, ntiles);                   \
        else                                                                                \
            hipLaunchKernelGGL((decompress_ternary_vec_kernel<k, false, kLoop>), grid,      \
                               block,                                                       \
                               lds_cap((decompress_ternary_vec_kernel<k, false, kLoop>),    \
                                       kDequantWgPerCu),                                    \
                               stream, tab, W, n, out, ntiles);                             \
        break;
        GCQ_TDEC_CASE(1)
        GCQ_TDEC_CASE(2)
        GCQ_TDEC_CASE(3)
        GCQ_TDEC_CASE(4)
        GCQ_TDEC_CASE(5)
        GCQ_TDEC_CASE(6)
        GCQ_TDEC_CASE(7)
        GCQ_TDEC_CASE(8)
#undef GCQ_TDEC_CASE
    default:
        if (kDword)
            hipLaunchKernelGGL((decompress_ternary_dword_kernel<0, false, kLoop>), grid, block, 0,
                               stream, tab, W, n, out, ntiles);
        else
            hipLaunchKernelGGL((decompress_ternary_vec_kernel<0, false, kLoop>), grid, block,
                               lds_cap((decompress_ternary_vec_kernel<0, false, kLoop>),
                                       kDequantWgPerCu),
                               stream, tab, W, n, out, ntiles);
    }
}

int launch_decompress(const PtrTable<uint32_t>& tab, int W, size_t n, float* out,
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

}  // namespace
}  // namespace gcq

using namespace gcq;

GCQ_API size_t gc_compressed_ternary_words(size_t n) { return 3 + payload_words(n); }

GCQ_API int compress_ternary(const float* grad, float* residual, size_t n, float neg_threshold,
                             float pos_threshold, uint32_t* compr, hipStream_t stream)
{
    clear_error();
    if (!compr)
        return fail(GC_EINVAL, "compress_ternary: compr is NULL");
    if (n > 0 && (!grad || !residual))
        return fail(GC_EINVAL, "compress_ternary: grad or residual is NULL with n > 0");
    if (int rc = check_thresholds(neg_threshold, pos_threshold))
        return rc;
    if (!aligned4(compr) || !aligned4(grad) || !aligned4(residual))
        return fail(GC_EINVAL, "compress_ternary: buffers must be 4-byte aligned");
    const float n_f = static_cast<float>(n);
    const size_t ntiles = ceil_div(n, kTileElems);
    const dim3 grid(grid_for_tiles(ntiles)), block(kThreads);
    const bool loop = tiles_need_loop(ntiles);
    const bool dword = n > 0 && !(aligned16(grad) && aligned16(residual));
#define GCQ_TCOMP(K, L, LDS)                                                                   \
    hipLaunchKernelGGL((K<L>), grid, block, LDS, stream, grad, residual, n, neg_threshold,   \
                       pos_threshold, n_f, compr, ntiles)
    if (loop && dword)
        GCQ_TCOMP(compress_ternary_dword_kernel, true, 0);
    else if (loop)
        GCQ_TCOMP(compress_ternary_vec_kernel, true,
                  lds_cap(compress_ternary_vec_kernel<true>, kCompressWgPerCu));
    else if (dword)
        GCQ_TCOMP(compress_ternary_dword_kernel, false, 0);
    else
        GCQ_TCOMP(compress_ternary_vec_kernel, false,
                  lds_cap(compress_ternary_vec_kernel<false>, kCompressWgPerCu));
#undef GCQ_TCOMP
    return check_launch("compress_ternary");
}

GCQ_API int decompress_ternary(const uint32_t* compr, size_t n, float* out, int accumulate,
                               hipStream_t stream)
{
    clear_error();
    if (!compr)
        return fail(GC_EINVAL, "decompress_ternary: compr is NULL");
    if (n > 0 && !out)
        return fail(GC_EINVAL, "decompress_ternary: out is NULL with n > 0");
    if (accumulate != 0 && accumulate != 1)
        return fail(GC_EINVAL, "decompress_ternary: accumulate must be 0 or 1");
    if (!aligned4(compr) || !aligned4(out))
        return fail(GC_EINVAL, "decompress_ternary: buffers must be 4-byte aligned");
    PtrTable<uint32_t> tab{};
    tab.p[0] = compr;
    return launch_decompress(tab, 1, n, out, accumulate, stream, "decompress_ternary");
}

GCQ_API int decompress_ternary_sum(const uint32_t* const* compr, int W, size_t n, float* out,
                                   hipStream_t stream)
{
    clear_error();
    if (!compr)
        return fail(GC_EINVAL, "decompress_ternary_sum: compr is NULL");
    if (W < 1 || W > GC_MAX_WORKERS)
        return fail(GC_EINVAL, "decompress_ternary_sum: W must be in [1, 64]");
    if (n > 0 && !out)
        return fail(GC_EINVAL, "decompress_ternary_sum: out is NULL with n > 0");
    if (!aligned4(out))
        return fail(GC_EINVAL, "decompress_ternary_sum: out must be 4-byte aligned");
    PtrTable<uint32_t> tab{};
    for (int w = 0; w < W; ++w) {
        if (!compr[w] || !aligned4(compr[w]))
            return fail(GC_EINVAL,
                        "decompress_ternary_sum: a block pointer is NULL or misaligned");
        tab.p[w] = compr[w];
    }
    return launch_decompress(tab, W, n, out, 0, stream, "decompress_ternary_sum");
}
