/*
 * oracle.c -- plain CPU oracle for the gradient-quantization hot path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h). Single-threaded, one element at a
 * time, in the order the method states its steps. Built with
 *   gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math
 * so every fp32 expression below is evaluated as written, one binary32
 * rounding per operation (x86-64 SSE arithmetic, FLT_EVAL_METHOD == 0).
 *
 * Readings taken where the pages are silent are marked READING.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static uint32_t bits_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float float_of(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ======================================================================
 * 2-bit threshold quantization with error feedback
 * [MX] "Two bit quantization" and "Format of compressed gradient".
 * ==================================================================== */

/* [MX] "Format of compressed gradient": two thresholds, the original size,
 * then one 32-bit element per group of up to 16 values. */
size_t oracle_compressed_2bit_words(size_t n)
{
    return 3 + (n + 15) / 16;
}

/* Code of one value [MX] "Two bit quantization": at or above the positive
 * threshold -> binary 01; at or below the negative threshold -> binary 10;
 * anything else -> 00. Inclusive comparisons on both sides. */
static uint32_t code_of(float v, float neg_threshold, float pos_threshold)
{
    if (v >= pos_threshold)
        return 1u;
    if (v <= neg_threshold)
        return 2u;
    return 0u;
}

/* Value a code stands for. READING: the header keeps exactly the two
 * thresholds because they are what dequantization needs ([MX] "Format of
 * compressed gradient"), so 01 -> pos_threshold, 10 -> neg_threshold,
 * 00 -> 0. The unused pattern 11 ([MX] notes one wasted bit) -> 0. */
static float value_of(uint32_t code, float neg_threshold, float pos_threshold)
{
    if (code == 1u)
        return pos_threshold;
    if (code == 2u)
        return neg_threshold;
    return 0.0f;
}

/* quantize_2bit(grad, residual, compr, neg, pos) of [MX] "Operators".
 * Step by step, per element i ([MX] "Approach", "Two bit quantization"):
 *   v = grad + residual          (the carried error is added first)
 *   c = code_of(v)
 *   residual = v - value_of(c)   (the quantization error is kept)
 *   the code goes into 32-bit element 3 + i/16, most significant pair first
 *   (the printed example's bit string puts element 0 in bits 31..30).
 * Header: [0] = neg threshold, [1] = pos threshold, [2] = size as fp32. */
void oracle_quantize_2bit(const float* grad, float* residual, size_t n,
                          float neg_threshold, float pos_threshold,
                          uint32_t* compr)
{
    size_t nwords = (n + 15) / 16;
    compr[0] = bits_of(neg_threshold);
    compr[1] = bits_of(pos_threshold);
    compr[2] = bits_of((float)n);
    for (size_t j = 0; j < nwords; ++j)
        compr[3 + j] = 0u;
    for (size_t i = 0; i < n; ++i) {
        float v = grad[i] + residual[i];
        uint32_t c = code_of(v, neg_threshold, pos_threshold);
        float d = value_of(c, neg_threshold, pos_threshold);
        residual[i] = v - d;
        unsigned shift = 30u - 2u * (unsigned)(i % 16);
        compr[3 + i / 16] |= c << shift;
    }
}

static uint32_t code_at(const uint32_t* compr, size_t i)
{
    unsigned shift = 30u - 2u * (unsigned)(i % 16);
    return (compr[3 + i / 16] >> shift) & 3u;
}

/* dequantize_2bit(compr, decompr) of [MX] "Operators": each code becomes
 * the threshold it stands for, using the thresholds in the header. The size
 * is taken from the caller. */
void oracle_dequantize_2bit(const uint32_t* compr, size_t n, float* out)
{
    float neg = float_of(compr[0]);
    float pos = float_of(compr[1]);
    for (size_t i = 0; i < n; ++i)
        out[i] = value_of(code_at(compr, i), neg, pos);
}

/* [MX] "Local kvstore": every device (the reducing one included) quantizes;
 * the reducing device dequantizes each buffer and sums. READING: the sum is
 * taken in fp32 in worker order 0, 1, ..., W-1, starting from worker 0's
 * dequantized value. */
void oracle_dequantize_2bit_sum(const uint32_t* const* compr, int W, size_t n,
                                float* out)
{
    for (size_t i = 0; i < n; ++i) {
        const uint32_t* b0 = compr[0];
        float acc = value_of(code_at(b0, i), float_of(b0[0]), float_of(b0[1]));
        for (int w = 1; w < W; ++w) {
            const uint32_t* b = compr[w];
            float d = value_of(code_at(b, i), float_of(b[0]), float_of(b[1]));
            acc = acc + d;
        }
        out[i] = acc;
    }
}

/* ======================================================================
 * Dense ternary packing: the optimization [MX] "Two bit quantization"
 * defers. Three codes need log2(3) ~ 1.58 bits, and five codes fit one byte
 * (3^5 = 243 <= 256), so the block shrinks from 2 to 1.6 bits per value.
 * READING: the header is the 2-bit block's; then a byte array in memory
 * order, byte j holding values 5j .. 5j+4 as base-3 digits, the first value
 * most significant (byte = c0*81 + c1*27 + c2*9 + c3*3 + c4); digits are the
 * 2-bit codes (0 zero, 1 pos, 2 neg); tail digits 0; the byte array is
 * padded with zero bytes to whole 32-bit elements. A byte above 242 (never
 * written) decodes digit by digit like any other, and a leading digit of 3
 * is an unused code, so it dequantizes to 0.
 * ==================================================================== */

static const unsigned pow3[5] = {1u, 3u, 9u, 27u, 81u};

size_t oracle_compressed_ternary_words(size_t n)
{
    size_t nbytes = (n + 4) / 5;
    return 3 + (nbytes + 3) / 4;
}

/* The same error-feedback arithmetic as oracle_quantize_2bit; only the
 * packing of the codes differs. */
void oracle_quantize_ternary(const float* grad, float* residual, size_t n,
                             float neg_threshold, float pos_threshold,
                             uint32_t* compr)
{
    size_t words = oracle_compressed_ternary_words(n);
    compr[0] = bits_of(neg_threshold);
    compr[1] = bits_of(pos_threshold);
    compr[2] = bits_of((float)n);
    for (size_t j = 3; j < words; ++j)
        compr[j] = 0u;
    unsigned char* bytes = (unsigned char*)(compr + 3);
    for (size_t i = 0; i < n; ++i) {
        float v = grad[i] + residual[i];
        uint32_t c = code_of(v, neg_threshold, pos_threshold);
        float d = value_of(c, neg_threshold, pos_threshold);
        residual[i] = v - d;
        bytes[i / 5] = (unsigned char)(bytes[i / 5] + c * pow3[4 - i % 5]);
    }
}

static uint32_t ternary_digit_at(const uint32_t* compr, size_t i)
{
    const unsigned char* bytes = (const unsigned char*)(compr + 3);
    unsigned b = bytes[i / 5];
    unsigned k = 4u - (unsigned)(i % 5);
    unsigned d = b / pow3[k];
    return k == 4u ? d : d % 3u; /* the leading digit is not reduced */
}

void oracle_dequantize_ternary(const uint32_t* compr, size_t n, float* out)
{
    float neg = float_of(compr[0]);
    float pos = float_of(compr[1]);
    for (size_t i = 0; i < n; ++i)
        out[i] = value_of(ternary_digit_at(compr, i), neg, pos);
}

void oracle_dequantize_ternary_sum(const uint32_t* const* compr, int W,
                                   size_t n, float* out)
{
    for (size_t i = 0; i < n; ++i) {
        const uint32_t* b0 = compr[0];
        float acc = value_of(ternary_digit_at(b0, i), float_of(b0[0]),
                             float_of(b0[1]));
        for (int w = 1; w < W; ++w) {
            const uint32_t* b = compr[w];
            float d = value_of(ternary_digit_at(b, i), float_of(b[0]),
                               float_of(b[1]));
            acc = acc + d;
        }
        out[i] = acc;
    }
}

/* ======================================================================
 * Philox-4x32-10 [PHX]: a 4x32-bit counter and a 2x32-bit key.
 * One round: two 32x32->64 products of counter words 0 and 2 with the two
 * Philox-4x32 multipliers; the new words are (hi of the second product XOR
 * word 1 XOR key 0, lo of the second product, hi of the first product XOR
 * word 3 XOR key 1, lo of the first product). Before every round after the
 * first, the key is bumped by the two Weyl constants (the golden ratio and
 * sqrt(3)-1 in 0.32 fixed point). Ten rounds.
 * ==================================================================== */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                          uint32_t out[4])
{
    const uint32_t mult_a = 0xD2511F53u;
    const uint32_t mult_b = 0xCD9E8D57u;
    const uint32_t weyl_a = 0x9E3779B9u;
    const uint32_t weyl_b = 0xBB67AE85u;

    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += weyl_a;
            k1 += weyl_b;
        }
        uint64_t prod_a = (uint64_t)mult_a * (uint64_t)x0;
        uint64_t prod_b = (uint64_t)mult_b * (uint64_t)x2;
        uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
        uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
        uint32_t y0 = hi_b ^ x1 ^ k0;
        uint32_t y1 = lo_b;
        uint32_t y2 = hi_a ^ x3 ^ k1;
        uint32_t y3 = lo_a;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* ======================================================================
 * QSGD max-norm quantization [QMN] "About The Project": the workers agree
 * on one scale (the largest |g| over all of them), so that their integer
 * levels can be summed by an all-reduce and dequantized once.
 * Per element: level = floor(|g| / norm * s + u), sign kept, u uniform.
 * ==================================================================== */

/* READING: u is the top 24 bits of one 32-bit Philox word, scaled by 2^-24:
 * a value in [0, 1 - 2^-24], exact in fp32. */
float oracle_uniform24(uint32_t r)
{
    return (float)(r >> 8) * 0x1p-24f;
}

/* READING: floor(x + u) taken in exact arithmetic over the fp32 values x
 * and u (a literal fp32 sum could round 127 + (1 - 2^-24) up to 128).
 * The binary64 sum is exact whenever it can reach an integer: for x >= 1
 * both terms are multiples of 2^-24 below 2^8; for 2^-29 <= x < 1 the sum
 * is below 2 with its lowest bit at or above 2^-52; for x < 2^-29 the sum
 * stays below 1 - 2^-25 whatever the rounding, so the floor is 0. */
int oracle_stochastic_level(float x, float u)
{
    return (int)floor((double)x + (double)u);
}

/* Largest |g| over all workers and elements (READING: NaN is outside the
 * domain; fmaxf ignores it). */
float oracle_maxnorm(const float* const* grads, int W, size_t n)
{
    float m = 0.0f;
    for (int w = 0; w < W; ++w)
        for (size_t i = 0; i < n; ++i)
            m = fmaxf(m, fabsf(grads[w][i]));
    return m;
}

/* READING of "Philox4x32-10(seed, worker, index)": key = (seed low 32 bits,
 * seed high 32 bits); counter = (index/4 low, index/4 high, worker, 0);
 * element `index` takes output word index % 4. Counter word 3 is a purpose
 * tag: 0 for rounding, 1 for the rand-K draw. */
static uint32_t philox_word(uint64_t seed, uint64_t block, uint32_t word2,
                            uint32_t word3, unsigned which)
{
    uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), word2, word3};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    oracle_philox4x32_10(ctr, key, r);
    return r[which];
}

/* One level. READINGS: x = (|g| / norm) * s with two fp32 roundings in that
 * order; norm == 0 gives level 0; the sign of g is kept (g = -0 -> 0). */
static int8_t qsgd_level(float g, uint64_t index, float norm, int s,
                         uint64_t seed, uint32_t worker)
{
    if (norm == 0.0f)
        return 0;
    uint32_t r = philox_word(seed, index / 4, worker, 0u, (unsigned)(index % 4));
    float u = oracle_uniform24(r);
    float a = fabsf(g);
    float q = a / norm;
    float x = q * (float)s;
    int m = oracle_stochastic_level(x, u);
    return (int8_t)(g < 0.0f ? -m : m);
}

void oracle_qsgd_quantize(const float* grad, size_t n, float norm, int s,
                          uint64_t seed, uint32_t worker, int8_t* levels)
{
    for (size_t i = 0; i < n; ++i)
        levels[i] = qsgd_level(grad[i], (uint64_t)i, norm, s, seed, worker);
}

/* The same definition evaluated only at chosen element indices: value k sits
 * at element index[k] of the worker's gradient. */
void oracle_qsgd_quantize_at(const float* values, const uint64_t* index,
                             size_t m, float norm, int s, uint64_t seed,
                             uint32_t worker, int8_t* levels)
{
    for (size_t k = 0; k < m; ++k)
        levels[k] = qsgd_level(values[k], index[k], norm, s, seed, worker);
}

/* All-reduce compatible aggregation [QMN]: the workers' integer levels are
 * summed exactly (int32). */
void oracle_level_sum(const int8_t* const* levels, int W, size_t n,
                      int32_t* sums)
{
    for (size_t i = 0; i < n; ++i) {
        int32_t acc = 0;
        for (int w = 0; w < W; ++w)
            acc += (int32_t)levels[w][i];
        sums[i] = acc;
    }
}

/* Dequantize the summed levels: norm * sum / s, two fp32 roundings, left to
 * right. READING: the sum, not the mean (the caller divides by W). */
void oracle_qsgd_dequantize(const int32_t* sums, size_t n, float norm, int s,
                            float* out)
{
    for (size_t i = 0; i < n; ++i) {
        float t = norm * (float)sums[i];
        out[i] = t / (float)s;
    }
}

/* ======================================================================
 * GlobalRandK [QMN] "Results": all workers share the same K random indices
 * (K = 10000 in the pages' experiments).
 * READING: a partial Fisher-Yates shuffle of 0..n-1, step i swapping
 * positions i and j, with j = i + floor(R * (n - i) / 2^64) for the 64-bit
 * R = (word1 << 32) | word0 of Philox(key = seed, counter = (i, 0, 0, 1)).
 * The K first positions are the indices. Returns -1 if K > n or n > 2^32.
 * ==================================================================== */
int oracle_randk_indices(size_t n, uint32_t K, uint64_t seed, uint32_t* idx)
{
    if ((size_t)K > n || n > ((size_t)1 << 32))
        return -1;
    if (K == 0)
        return 0;
    uint32_t* perm = (uint32_t*)malloc(n * sizeof *perm);
    if (!perm)
        return -2;
    for (size_t p = 0; p < n; ++p)
        perm[p] = (uint32_t)p;
    for (uint32_t i = 0; i < K; ++i) {
        uint32_t ctr[4] = {i, 0u, 0u, 1u};
        uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
        uint32_t r[4];
        oracle_philox4x32_10(ctr, key, r);
        uint64_t R = ((uint64_t)r[1] << 32) | (uint64_t)r[0];
        uint64_t range = (uint64_t)(n - i);
        uint64_t off = (uint64_t)(((unsigned __int128)R * range) >> 64);
        size_t j = (size_t)i + (size_t)off;
        uint32_t tmp = perm[i];
        perm[i] = perm[j];
        perm[j] = tmp;
        idx[i] = perm[i];
    }
    free(perm);
    return 0;
}

void oracle_gather(const float* x, const uint32_t* idx, size_t K, float* out)
{
    for (size_t k = 0; k < K; ++k)
        out[k] = x[idx[k]];
}

/* Dense result of a sparsified step: zero everywhere but the K indices. */
void oracle_scatter_dense(const float* vals, const uint32_t* idx, size_t K,
                          size_t dense_n, float* dense)
{
    for (size_t i = 0; i < dense_n; ++i)
        dense[i] = 0.0f;
    for (size_t k = 0; k < K; ++k)
        dense[idx[k]] = vals[k];
}
