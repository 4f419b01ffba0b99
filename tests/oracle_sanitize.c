/*
 * Drives every function of the oracle over edge-case sizes, built together
 * with oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitizers.py. It checks memory safety and undefined
 * behaviour only; the values are pinned by the other oracle tests. Exit
 * status 0 and no sanitizer report mean success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t lcg = 0x243F6A8885A308D3ull;

static float rnd(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((int32_t)(lcg >> 32)) * (1.0f / 2147483648.0f);
}

static float* vec(size_t n, float scale)
{
    float* v = (float*)malloc((n ? n : 1) * sizeof *v);
    for (size_t i = 0; i < n; ++i)
        v[i] = rnd() * scale;
    return v;
}

static void threshold_family(size_t n)
{
    float* g = vec(n, 1.0f);
    float* r2 = vec(n, 0.25f);
    float* r3 = (float*)malloc((n ? n : 1) * sizeof *r3);
    memcpy(r3, r2, n * sizeof *r2);
    uint32_t* c2 = (uint32_t*)malloc(oracle_compressed_2bit_words(n) * sizeof *c2);
    uint32_t* c3 = (uint32_t*)malloc(oracle_compressed_ternary_words(n) * sizeof *c3);
    oracle_quantize_2bit(g, r2, n, -0.4f, 0.3f, c2);
    oracle_quantize_ternary(g, r3, n, -0.4f, 0.3f, c3);
    float* out = (float*)malloc((n ? n : 1) * sizeof *out);
    oracle_dequantize_2bit(c2, n, out);
    oracle_dequantize_ternary(c3, n, out);
    const uint32_t* b2[3] = {c2, c2, c2};
    const uint32_t* b3[3] = {c3, c3, c3};
    oracle_dequantize_2bit_sum(b2, 3, n, out);
    oracle_dequantize_ternary_sum(b3, 3, n, out);
    free(g), free(r2), free(r3), free(c2), free(c3), free(out);
}

static void qsgd_family(size_t n, int W, int s)
{
    float* gs[8];
    const float* cg[8];
    int8_t* lv[8];
    const int8_t* clv[8];
    for (int w = 0; w < W; ++w) {
        gs[w] = vec(n, 0.02f);
        cg[w] = gs[w];
        lv[w] = (int8_t*)malloc(n ? n : 1);
    }
    const float norm = oracle_maxnorm(cg, W, n);
    for (int w = 0; w < W; ++w) {
        oracle_qsgd_quantize(gs[w], n, norm, s, 0x1234567890ABCDEFull, (uint32_t)w, lv[w]);
        clv[w] = lv[w];
    }
    int32_t* S = (int32_t*)malloc((n ? n : 1) * sizeof *S);
    float* out = (float*)malloc((n ? n : 1) * sizeof *out);
    oracle_level_sum(clv, W, n, S);
    oracle_qsgd_dequantize(S, n, norm, s, out);
    uint64_t* idx = (uint64_t*)malloc((n ? n : 1) * sizeof *idx);
    for (size_t i = 0; i < n; ++i)
        idx[i] = (uint64_t)i * 4099u;
    oracle_qsgd_quantize_at(gs[0], idx, n, norm, s, 7, 1, lv[0]);
    for (int w = 0; w < W; ++w)
        free(gs[w]), free(lv[w]);
    free(S), free(out), free(idx);
}

static int randk_family(size_t n, uint32_t K)
{
    uint32_t* idx = (uint32_t*)malloc((K ? K : 1) * sizeof *idx);
    const int rc = oracle_randk_indices(n, K, 99, idx);
    if (rc == 0 && K > 0) {
        float* x = vec(n, 1.0f);
        float* gk = (float*)malloc(K * sizeof *gk);
        float* dense = (float*)malloc((n ? n : 1) * sizeof *dense);
        oracle_gather(x, idx, K, gk);
        oracle_scatter_dense(gk, idx, K, n, dense);
        free(x), free(gk), free(dense);
    }
    free(idx);
    return rc;
}

int main(void)
{
    static const size_t sizes[] = {0, 1, 2, 3, 4, 5, 15, 16, 17, 19, 20, 21, 63, 64, 65,
                                   1023, 1024, 1025, 1279, 1280, 1281, 4097, 65543};
    for (size_t k = 0; k < sizeof sizes / sizeof sizes[0]; ++k) {
        threshold_family(sizes[k]);
        qsgd_family(sizes[k], 3, 127);
        qsgd_family(sizes[k], 1, 1);
    }
    uint32_t ctr[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 7u, 1u}, key[2] = {0xFFFFFFFFu, 1u}, o[4];
    oracle_philox4x32_10(ctr, key, o);
    (void)oracle_uniform24(0xFFFFFFFFu);
    (void)oracle_stochastic_level(126.99999f, 0.99999994f);
    if (randk_family(1, 1) || randk_family(7, 7) || randk_family(1000, 999) ||
        randk_family(100003, 10000))
        return 2;
    if (randk_family(10, 11) == 0)  /* K > n must be refused */
        return 3;
    puts("sanitized oracle run: ok");
    return 0;
}
