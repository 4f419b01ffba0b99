/*
 * oracle.h -- plain CPU oracle for the gradient-quantization hot path.
 *
 * TEST INFRASTRUCTURE ONLY. This is the independent reference the HIP
 * library is checked against. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Every function is single-threaded and written for clarity, not speed.
 * fp32 is used exactly where the method is defined in fp32: each operation
 * is one IEEE-754 binary32 rounding, built with -ffp-contract=off.
 *
 * Sources cited in oracle.c:
 *   [MX]  apache/incubator-mxnet PR #8342 "[WIP] 2bit gradient compression":
 *         sections "Approach", "Two bit quantization",
 *         "Format of compressed gradient", "Local kvstore", "Operators".
 *   [QMN] vineeths96 "Gradient-Compression" README ("Quantization for
 *         Distributed Optimization"): "About The Project" (all-reduce
 *         compatible QSGDMaxNorm) and "Results" (GRandK-MN, K = 10000).
 *   [PHX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *         1, 2, 3", SC'11: the Philox-4x32 bijection with 10 rounds.
 */
#ifndef GCQ_ORACLE_H
#define GCQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- 2-bit threshold quantization with residual error feedback [MX] ---- */
size_t oracle_compressed_2bit_words(size_t n);
void oracle_quantize_2bit(const float* grad, float* residual, size_t n,
                          float neg_threshold, float pos_threshold,
                          uint32_t* compr);
void oracle_dequantize_2bit(const uint32_t* compr, size_t n, float* out);
void oracle_dequantize_2bit_sum(const uint32_t* const* compr, int W, size_t n,
                                float* out);

/* ---- dense ternary packing of the same codes (5 per byte) [MX] ---- */
size_t oracle_compressed_ternary_words(size_t n);
void oracle_quantize_ternary(const float* grad, float* residual, size_t n,
                             float neg_threshold, float pos_threshold,
                             uint32_t* compr);
void oracle_dequantize_ternary(const uint32_t* compr, size_t n, float* out);
void oracle_dequantize_ternary_sum(const uint32_t* const* compr, int W,
                                   size_t n, float* out);

/* ---- Philox-4x32-10 [PHX] ---- */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                          uint32_t out[4]);

/* ---- QSGD max-norm quantization [QMN] ---- */
float oracle_uniform24(uint32_t r);
int oracle_stochastic_level(float x, float u);
float oracle_maxnorm(const float* const* grads, int W, size_t n);
void oracle_qsgd_quantize(const float* grad, size_t n, float norm, int s,
                          uint64_t seed, uint32_t worker, int8_t* levels);
void oracle_qsgd_quantize_at(const float* values, const uint64_t* index,
                             size_t m, float norm, int s, uint64_t seed,
                             uint32_t worker, int8_t* levels);
void oracle_level_sum(const int8_t* const* levels, int W, size_t n,
                      int32_t* sums);
void oracle_qsgd_dequantize(const int32_t* sums, size_t n, float norm, int s,
                            float* out);

/* ---- GlobalRandK [QMN] ---- */
int oracle_randk_indices(size_t n, uint32_t K, uint64_t seed, uint32_t* idx);
void oracle_gather(const float* x, const uint32_t* idx, size_t K, float* out);
void oracle_scatter_dense(const float* vals, const uint32_t* idx, size_t K,
                          size_t dense_n, float* dense);

#ifdef __cplusplus
}
#endif
#endif
