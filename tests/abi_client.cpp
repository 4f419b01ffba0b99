// abi_client.cpp -- a client of libgcq.so that uses nothing but the C ABI
// (include/gcq.h) and the HIP runtime: no Python, no torch. It allocates
// its own device buffers and stream, runs each method family's step through
// the entry points, and checks every output element bit for bit against the
// CPU oracle (oracle/oracle.h, test infrastructure). Prints "OK" and exits
// 0 when all match; prints the first mismatch and exits 1 otherwise.
//
// Inputs come from splitmix64 below (seeded, synthetic); both sides read
// the same bytes.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gcq.h"
#include "oracle.h"

namespace {

int g_failures = 0;

#define HIP_OK(x)                                                                          \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

#define GC_OK_OR_FAIL(x)                                                                   \
    do {                                                                                   \
        int rc_ = (x);                                                                     \
        if (rc_ != GC_OK) {                                                                \
            std::printf("%s returned %d: %s\n", #x, rc_, gc_last_error());                 \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

uint64_t splitmix64(uint64_t& s)
{
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// n values uniform in [-scale, scale), from 24 random bits each.
std::vector<float> inputs(uint64_t seed, size_t n, float scale)
{
    std::vector<float> v(n);
    for (size_t i = 0; i < n; ++i) {
        const float u = float(splitmix64(seed) >> 40) * (1.0f / 16777216.0f);
        v[i] = (2.0f * u - 1.0f) * scale;
    }
    return v;
}

template <typename T>
bool same_bits(const char* what, const std::vector<T>& got, const std::vector<T>& want)
{
    if (got.size() != want.size() ||
        std::memcmp(got.data(), want.data(), got.size() * sizeof(T)) != 0) {
        for (size_t i = 0; i < got.size() && i < want.size(); ++i)
            if (std::memcmp(&got[i], &want[i], sizeof(T)) != 0) {
                std::printf("FAIL %s: first difference at element %zu\n", what, i);
                break;
            }
        ++g_failures;
        return false;
    }
    return true;
}

template <typename T>
T* to_device(const std::vector<T>& h)
{
    T* d = nullptr;
    if (hipMalloc(&d, h.size() * sizeof(T) + 16) != hipSuccess)
        return nullptr;
    if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
        return nullptr;
    return d;
}

template <typename T>
std::vector<T> to_host(const T* d, size_t n, hipStream_t s)
{
    std::vector<T> h(n);
    if (hipStreamSynchronize(s) != hipSuccess ||
        hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess)
        std::printf("FAIL copy back\n"), ++g_failures;
    return h;
}

// Two error-feedback iterations of W workers' compress_2bit, then the
// dequantize-sum of their blocks.
int two_bit(hipStream_t s)
{
    const int W = 3;
    const size_t n = 100003;
    const float neg = -0.5f, pos = 0.5f;
    const size_t words = gc_compressed_2bit_words(n);
    if (words != oracle_compressed_2bit_words(n))
        return std::printf("FAIL block size\n"), 1;
    std::vector<std::vector<float>> res_h(W, std::vector<float>(n, 0.0f));
    std::vector<std::vector<uint32_t>> blk_h(W, std::vector<uint32_t>(words));
    std::vector<float*> g_d(W), r_d(W);
    std::vector<uint32_t*> b_d(W);
    for (int w = 0; w < W; ++w) {
        r_d[w] = to_device(res_h[w]);
        b_d[w] = to_device(blk_h[w]);
        if (!r_d[w] || !b_d[w])
            return std::printf("FAIL allocation\n"), 1;
    }
    for (int it = 0; it < 2; ++it) {
        for (int w = 0; w < W; ++w) {
            const std::vector<float> g = inputs(1000 * w + it, n, 0.8f);
            if (it > 0)
                HIP_OK(hipFree(g_d[w]));
            g_d[w] = to_device(g);
            if (!g_d[w])
                return std::printf("FAIL allocation\n"), 1;
            GC_OK_OR_FAIL(compress_2bit(g_d[w], r_d[w], n, neg, pos, b_d[w], s));
            oracle_quantize_2bit(g.data(), res_h[w].data(), n, neg, pos, blk_h[w].data());
        }
        for (int w = 0; w < W; ++w) {
            same_bits("2-bit block", to_host(b_d[w], words, s), blk_h[w]);
            same_bits("2-bit residual", to_host(r_d[w], n, s), res_h[w]);
        }
    }
    float* out_d = nullptr;
    HIP_OK(hipMalloc(&out_d, n * sizeof(float)));
    GC_OK_OR_FAIL(decompress_2bit_sum(const_cast<const uint32_t* const*>(b_d.data()), W, n,
                                      out_d, s));
    std::vector<const uint32_t*> bh(W);
    for (int w = 0; w < W; ++w)
        bh[w] = blk_h[w].data();
    std::vector<float> sum_h(n);
    oracle_dequantize_2bit_sum(bh.data(), W, n, sum_h.data());
    same_bits("2-bit dequantize-sum", to_host(out_d, n, s), sum_h);
    // a refused call enqueues nothing and says why
    if (compress_2bit(g_d[0], r_d[0], n, 0.5f, -0.5f, b_d[0], s) != GC_EINVAL ||
        std::strlen(gc_last_error()) == 0)
        std::printf("FAIL swapped thresholds were not refused\n"), ++g_failures;
    for (int w = 0; w < W; ++w) {
        HIP_OK(hipFree(g_d[w]));
        HIP_OK(hipFree(r_d[w]));
        HIP_OK(hipFree(b_d[w]));
    }
    HIP_OK(hipFree(out_d));
    return 0;
}

// The QSGD-MN step: max-norm, W quantizes, level sum and dequantize.
int qsgd(hipStream_t s)
{
    const int W = 3, S = 127;
    const size_t n = 70001;
    const uint64_t seed = 0x5EEDull;
    std::vector<std::vector<float>> g_h(W);
    std::vector<float*> g_d(W);
    std::vector<int8_t*> l_d(W);
    for (int w = 0; w < W; ++w) {
        g_h[w] = inputs(77 + w, n, 0.02f);
        g_d[w] = to_device(g_h[w]);
        HIP_OK(hipMalloc(&l_d[w], n));
        if (!g_d[w])
            return std::printf("FAIL allocation\n"), 1;
    }
    float* norm_d = nullptr;
    HIP_OK(hipMalloc(&norm_d, sizeof(float)));
    size_t ws_bytes = 0;
    GC_OK_OR_FAIL(qsgd_global_maxnorm(g_d.data(), W, n, norm_d, nullptr, &ws_bytes, s));
    void* ws = nullptr;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    GC_OK_OR_FAIL(qsgd_global_maxnorm(g_d.data(), W, n, norm_d, ws, &ws_bytes, s));
    for (int w = 0; w < W; ++w)
        GC_OK_OR_FAIL(qsgd_maxnorm_quantize(g_d[w], n, norm_d, S, seed, uint32_t(w), l_d[w], s));
    int32_t* sums_d = nullptr;
    float* out_d = nullptr;
    HIP_OK(hipMalloc(&sums_d, n * sizeof(int32_t)));
    HIP_OK(hipMalloc(&out_d, n * sizeof(float)));
    GC_OK_OR_FAIL(qsgd_dequant_sum(const_cast<const int8_t* const*>(l_d.data()), W, n, norm_d, S,
                                   sums_d, out_d, nullptr, 0, s));
    std::vector<const float*> gh(W);
    for (int w = 0; w < W; ++w)
        gh[w] = g_h[w].data();
    const float norm = oracle_maxnorm(gh.data(), W, n);
    same_bits("QSGD norm", to_host(norm_d, 1, s), std::vector<float>{norm});
    std::vector<std::vector<int8_t>> lv(W, std::vector<int8_t>(n));
    std::vector<const int8_t*> lh(W);
    for (int w = 0; w < W; ++w) {
        oracle_qsgd_quantize(g_h[w].data(), n, norm, S, seed, uint32_t(w), lv[w].data());
        same_bits("QSGD levels", to_host(l_d[w], n, s), lv[w]);
        lh[w] = lv[w].data();
    }
    std::vector<int32_t> sums(n);
    std::vector<float> out(n);
    oracle_level_sum(lh.data(), W, n, sums.data());
    oracle_qsgd_dequantize(sums.data(), n, norm, S, out.data());
    same_bits("QSGD sums", to_host(sums_d, n, s), sums);
    same_bits("QSGD dequantized", to_host(out_d, n, s), out);
    for (int w = 0; w < W; ++w) {
        HIP_OK(hipFree(g_d[w]));
        HIP_OK(hipFree(l_d[w]));
    }
    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(norm_d));
    HIP_OK(hipFree(sums_d));
    HIP_OK(hipFree(out_d));
    return 0;
}

// The one-call GlobalRandK-MN step.
int grandk(hipStream_t s)
{
    const int W = 3, S = 7;
    const size_t n = 200003;
    const uint32_t K = 3000;
    const uint64_t seed = 0xABCDEF12345ull;
    std::vector<std::vector<float>> g_h(W);
    std::vector<float*> g_d(W);
    for (int w = 0; w < W; ++w) {
        g_h[w] = inputs(500 + w, n, 0.01f);
        g_d[w] = to_device(g_h[w]);
        if (!g_d[w])
            return std::printf("FAIL allocation\n"), 1;
    }
    size_t ws_bytes = 0;
    GC_OK_OR_FAIL(grandk_mn_step(g_d.data(), W, n, K, seed, S, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, &ws_bytes, s));
    void* ws = nullptr;
    uint32_t* idx_d = nullptr;
    int32_t* sums_d = nullptr;
    float *dense_d = nullptr, *norm_d = nullptr;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    HIP_OK(hipMalloc(&idx_d, K * sizeof(uint32_t)));
    HIP_OK(hipMalloc(&sums_d, K * sizeof(int32_t)));
    HIP_OK(hipMalloc(&dense_d, n * sizeof(float)));
    HIP_OK(hipMalloc(&norm_d, sizeof(float)));
    GC_OK_OR_FAIL(grandk_mn_step(g_d.data(), W, n, K, seed, S, idx_d, sums_d, dense_d, norm_d,
                                 ws, &ws_bytes, s));
    std::vector<uint32_t> idx(K);
    if (oracle_randk_indices(n, K, seed, idx.data()) != 0)
        return std::printf("FAIL oracle draw\n"), 1;
    std::vector<std::vector<float>> gk(W, std::vector<float>(K));
    std::vector<const float*> gp(W);
    for (int w = 0; w < W; ++w) {
        oracle_gather(g_h[w].data(), idx.data(), K, gk[w].data());
        gp[w] = gk[w].data();
    }
    const float norm = oracle_maxnorm(gp.data(), W, K);
    std::vector<std::vector<int8_t>> lv(W, std::vector<int8_t>(K));
    std::vector<const int8_t*> lh(W);
    for (int w = 0; w < W; ++w) {
        oracle_qsgd_quantize(gk[w].data(), K, norm, S, seed, uint32_t(w), lv[w].data());
        lh[w] = lv[w].data();
    }
    std::vector<int32_t> sums(K);
    std::vector<float> vals(K), dense(n);
    oracle_level_sum(lh.data(), W, K, sums.data());
    oracle_qsgd_dequantize(sums.data(), K, norm, S, vals.data());
    oracle_scatter_dense(vals.data(), idx.data(), K, n, dense.data());
    same_bits("GRandK indices", to_host(idx_d, K, s), idx);
    same_bits("GRandK norm", to_host(norm_d, 1, s), std::vector<float>{norm});
    same_bits("GRandK sums", to_host(sums_d, K, s), sums);
    same_bits("GRandK dense", to_host(dense_d, n, s), dense);
    for (int w = 0; w < W; ++w)
        HIP_OK(hipFree(g_d[w]));
    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(idx_d));
    HIP_OK(hipFree(sums_d));
    HIP_OK(hipFree(dense_d));
    HIP_OK(hipFree(norm_d));
    return 0;
}

}  // namespace

int main()
{
    hipStream_t s = nullptr;
    HIP_OK(hipStreamCreate(&s));
    std::printf("[case] 2-bit W=3 n=100003, two iterations\n");
    std::fflush(stdout);
    if (two_bit(s))
        return 1;
    std::printf("[case] QSGD-MN W=3 n=70001 s=127\n");
    std::fflush(stdout);
    if (qsgd(s))
        return 1;
    std::printf("[case] GRandK-MN W=3 n=200003 K=3000 s=7\n");
    std::fflush(stdout);
    if (grandk(s))
        return 1;
    HIP_OK(hipStreamDestroy(s));
    if (g_failures) {
        std::printf("%d mismatches\n", g_failures);
        return 1;
    }
    std::printf("OK\n");
    return 0;
}
