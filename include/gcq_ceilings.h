/*
 * gcq_ceilings.h -- C ABI of libgcq_ceilings.so: plain streaming kernels
 * that measure what the HBM of the device gives each access mix of the
 * quantization hot path. They exist for the benchmark; they compute nothing
 * of the method.
 *
 * The benchmark needs these rates to say how close each hot-path kernel
 * comes to what the memory system allows for its mix of reads and writes
 * (the profile of apache/incubator-mxnet PR #8342, "Questions", is what
 * showed where that operator's time went; these kernels play the same role
 * here). Each kernel moves exactly the bytes of one hot-path kernel, in the
 * same tile shapes, with trivial arithmetic in place of the quantization.
 *
 * Conventions: device pointers on the current device, 16-byte aligned; work
 * is enqueued on `stream` and the call returns at once; n must be a positive
 * multiple of gcq_ceiling_quantum(). Return 0, or -1 with a message in
 * gcq_ceiling_last_error() (nothing enqueued) for bad arguments or a failed
 * launch. The caller owns every buffer; the contents written are
 * meaningless.
 */
#ifndef GCQ_CEILINGS_H
#define GCQ_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GCQ_CEIL_READ_CHUNKED = 0, /* one contiguous chunk per workgroup (the max-norm's grid) */
    GCQ_CEIL_READ_TILE = 1,    /* one 4 KB tile per wave */
    GCQ_CEIL_WRITE_TILE = 0,   /* one 4 KB tile per wave */
    GCQ_CEIL_WRITE_STRIDE = 1, /* grid-stride fill, 2048 workgroups */
    GCQ_CEIL_DEQ_TILE = 0,     /* one tile per wave, 256 B word loads (the kernel's) */
    GCQ_CEIL_DEQ_WIDE = 1,     /* two tiles per wave, 512 B word loads */
    GCQ_CEIL_DEQ_BURST = 2     /* 16 tiles per 1024-thread workgroup, words staged in LDS */
};

const char* gcq_ceiling_last_error(void);

/* n must be a multiple of this many values (16384). */
size_t gcq_ceiling_quantum(void);

/* Holds every later launch of the 256-thread kernels below (all but the
 * dequantize burst pattern) to at most per_cu resident workgroups per CU,
 * through an LDS reservation the kernels never touch; 0 restores what their
 * registers allow. Process-wide. Returns -1 for per_cu < 0. */
int gcq_ceiling_set_wg_per_cu(int per_cu);

/* 32-bit words each block of gcq_ceiling_compress / gcq_ceiling_dequant
 * must hold for n values: the 2-bit block's 3 + n/16, plus 4 of padding
 * that the 16-byte-aligned patterns may read. */
size_t gcq_ceiling_block_words(size_t n);

/* Read n fp32 from each of nbufs buffers (HOST array of device pointers,
 * 1..64): 4 n nbufs bytes. sink receives one word per workgroup or tile
 * and needs gcq_ceiling_read_sink_words(nbufs, n) words. */
size_t gcq_ceiling_read_sink_words(int nbufs, size_t n);
int gcq_ceiling_read(const float* const* bufs, int nbufs, size_t n, int pattern, uint32_t* sink,
                     size_t sink_words, hipStream_t stream);

/* Write n fp32 to dst: 4 n bytes. */
int gcq_ceiling_write(float* dst, size_t n, int pattern, hipStream_t stream);

/* The 2-bit compress's mix: read a[n] and b[n], write b[n] and the n/16
 * words 12 bytes into `words` (gcq_ceiling_block_words(n) capacity):
 * 12 n + n/4 bytes. */
int gcq_ceiling_compress(const float* a, float* b, size_t n, uint32_t* words, size_t words_cap,
                         hipStream_t stream);

/* The W-block dequantize-sum's mix, W = 8: read n/16 words 12 bytes into
 * each block (HOST array of W device pointers, each of block_cap_words >=
 * gcq_ceiling_block_words(n) words), write out[n]: W n/4 + 4 n bytes. */
int gcq_ceiling_dequant(const uint32_t* const* blocks, int W, size_t n, size_t block_cap_words,
                        int pattern, float* out, hipStream_t stream);

/* The ternary dequantize-sum's mix, W = 8: read n/20 elements 12 bytes into
 * each block (block_cap_words >= 3 + n/20), write out[n]: W n/5 + 4 n bytes.
 * n must be a multiple of gcq_ceiling_ternary_quantum() (81920). */
size_t gcq_ceiling_ternary_quantum(void);
int gcq_ceiling_dequant_ternary(const uint32_t* const* blocks, int W, size_t n,
                                size_t block_cap_words, float* out, hipStream_t stream);

/* The quantize's mix: read src[n] fp32, write dst[n/4] words: 5 n bytes. */
int gcq_ceiling_quantize(const float* src, size_t n, uint32_t* dst, hipStream_t stream);

/* The level sum's mix, W = 8: read n bytes from each of W buffers (HOST
 * array of device pointers, n/4 words each), write sums[n] int32 and
 * out[n] fp32: (W + 8) n bytes. */
int gcq_ceiling_levelsum(const uint32_t* const* levels, int W, size_t n, int32_t* sums,
                         float* out, hipStream_t stream);

/* The fused quantize-sum's mix, W = 8: read n fp32 from each of W
 * gradients (HOST array of device pointers), the workers in turn per tile,
 * write sums[n] int32 and out[n] fp32: (4 W + 8) n bytes. */
int gcq_ceiling_quantize_sum(const float* const* grads, int W, size_t n, int32_t* sums,
                             float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GCQ_CEILINGS_H */
