/*
 * gcq.h -- C ABI of libgcq.so: gradient quantization kernels for MI355X
 * (gfx950).
 *
 * Two families of element-wise gradient compression for data-parallel SGD:
 *
 *  (1) 2-bit threshold quantization with residual error feedback, from the
 *      apache/incubator-mxnet pull request #8342 "[WIP] 2bit gradient
 *      compression" (sections "Approach", "Two bit quantization", "Format of
 *      compressed gradient", "Local kvstore", "Operators").
 *  (2) QSGDMaxNorm stochastic quantization and its GlobalRandK sparsified
 *      variant, from the vineeths96 "Gradient-Compression" page
 *      ("Quantization for Distributed Optimization": "About The Project",
 *      "Results").
 *
 * Conventions for every entry point below:
 *  - Pointers are DEVICE pointers on the current HIP device unless the
 *    comment says "host". The caller owns every buffer.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without waiting for it. No entry point synchronizes with the host,
 *    reads device memory from the host, or allocates device memory -- the
 *    only exception is gc_plan_2bit_multi_create, which is set-up, not hot
 *    path.
 *  - Return value: GC_OK, or a negative gc_status. Arguments are validated
 *    on the host before anything is enqueued; on GC_EINVAL nothing was
 *    enqueued. GC_EHIP reports a failed launch, read from HIP's last-error
 *    state of the calling thread right after the launch (so an error left
 *    pending there by an earlier HIP call surfaces here too). gc_last_error()
 *    gives a message for the calling thread's last failure.
 *  - Inputs and outputs of one call must not overlap unless stated.
 *  - Alignment: float buffers need 4-byte alignment. 16-byte-aligned ones
 *    take float4 accesses; others (views into a flat bucket, say) take the
 *    same tiles through 4-byte accesses, at close to the same speed. int8
 *    level buffers may have any alignment (4-byte-aligned ones are read and
 *    written a word at a time). Results are identical in every case.
 */
#ifndef GCQ_H
#define GCQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gc_status {
    GC_OK = 0,
    GC_EINVAL = -1,       /* bad argument; nothing enqueued */
    GC_EHIP = -2,         /* a HIP call or kernel launch failed */
    GC_EUNSUPPORTED = -3  /* valid request outside what the library supports */
} gc_status;

/* Largest number of simulated workers a single call combines. */
#define GC_MAX_WORKERS 64

/* Message for the calling thread's most recent failed call ("" if none).
 * The pointer stays valid until that thread's next call into the library. */
const char* gc_last_error(void);

/* ====================================================================
 * 2-bit threshold quantization with error feedback
 * ==================================================================== */

/* Size, in 32-bit elements, of the compressed block for n values:
 * 3 + ceil(n / 16). (PR #8342 "Format of compressed gradient": two
 * thresholds, the original size, then one element per 16 values; this is
 * what its create_2bit operator allocates.) Host-only; enqueues nothing. */
size_t gc_compressed_2bit_words(size_t n);

/* quantize_2bit of PR #8342 ("Operators", "Two bit quantization",
 * "Approach"). For each i < n, in fp32:
 *     v = grad[i] + residual[i]
 *     code = 01 if v >= pos_threshold, 10 if v <= neg_threshold, else 00
 *     residual[i] = v - (pos_threshold | neg_threshold | 0 for that code)
 * and writes the block `compr` (gc_compressed_2bit_words(n) elements):
 *     compr[0] = neg_threshold (fp32 bits), compr[1] = pos_threshold,
 *     compr[2] = (float)n, compr[3 + j] = codes of values 16j..16j+15,
 *     value 16j in bits 31..30 (most significant first), unused tail codes 00.
 * Every element of `compr` is written; it needs no clearing beforehand.
 *   grad      [n] fp32, read only
 *   residual  [n] fp32, read and updated in place (start it at zero)
 *   thresholds: finite, neg_threshold < 0 < pos_threshold, else GC_EINVAL
 *   compr     [3 + ceil(n/16)] uint32, 4-byte aligned
 * n may be 0 (only the header is written). */
int compress_2bit(const float* grad, float* residual, size_t n,
                  float neg_threshold, float pos_threshold,
                  uint32_t* compr, hipStream_t stream);

/* dequantize_2bit of PR #8342 ("Operators"): code 01 -> compr[1] (the
 * positive threshold), 10 -> compr[0] (the negative threshold), 00 and the
 * unused 11 -> 0. The thresholds are read from the block on the device; the
 * size n comes from the caller (the fp32 size field is not exact above
 * 2^24).
 *   accumulate = 0: out[i] = value;  accumulate = 1: out[i] = out[i] + value
 *   out [n] fp32. */
int decompress_2bit(const uint32_t* compr, size_t n, float* out,
                    int accumulate, hipStream_t stream);

/* Dequantize-and-sum of W blocks, as the reducing device does in PR #8342
 * "Local kvstore" (every worker's gradient, the reducer's own included, is
 * quantized). out[i] = d_0(i) + d_1(i) + ... + d_{W-1}(i), summed in fp32
 * in that order, starting from worker 0's value.
 *   compr  HOST array of W device pointers, each a block of n values
 *   W      1 .. GC_MAX_WORKERS
 *   out    [n] fp32 */
int decompress_2bit_sum(const uint32_t* const* compr, int W, size_t n,
                        float* out, hipStream_t stream);

/* ---- many tensors in one launch ------------------------------------- */

/* A plan holds, in device memory, the descriptor table of T tensors and the
 * chunk map that spreads their elements evenly over workgroups. The block
 * table it writes is the concatenation of one compress_2bit block per
 * tensor, in order: tensor t's block starts at element
 * sum_{u<t} gc_compressed_2bit_words(n_u) of compr_base.
 * Create it once (it allocates and copies synchronously: set-up, not hot
 * path); it remembers the device pointers, which must stay valid.
 *   grads, residuals  HOST arrays of T device pointers (may be NULL where
 *                     ns[t] == 0)
 *   ns                HOST array of T element counts
 *   T                 >= 1 */
typedef struct gc_plan gc_plan;
int gc_plan_2bit_multi_create(const float* const* grads,
                              float* const* residuals, const size_t* ns,
                              int T, gc_plan** plan);
/* Total uint32 elements of the plan's block table. */
size_t gc_plan_compressed_words(const gc_plan* plan);
/* Writes the T block offsets (in uint32 elements) into the HOST array
 * `offsets`. */
int gc_plan_block_offsets(const gc_plan* plan, size_t* offsets);
/* compress_2bit on every tensor of the plan with one pair of thresholds, in
 * one launch. Same arithmetic, validation and format as compress_2bit. The
 * device that was current at gc_plan_2bit_multi_create must be current
 * here, else GC_EINVAL. */
int compress_2bit_multi(gc_plan* plan, float neg_threshold,
                        float pos_threshold, uint32_t* compr_base,
                        hipStream_t stream);
/* Frees the plan's device memory. Waits for the device first. */
void gc_plan_destroy(gc_plan* plan);

/* ---- dense ternary packing of the same codes ------------------------- */

/* PR #8342 "Two bit quantization" notes that its three codes leave one
 * 2-bit pattern unused and defers a denser packing. These entry points are
 * that packing: the same thresholds, codes, residual update and header as
 * compress_2bit, with five codes per byte as base-3 digits (1.6 bits per
 * value). Payload byte j (bytes in memory order from element 3 on) holds
 * values 5j .. 5j+4 as c0*81 + c1*27 + c2*9 + c3*3 + c4, the first value
 * most significant, digit = code (0 zero, 1 positive, 2 negative); zero
 * bytes pad the payload to whole elements.
 *
 * Size in 32-bit elements of the block for n values: 3 + ceil(n / 20).
 * Host-only; enqueues nothing. */
size_t gc_compressed_ternary_words(size_t n);

/* As compress_2bit (same arguments, same residual update, same
 * validation), writing the ternary block: every element of `compr`
 * (gc_compressed_ternary_words(n) of them, 4-byte aligned) is written. */
int compress_ternary(const float* grad, float* residual, size_t n,
                     float neg_threshold, float pos_threshold,
                     uint32_t* compr, hipStream_t stream);

/* As decompress_2bit, for a ternary block. Digit 1 -> compr[1], 2 ->
 * compr[0], 0 -> 0; a byte above 242 (never written) has leading digit 3,
 * which also reads as 0. */
int decompress_ternary(const uint32_t* compr, size_t n, float* out,
                       int accumulate, hipStream_t stream);

/* As decompress_2bit_sum, for W ternary blocks: fp32 sum in worker order,
 * starting from worker 0's value. */
int decompress_ternary_sum(const uint32_t* const* compr, int W, size_t n,
                           float* out, hipStream_t stream);

/* ====================================================================
 * QSGDMaxNorm (vineeths96 page, "About The Project": one max-norm shared by
 * all workers keeps the integer levels summable by an all-reduce)
 * ==================================================================== */

/* norm = max over workers w and elements i of |grads[w][i]| (fp32, exact).
 * Two launches: per-workgroup maxima into `ws`, then one workgroup.
 *   grads     HOST array of W device pointers, each [n] fp32
 *   norm      device fp32 scalar (output)
 *   ws        device workspace; pass ws = NULL to query: *ws_bytes is set
 *             to the size needed for (W, n) and nothing is enqueued.
 *             Otherwise *ws_bytes is its size and must be at least that.
 * NaN inputs are outside the domain (they are ignored by the max). */
int qsgd_global_maxnorm(const float* const* grads, int W, size_t n,
                        float* norm, void* ws, size_t* ws_bytes,
                        hipStream_t stream);

/* qsgd_global_maxnorm for callers that cannot allocate or hand in a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same result, same launches; the partial maxima
 * live in a fixed device array of the library (1 MiB, one per device, held
 * until the process ends) instead of `ws`. No device or host memory is
 * allocated by the call (the array's device address is looked up once per
 * device, on the first call there).
 *   grads  HOST array of W device pointers, each [n] fp32;  W 1 .. 64
 *   norm   device fp32 scalar (output)
 * Every valid (W, n) fits the array; GC_EUNSUPPORTED would name a size
 * beyond it. All calls on one device share that device's array: calls that
 * overlap on one device (other streams, other host threads) race and must
 * be serialized by the caller. */
int qsgd_global_maxnorm_noalloc(const float* const* grads, int W, size_t n, float* norm,
                                hipStream_t stream);

/* levels[i] = sign(grad[i]) * floor(|grad[i]| / norm * s + u_i), with
 *   x = (|grad[i]| / norm) * s rounded to fp32 after each operation,
 *   the floor of x + u_i taken exactly (never rounding up to s + 1),
 *   u_i = (r >> 8) * 2^-24 for the 32-bit Philox4x32-10 output word
 *   r = word (i mod 4) of Philox(key = (seed lo, seed hi),
 *                                counter = (i/4 lo, i/4 hi, worker, 0)),
 *   levels = 0 everywhere when *norm == 0.
 *   grad    [n] fp32, finite (a NaN or infinite value, or an infinite
 *           norm, gets an unspecified level);  norm  device fp32 scalar,
 *           >= max |grad|
 *   s       1 .. 127 (levels lie in [-s, s]);  levels [n] int8 */
int qsgd_maxnorm_quantize(const float* grad, size_t n, const float* norm,
                          int s, uint64_t seed, uint32_t worker,
                          int8_t* levels, hipStream_t stream);

/* Sum of the W workers' levels (the all-reduce, simulated on one device)
 * and its dequantization:
 *   S[k]   = sum_w levels[w][k]   (int32, exact)
 *   val[k] = (norm * (float)S[k]) / (float)s   (fp32, two roundings)
 * Dense form (scatter_idx == NULL): sums[k] = S[k] if sums != NULL,
 *   out[k] = val[k], for k < n; dense_n is ignored.
 * Sparse form (scatter_idx != NULL, the GlobalRandK step): out has dense_n
 *   elements; out = 0 everywhere, then out[scatter_idx[k]] = val[k] for
 *   k < n. scatter_idx must hold distinct values < dense_n.
 *   levels  HOST array of W device pointers, each [n] int8
 *   norm    device fp32 scalar;  s 1 .. 127;  W 1 .. GC_MAX_WORKERS */
int qsgd_dequant_sum(const int8_t* const* levels, int W, size_t n,
                     const float* norm, int s, int32_t* sums, float* out,
                     const uint32_t* scatter_idx, size_t dense_n,
                     hipStream_t stream);

/* The W quantizes and the dense level sum of one step in one pass, for a
 * single device that simulates all W workers (the pages' all-reduce of
 * levels, "About The Project"): sums and out are exactly those of
 * qsgd_maxnorm_quantize on grads[w] with worker = w, for w = 0 .. W-1,
 * followed by the dense qsgd_dequant_sum. The int8 levels themselves are
 * not written, which saves their write and read-back (5 W n + W n bytes
 * become 4 W n).
 *   grads  HOST array of W device pointers, each [n] fp32
 *   norm   device fp32 scalar (the shared max-norm);  s 1 .. 127
 *   sums   [n] int32, or NULL;  out [n] fp32;  W 1 .. GC_MAX_WORKERS */
int qsgd_quantize_sum(const float* const* grads, int W, size_t n,
                      const float* norm, int s, uint64_t seed,
                      int32_t* sums, float* out, hipStream_t stream);

/* ---- GlobalRandK (vineeths96 page, "Results": K shared indices) -------- */

/* The K indices every worker shares: the first K positions of a partial
 * Fisher-Yates shuffle of 0..n-1 whose step i swaps positions i and
 *   j = i + floor(R * (n - i) / 2^64),  R = (w1 << 32) | w0,
 * where (w0, w1) are words 0 and 1 of Philox4x32-10(key = (seed lo,
 * seed hi), counter = (i, 0, 0, 1)).
 *   n      1 .. 2^32;  K  0 .. n;  idx  [K] uint32 (output, distinct)
 *   ws     device workspace, queried like qsgd_global_maxnorm's. */
int grandk_indices(size_t n, uint32_t K, uint64_t seed, uint32_t* idx,
                   void* ws, size_t* ws_bytes, hipStream_t stream);

/* out[k] = x[idx[k]] for k < K. idx values must be < the length of x. */
int gather_f32(const float* x, const uint32_t* idx, size_t K, float* out,
               hipStream_t stream);

/* The whole GlobalRandK-MN step of [QMN] "Results" for W simulated workers,
 * in three launches instead of one per worker per stage. The results are
 * exactly those of the separate calls:
 *   grandk_indices(n, K, seed)            -> idx
 *   gather_f32(grads[w], idx) for each w  -> g_w (length K)
 *   qsgd_global_maxnorm(g_0 .. g_{W-1})   -> norm
 *   qsgd_maxnorm_quantize(g_w, norm, s, seed, worker = w) for each w
 *   qsgd_dequant_sum(levels, norm, s, dense, sums, scatter_idx = idx, n)
 * (one seed serves the draw and the rounding, as in those calls).
 *   grads  HOST array of W device pointers, each [n] fp32
 *   idx    [K] uint32 out;  sums [K] int32 out, or NULL
 *   dense  [n] fp32 out: 0 outside idx, the dequantized sum at idx[k]
 *   norm   device fp32 scalar out (the shared max-norm), or NULL
 *   ws     16-byte-aligned workspace; ws == NULL: *ws_bytes = its size
 *          (about 4 W K bytes), else *ws_bytes must be at least that
 *   1 <= n <= 2^32, K <= n, K <= 2^30, s 1 .. 127, W 1 .. GC_MAX_WORKERS */
int grandk_mn_step(const float* const* grads, int W, size_t n, uint32_t K,
                   uint64_t seed, int s, uint32_t* idx, int32_t* sums,
                   float* dense, float* norm, void* ws, size_t* ws_bytes,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GCQ_H */
