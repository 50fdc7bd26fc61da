/*
 * gq.h -- Global-QSGD gradient compression on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libgq.so.  The operator is the Allreduce-compatible quantizer of
 * "Global-QSGD: Practical Floatless Quantization for Distributed Learning
 * with Theoretical Guarantees" (Xin, Canini, Richtarik, Horvath):
 *   - Sec. 2 (notation) defines the (q,p)-norm of the concatenation
 *     x = [x_1 .. x_n] of the n workers' vectors;
 *   - Sec. 3 (Global-Q) divides every coordinate by that ONE global norm,
 *     instead of each worker's local norm, and rounds it at random, without
 *     bias, to a level grid: standard dithering Global-L_s (levels (s-i)/s)
 *     or exponential dithering Global-E_s (levels 0 and 2^-k);
 *   - Sec. 6 (implementation) runs quantization, an integer Allreduce and
 *     one dequantization per gradient bucket.
 * Here the n workers are the n rows of one device buffer x[n][d], and the
 * Allreduce is an exact integer sum over those rows.
 *
 * Conventions shared by every entry point
 *   - x is row-major [n][d]; row i is worker i.  dtype GQ_IN_F32 (float) or
 *     GQ_IN_BF16 (bfloat16, widened exactly to float).
 *   - q, p are reals >= 1 or +INFINITY (the (q,p)-norm: q inside a worker,
 *     p over the n per-worker norms).  The pairs from {2, inf} are exact
 *     forms; other orders go through fp64 pow.
 *   - s: number of level intervals.  L: 1 <= s <= 2^24; the integer code of
 *     a coordinate is in [-s, s].  E: 1 <= s <= 31; levels 2^-k (k < s)
 *     are coded as the integers 2^(s-1-k), so codes are in [-2^(s-1), 2^(s-1)].
 *     M denotes the top code (s for L, 2^(s-1) for E).
 *   - code_bits W: two's-complement width of packed codes and code sums;
 *     gq_min_code_bits(n, s, scheme) <= W <= 32 so that any sum of n codes
 *     is exact in W bits.
 *   - Packed layout: each row is a little-endian bitstream; coordinate j
 *     occupies bits [j W, j W + W); rows are gq_code_row_bytes(d, W) bytes
 *     apart (16-byte multiples); pad bits are zero.  W = 8, 16, 32 is
 *     exactly an int8 / int16 / int32 array.
 *   - Randomness: Philox4x32-10 (Salmon et al., SC'11), key = seed, counter
 *     (lo32(j/8), hi32(j/8), worker, draw).  Coordinate j of worker w uses the
 *     16-bit half (j%8)%2 of word (j%8)/2 of draw 0 as the high half of a
 *     32-bit uniform u and the same half of draw 1 as its low half; the
 *     upper level is taken iff u < F, F = floor(frac * 2^32).
 *   - Memory: every pointer is a DEVICE pointer owned by the caller.  x,
 *     mean and packed code buffers must be 16-byte aligned.  With d == 0
 *     the per-coordinate buffers (x, codes, sums, mean) may be NULL.  The library
 *     allocates nothing and keeps no state between calls, except the
 *     device array behind gq_compress_mean_noalloc (below).
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *     enqueue kernels and never synchronize; results are ready when the
 *     stream reaches them.  Scalars computed on the device (the norm) stay
 *     there and later calls read them there.
 *   - Errors: every argument check runs before any HIP call, and a failing
 *     check returns its status with nothing enqueued.  GQ_ERR_DEVICE means a
 *     launch failed (hipGetLastError); gq_last_error() describes the most
 *     recent failure of the calling thread.  Non-finite inputs give
 *     unspecified but in-range codes (|code| <= M) and never fault.
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GQ_SCHEME_L = 0, GQ_SCHEME_E = 1 };
enum { GQ_IN_F32 = 0, GQ_IN_BF16 = 1 };

enum {
    GQ_OK = 0,
    GQ_ERR_NULL = 1,        /* a required pointer is NULL */
    GQ_ERR_ARG = 2,         /* n, d, s, dtype or scheme out of range */
    GQ_ERR_UNSUPPORTED = 3, /* q or p not in {2, inf}; sizes beyond the launch limits */
    GQ_ERR_CODE_WIDTH = 4,  /* code_bits outside [gq_min_code_bits, 32] */
    GQ_ERR_WORKSPACE = 5,   /* workspace smaller than gq_workspace_bytes */
    GQ_ERR_ALIGN = 6,       /* a buffer is not 16-byte aligned */
    GQ_ERR_DEVICE = 7       /* a HIP launch failed */
};

/* Smallest code width that holds every sum of n codes of the scheme:
 * ceil(log2(n M + 1)) + 1.  Returns -1 for invalid (n, s, scheme).        */
int32_t gq_min_code_bits(int64_t n, int32_t s, int32_t scheme);

/* Bytes of one packed row of d W-bit fields: 16 * ceil(d W / 128).
 * Returns -1 for d < 0 or W outside [1, 32].                               */
int64_t gq_code_row_bytes(int64_t d, int32_t code_bits);

/* Device workspace needed by gq_global_norm, gq_compress_mean,
 * gq_qsgd_local_mean and gq_e8_compress_mean for an [n][d] input of either
 * type (per-block partial norms and the per-worker norms).  Its contents
 * need no initialization and are scratch between calls; calls that may run
 * concurrently (on different streams) need separate workspaces.  Returns -1
 * for invalid sizes.                                                       */
int64_t gq_workspace_bytes(int64_t n, int64_t d);

/* Workspace with which gq_compress_mean runs fastest: gq_workspace_bytes
 * plus gq_span_bounds_bytes(n, d) rounded up to 256, where the norm pass
 * leaves the span bounds of the zero-code skip (see gq_global_norm_bounds).
 * The results are the same bits either way; with only
 * gq_workspace_bytes(n, d) bytes the fused pass reads every coordinate.
 * Returns -1 for invalid sizes.                                            */
int64_t gq_compress_workspace_bytes(int64_t n, int64_t d);

/* Global (q,p)-norm of the concatenation (Sec. 2 notation):
 *   q = 2: S_i = sum_j x_ij^2 in fp64 (each square exact); q = inf:
 *   m_i = max_j |x_ij|; other q: S_i = sum_j |x_ij|^q (fp64 pow).
 *   (2,2): N = fp32(sqrt(sum_i S_i)); (inf,2): fp32(sqrt(sum_i m_i^2));
 *   (2,inf): fp32(sqrt(max_i S_i)); (inf,inf): max_i m_i.  Other pairs:
 *   w_i = m_i, sqrt(S_i) (q = 2) or S_i^(1/q); N = fp32 of max_i w_i (p = inf),
 *   sqrt(sum_i w_i^2) (p = 2) or (sum_i w_i^p)^(1/p).
 *   Writes N to norm_dev[0] (one float, device).
 * The reduction tree is fixed by (n, d) and the input type, so repeated
 * calls give identical bits.  d == 0 gives N = 0.                          */
int32_t gq_global_norm(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                       float *norm_dev, void *workspace, int64_t workspace_bytes, void *stream);

/* The same norm over workers held in shards, e.g. one per device (Sec. 2
 * notation; Sec. 6 places the norm before the quantized Allreduce).
 * gq_norm_term writes to term_dev[0] (one double, device) the combination
 * over its n rows that the norm takes before its root, with S_i, m_i and
 * w_i as above:
 *   (2,2): sum_i S_i    (inf,2): sum_i m_i^2    (2,inf): max_i S_i
 *   (inf,inf): max_i m_i;  other orders: max_i w_i (p = inf),
 *   sum_i w_i^2 (p = 2), sum_i w_i^p (other p).
 * Terms of disjoint shards combine by SUM for finite p and by MAX for
 * p = inf (one all-reduce of a double).  gq_norm_from_term then writes N
 * of the combined term to norm_dev[0]: fp32 of it for (inf,inf) and for
 * p = inf with other orders, of its square root for the other {2, inf}
 * pairs and for p = 2, of its 1/p-th power otherwise.
 * One shard holding every row reproduces gq_global_norm's N bit for bit.
 * Over several shards N agrees within 1e-6 relative (exactly for
 * q = p = inf): each shard's fp64 sums follow its own reduction tree,
 * fixed by its (n, d), and a SUM over shards adds in its own order.
 * Errors as gq_global_norm; gq_norm_from_term needs no workspace.         */
int32_t gq_norm_term(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                     double *term_dev, void *workspace, int64_t workspace_bytes, void *stream);
int32_t gq_norm_from_term(const double *term_dev, float q, float p, float *norm_dev,
                          void *stream);

/* Quantization (Sec. 3, Global-Q with the L or E levels), given the global
 * norm N in norm_dev[0]:
 *   pre = 2^64 if N < 2^-64 else 1 (exact);  L: sigma = fp32(s / (N pre)),
 *   E: sigma = fp32(1 / (N pre)), both divided in fp64;
 *   t = fp32(fp32(|x| pre) sigma) clamped to s (L) or 1 (E);
 *   L: magnitude floor(t) or floor(t)+1, F = floor((t - floor t) 2^32);
 *   E: t = 2^e (1+phi) >= 2^(1-s): magnitude 2^(e+s-1) or twice it,
 *      F = phi 2^32; t < 2^(1-s): magnitude 0 or 1, F = floor(t 2^(s-1) 2^32);
 *   code = (u < F ? upper : lower), negated when the sign bit of x is set.
 * N == 0 gives all-zero codes.  Row i uses worker index worker_base + i in
 * the Philox counter, so shards quantized on different devices with their
 * global row index reproduce one big quantization.
 * codes: n rows of gq_code_row_bytes(d, W) bytes.  W must hold a sum of n
 * codes (gq_min_code_bits(n, s, scheme) <= W <= 32).                       */
int32_t gq_quantize(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s, int32_t scheme,
                    const float *norm_dev, uint64_t seed, int64_t worker_base, int32_t code_bits,
                    void *codes, void *stream);

/* The integer Allreduce of Sec. 6 on one device: code_sum[j] = sum_i
 * code[i][j], exact, written as one packed row of W-bit fields.  The sum
 * is exact whenever the codes came from gq_quantize with the same n and W
 * (W >= gq_min_code_bits); otherwise it wraps modulo 2^W.                  */
int32_t gq_reduce_codes(const void *codes, int64_t n, int64_t d, int32_t code_bits,
                        void *code_sum, void *stream);

/* Dequantization to the mean (Sec. 6): mean[j] = fp32(code_sum[j] kappa),
 * kappa = fp64(N / (n M)), product in fp64.  mean: d floats, device.       */
int32_t gq_dequantize(const void *code_sum, int64_t n, int64_t d, int32_t s, int32_t scheme,
                      int32_t code_bits, const float *norm_dev, float *mean, void *stream);

/* ---- Word layout for a native integer all-reduce ----
 * Sec. 6 reduces the codes with the collective's own integer SUM.  A
 * collective without a 16-bit integer type still sums 32-bit words, so this
 * layout packs f = floor(32 / W) fields per 32-bit word: coordinate j sits
 * in word j / f at bits [W (j % f), W (j % f) + W) and holds its code plus
 * M (a value in [0, 2M]).  Bits above the last field of a word, fields past
 * d and pad words are 0.  Rows are gq_word_row_bytes(d, W) bytes (16-byte
 * multiples) apart.  A field summed over n rows holds sum_i code_ij + n M
 * <= 2 n M < 2^W whenever W >= gq_min_code_bits(n, s, scheme), so the
 * word-wise uint32 sum of the rows -- in any order, as any all-reduce
 * algorithm adds them -- never carries out of a field.  Bits on the wire
 * per coordinate: 32 / f (16 for W = 11..16, 10.7 for W = 9, 10, 8 for
 * W = 7, 8), against 32 for an int32 container.                          */

/* 16 * ceil(ceil(d / floor(32 / W)) / 4); -1 for d < 0 or W outside [2, 32]. */
int64_t gq_word_row_bytes(int64_t d, int32_t code_bits);

/* gq_quantize's codes (same rules, same draws, worker index worker_base + i
 * for row i) written in the word layout.  W must hold a sum of the codes
 * of every worker whose rows will be summed: with shards, choose W for the
 * total number of workers (this call checks it against its own n).
 * words: n rows of gq_word_row_bytes(d, W) bytes, 16-byte aligned.        */
int32_t gq_quantize_words(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                          int32_t scheme, const float *norm_dev, uint64_t seed,
                          int64_t worker_base, int32_t code_bits, void *words, void *stream);

/* A device's own n rows summed before the all-reduce, in one pass: the
 * word row whose fields hold sum_i (code_ij + M) over its rows -- the same
 * bits as gq_sum_words of gq_quantize_words' rows, with the codes summed in
 * registers and never written.  Rows use worker indices worker_base + i.
 * Summed word-wise over every device and decoded by gq_dequantize_words
 * with n = the total number of workers, it gives the mean over all of
 * them; W must hold that total (this call checks it against its own n).
 * word_sum: gq_word_row_bytes(d, W) bytes, 16-byte aligned.               */
int32_t gq_compress_words_from_norm(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                                   int32_t scheme, const float *norm_dev, uint64_t seed,
                                   int64_t worker_base, int32_t code_bits, void *word_sum,
                                   void *stream);

/* What a native uint32 SUM all-reduce computes, on one device: word_sum[w]
 * = sum_i words[i][w] modulo 2^32 over the n rows.                         */
int32_t gq_sum_words(const void *words, int64_t n, int64_t d, int32_t code_bits, void *word_sum,
                     void *stream);

/* Dequantization of a summed row in the word layout, n = the number of
 * rows summed: mean[j] = fp32((field_j - n M) kappa), kappa = fp64(N / (n M)),
 * product in fp64 -- the same bits as gq_dequantize of the same sums.
 * W must satisfy the width rule for n.  mean: d floats, 16-byte aligned.  */
int32_t gq_dequantize_words(const void *word_sum, int64_t n, int64_t d, int32_t s, int32_t scheme,
                            int32_t code_bits, const float *norm_dev, float *mean, void *stream);

/* Fused quantize + exact integer sum + dequantize in one streaming pass,
 * given N in norm_dev[0]: equals gq_quantize, gq_reduce_codes and
 * gq_dequantize in sequence, without materializing the codes.  If
 * code_sum_or_null is not NULL it also receives the packed W-bit code sums
 * (then W must satisfy the width rule; otherwise code_bits is ignored).    */
int32_t gq_compress_mean_from_norm(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                                   int32_t scheme, uint64_t seed, const float *norm_dev,
                                   int32_t code_bits, float *mean, void *code_sum_or_null,
                                   void *stream);

/* The zero-code skip: the same results as gq_global_norm followed by
 * gq_compress_mean_from_norm, bit for bit, without reading most of x a
 * second time.  The fused pass stochastically rounds t = |x| / N (times s
 * for L) onto the levels of Sec. 3 ("Global-QSGD: Practical Floatless
 * Quantization ...", Global-L_s and Global-E_s); where t is below the first
 * non-zero level the code is 1 with probability F / 2^32 and 0 otherwise,
 * decided by the 16-bit uniform h (and the second draw on a tie).  With one
 * norm over a long concatenation most t are tiny, so most codes are 0, and
 * h alone proves it: a coordinate whose h exceeds a bound on its F >> 16
 * rounds to 0 whatever its exact value.
 *   gq_span_bounds_bytes(n, d) = 2 n stride, stride = 16 ceil(d / 8192):
 *     one 16-bit bound per (row, span of 512 coordinates), row-major with
 *     rows stride entries apart (-1 for invalid sizes).
 *   gq_global_norm_bounds: gq_global_norm (same N, same workspace rule),
 *     and in the same pass over x, bounds[i * stride + k] = the smallest
 *     bf16 bit pattern whose value is >= |x_ij| for every j of span k of row
 *     i (patterns 0x7F80 and above: an inf or NaN there), for every
 *     k < ceil(d / 512); the entries past them may be written too.
 *     bounds: device, 16-byte aligned, caller-owned.
 *   gq_compress_mean_skip: gq_compress_mean_from_norm (same arguments and
 *     results) given N in norm_dev[0] and those bounds for this x.  Per
 *     span and worker it derives a threshold H from the bound and N; a
 *     group of 8 coordinates whose eight 16-bit uniforms all exceed H adds
 *     nothing to the sums and is not loaded.  A span whose bound allows a
 *     non-zero lower level (t >= 1 for L, t >= 2^(1-s) for E), an inf or
 *     NaN, is read whole.  Bounds that do not belong to this x make the
 *     results wrong; they are not checked.
 * Errors as gq_global_norm and gq_compress_mean_from_norm, plus
 * GQ_ERR_NULL for a NULL bounds and GQ_ERR_ALIGN for one not 16-byte
 * aligned.                                                                 */
int64_t gq_span_bounds_bytes(int64_t n, int64_t d);
int32_t gq_global_norm_bounds(const void *x, int32_t dtype, int64_t n, int64_t d, float q,
                              float p, float *norm_dev, uint16_t *bounds, void *workspace,
                              int64_t workspace_bytes, void *stream);
int32_t gq_compress_mean_skip(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                              int32_t scheme, uint64_t seed, const float *norm_dev,
                              const uint16_t *bounds, int32_t code_bits, float *mean,
                              void *code_sum_or_null, void *stream);

/* The zero-code skip for sharded workers, where each device sums its own
 * rows into the word layout (Sec. 6's integer Allreduce over devices):
 *   gq_norm_term_bounds: gq_norm_term (same term, same workspace rule) and
 *     the span bounds of the device's n rows, as gq_global_norm_bounds
 *     writes them (row i of the shard is bounds row i).
 *   gq_compress_words_skip: gq_compress_words_from_norm (same arguments,
 *     same word row, bit for bit) given N in norm_dev[0] -- the global norm,
 *     from gq_norm_from_term of the combined terms -- and those bounds for
 *     this shard's x.  Groups are skipped as in gq_compress_mean_skip; the
 *     rows' worker indices worker_base + i enter the draws as there.
 * Errors as gq_norm_term and gq_compress_words_from_norm, plus GQ_ERR_NULL
 * for a NULL bounds (d > 0) and GQ_ERR_ALIGN for one not 16-byte aligned. */
int32_t gq_norm_term_bounds(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                            double *term_dev, uint16_t *bounds, void *workspace,
                            int64_t workspace_bytes, void *stream);
int32_t gq_compress_words_skip(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                               int32_t scheme, const float *norm_dev, const uint16_t *bounds,
                               uint64_t seed, int64_t worker_base, int32_t code_bits,
                               void *word_sum, void *stream);

/* The whole path: gq_global_norm, then gq_compress_mean_from_norm.
 * Writes N to norm_dev[0] and the dequantized mean to mean[0..d).  With a
 * workspace of gq_compress_workspace_bytes(n, d) it runs as
 * gq_global_norm_bounds then gq_compress_mean_skip, the bounds in the
 * workspace (same results, faster: provably zero codes are skipped).      */
int32_t gq_compress_mean(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s, float q,
                         float p, int32_t scheme, uint64_t seed, int32_t code_bits, float *mean,
                         float *norm_dev, void *code_sum_or_null, void *workspace,
                         int64_t workspace_bytes, void *stream);

/* The compress step as two kernels with the sums staged in between (many
 * workers; the fused pass itself, split where its only write would be).
 * Staging buffer `sums8`, gq_sums8_bytes(d) bytes, 16-byte aligned: first a
 * mask of one bit per group of 8 coordinates (group g is bit g % 64 of the
 * 64-bit word g / 64; the part is 8 ceil(d / 512) bytes rounded up to 16,
 * and that padding is never written), then d bytes (rounded up to 16) of
 * sums.
 * gq_compress_sums8, given N in norm_dev[0]: the exact code sum of every
 * coordinate over the n workers, as in gq_compress_mean_from_norm.  Every
 * mask word is written; bit g is 1 iff group g holds a non-zero sum (bits
 * past the last group are 0).  Only such a
 * group's 8 bytes are written, each sum as one signed byte when it lies in
 * [-127, 127] and as the escape byte -128 otherwise; the bytes of groups
 * whose sums are all zero are left as they were.
 * gq_dequantize_sums8, with the same x, n, s, scheme, seed and N: the mean,
 * mean[j] = fp32(sum_j kappa) as in gq_dequantize, reading the bytes of the
 * marked groups only.  A byte -128 makes it recompute that group's sums
 * from x (the same codes, so the same integers).  Together they give
 * gq_compress_mean_from_norm's mean bit for bit.                          */
int64_t gq_sums8_bytes(int64_t d);
int32_t gq_compress_sums8(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                          int32_t scheme, uint64_t seed, const float *norm_dev, void *sums8,
                          void *stream);
int32_t gq_dequantize_sums8(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                            int32_t scheme, uint64_t seed, const float *norm_dev,
                            const void *sums8, float *mean, void *stream);

/* gq_compress_mean without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * gq_compress_mean, bit for bit, except that the norm pass keeps its
 * partial sums (and, when gq_compress_workspace_bytes(n, d) fits too, the
 * span bounds of the zero-code skip) in a library-owned device array of
 * GQ_NOALLOC_SCRATCH_BYTES (64 MiB) instead of a workspace; every GPU the
 * library runs on holds its own copy of that array until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 *   - Size limit: inputs with gq_workspace_bytes(n, d) >
 *     GQ_NOALLOC_SCRATCH_BYTES are rejected with GQ_ERR_WORKSPACE before
 *     any HIP call (fp32 inputs up to about 128 GiB fit, and up to about
 *     44 GiB with the span bounds; the per-worker values cap n at about
 *     2 million).
 *   - Device: the array used is the current device's; a non-NULL stream
 *     must belong to the current device (GQ_ERR_ARG otherwise).  The first
 *     call on a device looks up its copy's address (hipGetSymbolAddress);
 *     a failure there returns GQ_ERR_DEVICE.
 *   - Concurrency: every call on one GPU shares that GPU's array.  Calls
 *     that may overlap on one GPU (different streams, or host threads
 *     without ordering) race on it and give undefined results; serialize
 *     them, or use gq_compress_mean with separate workspaces.  No value
 *     carries between calls: each call writes every scratch word it reads
 *     before reading it, so nothing needs clearing.                       */
#define GQ_NOALLOC_SCRATCH_BYTES (64LL << 20)
int32_t gq_compress_mean_noalloc(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                                 float q, float p, int32_t scheme, uint64_t seed,
                                 int32_t code_bits, float *mean, float *norm_dev,
                                 void *code_sum_or_null, void *stream);

/* Ablation: QSGD with LOCAL norms, the scheme Global-QSGD replaces (Sec. 3:
 * each worker normalizes by its own norm).  Worker i uses
 * N_i = fp32(sqrt(sum_j x_ij^2)) and the L_s rules above with N_i; codes
 * are in [-s, s] and are not summable across workers.
 * mean[j] = fp32(sum_i fp64(code_ij kappa_i)), kappa_i = fp64(N_i / (n s)),
 * accumulated in fp64 in worker order.  norms_dev: n floats.  If
 * codes_or_null is not NULL it receives the per-worker packed codes at
 * code_bits (gq_min_code_bits(1, s, GQ_SCHEME_L) <= W <= 32).  With a
 * workspace of gq_compress_workspace_bytes(n, d) it takes the zero-code
 * skip of gq_compress_mean_skip with each worker's own scale (a worker
 * whose kappa_i is not finite is read whole); the results are the same
 * bits.                                                                    */
int32_t gq_qsgd_local_mean(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                           uint64_t seed, float *mean, float *norms_dev, void *codes_or_null,
                           int32_t code_bits, void *workspace, int64_t workspace_bytes,
                           void *stream);

/* ---- The 8-bit exponential-dithering wire format (next to the path) ----
 * The pages' own format for exponential dithering ("Global-QSGD: Practical
 * Floatless Quantization ...", Sec. 4 worked example: 1 sign bit and 7
 * level bits; Sec. 6: custom reduction inside the tree Allreduce).
 * Code byte: bit 7 sign, bits 0..6 level index k; k = 0 is the level 0,
 * k >= 1 the level 2^(1-k) (levels 2^-m, m = 0..126: Global-E_s, s = 127).
 * Codes are not summable: a tree node is the average of its two children,
 * added in fp64 and rounded again at random, without bias, onto the same
 * grid (neighbours 2^e / 2^(e+1) with F = the top 32 fraction bits of the
 * fp64 value, or 0 / 2^-126 below 2^-126).  The draws of tree level l >= 1
 * at node m use Philox counter words (lo32(j/8), hi32(j/8), m, 2 l + draw);
 * level 0 is the quantization, with the layout given above.  Trees need n a
 * power of two up to 1024.  Code rows are gq_e8_row_bytes(d) bytes apart;
 * the pad bytes after the d codes of a row are never written.             */

/* 16 * ceil(d / 16), or -1 for d < 0.                                      */
int64_t gq_e8_row_bytes(int64_t d);

/* Quantize n rows to 8-bit codes given N in norm_dev[0] (Global-E_s with
 * s = 127: sigma = fp32(1 / (N pre)), t = min(fp32(|x| pre sigma), 1)).     */
int32_t gq_e8_quantize(const void *x, int32_t dtype, int64_t n, int64_t d, const float *norm_dev,
                       uint64_t seed, int64_t worker_base, void *codes, void *stream);

/* The custom reduction of one tree step: out = round((a + b) / 2) with the
 * draws of (level, node); level >= 1.                                      */
int32_t gq_e8_reduce_pair(const void *a, const void *b, int64_t d, uint64_t seed, int32_t level,
                          int64_t node, void *out, void *stream);

/* The whole tree over n rows of codes: level l combines nodes 2m and 2m+1
 * of level l-1 into node m; root: one row of d codes.                      */
int32_t gq_e8_tree(const void *codes, int64_t n, int64_t d, uint64_t seed, void *root,
                   void *stream);

/* The subtree over n rows of workers worker_base .. worker_base + n - 1
 * (worker_base a multiple of n): the tree's nodes there, drawn with their
 * node indices in the whole tree, so that a device holding an aligned block
 * of workers computes its subtree root and the levels above it
 * (gq_e8_reduce_pair with level log2(n) + 1 ... and the whole tree's node
 * index) reproduce gq_e8_tree over all workers bit for bit.  The codes must
 * come from gq_e8_quantize with the same worker_base.  gq_e8_tree is this
 * call with worker_base = 0.                                               */
int32_t gq_e8_subtree(const void *codes, int64_t n, int64_t d, uint64_t seed, int64_t worker_base,
                      void *root, void *stream);

/* mean[j] = fp32(N value(root[j])), product in fp64.                        */
int32_t gq_e8_dequantize(const void *root, int64_t d, const float *norm_dev, float *mean,
                         void *stream);

/* Norm, quantization, tree and dequantization in one call (the tree runs on
 * chip, in registers and LDS; no codes are written to memory);
 * root_or_null receives the root.                                          */
int32_t gq_e8_compress_mean(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                            uint64_t seed, float *mean, float *norm_dev, void *root_or_null,
                            void *workspace, int64_t workspace_bytes, void *stream);

/* Name of a status code (static string).                                  */
const char *gq_status_str(int32_t status);

/* Description of the last failed call on this thread ("" if none).        */
const char *gq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
