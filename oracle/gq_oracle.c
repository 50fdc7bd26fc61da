/*
 * gq_oracle.c -- CPU oracle for the Global-QSGD compression operator.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, scalar C
 * implementation of what the HIP library computes.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark load it; the
 * product library never does.  It shares no source, header, table or helper
 * with the HIP path (allreduce_compatible_gradient_amd/csrc).
 *
 * What it follows (all from "Global-QSGD: Practical Floatless Quantization
 * for Distributed Learning with Theoretical Guarantees", Xin, Canini,
 * Richtarik, Horvath):
 *   - Sec. 2 (notation): the l_p norm of one vector and the (q,p)-norm of the
 *     concatenation x = [x_1..x_n], outer sum over the n workers.
 *   - Sec. 3 (Global-Q definition, stripped from the page; taken in the
 *     QSGD / dithering form the section builds on): every coordinate is
 *     divided by ONE global norm, then rounded at random, without bias, to
 *     one of the two neighbouring levels.
 *   - Sec. 3 (the two level families): standard dithering Global-L_s with
 *     levels (s-i)/s, and exponential dithering Global-E_s with levels
 *     {0} and the powers of two 2^-k, k = 0..s-1.
 *   - Sec. 6 (implementation): quantize, integer Allreduce (here: an exact
 *     sum over the n simulated workers), dequantize once; the word layout
 *     whose plain 32-bit word sum adds the codes (a collective's own
 *     integer SUM) and the re-rounding tree of the 8-bit exponential format
 *     (Sec. 4 worked example, Sec. 5-6 custom reduction).
 * Philox4x32-10 follows Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3" (SC'11), Sec. on the Philox family.
 *
 * Readings where the pages leave a step open (all listed in the design
 * notes of the repository): scale sigma and dequant factor kappa formed in
 * fp64 and rounded once; fp32 per-element decisions; 32-bit threshold
 * F = floor(f * 2^32) compared with a 32-bit uniform u (round up iff u < F);
 * E-scheme codes are fixed-point integers (level 2^-k -> 2^(s-1-k));
 * norms below 2^-64 are handled by an exact 2^64 pre-scale.
 *
 * Build: gcc -std=c11 -O2 -fPIC -shared -ffp-contract=off gq_oracle.c -lm
 * (no -ffast-math: every float operation here is one IEEE-rounded step).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_SCHEME_L 0
#define ORACLE_SCHEME_E 1
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (SC'11).  Two 32x32->64 products per round on counter words
 * 0 and 2; the new state takes the high halves xor-ed with the other counter
 * words and the round key, and the low halves as they are.  The key is
 * advanced by the Weyl constants before every round after the first.       */

static void philox_round(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    uint32_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        philox_round(c, k0, k1);
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* The 32-bit uniform used for element j of worker `worker`.
 * Block b = j / 8 of a worker's row owns two Philox outputs:
 *   A = Philox(key = seed, ctr = (lo32(b), hi32(b), worker, 0))
 *   B = Philox(key = seed, ctr = (lo32(b), hi32(b), worker, 1))
 * Element e = j % 8 takes 16-bit half (e % 2) of word e / 2 of A as the high
 * half of u, and the same half of B as the low half.                       */
uint32_t oracle_uniform32(uint64_t seed, uint64_t worker, uint64_t j)
{
    uint64_t b = j / 8;
    unsigned e = (unsigned)(j % 8);
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t ca[4] = {(uint32_t)(b & 0xFFFFFFFFu), (uint32_t)(b >> 32), (uint32_t)worker, 0u};
    uint32_t cb[4] = {(uint32_t)(b & 0xFFFFFFFFu), (uint32_t)(b >> 32), (uint32_t)worker, 1u};
    uint32_t A[4], B[4];
    oracle_philox4x32_10(ca, key, A);
    oracle_philox4x32_10(cb, key, B);
    unsigned shift = 16u * (e % 2u);
    uint32_t hi16 = (A[e / 2] >> shift) & 0xFFFFu;
    uint32_t lo16 = (B[e / 2] >> shift) & 0xFFFFu;
    return (hi16 << 16) | lo16;
}

/* ------------------------------------------------------------------------ */
/* Inputs: row-major x[n][d], fp32 or bf16 (bf16 widened exactly).           */

static float load_x(const void *x, int dtype, uint64_t idx)
{
    if (dtype == ORACLE_F32)
        return ((const float *)x)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)x)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static uint32_t float_bits(float f)
{
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return b;
}

/* Compensated (Neumaier) running sum in fp64: the result is the exact sum
 * of the terms up to a couple of fp64 roundings, independent of length.   */
typedef struct { double s, c; } nsum;

static void nsum_add(nsum *a, double v)
{
    double t = a->s + v;
    if (fabs(a->s) >= fabs(v))
        a->c += (a->s - t) + v;
    else
        a->c += (v - t) + a->s;
    a->s = t;
}

/* ------------------------------------------------------------------------ */
/* (q,p)-norm of the concatenation, Sec. 2.  q selects the per-worker norm,
 * p the norm taken over the n per-worker norms; each is a real >= 1 or
 * +infinity (Sec. 2 allows (1, inf) and inf; 1 is admitted as well).
 * per_worker[i] receives max_j |x_ij| (q = inf) or sum_j |x_ij|^q (finite q;
 * for q = 2 every square is exact in fp64, other q use fp64 pow).
 * The four combinations of {2, inf} are formed without pow:
 *   (2,2) sqrt(sum_i S_i)   (2,inf) sqrt(max_i S_i)
 *   (inf,2) sqrt(sum_i m_i^2)   (inf,inf) max_i m_i
 * Any other pair: w_i = m_i, sqrt(S_i) (q = 2) or S_i^(1/q); then
 * N = max_i w_i (p = inf), sqrt(sum_i w_i^2) (p = 2) or (sum_i w_i^p)^(1/p).
 * N is that fp64 value rounded once to fp32.                               */

static int is_inf_order(float v) { return isinf(v) && v > 0; }

/* Combination over workers of the per-worker values. */
float oracle_norm_from_partials(const double *per_worker, int64_t n, float q, float p)
{
    int q_inf = is_inf_order(q), p_inf = is_inf_order(p);
    int q_two = (q == 2.0f), p_two = (p == 2.0f);
    if ((q_inf || q_two) && (p_inf || p_two)) {
        if (p_inf) {
            double m = 0.0;
            for (int64_t i = 0; i < n; ++i)
                if (per_worker[i] > m)
                    m = per_worker[i];
            return q_inf ? (float)m : (float)sqrt(m);
        }
        nsum tot = {0.0, 0.0};
        for (int64_t i = 0; i < n; ++i)
            nsum_add(&tot, q_inf ? per_worker[i] * per_worker[i] : per_worker[i]);
        return (float)sqrt(tot.s + tot.c);
    }
    /* general orders */
    double m = 0.0;
    nsum tot = {0.0, 0.0};
    for (int64_t i = 0; i < n; ++i) {
        double w = q_inf ? per_worker[i]
                         : (q_two ? sqrt(per_worker[i]) : pow(per_worker[i], 1.0 / (double)q));
        if (p_inf) {
            if (w > m)
                m = w;
        } else {
            nsum_add(&tot, p_two ? w * w : pow(w, (double)p));
        }
    }
    if (p_inf)
        return (float)m;
    double t = tot.s + tot.c;
    return (float)(p_two ? sqrt(t) : pow(t, 1.0 / (double)p));
}

float oracle_global_norm(const void *x, int dtype, int64_t n, int64_t d,
                         float q, float p, double *per_worker)
{
    int q_inf = is_inf_order(q);
    for (int64_t i = 0; i < n; ++i) {
        if (q_inf) {
            float m = 0.0f;
            for (int64_t j = 0; j < d; ++j) {
                float a = fabsf(load_x(x, dtype, (uint64_t)(i * d + j)));
                if (a > m)
                    m = a;
            }
            per_worker[i] = (double)m;
        } else {
            nsum acc = {0.0, 0.0};
            for (int64_t j = 0; j < d; ++j) {
                double v = (double)load_x(x, dtype, (uint64_t)(i * d + j));
                /* q = 2: exact, a 24-bit significand squared; else fp64 pow */
                nsum_add(&acc, q == 2.0f ? v * v : pow(fabs(v), (double)q));
            }
            per_worker[i] = acc.s + acc.c;
        }
    }
    return oracle_norm_from_partials(per_worker, n, q, p);
}

/* ------------------------------------------------------------------------ */
/* Scalars of one quantization: pre-scale, scale sigma, dequant factor kappa.
 *   M      = s (L) or 2^(s-1) (E): the integer code of the top level 1.
 *   pre    = 2^64 if N < 2^-64, else 1 (exact; keeps sigma finite).
 *   sigma  = fp32(s / (N*pre)) for L, fp32(1 / (N*pre)) for E, both in fp64.
 *   kappa  = fp64(N / (n*M)): the value of one code unit in the mean.       */

int64_t oracle_top_code(int s, int scheme)
{
    return scheme == ORACLE_SCHEME_L ? (int64_t)s : ((int64_t)1 << (s - 1));
}

void oracle_scale_params(float N, int64_t n, int s, int scheme,
                         float *pre, float *sigma, double *kappa)
{
    float pr = (N < 0x1p-64f) ? 0x1p64f : 1.0f;
    float Np = N * pr;
    double num = (scheme == ORACLE_SCHEME_L) ? (double)s : 1.0;
    *pre = pr;
    *sigma = (float)(num / (double)Np);
    *kappa = (double)N / ((double)n * (double)oracle_top_code(s, scheme));
}

/* The deterministic half of the rounding for one coordinate: the two integer
 * codes (magnitudes) that bracket |x|/N on the level grid and the 32-bit
 * threshold F.  The random half picks m_hi with probability F / 2^32.
 *   L: t = min(fp32(|x|*pre*sigma), s); m_lo = floor(t); m_hi = m_lo + 1;
 *      F = floor((t - floor(t)) * 2^32).
 *   E: r = min(fp32(|x|*pre*sigma), 1), c = 2^(1-s).
 *      r >= c, r = 2^e (1 + phi): m_lo = 2^(e+s-1), m_hi = 2 m_lo,
 *      F = phi * 2^32 (exact: the 23 fraction bits of r, shifted).
 *      r <  c: m_lo = 0, m_hi = 1, F = floor(r 2^(s-1) 2^32).
 * N == 0 gives m_lo = m_hi = 0, F = 0.                                    */
void oracle_bracket(float xv, float pre, float sigma, int zero_norm, int s, int scheme,
                    int32_t *m_lo, int32_t *m_hi, uint32_t *F)
{
    if (zero_norm) {
        *m_lo = 0; *m_hi = 0; *F = 0u;
        return;
    }
    float a = fabsf(xv);
    float t = (a * pre) * sigma;
    if (scheme == ORACLE_SCHEME_L) {
        float top = (float)s;
        if (!(t <= top)) /* clamp; a NaN also lands on the top level */
            t = top;
        float lo = floorf(t);
        float f = t - lo;
        *m_lo = (int32_t)lo;
        *m_hi = (int32_t)lo + 1;
        *F = (uint32_t)(f * 0x1p32f);
        return;
    }
    if (!(t <= 1.0f))
        t = 1.0f;
    float c = ldexpf(1.0f, 1 - s);
    if (t >= c) {
        uint32_t tb = float_bits(t);
        int e = (int)((tb >> 23) & 0xFFu) - 127;
        uint32_t mant = tb & 0x7FFFFFu;
        int32_t lo = (int32_t)1 << (e + s - 1);
        *m_lo = lo;
        *m_hi = (int32_t)(2u * (uint32_t)lo); /* unused when F == 0 (t = 1, s = 31) */
        *F = mant << 9;
    } else {
        float f = t * ldexpf(1.0f, s - 1);
        *m_lo = 0;
        *m_hi = 1;
        *F = (uint32_t)(f * 0x1p32f);
    }
}

/* One signed code: pick the upper magnitude iff u < F, then apply the sign
 * bit of x.                                                               */
int32_t oracle_code(float xv, float pre, float sigma, int zero_norm, int s, int scheme, uint32_t u)
{
    int32_t m_lo, m_hi;
    uint32_t F;
    oracle_bracket(xv, pre, sigma, zero_norm, s, scheme, &m_lo, &m_hi, &F);
    int32_t m = (u < F) ? m_hi : m_lo;
    return (float_bits(xv) >> 31) ? -m : m;
}

/* ------------------------------------------------------------------------ */
/* Quantize all n rows given the norm.  Row i is worker worker_base + i.    */
void oracle_quantize(const void *x, int dtype, int64_t n, int64_t d, float N,
                     int s, int scheme, uint64_t seed, int64_t worker_base, int32_t *codes)
{
    float pre, sigma;
    double kappa;
    oracle_scale_params(N, n, s, scheme, &pre, &sigma, &kappa);
    int zero = (N == 0.0f);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < d; ++j) {
            uint64_t g = (uint64_t)(i * d + j);
            uint32_t u = oracle_uniform32(seed, (uint64_t)(worker_base + i), (uint64_t)j);
            codes[g] = oracle_code(load_x(x, dtype, g), pre, sigma, zero, s, scheme, u);
        }
}

/* Smallest two's-complement width that holds every sum of n codes:
 * |sum| <= n*M needs ceil(log2(n*M + 1)) + 1 bits.                         */
int oracle_min_code_bits(int64_t n, int s, int scheme)
{
    int64_t nm = n * oracle_top_code(s, scheme);
    int bits = 0;
    while (((int64_t)1 << bits) < nm + 1)
        ++bits;
    return bits + 1;
}

/* Bytes of one packed row: d fields of W bits, padded to 16 bytes.         */
int64_t oracle_row_bytes(int64_t d, int W)
{
    int64_t bits = d * (int64_t)W;
    return ((bits + 127) / 128) * 16;
}

/* Little-endian bitstream: bit k of a row is bit k % 8 of byte k / 8;
 * element j occupies bits [j W, j W + W) in two's complement.             */
void oracle_pack(const int32_t *codes, int64_t n, int64_t d, int W, uint8_t *out)
{
    int64_t rb = oracle_row_bytes(d, W);
    memset(out, 0, (size_t)(n * rb));
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < d; ++j) {
            uint32_t field = (uint32_t)codes[i * d + j];
            for (int b = 0; b < W; ++b)
                if ((field >> b) & 1u) {
                    int64_t k = j * W + b;
                    out[i * rb + k / 8] |= (uint8_t)(1u << (k % 8));
                }
        }
}

void oracle_unpack(const uint8_t *in, int64_t n, int64_t d, int W, int32_t *codes)
{
    int64_t rb = oracle_row_bytes(d, W);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < d; ++j) {
            int64_t v = 0;
            for (int b = 0; b < W; ++b) {
                int64_t k = j * W + b;
                if ((in[i * rb + k / 8] >> (k % 8)) & 1u)
                    v |= (int64_t)1 << b;
            }
            if (v >> (W - 1)) /* sign bit set */
                v -= (int64_t)1 << W;
            codes[i * d + j] = (int32_t)v;
        }
}

/* Exact integer sum over workers, per coordinate.                          */
void oracle_sum_codes(const int32_t *codes, int64_t n, int64_t d, int64_t *sums)
{
    for (int64_t j = 0; j < d; ++j) {
        int64_t acc = 0;
        for (int64_t i = 0; i < n; ++i)
            acc += codes[i * d + j];
        sums[j] = acc;
    }
}

/* Dequantize once to the mean: mean_j = fp32(sum_j * kappa) (fp64 product). */
void oracle_dequantize(const int64_t *sums, int64_t n, int64_t d, float N, int s, int scheme,
                       float *mean)
{
    float pre, sigma;
    double kappa;
    oracle_scale_params(N, n, s, scheme, &pre, &sigma, &kappa);
    for (int64_t j = 0; j < d; ++j)
        mean[j] = (float)((double)sums[j] * kappa);
}

/* ------------------------------------------------------------------------ */
/* Word layout for a native integer all-reduce (Sec. 6: the codes are summed
 * by the collective's own integer SUM; a collective without a 16-bit integer
 * type still sums 32-bit words).  Field width W, f = floor(32 / W) fields per
 * 32-bit word: coordinate j sits in word j / f at bits [W (j % f),
 * W (j % f) + W) and holds its code plus M, a value in [0, 2M].  Bits above
 * the last field of a word, fields past d and the row's pad words are 0;
 * rows are padded to 16 bytes.  Summed over n rows, a field holds
 * sum_i code_ij + n M <= 2 n M, below 2^W whenever W is at least the
 * minimal width (2^(W-1) > n M), so the 32-bit sum of the words never
 * carries out of a field and never wraps.                                  */

int oracle_word_fields(int W) { return 32 / W; }

int64_t oracle_word_row_bytes(int64_t d, int W)
{
    int64_t f = 32 / W;
    int64_t words = (d + f - 1) / f;
    return ((words + 3) / 4) * 16;
}

void oracle_pack_words(const int32_t *codes, int64_t n, int64_t d, int W, int64_t M,
                       uint32_t *out)
{
    int64_t f = 32 / W, rw = oracle_word_row_bytes(d, W) / 4;
    memset(out, 0, (size_t)(n * rw) * sizeof(uint32_t));
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < d; ++j) {
            uint32_t biased = (uint32_t)((int64_t)codes[i * d + j] + M);
            out[i * rw + j / f] |= biased << (W * (int)(j % f));
        }
}

/* What the collective computes: the word-wise sum of n rows, modulo 2^32.  */
void oracle_sum_words(const uint32_t *rows, int64_t n, int64_t nwords, uint32_t *sum)
{
    for (int64_t w = 0; w < nwords; ++w) {
        uint32_t acc = 0;
        for (int64_t i = 0; i < n; ++i)
            acc += rows[i * nwords + w];
        sum[w] = acc;
    }
}

/* Field j of a summed row, minus the n biases: the exact code sum.         */
void oracle_unpack_word_sums(const uint32_t *sum, int64_t n, int64_t d, int W, int64_t M,
                             int64_t *sums)
{
    int64_t f = 32 / W;
    uint32_t mask = W == 32 ? 0xFFFFFFFFu : ((1u << W) - 1u);
    for (int64_t j = 0; j < d; ++j) {
        uint32_t field = (sum[j / f] >> (W * (int)(j % f))) & mask;
        sums[j] = (int64_t)field - n * M;
    }
}

/* Selected columns of the whole pipeline, given the norm: for each listed
 * coordinate j, the exact code sum over the n workers and the mean.        */
void oracle_compress_mean_cols(const void *x, int dtype, int64_t n, int64_t d, float N,
                               int s, int scheme, uint64_t seed,
                               const int64_t *cols, int64_t ncols, int64_t *sums, float *mean)
{
    float pre, sigma;
    double kappa;
    oracle_scale_params(N, n, s, scheme, &pre, &sigma, &kappa);
    int zero = (N == 0.0f);
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t j = cols[c];
        int64_t acc = 0;
        for (int64_t i = 0; i < n; ++i) {
            uint64_t g = (uint64_t)(i * d + j);
            uint32_t u = oracle_uniform32(seed, (uint64_t)i, (uint64_t)j);
            acc += oracle_code(load_x(x, dtype, g), pre, sigma, zero, s, scheme, u);
        }
        sums[c] = acc;
        mean[c] = (float)((double)acc * kappa);
    }
}

/* Whole pipeline: norm, codes, exact sum, one dequantization.              */
float oracle_compress_mean(const void *x, int dtype, int64_t n, int64_t d, int s,
                           float q, float p, int scheme, uint64_t seed,
                           int64_t *sums, float *mean)
{
    double *pw = (double *)malloc((size_t)n * sizeof(double));
    int64_t *cols = (int64_t *)malloc((size_t)d * sizeof(int64_t));
    if (!pw || !cols) {
        free(pw);
        free(cols);
        return NAN;
    }
    float N = oracle_global_norm(x, dtype, n, d, q, p, pw);
    for (int64_t j = 0; j < d; ++j)
        cols[j] = j;
    oracle_compress_mean_cols(x, dtype, n, d, N, s, scheme, seed, cols, d, sums, mean);
    free(pw);
    free(cols);
    return N;
}

/* ------------------------------------------------------------------------ */
/* Ablation: QSGD with LOCAL norms (the baseline Global-QSGD replaces).
 * Worker i scales by its own N_i = fp32(sqrt(sum_j x_ij^2)) and rounds to
 * the L_s levels with the same uniforms as above; codes are in [-s, s].
 * The mean is not an integer sum any more: mean_j = fp32(sum_i code_ij *
 * kappa_i) with kappa_i = fp64(N_i / (n s)), accumulated in fp64 in worker
 * order 0..n-1.                                                           */
void oracle_local_norms(const void *x, int dtype, int64_t n, int64_t d, float *norms)
{
    for (int64_t i = 0; i < n; ++i) {
        nsum acc = {0.0, 0.0};
        for (int64_t j = 0; j < d; ++j) {
            double v = (double)load_x(x, dtype, (uint64_t)(i * d + j));
            nsum_add(&acc, v * v);
        }
        norms[i] = (float)sqrt(acc.s + acc.c);
    }
}

/* Listed coordinates of the ablation, given the per-worker norms; codes_or_null
 * (n x ncols, row-major) receives the per-worker codes of those coordinates. */
void oracle_qsgd_local_cols(const void *x, int dtype, int64_t n, int64_t d, int s, uint64_t seed,
                            const float *norms, const int64_t *cols, int64_t ncols,
                            int32_t *codes_or_null, float *mean)
{
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t j = cols[c];
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            float pre, sigma;
            double kappa;
            oracle_scale_params(norms[i], 1, s, ORACLE_SCHEME_L, &pre, &sigma, &kappa);
            kappa = (double)norms[i] / ((double)n * (double)s);
            uint64_t g = (uint64_t)(i * d + j);
            uint32_t u = oracle_uniform32(seed, (uint64_t)i, (uint64_t)j);
            int32_t code = oracle_code(load_x(x, dtype, g), pre, sigma, norms[i] == 0.0f, s,
                                       ORACLE_SCHEME_L, u);
            if (codes_or_null)
                codes_or_null[i * ncols + c] = code;
            acc = acc + (double)code * kappa;
        }
        mean[c] = (float)acc;
    }
}

void oracle_qsgd_local_mean(const void *x, int dtype, int64_t n, int64_t d, int s, uint64_t seed,
                            float *norms, int32_t *codes_or_null, float *mean)
{
    int64_t *cols = (int64_t *)malloc((size_t)(d > 0 ? d : 1) * sizeof(int64_t));
    if (!cols)
        return;
    oracle_local_norms(x, dtype, n, d, norms);
    for (int64_t j = 0; j < d; ++j)
        cols[j] = j;
    /* with every column listed in order, the [n][ncols] codes are the [n][d] codes */
    oracle_qsgd_local_cols(x, dtype, n, d, s, seed, norms, cols, d, codes_or_null, mean);
    free(cols);
}

/* ------------------------------------------------------------------------ */
/* The pages' own wire format for exponential dithering (Sec. 4 worked
 * example, Sec. 6 custom reduction): 8-bit codes, bit 7 the sign, bits 0..6
 * a level index.  Index 0 is the level 0; index k in [1, 127] is the level
 * 2^(1-k), so the levels are {0} and 2^-m for m = 0..126 (s = 127).
 * A tree Allreduce combines two children into their average, rounded again
 * at random, without bias, onto the same grid ("extra variance due to
 * stochastic rounding during AllReduce").  Readings: the average (not the
 * sum) keeps every node inside [-1, 1]; the pair is added in fp64; n is a
 * power of two; the draws of tree level l >= 1, node m use Philox counter
 * words (lo32(j/8), hi32(j/8), m, 2 l + draw), so level 0 is the
 * quantization layout above.                                               */

/* Uniform of element j from counter words 2 and 3 = (c2, 2 c3pair + draw). */
uint32_t oracle_uniform32_ctr(uint64_t seed, uint32_t c2, uint32_t c3pair, uint64_t j)
{
    uint64_t b = j / 8;
    unsigned e = (unsigned)(j % 8);
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t ca[4] = {(uint32_t)(b & 0xFFFFFFFFu), (uint32_t)(b >> 32), c2, 2u * c3pair};
    uint32_t cb[4] = {(uint32_t)(b & 0xFFFFFFFFu), (uint32_t)(b >> 32), c2, 2u * c3pair + 1u};
    uint32_t A[4], B[4];
    oracle_philox4x32_10(ca, key, A);
    oracle_philox4x32_10(cb, key, B);
    unsigned shift = 16u * (e % 2u);
    return (((A[e / 2] >> shift) & 0xFFFFu) << 16) | ((B[e / 2] >> shift) & 0xFFFFu);
}

/* Value of a code in units of the global norm.                             */
double oracle_e8_value(uint8_t c)
{
    int idx = c & 0x7F;
    if (idx == 0)
        return 0.0;
    double v = ldexp(1.0, 1 - idx);
    return (c & 0x80) ? -v : v;
}

/* Round r = |v| <= 1 (fp64) at random onto the grid, sign from v: the upper
 * neighbour with probability F / 2^32.
 *   r >= 2^-126, r = 2^e (1 + phi): neighbours 2^e and 2^(e+1),
 *     F = floor(phi 2^32) (the top 32 of phi's 52 fraction bits);
 *   0 < r < 2^-126: neighbours 0 and 2^-126, F = floor(r 2^126 2^32).      */
uint8_t oracle_e8_round(double v, uint32_t u)
{
    double r = fabs(v);
    if (!(r <= 1.0))
        r = 1.0; /* clamp; NaN lands on the top level */
    if (r == 0.0)
        return 0;
    uint8_t sign = (v < 0.0) ? 0x80 : 0x00;
    if (r >= 0x1p-126) {
        int e;
        double m = frexp(r, &e); /* r = m 2^e, m in [0.5, 1) */
        e -= 1;                  /* r = 2^e (1 + phi), phi = 2 m - 1 */
        double phi = 2.0 * m - 1.0;
        uint32_t F = (uint32_t)(phi * 0x1p32);
        int up = u < F;
        int idx = 1 - (e + up); /* level 2^(e+up) */
        return (uint8_t)(sign | idx);
    }
    uint32_t F = (uint32_t)((r * 0x1p126) * 0x1p32);
    return (uint8_t)(u < F ? (sign | 127) : 0);
}

/* One 8-bit code of the quantization (Global-E_s, s = 127): t =
 * min(fp32(|x| pre sigma), 1) with sigma = fp32(1 / (N pre)), the random
 * rounding above, then the sign bit of x on a non-zero code.              */
static uint8_t e8_code(float xv, float N, float pre, float sigma, uint32_t u)
{
    if (N == 0.0f)
        return 0;
    float t = (fabsf(xv) * pre) * sigma;
    if (!(t <= 1.0f))
        t = 1.0f;
    uint8_t c = oracle_e8_round((double)t, u);
    if ((float_bits(xv) >> 31) && c)
        return (uint8_t)(c | 0x80);
    return (uint8_t)(c & 0x7F);
}

/* Quantize n rows to 8-bit codes given the norm, with the level-0 uniforms
 * of worker worker_base + i.                                               */
void oracle_e8_quantize(const void *x, int dtype, int64_t n, int64_t d, float N, uint64_t seed,
                        int64_t worker_base, uint8_t *codes)
{
    float pre, sigma;
    double kappa;
    oracle_scale_params(N, n, 127, ORACLE_SCHEME_E, &pre, &sigma, &kappa);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < d; ++j) {
            uint64_t g = (uint64_t)(i * d + j);
            uint32_t u = oracle_uniform32_ctr(seed, (uint32_t)(worker_base + i), 0, (uint64_t)j);
            codes[g] = e8_code(load_x(x, dtype, g), N, pre, sigma, u);
        }
}

/* The custom reduction of two code vectors at tree level `level`, node `node`. */
void oracle_e8_reduce_pair(const uint8_t *a, const uint8_t *b, int64_t d, uint64_t seed,
                           uint32_t level, uint32_t node, uint8_t *out)
{
    for (int64_t j = 0; j < d; ++j) {
        double v = 0.5 * (oracle_e8_value(a[j]) + oracle_e8_value(b[j]));
        out[j] = oracle_e8_round(v, oracle_uniform32_ctr(seed, node, level, (uint64_t)j));
    }
}

/* The whole tree over n = 2^L rows of codes (row-major [n][d]): level l
 * combines nodes 2m and 2m+1 of level l-1 into node m.  scratch: n*d bytes. */
int oracle_e8_tree(const uint8_t *codes, int64_t n, int64_t d, uint64_t seed, uint8_t *root,
                   uint8_t *scratch)
{
    if (n < 1 || (n & (n - 1)) != 0)
        return -1;
    memcpy(scratch, codes, (size_t)(n * d));
    int64_t nodes = n;
    for (uint32_t level = 1; nodes > 1; ++level) {
        for (int64_t m = 0; m < nodes / 2; ++m)
            oracle_e8_reduce_pair(scratch + (2 * m) * d, scratch + (2 * m + 1) * d, d, seed, level,
                                  (uint32_t)m, scratch + m * d);
        nodes /= 2;
    }
    memcpy(root, scratch, (size_t)d);
    return 0;
}

/* Dequantize the root: mean_j = fp32(N value_j) (fp64 product).            */
void oracle_e8_dequantize(const uint8_t *root, int64_t d, float N, float *mean)
{
    for (int64_t j = 0; j < d; ++j)
        mean[j] = (float)((double)N * oracle_e8_value(root[j]));
}

/* Listed coordinates of the whole 8-bit pipeline given the norm: for each
 * coordinate j, the n codes, the tree over them, the root and its mean.     */
void oracle_e8_compress_cols(const void *x, int dtype, int64_t n, int64_t d, float N,
                             uint64_t seed, const int64_t *cols, int64_t ncols, uint8_t *root,
                             float *mean)
{
    float pre, sigma;
    double kappa;
    oracle_scale_params(N, n, 127, ORACLE_SCHEME_E, &pre, &sigma, &kappa);
    uint8_t *node = (uint8_t *)malloc((size_t)n);
    if (!node)
        return;
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t j = cols[c];
        for (int64_t i = 0; i < n; ++i)
            node[i] = e8_code(load_x(x, dtype, (uint64_t)(i * d + j)), N, pre, sigma,
                              oracle_uniform32_ctr(seed, (uint32_t)i, 0, (uint64_t)j));
        int64_t nodes = n;
        for (uint32_t level = 1; nodes > 1; ++level) {
            for (int64_t m = 0; m < nodes / 2; ++m) {
                double v = 0.5 * (oracle_e8_value(node[2 * m]) + oracle_e8_value(node[2 * m + 1]));
                node[m] = oracle_e8_round(v, oracle_uniform32_ctr(seed, (uint32_t)m, level, (uint64_t)j));
            }
            nodes /= 2;
        }
        root[c] = node[0];
        mean[c] = (float)((double)N * oracle_e8_value(node[0]));
    }
    free(node);
}
