// gq.hip -- Global-QSGD compression on AMD Instinct MI355X (gfx950, CDNA4).
//
// Kernels and C ABI of libgq.so (declarations and the full contract are in
// include/gq.h).  The operator is Global-Q of "Global-QSGD: Practical
// Floatless Quantization for Distributed Learning with Theoretical
// Guarantees": one global (q,p)-norm over all workers (Sec. 2 notation),
// unbiased random rounding of |x|/N to the standard-dithering levels
// (s-i)/s or the exponential-dithering levels 2^-k (Sec. 3), integer codes
// whose sum over workers is exact, one dequantization (Sec. 6).
//
// Design (all bandwidth-bound work; nothing here is a dense contraction, so
// no MFMA):
//   k_norm_partial   pass 1: streams x once, fp64 sum of squares (or max|x|)
//                    per (worker, chunk) into a fixed slot -- no atomics, so
//                    the result bits depend only on (n, d).
//   k_norm_finalize  one 1024-thread block: every thread loads ~8 partials
//                    at once, fixed-order segmented tree per worker, then the
//                    (q,p) combination over workers, sqrt in fp64, one fp32
//                    rounding.
//   k_compress_mean  pass 2: each thread owns 8 consecutive coordinates (one
//                    Philox block) and walks the n workers, so the integer sum
//                    stays in registers; 128-bit loads, one Philox4x32-10 call
//                    per 8 coordinates (16 random bits each, a second call only
//                    when the first 16 bits tie the threshold, p ~ 2^-16), and
//                    the mean is written once.  One block per 2048-coordinate
//                    tile (short-lived blocks streaming 2 KB per wave read
//                    HBM faster than grid-stride loops on this part), tiles in
//                    reverse of pass 1's order.  For bf16 standard dithering
//                    with n s < 2^15 (vector-ALU bound), the rounding is one
//                    integer add per coordinate and pairs of coordinates are
//                    signed and summed in packed int16 lanes.
//   k_norm_oneshot / k_norm_mid: pass 1 for inputs above 256 MiB, 16 KB
//                    one-shot blocks, then a fixed-order middle reduction.
//   k_quantize / k_reduce_codes / k_dequantize: the same steps unfused, with
//                    W-bit codes packed through LDS into coalesced words.
//   k_quantize_words / k_compress_words / k_sum_words / k_dequantize_words:
//                    floor(32/W) biased fields per 32-bit word, the layout a
//                    native uint32 SUM all-reduce adds exactly (Sec. 6).
//   k_local_mean     ablation: per-worker norms (QSGD), fp64 mean.
//   k_e8_*           the pages' 8-bit exponential format (sign + 7-bit level
//                    index): quantization, the re-rounding pair step, the
//                    averaging tree as a binary counter with its stack in
//                    LDS, dequantization, and the fused norm-to-mean path.
//
// Sections below: constants and host-side geometry; device helpers (Philox,
// bracketing, loads, stores, packing); the norm kernels; the fused and
// unfused code kernels with the ablation; the word layout; the 8-bit format;
// launch helpers; the C ABI.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>
#include <type_traits>

#include "gq.h"

// Library-owned scratch of gq_compress_mean_noalloc: the norm pass's
// partial sums for callers that cannot allocate.  Each device holds its own
// copy; host code never uses this name as an address (in host code it is a
// stand-in, not device memory) -- the device address comes from
// hipGetSymbolAddress, once per device, below.
static __device__ __align__(256) uint8_t scratch[GQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kThreads = 256;               // 4 wave64 per block
constexpr int kPer = 8;                     // coordinates per thread: one Philox output block
constexpr int kTile = kThreads * kPer;      // 2048 coordinates per block
constexpr int64_t kNormTargetBlocks = 8192; // pass-1 blocks: ~32 per CU on 256 CUs
constexpr int64_t kMaxGrid = 0x7FFFFFFF;
constexpr int64_t kSums8MinN = 32;          // workers from which fp32 compress stages its sums

thread_local char g_err[512];

int32_t fail(int32_t status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

inline int32_t ok()
{
    g_err[0] = 0;
    return GQ_OK;
}

// ---------------------------------------------------------------------------
// Host-side sizes

// q and p: a real >= 1 or +inf ("Global-QSGD: Practical Floatless Quantization ...",
// Sec. 2 allows (1, inf) and inf; 1 is admitted as well)
inline bool order_ok(float v) { return v >= 1.0f; }

inline bool is_two(float v) { return v == 2.0f; }
inline bool is_inf_order(float v) { return isinf(v) && v > 0.0f; }

inline int64_t top_code(int32_t s, int32_t scheme)
{
    return scheme == GQ_SCHEME_L ? (int64_t)s : ((int64_t)1 << (s - 1));
}

inline bool s_ok(int32_t s, int32_t scheme)
{
    if (scheme == GQ_SCHEME_L)
        return s >= 1 && s <= (1 << 24);
    if (scheme == GQ_SCHEME_E)
        return s >= 1 && s <= 31;
    return false;
}

int32_t min_bits(int64_t n, int32_t s, int32_t scheme)
{
    if (n < 1 || n > ((int64_t)1 << 40) || !s_ok(s, scheme))
        return -1;
    const int64_t nm = n * top_code(s, scheme); // < 2^71 is impossible here: n < 2^40, M <= 2^30
    int bits = 0;
    while (bits < 62 && ((int64_t)1 << bits) < nm + 1)
        ++bits;
    return bits + 1;
}

__host__ __device__ inline int64_t row_bytes(int64_t d, int32_t W) { return ((d * W + 127) / 128) * 16; }

// Staged 1-byte sums (the many-worker compress step): a mask with one bit
// per 8-coordinate group (64-bit words, one per 64 groups: one per wave of
// the pass), then one byte per coordinate, each part 16-byte aligned.
__host__ __device__ inline int64_t sums8_mask_bytes(int64_t d) { return ((d + 511) / 512 * 8 + 15) / 16 * 16; }
__host__ __device__ inline int64_t sums8_bytes(int64_t d) { return sums8_mask_bytes(d) + (d + 15) / 16 * 16; }

// Bounds of |x| that let the fused pass skip coordinates whose code is
// provably 0: one 16-bit bound per (row, 512-coordinate span), the span one
// wave of the fused pass covers; written by pass 1, row-major.
constexpr int kSpan = 512;
__host__ __device__ inline int64_t bound_spans(int64_t d) { return (d + kSpan - 1) / kSpan; }
// Entries per row: the spans rounded up to 16, so that a one-shot pass-1
// block's 8 (fp32) or 16 (bf16) bounds are one aligned 16- or 32-byte store.
__host__ __device__ inline int64_t bound_stride(int64_t d) { return (bound_spans(d) + 15) / 16 * 16; }

inline int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Pass-1 geometry: each row is cut into `chunks` ranges of `chunk_len`
// coordinates (a multiple of the 2048-coordinate tile); one block per
// (chunk, worker).  It and the one-shot geometry below depend on (n, d) and
// the input type only, so the partial-sum tree -- and the norm's bits --
// are the same on every call.
struct NormGeom {
    int64_t chunks, chunk_len, blocks;
};
NormGeom norm_geom(int64_t n, int64_t d)
{
    NormGeom g{0, kTile, 0};
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return g;
    int64_t want = (kNormTargetBlocks + n - 1) / n;
    if (want < 1)
        want = 1;
    if (want > tiles)
        want = tiles;
    const int64_t tiles_per_chunk = (tiles + want - 1) / want;
    g.chunk_len = tiles_per_chunk * kTile;
    g.chunks = (d + g.chunk_len - 1) / g.chunk_len;
    g.blocks = g.chunks * n;
    return g;
}

// Pass 1 for inputs above 256 MiB: one-shot blocks of 512 threads reading
// 16 KB of one row each (row-major block order, one partial per block), then
// a middle kernel that reduces every 2048 consecutive partials of a row in a
// fixed order.  Measured on the 7 and 16 GB fp32 inputs: the whole operation
// -2.5%; with the wave sums by DPP moves, on the 5.7 GB bf16 input the pass
// 978 -> 920 us (whole operation -4.5%) and on the 0.8 GB fp32 input
// 146 -> 134 us (whole operation -2%).  Smaller inputs keep the chunk-major
// blocks: fewer, longer-lived blocks and no middle launch.
constexpr int kOsThreads = 512;
constexpr int64_t kOsBlockBytes = 16 * 1024;
constexpr double kOsMinBytes = 268435456.0;
constexpr int kMidThreads = 256;
constexpr int64_t kMidPer = 8 * kMidThreads; // partials per middle block

struct OneShotGeom {
    bool on;
    int64_t span, bpr, gpr; // elements per block, blocks and middle blocks per row
};
OneShotGeom oneshot_geom(int64_t n, int64_t d, int64_t elem_bytes)
{
    OneShotGeom o{false, kOsBlockBytes / elem_bytes, 0, 0};
    if ((double)n * (double)d * (double)elem_bytes <= kOsMinBytes)
        return o;
    o.on = true;
    o.bpr = (d + o.span - 1) / o.span;
    o.gpr = (o.bpr + kMidPer - 1) / kMidPer;
    return o;
}

struct WsLayout {
    int64_t partials, mid, per_worker, params, total;
    // gq_compress_mean's optional span bounds (u16 [n][bound_stride(d)])
    int64_t bounds, total_compress;
};

// The layout covers the pass-1 geometry of either input type.
WsLayout ws_layout(int64_t n, int64_t d)
{
    const NormGeom g = norm_geom(n, d);
    const OneShotGeom o = oneshot_geom(n, d, 4);
    int64_t part = 8 * n * g.chunks, mid = 0;
    if (o.on) {
        if (8 * n * o.bpr > part)
            part = 8 * n * o.bpr;
        mid = 8 * n * o.gpr;
    }
    WsLayout w;
    w.partials = 0;
    w.mid = align256(part);
    w.per_worker = w.mid + align256(mid);
    w.params = w.per_worker + align256(8 * n);
    w.total = w.params + align256(16 * n);
    w.bounds = w.total;
    w.total_compress = d > 0 ? w.total + align256(2 * n * bound_stride(d)) : w.total;
    return w;
}

// ---------------------------------------------------------------------------
// Device helpers

struct WorkerParams { // per-worker scalars of the local-norm ablation
    float pre, sigma;
    double kappa;
};

struct QParams {
    float pre;   // 2^64 when N < 2^-64, else 1 (exact pre-scale of |x|)
    float sigma; // fp32(s / (N pre)) for L, fp32(1 / (N pre)) for E
    float top;   // clamp of t: s (L) or 1 (E)
    float cE;    // 2^(1-s): the smallest non-zero E level
    float p2E;   // 2^(s+31): maps t < 2^(1-s) to the threshold scale
    float twoE;  // 2^(s-1): integer code of the level 1
    float p2E16; // 2^(s+15): t 2^(s+15) = F 2^-16 for t < 2^(1-s)
    uint32_t eoff; // (s-1) << 23: adds s-1 to an fp32 exponent field
    double kappa;
    int s;
    bool zero;
    bool prescale;
};

__device__ __forceinline__ QParams make_qparams(float N, int64_t n, int s, int scheme)
{
    QParams q;
    q.zero = (N == 0.0f);
    q.prescale = (N < 0x1p-64f);
    q.pre = q.prescale ? 0x1p64f : 1.0f;
    const float Np = N * q.pre;
    q.sigma = (float)((scheme == GQ_SCHEME_L ? (double)s : 1.0) / (double)Np);
    q.top = (scheme == GQ_SCHEME_L) ? (float)s : 1.0f;
    q.cE = __uint_as_float((uint32_t)(128 - s) << 23);
    q.p2E = __uint_as_float((uint32_t)(158 + s) << 23);
    q.twoE = __uint_as_float((uint32_t)(126 + s) << 23);
    q.p2E16 = __uint_as_float((uint32_t)(142 + s) << 23);
    q.eoff = (uint32_t)(s - 1) << 23;
    const double M = (scheme == GQ_SCHEME_L) ? (double)s : ldexp(1.0, s - 1);
    q.kappa = (double)N / ((double)n * M);
    q.s = s;
    return q;
}

// Philox4x32-10 (SC'11): per round, two 32x32->64 products of counter words
// 0 and 2 by the Philox multipliers; high halves are xor-ed with counter
// words 1 / 3 and the round key, low halves move over; the key advances by
// the Weyl constants.  The key (the seed) is wave-uniform and lives in SGPRs.
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)c.x * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c.z * 0xCD9E8D57u;
        // v_bitop3_b32 with truth table 0x96 is a three-input xor
        c = make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96),
                       (uint32_t)p1,
                       __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96),
                       (uint32_t)p0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

__device__ __forceinline__ uint32_t half16(const uint4 &w, int k)
{
    const uint32_t word = (k >> 1) == 0 ? w.x : (k >> 1) == 1 ? w.y : (k >> 1) == 2 ? w.z : w.w;
    return (k & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// Single instructions the compiler does not form by itself here (it goes
// through extra masks, shifts and perms).  Each SDWA or 16-bit form is
// preceded by one wait state, so no VALU-to-SDWA or 16-bit operand
// forwarding hazard has to be known to the compiler's hazard recognizer.
//   add_half16<H>(a, w) = a + (16-bit half H of w)
//   max3_lo16(a, b, c)  = max of the low halves, in the low half (high half unused)
//   cvt_u32_sat(f)      = v_cvt_u32_f32: truncation, saturating outside [0, 2^32)
//                         (a C conversion of an out-of-range value is undefined)
template <int H>
__device__ __forceinline__ uint32_t add_half16(uint32_t a, uint32_t w)
{
    uint32_t r;
    if (H == 0)
        asm("s_nop 0\n\tv_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD "
            "src0_sel:WORD_0 src1_sel:DWORD" : "=v"(r) : "v"(w), "v"(a));
    else
        asm("s_nop 0\n\tv_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD "
            "src0_sel:WORD_1 src1_sel:DWORD" : "=v"(r) : "v"(w), "v"(a));
    return r;
}

__device__ __forceinline__ uint32_t max3_lo16(uint32_t a, uint32_t b, uint32_t c)
{
    uint32_t r;
    asm("s_nop 0\n\tv_max3_u16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ uint32_t cvt_u32_sat(float f)
{
    uint32_t r;
    asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(f));
    return r;
}

// Deterministic half of the rounding for one coordinate, in fp32 exactly as
// the contract states: the lower candidate magnitude lo (an integer held
// exactly in a float), the step to the upper one, and the 32-bit threshold
// F (upper iff u < F).  Returns F >> 16 through Fh; F itself is only formed
// on the rare path that needs its low half.
template <int SCH, bool PRE>
__device__ __forceinline__ void bracket(float v, const QParams &q, float &lo, float &step,
                                        uint32_t &Fh, uint32_t *F_full)
{
    float a = fabsf(v);
    if (PRE)
        a = a * q.pre;
    if (SCH == GQ_SCHEME_L) {
        const float t = fminf(a * q.sigma, q.top); // v_min: a NaN lands on the top level
        lo = floorf(t);
        const float f = t - lo; // exact
        step = 1.0f;
        Fh = (uint32_t)(f * 0x1p16f); // floor(f 2^16) = F >> 16
        if (F_full)
            *F_full = (uint32_t)(f * 0x1p32f);
    } else {
        // Both cases are formed and one is selected (no divergent branch):
        //   t >= 2^(1-s), t = 2^e (1 + phi): lower level 2^e -> code 2^(e+s-1),
        //     step to 2^(e+1) equal to it, F = phi 2^32 (the fraction bits);
        //   t <  2^(1-s): codes 0 or 1, F = floor(t 2^(s-1) 2^32).
        const float t = fminf(a * q.sigma, 1.0f);
        const uint32_t tb = __float_as_uint(t);
        const bool big = t >= q.cE;
        const float lo_big = __uint_as_float(tb & 0xFF800000u) * q.twoE;
        const float y = t * q.p2E; // exact; < 2^32 when t < 2^(1-s)
        lo = big ? lo_big : 0.0f;
        step = big ? lo_big : 1.0f;
        Fh = big ? ((tb >> 7) & 0xFFFFu) : (uint32_t)(y * 0x1p-16f);
        if (F_full)
            *F_full = big ? (tb << 9) : (uint32_t)y;
    }
}

// Exponential dithering in carry form: the same magnitudes and ties as
// bracket() with the comparison in quant_group.  Every coordinate first takes
// the bracket below 2^(1-s), where F >> 16 = (uint)(t 2^(s+15)) < 2^16 and
// Z = (F >> 16) + (0xFFFF - h) carries into bit 16 iff h < F >> 16: byte 2
// of Z is the code, 0 or 1.  For t >= 2^(1-s), t = 2^e (1 + phi), F >> 16
// is bits 7..22 of t's fp32 pattern; adding (0xFFFF - h) << 7 carries into
// the exponent iff h < F >> 16, and with s - 1 added to the exponent and the
// fraction cleared the pattern is the code 2^(e+s-1) or 2^(e+s) as an fp32.
// That step runs only in waves holding such a coordinate.  A tie
// (h == F >> 16) leaves the 16 bits below the carry all ones; the group flag
// is raised when any coordinate's sum in either bracket shows this (a
// superset: settle_ties re-derives each coordinate's own bracket).
template <bool PRE>
__device__ __forceinline__ void quant_group_e(const float (&v)[kPer], const uint4 &A,
                                              const QParams &q, float (&m)[kPer], bool &tie)
{
    const uint32_t hx[kPer / 2] = {~A.x, ~A.y, ~A.z, ~A.w}; // 0xFFFF - h, two per word
    float t[kPer];
    uint32_t Z[kPer];
    bool big = false;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        float a = fabsf(v[k]);
        if (PRE)
            a = a * q.pre;
        t[k] = fminf(a * q.sigma, 1.0f); // v_min: a NaN lands on the top level
        const uint32_t Fs = cvt_u32_sat(t[k] * q.p2E16);
        Z[k] = (k & 1) ? add_half16<1>(Fs, hx[k >> 1]) : add_half16<0>(Fs, hx[k >> 1]);
        m[k] = (float)((Z[k] >> 16) & 0xFFu);
        big |= t[k] >= q.cE;
    }
    const uint32_t mx = max3_lo16(Z[6], Z[7], max3_lo16(Z[0], Z[1], Z[2]));
    tie |= ((uint16_t)mx == 0xFFFFu) | ((uint16_t)max3_lo16(Z[3], Z[4], Z[5]) == 0xFFFFu);
    if (big) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const uint32_t h7 = ((k & 1) ? (hx[k >> 1] >> 16) : (hx[k >> 1] & 0xFFFFu)) << 7;
            const uint32_t tc = __float_as_uint(t[k]) + h7 + q.eoff;
            if (t[k] >= q.cE) {
                m[k] = __uint_as_float(tc & 0xFF800000u);
                tie |= (tc & 0x7FFF80u) == 0x7FFF80u;
            }
        }
    }
}

// Magnitudes of one 8-coordinate group from draw 0: the high 16 bits h of
// each uniform decide unless h == F >> 16; such coordinates keep the lower
// level here and `tie` is raised for the rare second draw.  ECARRY selects
// quant_group_e for exponential dithering: 35% fewer VALU instructions,
// 5% faster quantization to 13-bit codes of a 16 x 110M fp32 input; in the
// memory-bound fused pass the select form below measured 2% faster.
template <int SCH, bool PRE, bool ECARRY = true>
__device__ __forceinline__ void quant_group(const float (&v)[kPer], const uint4 &A, const QParams &q,
                                            float (&m)[kPer], bool &tie)
{
    if constexpr (SCH == GQ_SCHEME_E && ECARRY) {
        quant_group_e<PRE>(v, A, q, m, tie);
        return;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        float lo, step;
        uint32_t Fh;
        bracket<SCH, PRE>(v[k], q, lo, step, Fh, nullptr);
        const uint32_t h = half16(A, k);
        m[k] = (h < Fh) ? lo + step : lo;
        tie |= (h == Fh);
    }
}

// The rare path: for each coordinate whose 16 bits tied, draw 1 supplies the
// low 16 bits of its uniform; adds the step to the magnitude when the full
// 32-bit uniform is below F.
template <int SCH, bool PRE>
__device__ __forceinline__ void settle_ties(const float (&v)[kPer], const uint4 &A, const uint4 &B,
                                            const QParams &q, float (&m)[kPer])
{
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        float lo, step;
        uint32_t Fh, F;
        bracket<SCH, PRE>(v[k], q, lo, step, Fh, &F);
        if ((half16(A, k) == Fh) && (half16(B, k) < (F & 0xFFFFu)))
            m[k] += step;
    }
}

// 8 consecutive inputs widened to fp32.  Fast path: the group lies inside
// the row and the row starts 16-byte aligned (d % 8 == 0): 128-bit loads.
template <int DT>
__device__ __forceinline__ void load_group(const void *__restrict__ x, int64_t row_off, int64_t j0,
                                           int64_t d, bool vec, float (&v)[kPer])
{
    if (DT == GQ_IN_F32) {
        const float *p = (const float *)x + row_off + j0;
        if (vec) {
            const float4 a = *(const float4 *)p;
            const float4 b = *(const float4 *)(p + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                v[k] = (j0 + k < d) ? p[k] : 0.0f;
        }
    } else {
        const uint16_t *p = (const uint16_t *)x + row_off + j0;
        if (vec) {
            const uint4 r = *(const uint4 *)p;
            v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xFFFF0000u);
            v[2] = __uint_as_float(r.y << 16); v[3] = __uint_as_float(r.y & 0xFFFF0000u);
            v[4] = __uint_as_float(r.z << 16); v[5] = __uint_as_float(r.z & 0xFFFF0000u);
            v[6] = __uint_as_float(r.w << 16); v[7] = __uint_as_float(r.w & 0xFFFF0000u);
        } else {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                v[k] = (j0 + k < d) ? __uint_as_float((uint32_t)p[k] << 16) : 0.0f;
        }
    }
}

// Results are written once and never re-read by these kernels.  Where a
// write stream interleaves with a heavier read stream (the fused, reduce and
// ablation passes, quantization to codes of up to 16 bits), non-temporal
// 128-bit stores are faster (measured: the fused pass 4.5% on an
// 8 x 25.6M input, neutral on larger ones; quantization of fp32 input to
// 16-bit codes 4%; non-temporal loads do worse).  Where writes dominate
// (dequantization; quantization to 32-bit codes, 31% faster for fp32 input)
// plain stores are faster.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void nt_store(float *p, float a, float b, float c, float d)
{
    const f32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, (f32x4 *)p);
}

__device__ __forceinline__ void nt_store(uint8_t *p, const uint4 &w)
{
    const u32x4 v = {w.x, w.y, w.z, w.w};
    __builtin_nontemporal_store(v, (u32x4 *)p);
}

__device__ __forceinline__ void nt_store(uint8_t *p, const uint2 &w)
{
    const u32x2 v = {w.x, w.y};
    __builtin_nontemporal_store(v, (u32x2 *)p);
}

// 8 consecutive floats of the mean: two 128-bit stores when the group lies
// inside an aligned row (d % 8 == 0), else per-element stores up to d.
template <bool NT = true>
__device__ __forceinline__ void store_mean8(float *__restrict__ mean, int64_t j0, int64_t d,
                                            const float (&m)[kPer])
{
    if ((d & 7) == 0) {
        if (NT) {
            nt_store(mean + j0, m[0], m[1], m[2], m[3]);
            nt_store(mean + j0 + 4, m[4], m[5], m[6], m[7]);
        } else {
            *(float4 *)(mean + j0) = make_float4(m[0], m[1], m[2], m[3]);
            *(float4 *)(mean + j0 + 4) = make_float4(m[4], m[5], m[6], m[7]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if (j0 + k < d)
                mean[j0 + k] = m[k];
    }
}

// Orders one wave's LDS accesses before and after a phase of the wave-level
// packing (a wave's LDS operations execute in order; this keeps the
// compiler from moving them across the phase boundary).
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Store 8 W-bit fields per thread (thread-major: coordinate tile*2048 +
// 8*t + k) into one packed row.  W = 8/16/32: direct vector stores.  Other
// W: each wave assembles its whole words in LDS and writes them with 16-byte
// stores.  Every thread of the block must call this.  Bytes past the row's
// end are never written; pad fields are zero.  wave_lds, if given, is this
// wave's own region of at least 16 W words (else lds + wave 16 W).
template <bool NT = true>
__device__ __forceinline__ void store_tile_packed(uint32_t *lds, const int (&val)[kPer], int W, uint8_t *row,
                                  int64_t tile, int64_t rbytes, uint32_t *wave_lds = nullptr)
{
    const int t = threadIdx.x;
    const int64_t j0 = tile * kTile + (int64_t)t * kPer;
    if (W == 8) {
        const int64_t off = j0;
        if (off < rbytes) {
            uint2 o;
            o.x = (val[0] & 0xFF) | (val[1] & 0xFF) << 8 | (val[2] & 0xFF) << 16 | (uint32_t)val[3] << 24;
            o.y = (val[4] & 0xFF) | (val[5] & 0xFF) << 8 | (val[6] & 0xFF) << 16 | (uint32_t)val[7] << 24;
            if (NT)
                nt_store(row + off, o);
            else
                *(decltype(o) *)(row + off) = o;
        }
        return;
    }
    if (W == 16) {
        const int64_t off = 2 * j0;
        if (off < rbytes) {
            uint4 o;
            o.x = (val[0] & 0xFFFF) | (uint32_t)val[1] << 16;
            o.y = (val[2] & 0xFFFF) | (uint32_t)val[3] << 16;
            o.z = (val[4] & 0xFFFF) | (uint32_t)val[5] << 16;
            o.w = (val[6] & 0xFFFF) | (uint32_t)val[7] << 16;
            if (NT)
                nt_store(row + off, o);
            else
                *(decltype(o) *)(row + off) = o;
        }
        return;
    }
    if (W == 32) {
        const int64_t off = 4 * j0;
        const uint4 lo = make_uint4(val[0], val[1], val[2], val[3]);
        const uint4 hi = make_uint4(val[4], val[5], val[6], val[7]);
        if (NT) {
            if (off < rbytes)
                nt_store(row + off, lo);
            if (off + 16 < rbytes)
                nt_store(row + off + 16, hi);
        } else {
            if (off < rbytes)
                *(uint4 *)(row + off) = lo;
            if (off + 16 < rbytes)
                *(uint4 *)(row + off + 16) = hi;
        }
        return;
    }
    // Other widths, one wave at a time (no block barrier): wave v holds the
    // tile's coordinates [512 v, 512 v + 512), whose bits [512 v W,
    // 512 (v + 1) W) are 16 W whole words.  The wave clears its own LDS
    // region of 16 W words, ORs every field into place (LDS atomics; a field
    // may straddle two words), then writes the region out as 16-byte stores.
    const int lane = t & 63, wave = t >> 6;
    const int nw = 16 * W;
    uint32_t *wl = wave_lds ? wave_lds : lds + wave * nw;
    for (int j = lane; j < nw; j += 64)
        wl[j] = 0u;
    wave_lds_fence();
    const uint32_t mask = (1u << W) - 1u;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int bit = (lane * kPer + k) * W;
        const int wi = bit >> 5, sh = bit & 31;
        const uint32_t f = (uint32_t)val[k] & mask;
        atomicOr(&wl[wi], f << sh);
        if (sh + W > 32)
            atomicOr(&wl[wi + 1], f >> (32 - sh));
    }
    wave_lds_fence();
    const int64_t wbase = tile * 64 * W + (int64_t)wave * nw; // first word of the region
    for (int u = lane; u < 4 * W; u += 64) {
        const int64_t off = (wbase + 4 * u) * 4;
        if (off < rbytes) {
            const uint4 o = ((const uint4 *)wl)[u];
            if (NT)
                nt_store(row + off, o);
            else
                *(uint4 *)(row + off) = o;
        }
    }
    wave_lds_fence();
}

// Lane `lane`'s 8 sign-extended W-bit fields from a wave's staged region of
// nw words (the lane's fields start at bit 8 lane W).
__device__ __forceinline__ void extract_fields_wave(const uint32_t *wl, int nw, int W, int lane,
                                                    int (&val)[kPer])
{
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int bit = (lane * kPer + k) * W;
        const int wi = bit >> 5, sh = bit & 31;
        const uint64_t two = (uint64_t)wl[wi] | ((uint64_t)(wi + 1 < nw ? wl[wi + 1] : 0u) << 32);
        const uint32_t f = (uint32_t)(two >> sh);
        val[k] = (int)(f << (32 - W)) >> (32 - W);
    }
}

// Inverse of store_tile_packed: 8 sign-extended fields per thread.  Fields
// past the row's end read as 0.  Every thread of the block must call this;
// the LDS staging is per wave, so no block barrier is taken.
__device__ __forceinline__ void load_tile_fields(uint32_t *lds, const uint8_t *row, int W, int64_t tile,
                                 int64_t rbytes, int (&val)[kPer])
{
    const int t = threadIdx.x;
    const int64_t j0 = tile * kTile + (int64_t)t * kPer;
    if (W == 8) {
        uint2 r = make_uint2(0, 0);
        if (j0 < rbytes)
            r = *(const uint2 *)(row + j0);
        val[0] = (int8_t)(r.x); val[1] = (int8_t)(r.x >> 8);
        val[2] = (int8_t)(r.x >> 16); val[3] = (int8_t)(r.x >> 24);
        val[4] = (int8_t)(r.y); val[5] = (int8_t)(r.y >> 8);
        val[6] = (int8_t)(r.y >> 16); val[7] = (int8_t)(r.y >> 24);
        return;
    }
    if (W == 16) {
        uint4 r = make_uint4(0, 0, 0, 0);
        if (2 * j0 < rbytes)
            r = *(const uint4 *)(row + 2 * j0);
        val[0] = (int16_t)(r.x); val[1] = (int16_t)(r.x >> 16);
        val[2] = (int16_t)(r.y); val[3] = (int16_t)(r.y >> 16);
        val[4] = (int16_t)(r.z); val[5] = (int16_t)(r.z >> 16);
        val[6] = (int16_t)(r.w); val[7] = (int16_t)(r.w >> 16);
        return;
    }
    if (W == 32) {
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (4 * j0 < rbytes)
            a = *(const uint4 *)(row + 4 * j0);
        if (4 * j0 + 16 < rbytes)
            b = *(const uint4 *)(row + 4 * j0 + 16);
        val[0] = (int)a.x; val[1] = (int)a.y; val[2] = (int)a.z; val[3] = (int)a.w;
        val[4] = (int)b.x; val[5] = (int)b.y; val[6] = (int)b.z; val[7] = (int)b.w;
        return;
    }
    // Other widths, one wave at a time (no block barrier): the wave loads
    // its 16 W words (see store_tile_packed) with 16-byte loads into its own
    // LDS region, then every lane extracts its 8 fields from a 64-bit window.
    const int lane = t & 63, wave = t >> 6;
    const int nw = 16 * W;
    uint32_t *wl = lds + wave * nw;
    const int64_t wbase = tile * 64 * W + (int64_t)wave * nw;
    for (int u = lane; u < 4 * W; u += 64) {
        const int64_t off = (wbase + 4 * u) * 4;
        ((uint4 *)wl)[u] = off < rbytes ? *(const uint4 *)(row + off) : make_uint4(0u, 0u, 0u, 0u);
    }
    wave_lds_fence();
    extract_fields_wave(wl, nw, W, lane, val);
    wave_lds_fence();
}

// One DPP move of a double (both halves, the same pattern; every source lane
// of the patterns used here lies in the same row of 16).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the wave (every lane active), in a fixed order: within each row
// of 16 lanes the partners lane ^ 1, lane ^ 2, the mirrored 8-lane half and
// the mirrored row (each lane adds the same two values, so every lane of a
// row ends with the row's sum), then the four rows read from lanes 0, 16, 32
// and 48 and added as (r0 + r1) + (r2 + r3).  The result is in every lane.
__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_f64<0xB1>(v);  // quad_perm 1,0,3,2
    v += dpp_f64<0x4E>(v);  // quad_perm 2,3,0,1
    v += dpp_f64<0x141>(v); // row_half_mirror
    v += dpp_f64<0x140>(v); // row_mirror
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    auto row = [&](int lane) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, lane);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), lane);
        return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    };
    return (row(0) + row(16)) + (row(32) + row(48));
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// acc + v^2 in fp64 as one fused multiply-add: the square of a float (24
// significant bits) is exact in fp64, so the fused form rounds the same
// single sum as a separate product and add would.
__device__ __forceinline__ double add_square(double acc, float v)
{
    return fma((double)v, (double)v, acc);
}

// Span bounds.  The largest |x| of 8 widened inputs as an ordered integer:
// max of (bits & 0x7FFFFFFF), so an inf or a NaN exceeds every finite value.
__device__ __forceinline__ uint32_t abs_bits_max(const float (&v)[kPer])
{
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        m = max(m, __float_as_uint(v[k]) & 0x7FFFFFFFu);
    return m;
}

// Every lane of the wave must be active.  Within each row of 16 lanes the
// partners are lane ^ 1 and lane ^ 2 (quad permutations), then the mirror
// of each 8-lane half and of the row (DPP moves, no LDS round trip); the
// four rows' maxima are then read from lanes 0, 16, 32 and 48.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    // each move yields 0 (the identity of the max) for an invalid source
    // lane, so the compiler folds it into the max as one DPP instruction
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true)); // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true)); // row_mirror
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// The stored bound: the high half of the largest pattern, rounded up, i.e.
// the smallest bf16 pattern whose value is >= every |x| of the span.  Values
// 0x7F80 and above stand for inf or NaN (or a finite value that rounds up
// to inf) and make the span dense.
__device__ __forceinline__ uint16_t bound16(uint32_t m) { return (uint16_t)((m + 0xFFFFu) >> 16); }

// One wave's bound for the span starting at coordinate jw of row i (all
// lanes active; lane 0 stores it when the span starts inside the row).
// stride: entries per row (bound_stride).  jw is the same in every lane;
// taken from lane 0 the index arithmetic runs in scalar registers.
__device__ __forceinline__ void store_bound(uint16_t *__restrict__ bounds, int64_t stride,
                                            int64_t i, int64_t jw, int64_t d, uint32_t lane_max)
{
    const uint32_t m = wave_max_u32(lane_max);
    const uint64_t jw0 = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(jw >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)jw);
    if ((threadIdx.x & 63) == 0 && (int64_t)jw0 < d)
        bounds[i * stride + (int64_t)(jw0 >> 9)] = bound16(m);
}

// Block reduction with a fixed tree: butterflies inside each wave, then the
// WAVES wave results in order.  Result valid in thread 0.
template <bool MAX, int WAVES = kThreads / 64>
__device__ __forceinline__ double block_reduce(double v, double *lds)
{
    if (MAX)
        v = (double)wave_max((float)v);
    else
        v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        lds[wave] = v;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
        r = lds[0];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            r = MAX ? fmax(r, lds[w]) : r + lds[w];
    }
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------------------
// Pass 1: per-(chunk, worker) partial norms.  Block b reads chunk b / n of
// row b % n, so the last blocks to run read the ends of all rows.  With
// `bounds`, each wave also stores the bound of every 512-coordinate span it
// reads (see bound16).

// QM: 0 = q 2 (exact squares), 1 = q inf (max |x|), 2 = other q (fp64 pow)
template <int DT, int QM>
__global__ __launch_bounds__(kThreads) void k_norm_partial(const void *__restrict__ x, int64_t n,
                                                           int64_t d, int64_t chunks,
                                                           int64_t chunk_len, double qd,
                                                           double *__restrict__ partials,
                                                           uint16_t *__restrict__ bounds,
                                                           int64_t bstride)
{
    constexpr bool QINF = QM == 1;
    __shared__ double red[4];
    const int64_t b = blockIdx.x;
    const int64_t c = b / n, i = b % n;
    const int64_t jb = c * chunk_len;
    const int64_t je = (jb + chunk_len < d) ? jb + chunk_len : d;
    const bool vec_row = (d & 7) == 0;
    const int64_t row_off = i * d;
    // lanes run the loops below in lockstep until the last lane's group
    // leaves the chunk: a wave's bounds are formed in the steps where its
    // last lane is still inside (so is every other), and the steps where it
    // is not -- only at a row end that is not a whole tile, within the last
    // four tiles -- are redone after the loops
    const int64_t to_last = 8 * (63 - (int64_t)(threadIdx.x & 63));
    double s0 = 0.0, s1 = 0.0;
    float mx = 0.0f;
    int64_t j = jb + (int64_t)threadIdx.x * kPer;
    // the sums of four groups (tiles j .. j + 3 kTile) and, where the wave's
    // last lane is inside, their span bounds
    auto four = [&](const float (&v0)[kPer], const float (&v1)[kPer], const float (&v2)[kPer],
                    const float (&v3)[kPer]) {
        if (bounds && j + to_last + 3 * kTile < je) {
            const int64_t jw = j - 8 * (int64_t)(threadIdx.x & 63);
            store_bound(bounds, bstride, i, jw, d, abs_bits_max(v0));
            store_bound(bounds, bstride, i, jw + kTile, d, abs_bits_max(v1));
            store_bound(bounds, bstride, i, jw + 2 * kTile, d, abs_bits_max(v2));
            store_bound(bounds, bstride, i, jw + 3 * kTile, d, abs_bits_max(v3));
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            if (QINF) {
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v0[k]), fabsf(v1[k])),
                                     fmaxf(fabsf(v2[k]), fabsf(v3[k]))));
            } else if (QM == 0) {
                s0 = add_square(s0, v0[k]);
                s1 = add_square(s1, v1[k]);
                s0 = add_square(s0, v2[k]);
                s1 = add_square(s1, v3[k]);
            } else {
                s0 += pow(fabs((double)v0[k]), qd);
                s1 += pow(fabs((double)v1[k]), qd);
                s0 += pow(fabs((double)v2[k]), qd);
                s1 += pow(fabs((double)v3[k]), qd);
            }
        }
    };
    if (DT == GQ_IN_BF16 && vec_row) {
        // bf16: eight groups' 16-byte words requested together, then summed
        // as two steps of four in the same order as below (the span bounds
        // lengthen the work between loads; more bytes in flight cover it)
        const uint16_t *rowp = (const uint16_t *)x + row_off;
        auto widen = [](const uint4 &w, float (&v)[kPer]) {
            const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = __uint_as_float(a[k] << 16);
                v[2 * k + 1] = __uint_as_float(a[k] & 0xFFFF0000u);
            }
        };
        for (; j + 7 * kTile < je; j += 4 * kTile) {
            uint4 w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                w[u] = *(const uint4 *)(rowp + j + u * kTile);
            float v0[kPer], v1[kPer], v2[kPer], v3[kPer];
            widen(w[0], v0); widen(w[1], v1); widen(w[2], v2); widen(w[3], v3);
            four(v0, v1, v2, v3);
            j += 4 * kTile;
            widen(w[4], v0); widen(w[5], v1); widen(w[6], v2); widen(w[7], v3);
            four(v0, v1, v2, v3);
        }
    }
    if (vec_row) {
        // four groups in flight per thread
        for (; j + 3 * kTile < je; j += 4 * kTile) {
            float v0[kPer], v1[kPer], v2[kPer], v3[kPer];
            load_group<DT>(x, row_off, j, d, true, v0);
            load_group<DT>(x, row_off, j + kTile, d, true, v1);
            load_group<DT>(x, row_off, j + 2 * kTile, d, true, v2);
            load_group<DT>(x, row_off, j + 3 * kTile, d, true, v3);
            four(v0, v1, v2, v3);
        }
    }
    for (; j < je; j += kTile) {
        float v[kPer];
        load_group<DT>(x, row_off, j, je, vec_row, v);
        if (bounds && j + to_last < je)
            store_bound(bounds, bstride, i, j - 8 * (int64_t)(threadIdx.x & 63), d,
                        abs_bits_max(v));
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            if (QINF)
                mx = fmaxf(mx, fabsf(v[k]));
            else if (QM == 0)
                s0 = add_square(s0, v[k]);
            else
                s0 += pow(fabs((double)v[k]), qd);
        }
    }
    if (bounds && (je - jb) % kTile != 0) {
        // the last four tiles of a chunk ending inside a tile, with every
        // lane of the block active (loads past the end give 0)
        const int64_t last = jb + (je - jb - 1) / kTile * kTile;
        for (int64_t jt = (last - 3 * kTile > jb) ? last - 3 * kTile : jb; jt < je; jt += kTile) {
            const int64_t jj = jt + (int64_t)threadIdx.x * kPer;
            float v[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (jj < je)
                load_group<DT>(x, row_off, jj, je, vec_row, v);
            store_bound(bounds, bstride, i, jt + (int64_t)(threadIdx.x >> 6) * kSpan, d,
                        abs_bits_max(v));
        }
    }
    const double r = QINF ? block_reduce<true>((double)mx, red) : block_reduce<false>(s0 + s1, red);
    if (threadIdx.x == 0)
        partials[i * chunks + c] = r;
}

// Pass 1, one-shot: block b reads elements [g span, (g + 1) span) of row
// i = b / bpr, g = b % bpr: groups of 8 at (u * 512 + thread) * 8 for
// u < 16 KB / (8 * 512 * element bytes), all loads issued before the sums.
// With `bounds`, each wave stores the bound of each 512-coordinate span it
// reads (see bound16).
template <int DT, int QM>
__global__ __launch_bounds__(kOsThreads) void k_norm_oneshot(const void *__restrict__ x, int64_t d,
                                                             int64_t bpr, int64_t span, double qd,
                                                             double *__restrict__ partials,
                                                             uint16_t *__restrict__ bounds,
                                                             int64_t bstride)
{
    constexpr bool QINF = QM == 1;
    constexpr int G = DT == GQ_IN_F32 ? 1 : 2; // 8-element groups per thread
    __shared__ double red[kOsThreads / 64];
    __shared__ alignas(16) uint16_t blk_bounds[G * (kOsThreads / 64)];
    const int64_t i = blockIdx.x / bpr, g = blockIdx.x % bpr;
    float v[G][kPer];
    if ((d & 7) == 0) {
        // every 128-bit load is issued before any is used
        uint4 r[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            // fp32: the two halves of one group; bf16: one group each
            const int64_t j = DT == GQ_IN_F32
                ? g * span + (int64_t)threadIdx.x * kPer + 4 * q
                : g * span + ((int64_t)q * kOsThreads + threadIdx.x) * kPer;
            const char *p = (const char *)x + (i * d + j) * (DT == GQ_IN_F32 ? 4 : 2);
            r[q] = j < d ? *(const uint4 *)p : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t w[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (DT == GQ_IN_F32) {
                    v[0][4 * q + e] = __uint_as_float(w[e]);
                } else {
                    v[q][2 * e] = __uint_as_float(w[e] << 16);
                    v[q][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int64_t j = g * span + ((int64_t)u * kOsThreads + threadIdx.x) * kPer;
            if (j < d) {
                load_group<DT>(x, i * d, j, d, false, v[u]);
            } else {
#pragma unroll
                for (int k = 0; k < kPer; ++k)
                    v[u][k] = 0.0f;
            }
        }
    }
    if (bounds) {
        // group u of lane l of wave w starts at g span + (u 512 + 64 w + l) 8,
        // so wave w's bound for group u is the block's entry u 8 + w; the
        // block's 8 G entries go out together below (one aligned store:
        // the row stride is a multiple of 16 entries)
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const uint32_t m = wave_max_u32(abs_bits_max(v[u]));
            if ((threadIdx.x & 63) == 0)
                blk_bounds[u * (kOsThreads / 64) + (threadIdx.x >> 6)] = bound16(m);
        }
    }
    double s0 = 0.0, s1 = 0.0;
    float mx = 0.0f;
#pragma unroll
    for (int u = 0; u < G; ++u) {
#pragma unroll
        for (int k = 0; k < kPer; k += 2) {
            if (QINF) {
                mx = fmaxf(mx, fmaxf(fabsf(v[u][k]), fabsf(v[u][k + 1])));
            } else if (QM == 0) {
                s0 = add_square(s0, v[u][k]);
                s1 = add_square(s1, v[u][k + 1]);
            } else {
                s0 += pow(fabs((double)v[u][k]), qd);
                s1 += pow(fabs((double)v[u][k + 1]), qd);
            }
        }
    }
    const double r = QINF ? block_reduce<true, kOsThreads / 64>((double)mx, red)
                          : block_reduce<false, kOsThreads / 64>(s0 + s1, red);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = r;
    // entries past the row's last span land in the row's padding
    if (bounds && threadIdx.x < G)
        *(uint4 *)(bounds + i * bstride + g * (span / kSpan) + 8 * threadIdx.x) =
            *(const uint4 *)(blk_bounds + 8 * threadIdx.x);
}

// Middle reduction of the one-shot partials: block b sums (or maxes) the
// partials [grp 2048, (grp + 1) 2048) of row i = b / gpr, grp = b % gpr: each
// thread its 8 at stride 256 in order, then the block tree.  Past the end a
// partial is 0, the identity of both (partials are non-negative).
template <bool QINF>
__global__ __launch_bounds__(kMidThreads) void k_norm_mid(const double *__restrict__ partials,
                                                          int64_t bpr, int64_t gpr,
                                                          double *__restrict__ mid)
{
    __shared__ double red[kMidThreads / 64];
    const int64_t i = blockIdx.x / gpr, grp = blockIdx.x % gpr;
    const double *p = partials + i * bpr;
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t c = grp * kMidPer + (int64_t)u * kMidThreads + threadIdx.x;
        v[u] = c < bpr ? p[c] : 0.0;
    }
    double acc = v[0];
#pragma unroll
    for (int u = 1; u < 8; ++u)
        acc = QINF ? fmax(acc, v[u]) : acc + v[u];
    const double r = block_reduce<QINF, kMidThreads / 64>(acc, red);
    if (threadIdx.x == 0)
        mid[blockIdx.x] = r;
}

// Pass 1b: one block of kFinThreads.  Worker i's partials are summed by a
// segment of `seg` consecutive threads (a power of two, seg * workers per
// pass = kFinThreads); each thread adds its partials c = lane, lane + seg,
// ... in order, eight loads in flight, then the segment reduces with a fixed
// butterfly (and, for segments wider than a wave, the wave results in
// order through LDS).  The per-worker values are then combined over workers
// by a block-wide fixed tree.  LOCAL: per-worker norms and the per-worker
// scalars of the local-norm ablation instead of one global norm.
constexpr int kFinThreads = 1024;

template <bool MAX>
__device__ __forceinline__ double combine(double a, double b) { return MAX ? fmax(a, b) : a + b; }

template <bool MAX>
__device__ __forceinline__ double butterfly(double v, int width)
{
    for (int off = width >> 1; off > 0; off >>= 1)
        v = combine<MAX>(v, __shfl_xor(v, off));
    return v;
}

// N from the combination `tot` over workers (the term): fp32 of tot for
// (inf, inf) and of its square root for the other {2, inf} pairs; for GEN
// orders fp32 of tot (p = inf), sqrt(tot) (p = 2) or tot^(1/p).
template <bool QINF, bool PINF, bool GEN>
__device__ __forceinline__ float norm_from_term(double tot, double pd)
{
    if (GEN)
        return PINF ? (float)tot : (float)(pd == 2.0 ? sqrt(tot) : pow(tot, 1.0 / pd));
    return (QINF && PINF) ? (float)tot : (float)sqrt(tot);
}

// GEN: (q, p) not both in {2, inf}: w_i = m_i, sqrt(S_i) (q = 2) or S_i^(1/q),
// then N = max_i w_i, sqrt(sum_i w_i^2) (p = 2) or (sum_i w_i^p)^(1/p), in fp64.
// With term_out set, the combination over workers (before the root) goes
// there in fp64 instead of N to norm_out.
template <bool QINF, bool PINF, bool LOCAL, bool GEN>
__global__ __launch_bounds__(kFinThreads) void k_norm_finalize(const double *__restrict__ partials,
                                                               int64_t n, int64_t chunks,
                                                               double *__restrict__ per_worker,
                                                               float *__restrict__ norm_out, int s,
                                                               WorkerParams *__restrict__ params,
                                                               double qd, double pd,
                                                               double *__restrict__ term_out)
{
    __shared__ double red[kFinThreads / 64];
    const int t = threadIdx.x, lane64 = t & 63, wave = t >> 6;
    int seg = kFinThreads;
    while (seg > 1 && (int64_t)seg * n > kFinThreads)
        seg >>= 1;
    const int rows_per_pass = kFinThreads / seg;
    for (int64_t r0 = 0; r0 < n; r0 += rows_per_pass) {
        const int64_t i = r0 + t / seg;
        const int lane = t % seg;
        double acc = 0.0;
        if (i < n) {
            // rounds of eight loads issued together; past the end a load is
            // replaced by 0, the identity of both the sum and the max of
            // non-negative partials, so a short tail costs one round trip
            // instead of one per partial
            const double *p = partials + i * chunks;
            for (int64_t c = lane; c < chunks; c += 8 * (int64_t)seg) {
                double v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t cu = c + u * (int64_t)seg;
                    v[u] = cu < chunks ? p[cu] : 0.0;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    acc = combine<QINF>(acc, v[u]);
            }
        }
        acc = butterfly<QINF>(acc, seg < 64 ? seg : 64);
        if (seg > 64) {
            if (lane64 == 0)
                red[wave] = acc;
            __syncthreads();
            if (lane == 0) {
                double r = red[wave];
                for (int w = 1; w < seg / 64; ++w)
                    r = combine<QINF>(r, red[wave + w]);
                acc = r;
            }
            __syncthreads();
        }
        if (lane == 0 && i < n)
            per_worker[i] = acc;
    }
    __syncthreads();
    if (LOCAL) {
        for (int64_t i = t; i < n; i += kFinThreads) {
            const float Ni = (float)sqrt(per_worker[i]);
            norm_out[i] = Ni;
            const float pre = (Ni < 0x1p-64f) ? 0x1p64f : 1.0f;
            WorkerParams w;
            w.pre = pre;
            w.sigma = (float)((double)s / (double)(Ni * pre));
            w.kappa = (double)Ni / ((double)n * (double)s);
            params[i] = w;
        }
        return;
    }
    // combine over workers: strided in-order partial per thread, then a fixed tree
    const bool q2 = qd == 2.0, p2 = pd == 2.0;
    double acc = 0.0;
    for (int64_t i = t; i < n; i += kFinThreads) {
        const double w = per_worker[i];
        if (GEN) {
            const double wi = QINF ? w : (q2 ? sqrt(w) : pow(w, 1.0 / qd));
            acc = combine<PINF>(acc, PINF ? wi : (p2 ? wi * wi : pow(wi, pd)));
        } else {
            acc = combine<PINF>(acc, (QINF && !PINF) ? w * w : w);
        }
    }
    acc = butterfly<PINF>(acc, 64);
    if (lane64 == 0)
        red[wave] = acc;
    __syncthreads();
    if (t == 0) {
        double tot = red[0];
        for (int w = 1; w < kFinThreads / 64; ++w)
            tot = combine<PINF>(tot, red[w]);
        if (term_out)
            term_out[0] = tot;
        else
            norm_out[0] = norm_from_term<QINF, PINF, GEN>(tot, pd);
    }
}

// N of the whole from the term combined over shards (one thread).
template <bool QINF, bool PINF, bool GEN>
__global__ __launch_bounds__(64) void k_norm_from_term(const double *__restrict__ term, double pd,
                                                       float *__restrict__ norm_out)
{
    if (threadIdx.x == 0)
        norm_out[0] = norm_from_term<QINF, PINF, GEN>(term[0], pd);
}

// ---------------------------------------------------------------------------
// Pass 2, fused: quantize + exact integer sum over workers + dequantize.

// Walk the n workers for one 8-coordinate group, adding the signed codes.
// FACC: the sum is kept in fp32, exact because every partial sum is an
// integer of magnitude <= n M <= 2^24; the sign is applied by an fma with
// +-1.  Otherwise int32.  (Prefetching the next worker's inputs into
// registers was measured to give nothing for fp32 and to cost 3% for bf16.)
// wb: Philox worker index of row 0 (rows held by one device of several).
template <int DT, int SCH, bool PRE, bool FACC>
__device__ __forceinline__ void accumulate_workers(const void *__restrict__ x, int64_t n, int64_t d,
                                                   int64_t j0, bool vec, const QParams &q,
                                                   uint32_t k0, uint32_t k1, float (&accf)[kPer],
                                                   int (&acci)[kPer], uint32_t wb = 0)
{
    const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
    for (int64_t i = 0; i < n; ++i) {
        float v[kPer];
        load_group<DT>(x, i * d, j0, d, vec, v);
        const uint4 A = philox10(make_uint4(blo, bhi, wb + (uint32_t)i, 0u), k0, k1);
        float m[kPer];
        bool tie = false;
        quant_group<SCH, PRE, false>(v, A, q, m, tie);
        if (tie) {
            const uint4 B = philox10(make_uint4(blo, bhi, wb + (uint32_t)i, 1u), k0, k1);
            settle_ties<SCH, PRE>(v, A, B, q, m);
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            if (FACC)
                accf[k] = fmaf(copysignf(1.0f, v[k]), m[k], accf[k]);
            else
                acci[k] += (int)copysignf(m[k], v[k]);
        }
    }
}

// Accumulators of the fused pass: int32, fp32 (exact while every partial
// sum is an integer of magnitude <= 2^24), or packed int16 pairs.
enum { kAccInt = 0, kAccF32 = 1, kAccPk16 = 2 };

// Standard dithering with n s < 2^15: the per-coordinate sums fit int16,
// so the magnitudes are formed with one 32-bit add each and pairs of
// coordinates are signed and summed in packed 16-bit lanes.  With
// sigma16 = sigma 2^16 and top16 = s 2^16, min(|x| pre sigma16, top16) equals
// t 2^16 exactly (a power-of-two scaling of the same rounding; a t below
// fp32's normal range gives lo = 0 and F < 2^16 either way), so
// T = (uint32)(t 2^16) = lo 2^16 + (F >> 16).  Adding 0xFFFF - h, h the 16-bit
// half of the uniform, carries into bit 16 iff F >> 16 > h, so the magnitude
// lo + [h < F >> 16] is the high half of T + (0xFFFF - h).  A tie
// (h == F >> 16) is settled with the second draw exactly as in the other
// paths.  The sign is applied as a multiply by +-1 from the sign bit.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ i16x2 as_i16x2(uint32_t w) { return __builtin_bit_cast(i16x2, w); }

// ---------------------------------------------------------------------------
// Zero-code skip of the fused pass.  With one global norm over a long
// concatenation |x| / N is small, and most coordinates round to code 0.  Let
// K = 16 (L) or s + 15 (E) and sigK = sigma 2^K (exact, a power-of-two
// scaling), so that t 2^K = |x| pre sigK.  Where t is below the first
// non-zero level -- t < 1 (L) or t < 2^(1-s) (E), i.e. t 2^K < 2^16 -- the
// lower level is 0 and F >> 16 = floor(t 2^K) = (uint)(|x| pre sigK): the
// code is non-zero only if the 16-bit uniform h is below it, or equal to it
// and the second draw decides.  Pass 1 stores, per (row, 512-coordinate
// span), a bf16 pattern B >= every |x| of the span (bound16).  The
// threshold H = (uint)(B pre sigK) is then >= F >> 16 of every coordinate of
// the span, fp32 multiplication and truncation being monotone, so a group
// whose eight h all exceed H has eight zero codes and is never loaded.  A
// span whose H would reach 2^16 (some t may reach the first level), whose B
// is inf or NaN, or a sigK that overflows, is dense: every group is loaded
// and quantized as without the skip.

// Lane l: the threshold of row c + l for this wave's span (0x10000: dense).
template <bool PRE>
__device__ __forceinline__ uint32_t span_threshold(const uint16_t *__restrict__ bounds,
                                                   int64_t bstride, int64_t span, int64_t c,
                                                   int64_t n, const QParams &q, float sigK,
                                                   bool sparse_ok)
{
    const int64_t r = c + (int64_t)(threadIdx.x & 63);
    uint32_t H = 0x10000u;
    if (sparse_ok && r < n) {
        const uint32_t b = bounds[r * bstride + span];
        if (b < 0x7F80u) {
            float a = __uint_as_float(b << 16);
            if (PRE)
                a = a * q.pre;
            const float th = a * sigK;
            if (th < 65536.0f)
                H = (uint32_t)th;
        }
    }
    return H;
}

// The smallest of the eight 16-bit uniform halves of one Philox block.
__device__ __forceinline__ uint32_t min_half16(const uint4 &A)
{
    const u16x2 m = __builtin_elementwise_min(
        __builtin_elementwise_min(__builtin_bit_cast(u16x2, A.x), __builtin_bit_cast(u16x2, A.y)),
        __builtin_elementwise_min(__builtin_bit_cast(u16x2, A.z), __builtin_bit_cast(u16x2, A.w)));
    return min((uint32_t)m.x, (uint32_t)m.y);
}

// Magnitudes (0 or 1) of a group in a sparse span, from draw 0: T = F >> 16
// as above, and S = T + (0xFFFF - h) carries into bit 16 iff h < T; its low
// half is all ones iff h == T, a tie for the second draw.
template <bool PRE>
__device__ __forceinline__ void quant_group_sparse(const float (&v)[kPer], const uint4 &A,
                                                   const QParams &q, float sigK,
                                                   float (&m)[kPer], bool &tie)
{
    const uint32_t hx[kPer / 2] = {~A.x, ~A.y, ~A.z, ~A.w}; // 0xFFFF - h, two per word
    uint32_t S[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        float a = fabsf(v[k]);
        if (PRE)
            a = a * q.pre;
        const uint32_t T = cvt_u32_sat(a * sigK);
        S[k] = (k & 1) ? add_half16<1>(T, hx[k >> 1]) : add_half16<0>(T, hx[k >> 1]);
        m[k] = (float)((S[k] >> 16) & 0xFFu);
    }
    const uint32_t mx = max3_lo16(S[6], S[7], max3_lo16(S[0], S[1], S[2]));
    tie |= ((uint16_t)mx == 0xFFFFu) | ((uint16_t)max3_lo16(S[3], S[4], S[5]) == 0xFFFFu);
}

// Candidate queue of the zero-code skip.  A sparse row is tested with one
// Philox block per lane (its group), and only now and then does a lane's
// group pass h <= H; quantized in its own lane, that group would run the
// load and the quantization with the rest of the wave masked off.  Instead
// each wave queues its passing (row, group) pairs in LDS, and whenever 64
// are waiting every lane takes one: it draws the group's block again, loads
// the group, quantizes it and adds its codes to the span's 512 integer sums
// in LDS (integer atomic adds: exact in any order).  Drawing again costs
// less than keeping the blocks: 16 KB of LDS per block instead of 32 KB
// leaves room for more waves (measured 2-7% faster).  The queue is drained
// after every step of two rows, which add at most 128 entries to at most 63
// waiting, so 256 slots suffice.
constexpr int kQueue = 256;
struct SkipQueue {
    uint2 rg[kQueue]; // row, group of the span (0..63)
    int sum[kSpan];   // queued codes summed per coordinate of the span
};

// One queue per wave of the block, shared by every instantiation in a kernel.
__device__ __forceinline__ SkipQueue &wave_skip_queue()
{
    __shared__ SkipQueue queues[kThreads / 64];
    return queues[threadIdx.x >> 6];
}

// Lanes < count each take entry head + lane of the queue.
template <int DT, int SCH, bool PRE>
__device__ __forceinline__ void drain_queue(SkipQueue &sq, uint32_t head, uint32_t count,
                                            const void *__restrict__ x, int64_t d, int64_t span,
                                            bool vec, const QParams &q, float sigK, uint32_t k0,
                                            uint32_t k1, uint32_t wb)
{
    const uint32_t lane = threadIdx.x & 63;
    if (lane < count) {
        const uint32_t e = (head + lane) % kQueue;
        const uint2 rg = sq.rg[e];
        const int64_t jg = span * kSpan + 8 * (int64_t)rg.y;
        const uint4 A = philox10(make_uint4((uint32_t)((uint64_t)jg >> 3),
                                            (uint32_t)((uint64_t)jg >> 35), wb + rg.x, 0u), k0, k1);
        float v[kPer], m[kPer];
        bool tie = false;
        load_group<DT>(x, (int64_t)rg.x * d, jg, d, vec, v);
        quant_group_sparse<PRE>(v, A, q, sigK, m, tie);
        if (tie) {
            const uint4 B = philox10(make_uint4((uint32_t)((uint64_t)jg >> 3),
                                                (uint32_t)((uint64_t)jg >> 35), wb + rg.x, 1u),
                                     k0, k1);
            settle_ties<SCH, PRE>(v, A, B, q, m);
        }
        // every code, zeros included: no per-coordinate branches (measured
        // 1-3% faster than adding only the non-zero ones)
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            atomicAdd(&sq.sum[8 * rg.y + k], (int)copysignf(m[k], v[k]));
    }
}

// The wave's queue state: entries [head, tail) wait (wave-uniform counts).
template <int DT, int SCH, bool PRE>
struct SkipQueueWalk {
    SkipQueue *sq;
    const void *__restrict__ x;
    int64_t d, span;
    bool vec;
    const QParams &q;
    float sigK;
    uint32_t k0, k1, wb;
    uint32_t head = 0, tail = 0;

    __device__ __forceinline__ void start()
    {
        const int b = 8 * (int)(threadIdx.x & 63);
        *(int4 *)&sq->sum[b] = make_int4(0, 0, 0, 0);
        *(int4 *)&sq->sum[b + 4] = make_int4(0, 0, 0, 0);
        wave_lds_fence();
    }
    // Row i of a sparse span: queue the lanes whose group passes.
    __device__ __forceinline__ void offer(int64_t i, bool cand)
    {
        const uint64_t mask = __ballot(cand);
        if (cand) {
            const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
            const uint32_t e = (tail + below) % kQueue;
            sq->rg[e] = make_uint2((uint32_t)i, threadIdx.x & 63);
        }
        tail += (uint32_t)__popcll(mask);
    }
    // Between steps: every lane busy while 64 or more entries wait.
    __device__ __forceinline__ void drain_full()
    {
        while (tail - head >= 64) {
            wave_lds_fence();
            drain_queue<DT, SCH, PRE>(*sq, head, 64, x, d, span, vec, q, sigK, k0, k1, wb);
            head += 64;
            wave_lds_fence();
        }
    }
    // After the last row: drain the rest; returns this lane's 8 queued sums.
    __device__ __forceinline__ void finish(int (&qs)[kPer])
    {
        drain_full();
        wave_lds_fence();
        if (tail != head)
            drain_queue<DT, SCH, PRE>(*sq, head, tail - head, x, d, span, vec, q, sigK, k0, k1, wb);
        wave_lds_fence();
        const int b = 8 * (int)(threadIdx.x & 63);
        const int4 s0 = *(const int4 *)&sq->sum[b], s1 = *(const int4 *)&sq->sum[b + 4];
        qs[0] = s0.x; qs[1] = s0.y; qs[2] = s0.z; qs[3] = s0.w;
        qs[4] = s1.x; qs[5] = s1.y; qs[6] = s1.z; qs[7] = s1.w;
        wave_lds_fence(); // the next call's clearing comes after these reads
    }
};

// accumulate_workers with the zero-code skip: every lane of the wave must be
// here (the thresholds are shared through lane reads); `live` marks lanes
// whose group is inside the row.  Rows of a dense span take quant_group in
// every lane; the passing groups of sparse rows go through the wave's
// candidate queue.
template <int DT, int SCH, bool PRE, bool FACC>
__device__ __forceinline__ void accumulate_workers_skip(const void *__restrict__ x, int64_t n,
                                                        int64_t d, int64_t j0, bool vec,
                                                        bool live, const QParams &q,
                                                        uint32_t k0, uint32_t k1,
                                                        const uint16_t *__restrict__ bounds,
                                                        int64_t bstride, int64_t span, float sigK,
                                                        bool sparse_ok, float (&accf)[kPer],
                                                        int (&acci)[kPer], uint32_t wb = 0)
{
    SkipQueueWalk<DT, SCH, PRE> walk{&wave_skip_queue(), x, d, span, vec, q, sigK, k0, k1, wb};
    walk.start();
    const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
    // one worker's group of a dense span, in its own lane
    auto own = [&](int64_t i, const uint4 &A) {
        float v[kPer], m[kPer];
        bool tie = false;
        load_group<DT>(x, i * d, j0, d, vec, v);
        quant_group<SCH, PRE, false>(v, A, q, m, tie);
        if (tie) {
            const uint4 B = philox10(make_uint4(blo, bhi, wb + (uint32_t)i, 1u), k0, k1);
            settle_ties<SCH, PRE>(v, A, B, q, m);
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            if (FACC)
                accf[k] = fmaf(copysignf(1.0f, v[k]), m[k], accf[k]);
            else
                acci[k] += (int)copysignf(m[k], v[k]);
        }
    };
    auto row = [&](int64_t i, uint32_t H, const uint4 &A) {
        if (H <= 0xFFFFu)
            walk.offer(i, live && min_half16(A) <= H);
        else if (live)
            own(i, A);
    };
    for (int64_t c = 0; c < n; c += 64) {
        const uint32_t Hl = span_threshold<PRE>(bounds, bstride, span, c, n, q, sigK, sparse_ok);
        const int cnt = (int)(n - c < 64 ? n - c : 64);
        int r = 0;
        // two workers per step: two independent Philox chains in flight
        // (measured 1-4% faster than one)
        for (; r + 1 < cnt; r += 2) {
            const uint4 A0 = philox10(make_uint4(blo, bhi, wb + (uint32_t)(c + r), 0u), k0, k1);
            const uint4 A1 = philox10(make_uint4(blo, bhi, wb + (uint32_t)(c + r + 1), 0u), k0, k1);
            row(c + r, __builtin_amdgcn_readlane(Hl, r), A0);
            row(c + r + 1, __builtin_amdgcn_readlane(Hl, r + 1), A1);
            walk.drain_full();
        }
        if (r < cnt)
            row(c + r, __builtin_amdgcn_readlane(Hl, r),
                philox10(make_uint4(blo, bhi, wb + (uint32_t)(c + r), 0u), k0, k1));
    }
    int qs[kPer];
    walk.finish(qs);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        if (FACC)
            accf[k] += (float)qs[k]; // integers below 2^24: exact
        else
            acci[k] += qs[k];
    }
}

template <int DT, bool PRE>
__device__ __forceinline__ void pk16_row(const void *__restrict__ x, int64_t d, int64_t j0,
                                         bool vec, int64_t i, const uint4 &A, const QParams &q,
                                         float sigma16, float top16, uint32_t blo, uint32_t bhi,
                                         uint32_t wi, uint32_t k0, uint32_t k1,
                                         i16x2 (&acc2)[kPer / 2])
{
    static_assert(DT == GQ_IN_BF16, "packed 16-bit sums take bf16 input");
    // raw bf16 pairs (0 past the end of the row): the sign bits of both
    // coordinates sit at bits 15 and 31 of each word
    uint32_t rw[kPer / 2];
    const uint16_t *row = (const uint16_t *)x + i * d + j0;
    if (vec) {
        const uint4 r = *(const uint4 *)row;
        rw[0] = r.x; rw[1] = r.y; rw[2] = r.z; rw[3] = r.w;
    } else {
#pragma unroll
        for (int k = 0; k < kPer / 2; ++k)
            rw[k] = ((j0 + 2 * k < d) ? (uint32_t)row[2 * k] : 0u) |
                    ((j0 + 2 * k + 1 < d) ? (uint32_t)row[2 * k + 1] << 16 : 0u);
    }
    float v[kPer];
#pragma unroll
    for (int k = 0; k < kPer / 2; ++k) {
        v[2 * k] = __uint_as_float(rw[k] << 16);
        v[2 * k + 1] = __uint_as_float(rw[k] & 0xFFFF0000u);
    }
    const uint32_t Aw[kPer / 2] = {A.x, A.y, A.z, A.w};
    uint32_t T[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        float a = fabsf(v[k]);
        if (PRE)
            a = a * q.pre;
        T[k] = (uint32_t)fminf(a * sigma16, top16);
    }
    // S = T + (0xFFFF - h): its low half is 0xFFFF exactly when h equals
    // the low half of T (a tie), so the max of the 8 low halves finds any
    // tie in the group.  As SDWA adds and 16-bit max3 these steps take 8
    // fewer VALU instructions per worker than the compiler's own lowering
    // (measured -2.8% on this pass).
    uint32_t m2[kPer / 2], S[kPer];
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) {
        const uint32_t hx = ~Aw[p]; // 0xFFFF - h of both coordinates
        S[2 * p] = add_half16<0>(T[2 * p], hx);
        S[2 * p + 1] = add_half16<1>(T[2 * p + 1], hx);
        m2[p] = __builtin_amdgcn_perm(S[2 * p + 1], S[2 * p], 0x07060302u); // high halves
    }
    const uint32_t mx = max3_lo16(S[6], S[7], max3_lo16(S[0], S[1], S[2]));
    const bool tie = ((uint16_t)mx == 0xFFFFu) | ((uint16_t)max3_lo16(S[3], S[4], S[5]) == 0xFFFFu);
    if (tie) {
        const uint4 B = philox10(make_uint4(blo, bhi, wi, 1u), k0, k1);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            if ((S[k] & 0xFFFFu) == 0xFFFFu) { // tie: h == F >> 16
                float lo, step;
                uint32_t Fh, F;
                bracket<GQ_SCHEME_L, PRE>(v[k], q, lo, step, Fh, &F);
                if (half16(B, k) < (F & 0xFFFFu))
                    m2[k >> 1] += (k & 1) ? 0x00010000u : 0x00000001u;
            }
        }
    }
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) {
        // +1 / -1 per lane from the sign bits of the two inputs
        const i16x2 sgn = (as_i16x2(rw[p]) >> (i16x2)15) | (i16x2)1;
        acc2[p] += as_i16x2(m2[p]) * sgn;
    }
}

// SKIP: the zero-code skip of the fused pass (see span_thresholds); then
// every lane of the wave must be here, `live` marking those with
// coordinates in the row.
template <int DT, bool PRE, bool SKIP>
__device__ __forceinline__ void accumulate_workers_pk16(const void *__restrict__ x, int64_t n,
                                                        int64_t d, int64_t j0, bool vec,
                                                        const QParams &q, uint32_t k0,
                                                        uint32_t k1, int (&acc)[kPer],
                                                        uint32_t wb = 0, bool live = true,
                                                        const uint16_t *__restrict__ bounds = nullptr,
                                                        int64_t bstride = 0, int64_t span = 0,
                                                        bool sparse_ok = false)
{
    const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
    const float sigma16 = q.sigma * 0x1p16f, top16 = q.top * 0x1p16f;
    i16x2 acc2[kPer / 2];
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p)
        acc2[p] = as_i16x2(0u);
    int qs[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (SKIP) {
        SkipQueueWalk<DT, GQ_SCHEME_L, PRE> walk{&wave_skip_queue(), x, d, span, vec, q, sigma16,
                                                 k0, k1, wb};
        walk.start();
        for (int64_t c = 0; c < n; c += 64) {
            const uint32_t Hl = span_threshold<PRE>(bounds, bstride, span, c, n, q, sigma16, sparse_ok);
            const int cnt = (int)(n - c < 64 ? n - c : 64);
            auto row = [&](int64_t i, uint32_t H, const uint4 &A) {
                if (H <= 0xFFFFu)
                    walk.offer(i, live && min_half16(A) <= H);
                else if (live)
                    pk16_row<DT, PRE>(x, d, j0, vec, i, A, q, sigma16, top16, blo, bhi,
                                      wb + (uint32_t)i, k0, k1, acc2);
            };
            int r = 0;
            for (; r + 1 < cnt; r += 2) {
                const uint4 A0 = philox10(make_uint4(blo, bhi, wb + (uint32_t)(c + r), 0u), k0, k1);
                const uint4 A1 = philox10(make_uint4(blo, bhi, wb + (uint32_t)(c + r + 1), 0u), k0, k1);
                row(c + r, __builtin_amdgcn_readlane(Hl, r), A0);
                row(c + r + 1, __builtin_amdgcn_readlane(Hl, r + 1), A1);
                walk.drain_full();
            }
            if (r < cnt)
                row(c + r, __builtin_amdgcn_readlane(Hl, r),
                    philox10(make_uint4(blo, bhi, wb + (uint32_t)(c + r), 0u), k0, k1));
        }
        walk.finish(qs);
    } else {
        for (int64_t i = 0; i < n; ++i) {
            const uint4 A = philox10(make_uint4(blo, bhi, wb + (uint32_t)i, 0u), k0, k1);
            pk16_row<DT, PRE>(x, d, j0, vec, i, A, q, sigma16, top16, blo, bhi, wb + (uint32_t)i,
                              k0, k1, acc2);
        }
    }
#pragma unroll
    for (int p = 0; p < kPer / 2; ++p) {
        acc[2 * p] = acc2[p].x + qs[2 * p];
        acc[2 * p + 1] = acc2[p].y + qs[2 * p + 1];
    }
}
// SKIP: with pass 1's span bounds (u16 [n][bstride]), groups whose codes are
// provably all 0 are neither loaded nor quantized (the zero-code skip); the
// rest of sparse spans go through the wave's candidate queue.
// With SKIP and standard dithering the registers are capped for 6 waves per
// SIMD (measured 2-5% faster than 5; exponential dithering would spill).
template <int DT, int SCH, int ACC, bool SKIP>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(SKIP && SCH == GQ_SCHEME_L ? 6 : 1))) void k_compress_mean(const void *__restrict__ x, int64_t n,
                                                            int64_t d, int s, uint64_t seed,
                                                            const float *__restrict__ norm_dev,
                                                            float *__restrict__ mean,
                                                            uint8_t *__restrict__ code_sum, int W,
                                                            const uint16_t *__restrict__ bounds,
                                                            int64_t bstride)
{
    // fp32: 32 KB of LDS caps residency at 5 blocks (20 waves) per CU.
    // Fewer concurrent waves interleave fewer HBM read and write streams:
    // measured -6% on this pass for fp32 at 0.8-16 GB (4 and 5 blocks alike,
    // 6 no gain); bf16, bound by vector ALU work, needs the full residency
    // (5 blocks: +15%).  Only the code-sum packing uses the first 8 KB.
    // With SKIP each wave packs in its own candidate queue (free by then).
    __shared__ alignas(16) uint32_t lds[SKIP ? 4 : DT == GQ_IN_F32 ? 8192 : kTile];
    // Reverse of pass 1's order: the chunk-major pass 1 (inputs up to 256 MiB)
    // finishes on the last chunks of every row, so starting pass 2 there
    // re-reads data the memory-side cache still holds (measured: -7% time on
    // an 0.8 GB input when it took that pass; neutral on 7-16 GB).
    const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t j0 = tile * kTile + (int64_t)threadIdx.x * kPer;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    float accf[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    int acc[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (SKIP) {
        // one span per wave; the whole wave enters when its span starts
        // inside the row
        const int64_t span = tile * (kTile / kSpan) + (int64_t)(threadIdx.x >> 6);
        if (!q.zero && span * kSpan < d) {
            const bool vec = (d & 7) == 0, live = j0 < d;
            const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
            const float sigK = q.sigma * (SCH == GQ_SCHEME_L ? 0x1p16f : q.p2E16);
            const bool sparse_ok = sigK < INFINITY; // false for NaN too
            if constexpr (ACC == kAccPk16) {
                if (q.prescale)
                    accumulate_workers_pk16<DT, true, true>(x, n, d, j0, vec, q, k0, k1, acc, 0u,
                                                            live, bounds, bstride, span, sparse_ok);
                else
                    accumulate_workers_pk16<DT, false, true>(x, n, d, j0, vec, q, k0, k1, acc, 0u,
                                                             live, bounds, bstride, span, sparse_ok);
            } else if (q.prescale)
                accumulate_workers_skip<DT, SCH, true, ACC == kAccF32>(
                    x, n, d, j0, vec, live, q, k0, k1, bounds, bstride, span, sigK, sparse_ok, accf, acc);
            else
                accumulate_workers_skip<DT, SCH, false, ACC == kAccF32>(
                    x, n, d, j0, vec, live, q, k0, k1, bounds, bstride, span, sigK, sparse_ok, accf, acc);
            if (ACC == kAccF32) {
#pragma unroll
                for (int k = 0; k < kPer; ++k)
                    acc[k] = (int)accf[k];
            }
        }
    } else if (!q.zero && j0 < d) {
        const bool vec = (d & 7) == 0;
        const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
        if constexpr (ACC == kAccPk16) {
            if (q.prescale)
                accumulate_workers_pk16<DT, true, false>(x, n, d, j0, vec, q, k0, k1, acc);
            else
                accumulate_workers_pk16<DT, false, false>(x, n, d, j0, vec, q, k0, k1, acc);
        } else if (q.prescale)
            accumulate_workers<DT, SCH, true, ACC == kAccF32>(x, n, d, j0, vec, q, k0, k1, accf, acc);
        else
            accumulate_workers<DT, SCH, false, ACC == kAccF32>(x, n, d, j0, vec, q, k0, k1, accf, acc);
        if (ACC == kAccF32) {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc[k] = (int)accf[k];
        }
    }
    if (j0 < d) {
        float m[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            m[k] = (float)((double)acc[k] * q.kappa);
        store_mean8(mean, j0, d, m);
    }
    if (code_sum)
        store_tile_packed(lds, acc, W, code_sum, tile, row_bytes(d, W),
                          SKIP ? (uint32_t *)wave_skip_queue().sum : nullptr);
}

// Many workers (n >= kSums8MinN, fp32): the compress step in two kernels.
// While the pass streams n rows per tile, every byte it writes costs far
// more than its share of bandwidth: on a 64 x 64M fp32 input the pass takes
// 2.66 ms without writes, 2.95 ms with the 256 MB mean interleaved, 2.75 ms
// with 64 MB of 1-byte sums (about 1.2 us per MB written).  So the pass
// writes as little as it can: one bit per 8-coordinate group (a wave's 64
// groups in one 64-bit word, from a ballot, so no atomics and no clearing),
// and only for groups holding a non-zero sum their 8 bytes, each sum in
// [-127, 127] as itself, beyond it the escape -128.  With one global norm
// over a large concatenation |x| / N is tiny and most groups sum to zero
// (1-2% of groups are non-zero on the gradient-like inputs).  A second
// streaming kernel writes the mean from the mask and the bytes,
// recomputing an escaped group's sums from x (the same accumulation, so the
// same integers).  An input where every group escapes is still exact, at
// the cost of a second full pass.
constexpr int kSums8Escape = -128;

template <int DT, int SCH, int ACC>
__global__ __launch_bounds__(kThreads) void k_compress_sums8(const void *__restrict__ x, int64_t n,
                                                             int64_t d, int s, uint64_t seed,
                                                             const float *__restrict__ norm_dev,
                                                             uint8_t *__restrict__ staged)
{
    // the residency cap of the fused pass (32 KB of LDS: 5 blocks per CU)
    __shared__ alignas(16) uint32_t lds[8192];
    if (n < 0)
        lds[threadIdx.x] = 0;
    const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t g = tile * kThreads + threadIdx.x; // this thread's 8-coordinate group
    const int64_t j0 = g * kPer;
    if (j0 >= d)
        return;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    float accf[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    int acc[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (!q.zero) {
        const bool vec = (d & 7) == 0;
        const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
        if (q.prescale)
            accumulate_workers<DT, SCH, true, ACC == kAccF32>(x, n, d, j0, vec, q, k0, k1, accf, acc);
        else
            accumulate_workers<DT, SCH, false, ACC == kAccF32>(x, n, d, j0, vec, q, k0, k1, accf, acc);
        if (ACC == kAccF32) {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc[k] = (int)accf[k];
        }
    }
    bool nz = false;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        nz |= acc[k] != 0;
    // lanes past the end have returned and count as zero groups; lane 0 holds
    // the wave's first group, so it is active whenever the word is in range
    const uint64_t bits = __ballot(nz);
    if ((threadIdx.x & 63) == 0)
        ((uint64_t *)staged)[g >> 6] = bits;
    if (!nz)
        return;
    int8_t *sums8 = (int8_t *)(staged + sums8_mask_bytes(d));
    uint32_t b[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        b[k] = (uint32_t)((acc[k] >= -127 && acc[k] <= 127) ? acc[k] : kSums8Escape) & 0xFFu;
    if (j0 + kPer <= d && (d & 7) == 0) {
        const uint2 o = make_uint2(b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24,
                                   b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24);
        nt_store((uint8_t *)sums8 + j0, o);
    } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            if (j0 + k < d)
                sums8[j0 + k] = (int8_t)b[k];
    }
}

template <int DT, int SCH, int ACC>
__global__ __launch_bounds__(kThreads) void k_dequantize_sums8(const void *__restrict__ x, int64_t n,
                                                               int64_t d, int s, uint64_t seed,
                                                               const float *__restrict__ norm_dev,
                                                               const uint8_t *__restrict__ staged,
                                                               float *__restrict__ mean)
{
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t j0 = g * kPer;
    if (j0 >= d)
        return;
    // the mask word and the group's bytes are loaded together (one round
    // trip; the bytes of an unmarked group are stale and ignored): waiting
    // for the mask before loading the bytes measured 154 against 126 us on
    // a 110M-coordinate row (the same on a 64M one)
    const uint64_t word = ((const uint64_t *)staged)[g >> 6]; // one word per wave
    const int8_t *sums8 = (const int8_t *)(staged + sums8_mask_bytes(d));
    const bool full = j0 + kPer <= d && (d & 7) == 0;
    uint2 w = make_uint2(0u, 0u);
    if (full)
        w = *(const uint2 *)(sums8 + j0);
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    int acc[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    if ((word >> (g & 63)) & 1u) {
        bool esc = false;
        if (full) {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc[k] = (int)(int8_t)(((k < 4 ? w.x : w.y) >> (8 * (k & 3))) & 0xFFu);
        } else {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc[k] = j0 + k < d ? (int)sums8[j0 + k] : 0;
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            esc |= acc[k] == kSums8Escape;
        if (esc) {
            // a sum outside [-127, 127] in this group: recompute the group's
            // exact sums over the n workers, as the pass formed them
            float accf[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
            int acci[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
            const bool vec = (d & 7) == 0;
            const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
            if (q.prescale)
                accumulate_workers<DT, SCH, true, ACC == kAccF32>(x, n, d, j0, vec, q, k0, k1, accf, acci);
            else
                accumulate_workers<DT, SCH, false, ACC == kAccF32>(x, n, d, j0, vec, q, k0, k1, accf, acci);
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc[k] = ACC == kAccF32 ? (int)accf[k] : acci[k];
        }
    }
    float m[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        m[k] = (float)((double)acc[k] * q.kappa);
    store_mean8<false>(mean, j0, d, m);
}

// Codes of one 8-coordinate group of worker wk (v already loaded).
template <int SCH>
__device__ __forceinline__ void quantize_group_codes(const float (&v)[kPer], const QParams &q,
                                                     int64_t j0, uint64_t wk, uint64_t seed,
                                                     int (&code)[kPer])
{
    const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const uint4 A = philox10(make_uint4(blo, bhi, (uint32_t)wk, 0u), k0, k1);
    float m[kPer];
    bool tie = false;
    if (q.prescale)
        quant_group<SCH, true>(v, A, q, m, tie);
    else
        quant_group<SCH, false>(v, A, q, m, tie);
    if (tie) {
        const uint4 B = philox10(make_uint4(blo, bhi, (uint32_t)wk, 1u), k0, k1);
        if (q.prescale)
            settle_ties<SCH, true>(v, A, B, q, m);
        else
            settle_ties<SCH, false>(v, A, B, q, m);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        code[k] = (int)copysignf(m[k], v[k]);
}

// Unfused quantize: block b encodes tile b % tiles of row b / tiles.
template <int DT, int SCH, bool NT>
__global__ __launch_bounds__(kThreads) void k_quantize(const void *__restrict__ x, int64_t n,
                                                       int64_t d, int s, uint64_t seed,
                                                       int64_t worker_base,
                                                       const float *__restrict__ norm_dev,
                                                       uint8_t *__restrict__ codes, int W,
                                                       int64_t rbytes, int64_t tiles)
{
    __shared__ alignas(16) uint32_t lds[kTile];
    const int64_t i = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int64_t j0 = tile * kTile + (int64_t)threadIdx.x * kPer;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    int code[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (!q.zero && j0 < d) {
        float v[kPer];
        load_group<DT>(x, i * d, j0, d, (d & 7) == 0, v);
        quantize_group_codes<SCH>(v, q, j0, (uint64_t)(worker_base + i), seed, code);
    }
    store_tile_packed<NT>(lds, code, W, codes + i * rbytes, tile, rbytes);
}

// The same with two consecutive tiles per block (tiles 2 (b % ceil(tiles/2))
// and the next, of row b / ceil(tiles/2)), the loads of both issued first:
// bf16 rows (4 KB of input per tile) measured 7-9% faster this way; fp32
// rows keep one tile per block.
template <int DT, int SCH, bool NT>
__global__ __launch_bounds__(kThreads) void k_quantize2(const void *__restrict__ x, int64_t n,
                                                        int64_t d, int s, uint64_t seed,
                                                        int64_t worker_base,
                                                        const float *__restrict__ norm_dev,
                                                        uint8_t *__restrict__ codes, int W,
                                                        int64_t rbytes, int64_t tiles)
{
    __shared__ alignas(16) uint32_t lds[kTile];
    const int64_t pairs = (tiles + 1) / 2;
    const int64_t i = blockIdx.x / pairs, t0 = (blockIdx.x % pairs) * 2;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    const bool vec = (d & 7) == 0;
    float v[2][kPer];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int64_t j0 = (t0 + r) * kTile + (int64_t)threadIdx.x * kPer;
        if (!q.zero && j0 < d)
            load_group<DT>(x, i * d, j0, d, vec, v[r]);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int64_t tile = t0 + r;
        if (tile >= tiles) // uniform over the block
            break;
        const int64_t j0 = tile * kTile + (int64_t)threadIdx.x * kPer;
        int code[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (!q.zero && j0 < d)
            quantize_group_codes<SCH>(v[r], q, j0, (uint64_t)(worker_base + i), seed, code);
        if (r > 0)
            __syncthreads(); // the packer's LDS is reused
        store_tile_packed<NT>(lds, code, W, codes + i * rbytes, tile, rbytes);
    }
}

// Unfused integer sum over the n packed rows of one tile.
__global__ __launch_bounds__(kThreads) void k_reduce_codes(const uint8_t *__restrict__ codes,
                                                           int64_t n, int W, int64_t rbytes,
                                                           uint8_t *__restrict__ out)
{
    __shared__ alignas(16) uint32_t lds[kTile];
    const int64_t tile = blockIdx.x;
    int acc[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (W == 8 || W == 16 || W == 32) {
        for (int64_t i = 0; i < n; ++i) {
            int v[kPer];
            load_tile_fields(lds, codes + i * rbytes, W, tile, rbytes, v);
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc[k] += v[k]; // exact when W holds n M; otherwise wraps below
        }
    } else {
        // the wave-level staging of load_tile_fields with the next row's
        // 16-byte chunks (u = lane and lane + 64 of the 4 W) loaded into
        // registers while the current row is extracted
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int nw = 16 * W, nq = 4 * W;
        uint32_t *wl = lds + wave * nw;
        const int64_t wbase = tile * 64 * W + (int64_t)wave * nw;
        uint4 nxt[2];
        auto fetch = [&](int64_t i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int u = lane + 64 * h;
                const int64_t off = (wbase + 4 * u) * 4;
                nxt[h] = (u < nq && off < rbytes) ? *(const uint4 *)(codes + i * rbytes + off)
                                                  : make_uint4(0u, 0u, 0u, 0u);
            }
        };
        fetch(0);
        for (int64_t i = 0; i < n; ++i) {
            const uint4 cur0 = nxt[0], cur1 = nxt[1];
            if (i + 1 < n)
                fetch(i + 1);
            if (lane < nq)
                ((uint4 *)wl)[lane] = cur0;
            if (lane + 64 < nq)
                ((uint4 *)wl)[lane + 64] = cur1;
            wave_lds_fence();
            int v[kPer];
            extract_fields_wave(wl, nw, W, lane, v);
            wave_lds_fence();
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc[k] += v[k];
        }
    }
    if (W < 32) {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            acc[k] = (int)((uint32_t)acc[k] << (32 - W)) >> (32 - W);
    }
    store_tile_packed(lds, acc, W, out, tile, rbytes);
}

// Unfused dequantization of one packed row of code sums.
template <int SCH>
__global__ __launch_bounds__(kThreads) void k_dequantize(const uint8_t *__restrict__ code_sum,
                                                         int64_t n, int64_t d, int s, int W,
                                                         const float *__restrict__ norm_dev,
                                                         float *__restrict__ mean)
{
    __shared__ alignas(16) uint32_t lds[kTile];
    const int64_t tile = blockIdx.x;
    const int64_t j0 = tile * kTile + (int64_t)threadIdx.x * kPer;
    int v[kPer];
    load_tile_fields(lds, code_sum, W, tile, row_bytes(d, W), v);
    if (j0 >= d)
        return;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    float m[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        m[k] = (float)((double)v[k] * q.kappa);
    store_mean8<false>(mean, j0, d, m);
}

// ---------------------------------------------------------------------------
// Word layout for a native integer all-reduce (Sec. 6: the collective's own
// integer SUM adds the codes).  FPW = floor(32 / W) fields per 32-bit word;
// coordinate j sits in word j / FPW at bits W (j % FPW) and holds code + M
// (0 past d).  A block covers 2048 words of one row, i.e. 2048 FPW
// coordinates.  Quantization is coalesced per 8-coordinate Philox group:
// group g of thread t is coordinates g 2048 + 8 t .. + 8 of the block; the
// biased fields go to LDS (one byte each for W <= 8, two for W <= 16), and
// after one barrier thread t assembles words 4 t .. 4 t + 3 and
// 1024 + 4 t .. + 3 and stores each quad with one 16-byte store.  With
// FPW = 1 (W >= 17) the 8 fields of a thread are its 8 words, no LDS.
constexpr int kWordsPerBlock = 2048;

__host__ __device__ constexpr int word_fields(int W) { return 32 / W; }

template <int FPW>
using WordLdsT = typename std::conditional<(FPW >= 4), uint8_t, uint16_t>::type;

// PK: bf16 standard dithering, codes formed by the fused pass's packed
// 16-bit loop over one row (the row's codes are its one-row sum).
template <int DT, int SCH, int FPW, bool PK = false>
__global__ __launch_bounds__(kThreads) void k_quantize_words(const void *__restrict__ x, int64_t n,
                                                             int64_t d, int s, uint64_t seed,
                                                             int64_t worker_base,
                                                             const float *__restrict__ norm_dev,
                                                             uint32_t *__restrict__ words, int W,
                                                             uint32_t M, int64_t rwords,
                                                             int64_t tiles)
{
    static_assert(kThreads * kPer == kWordsPerBlock, "one Philox group per thread and word group");
    using E = WordLdsT<FPW>;
    __shared__ alignas(16) E lds[FPW > 1 ? kWordsPerBlock * FPW : 1];
    const int64_t i = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int64_t c_base = tile * kWordsPerBlock * FPW; // first coordinate of the block
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    const bool vec = (d & 7) == 0;
    uint32_t *row = words + i * rwords;
    if constexpr (FPW == 1) {
        const int64_t j0 = c_base + (int64_t)threadIdx.x * kPer;
        int code[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (!q.zero && j0 < d) {
            float v[kPer];
            load_group<DT>(x, i * d, j0, d, vec, v);
            quantize_group_codes<SCH>(v, q, j0, (uint64_t)(worker_base + i), seed, code);
        }
        uint32_t w[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            w[k] = (j0 + k < d) ? (uint32_t)code[k] + M : 0u;
        if (j0 < rwords)
            nt_store((uint8_t *)(row + j0), make_uint4(w[0], w[1], w[2], w[3]));
        if (j0 + 4 < rwords)
            nt_store((uint8_t *)(row + j0 + 4), make_uint4(w[4], w[5], w[6], w[7]));
    } else {
#pragma unroll
        for (int g = 0; g < FPW; ++g) {
            const int rel = g * kWordsPerBlock + (int)threadIdx.x * kPer;
            const int64_t j0 = c_base + rel;
            int code[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (!q.zero && j0 < d) {
                if constexpr (PK) {
                    const void *xrow = (const uint16_t *)x + i * d;
                    const uint32_t wk = (uint32_t)(worker_base + i);
                    if (q.prescale)
                        accumulate_workers_pk16<DT, true, false>(xrow, 1, d, j0, vec, q, (uint32_t)seed,
                                                          (uint32_t)(seed >> 32), code, wk);
                    else
                        accumulate_workers_pk16<DT, false, false>(xrow, 1, d, j0, vec, q, (uint32_t)seed,
                                                           (uint32_t)(seed >> 32), code, wk);
                } else {
                    float v[kPer];
                    load_group<DT>(x, i * d, j0, d, vec, v);
                    quantize_group_codes<SCH>(v, q, j0, (uint64_t)(worker_base + i), seed, code);
                }
            }
            E b[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                b[k] = (E)((j0 + k < d) ? (uint32_t)code[k] + M : 0u);
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                lds[rel + k] = b[k];
        }
        __syncthreads();
        const int64_t w_base = tile * kWordsPerBlock;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int wr = h * (kWordsPerBlock / 2) + 4 * (int)threadIdx.x;
            uint32_t w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t acc = 0;
#pragma unroll
                for (int f = 0; f < FPW; ++f)
                    acc |= (uint32_t)lds[(wr + u) * FPW + f] << (W * f);
                w[u] = acc;
            }
            if (w_base + wr < rwords)
                nt_store((uint8_t *)(row + w_base + wr), make_uint4(w[0], w[1], w[2], w[3]));
        }
    }
}

// The same for 3, 5, 6 or 10 fields per word, where a thread's 8
// coordinates straddle unaligned words: a block covers 2048 words
// (2048 FPW coordinates); thread t loads words 8 t .. 8 t + 7 with two
// 16-byte loads, decodes their 8 FPW values into LDS, and after one barrier
// the block stores the mean with 16-byte stores, 4 KB per instruction.
template <int SCH, int FPW>
__global__ __launch_bounds__(kThreads) void k_dequantize_words_lds(
    const uint32_t *__restrict__ wsum, int64_t n, int64_t d, int s, int W, uint32_t M,
    int64_t rwords, const float *__restrict__ norm_dev, float *__restrict__ mean)
{
    static_assert(FPW == 3 || FPW == 5 || FPW == 6 || FPW == 10,
                  "field counts whose words do not align with 8 coordinates");
    constexpr int kCoords = kWordsPerBlock * FPW; // coordinates per block
    __shared__ alignas(16) float lds[kCoords];
    const int64_t c_base = (int64_t)blockIdx.x * kCoords;
    const int64_t w0 = (int64_t)blockIdx.x * kWordsPerBlock + (int64_t)threadIdx.x * kPer;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    const uint32_t mask = (1u << W) - 1u; // W <= 10 here
    const uint32_t bias = (uint32_t)(n * (int64_t)M);
    uint32_t w[kPer];
    {
        const uint4 a = (w0 < rwords) ? *(const uint4 *)(wsum + w0) : make_uint4(0, 0, 0, 0);
        const uint4 b = (w0 + 4 < rwords) ? *(const uint4 *)(wsum + w0 + 4) : make_uint4(0, 0, 0, 0);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
            const int32_t v = (int32_t)(((w[u] >> (W * f)) & mask) - bias);
            lds[((int)threadIdx.x * kPer + u) * FPW + f] = (float)((double)v * q.kappa);
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kCoords / (4 * kThreads); ++r) {
        const int c = (r * kThreads + (int)threadIdx.x) * 4;
        const int64_t j = c_base + c;
        if (j + 4 <= d) {
            *(float4 *)(mean + j) = *(const float4 *)(lds + c);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (j + k < d)
                    mean[j + k] = lds[c + k];
        }
    }
}

// A device's own rows summed before the all-reduce: the word row whose
// fields hold sum_i (code_ij + M) over its n rows, as gq_sum_words of the
// rows of k_quantize_words, in one pass with the sum in registers.  Block =
// 2048 words (2048 FPW coordinates); for each of its FPW groups a thread
// walks the n rows for 8 coordinates with the fused pass's accumulators
// (ACC as in k_compress_mean: fp32 sums, int32, or packed 16-bit pairs for
// bf16 standard dithering), then the biased sums go to LDS and are
// assembled into word quads as in k_quantize_words.
// SKIP: with pass 1's span bounds, as the fused pass (each 2048-coordinate
// segment is one fused-pass tile: a wave per 512-coordinate span).
template <int DT, int SCH, int FPW, int ACC, bool SKIP>
__global__ __launch_bounds__(kThreads) void k_compress_words(const void *__restrict__ x, int64_t n,
                                                             int64_t d, int s, uint64_t seed,
                                                             int64_t worker_base,
                                                             const float *__restrict__ norm_dev,
                                                             uint32_t *__restrict__ out, int W,
                                                             uint32_t bias, int64_t rwords,
                                                             const uint16_t *__restrict__ bounds,
                                                             int64_t bstride)
{
    using E = WordLdsT<FPW>;
    __shared__ alignas(16) E lds[FPW > 1 ? kWordsPerBlock * FPW : 1];
    const int64_t tile = blockIdx.x;
    const int64_t c_base = tile * kWordsPerBlock * FPW;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    const bool vec = (d & 7) == 0;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32), wb = (uint32_t)worker_base;
    uint32_t w1[kPer]; // FPW == 1: the thread's 8 words
#pragma unroll(SKIP ? 1 : FPW)
    for (int g = 0; g < FPW; ++g) {
        const int rel = g * kWordsPerBlock + (int)threadIdx.x * kPer;
        const int64_t j0 = c_base + rel;
        int acc[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
        const int64_t span = (c_base + g * kWordsPerBlock) / kSpan + (int64_t)(threadIdx.x >> 6);
        if (SKIP && !q.zero && span * kSpan < d) { // the whole wave
            const bool live = j0 < d;
            const float sigK = q.sigma * (SCH == GQ_SCHEME_L ? 0x1p16f : q.p2E16);
            const bool sparse_ok = sigK < INFINITY;
            if constexpr (ACC == kAccPk16) {
                if (q.prescale)
                    accumulate_workers_pk16<DT, true, true>(x, n, d, j0, vec, q, k0, k1, acc, wb,
                                                            live, bounds, bstride, span, sparse_ok);
                else
                    accumulate_workers_pk16<DT, false, true>(x, n, d, j0, vec, q, k0, k1, acc, wb,
                                                             live, bounds, bstride, span, sparse_ok);
            } else {
                float accf[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (q.prescale)
                    accumulate_workers_skip<DT, SCH, true, ACC == kAccF32>(
                        x, n, d, j0, vec, live, q, k0, k1, bounds, bstride, span, sigK, sparse_ok,
                        accf, acc, wb);
                else
                    accumulate_workers_skip<DT, SCH, false, ACC == kAccF32>(
                        x, n, d, j0, vec, live, q, k0, k1, bounds, bstride, span, sigK, sparse_ok,
                        accf, acc, wb);
                if (ACC == kAccF32) {
#pragma unroll
                    for (int k = 0; k < kPer; ++k)
                        acc[k] = (int)accf[k];
                }
            }
        } else if (!SKIP && !q.zero && j0 < d) {
            if constexpr (ACC == kAccPk16) {
                if (q.prescale)
                    accumulate_workers_pk16<DT, true, false>(x, n, d, j0, vec, q, k0, k1, acc, wb);
                else
                    accumulate_workers_pk16<DT, false, false>(x, n, d, j0, vec, q, k0, k1, acc, wb);
            } else {
                float accf[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (q.prescale)
                    accumulate_workers<DT, SCH, true, ACC == kAccF32>(x, n, d, j0, vec, q, k0, k1,
                                                                      accf, acc, wb);
                else
                    accumulate_workers<DT, SCH, false, ACC == kAccF32>(x, n, d, j0, vec, q, k0,
                                                                       k1, accf, acc, wb);
                if (ACC == kAccF32) {
#pragma unroll
                    for (int k = 0; k < kPer; ++k)
                        acc[k] = (int)accf[k];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const uint32_t b = (j0 + k < d) ? (uint32_t)acc[k] + bias : 0u;
            if constexpr (FPW == 1)
                w1[k] = b;
            else
                lds[rel + k] = (E)b;
        }
    }
    if constexpr (FPW == 1) {
        const int64_t w0 = c_base + (int64_t)threadIdx.x * kPer;
        if (w0 < rwords)
            nt_store((uint8_t *)(out + w0), make_uint4(w1[0], w1[1], w1[2], w1[3]));
        if (w0 + 4 < rwords)
            nt_store((uint8_t *)(out + w0 + 4), make_uint4(w1[4], w1[5], w1[6], w1[7]));
    } else {
        __syncthreads();
        const int64_t w_base = tile * kWordsPerBlock;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int wr = h * (kWordsPerBlock / 2) + 4 * (int)threadIdx.x;
            uint32_t w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t a = 0;
#pragma unroll
                for (int f = 0; f < FPW; ++f)
                    a |= (uint32_t)lds[(wr + u) * FPW + f] << (W * f);
                w[u] = a;
            }
            if (w_base + wr < rwords)
                nt_store((uint8_t *)(out + w_base + wr), make_uint4(w[0], w[1], w[2], w[3]));
        }
    }
}

// The accumulator of k_compress_words for one fields-per-word count: packed
// 16-bit pairs for bf16 standard dithering with n M < 2^15, else fp32 sums
// while n M <= 2^24 (always true for W <= 16), else int32.
// bounds != nullptr: the zero-code skip with pass 1's span bounds.
template <int DT, int SCH, int F, bool SKIP>
void launch_compress_words_as(dim3 grid, hipStream_t st, bool pk16, bool facc, const void *x,
                              int64_t n, int64_t d, int s, uint64_t seed, int64_t worker_base,
                              const float *norm_dev, uint32_t *out, int W, uint32_t bias,
                              int64_t rwords, const uint16_t *bounds, int64_t bstride)
{
    const dim3 block(kThreads);
    if constexpr (DT == GQ_IN_BF16 && SCH == GQ_SCHEME_L && F > 1) {
        if (pk16) {
            k_compress_words<DT, SCH, F, kAccPk16, SKIP><<<grid, block, 0, st>>>(
                x, n, d, s, seed, worker_base, norm_dev, out, W, bias, rwords, bounds, bstride);
            return;
        }
    }
    if constexpr (F > 1) {
        k_compress_words<DT, SCH, F, kAccF32, SKIP><<<grid, block, 0, st>>>(
            x, n, d, s, seed, worker_base, norm_dev, out, W, bias, rwords, bounds, bstride);
    } else {
        if (facc)
            k_compress_words<DT, SCH, F, kAccF32, SKIP><<<grid, block, 0, st>>>(
                x, n, d, s, seed, worker_base, norm_dev, out, W, bias, rwords, bounds, bstride);
        else
            k_compress_words<DT, SCH, F, kAccInt, SKIP><<<grid, block, 0, st>>>(
                x, n, d, s, seed, worker_base, norm_dev, out, W, bias, rwords, bounds, bstride);
    }
}

template <int DT, int SCH, int F>
void launch_compress_words(dim3 grid, hipStream_t st, bool pk16, bool facc, const void *x,
                           int64_t n, int64_t d, int s, uint64_t seed, int64_t worker_base,
                           const float *norm_dev, uint32_t *out, int W, uint32_t bias,
                           int64_t rwords, const uint16_t *bounds)
{
    if (bounds)
        launch_compress_words_as<DT, SCH, F, true>(grid, st, pk16, facc, x, n, d, s, seed,
                                                   worker_base, norm_dev, out, W, bias, rwords,
                                                   bounds, bound_stride(d));
    else
        launch_compress_words_as<DT, SCH, F, false>(grid, st, pk16, facc, x, n, d, s, seed,
                                                    worker_base, norm_dev, out, W, bias, rwords,
                                                    nullptr, 0);
}

// What a native integer SUM over the n rows computes: the word-wise sum
// modulo 2^32.  Thread = 8 consecutive words, the n rows in order.
__global__ __launch_bounds__(kThreads) void k_sum_words(const uint32_t *__restrict__ words,
                                                        int64_t n, int64_t rwords,
                                                        uint32_t *__restrict__ out)
{
    const int64_t w0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    if (w0 >= rwords)
        return;
    const bool two = w0 + 4 < rwords; // rwords is a multiple of 4
    uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t *r = words + i * rwords + w0;
        const uint4 u = *(const uint4 *)r;
        a.x += u.x; a.y += u.y; a.z += u.z; a.w += u.w;
        if (two) {
            const uint4 v = *(const uint4 *)(r + 4);
            b.x += v.x; b.y += v.y; b.z += v.z; b.w += v.w;
        }
    }
    nt_store((uint8_t *)(out + w0), a);
    if (two)
        nt_store((uint8_t *)(out + w0 + 4), b);
}

// Dequantization of a summed row in the word layout: field - n M, times
// kappa (fp64 product, one rounding).  Thread = 8 consecutive coordinates,
// as in k_dequantize, so the mean stores of a wave are contiguous; each
// coordinate reads its own word (neighbours share words through the cache).
// One 64-bit division per thread finds the first word and field; the 8
// offsets from there are small constant divisions.
template <int SCH, int FPW>
__global__ __launch_bounds__(kThreads) void k_dequantize_words(const uint32_t *__restrict__ wsum,
                                                               int64_t n, int64_t d, int s, int W,
                                                               uint32_t M,
                                                               const float *__restrict__ norm_dev,
                                                               float *__restrict__ mean)
{
    const int64_t j0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    if (j0 >= d)
        return;
    const QParams q = make_qparams(*norm_dev, n, s, SCH);
    const uint32_t mask = W == 32 ? 0xFFFFFFFFu : ((1u << W) - 1u);
    // n M < 2^31 (the width rule), so field - n M is an int32 and converts
    // to fp64 in one instruction (an int64 conversion is a long sequence)
    const uint32_t bias = (uint32_t)(n * (int64_t)M);
    const int64_t w0 = j0 / FPW;
    const uint32_t r0 = (uint32_t)(j0 - w0 * FPW); // field of coordinate j0, < FPW
    const uint32_t *row = wsum + w0;
    // all loads first, unconditional inside the row (loads each behind its
    // own branch were issued one round trip at a time: 37 vs 27 us on
    // 25.6M coordinates); fields past d read 0 and are not stored
    uint32_t wv[kPer];
    if (j0 + kPer <= d) {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            wv[k] = row[(r0 + (uint32_t)k) / FPW];
    } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            wv[k] = (j0 + k < d) ? row[(r0 + (uint32_t)k) / FPW] : 0u;
    }
    float m[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint32_t r = r0 + (uint32_t)k, f = r - (r / FPW) * FPW;
        const int32_t v = (int32_t)(((wv[k] >> (W * f)) & mask) - bias);
        m[k] = (float)((double)v * q.kappa);
    }
    store_mean8<false>(mean, j0, d, m);
}

// Ablation: local-norm QSGD.  Worker i uses its own scalars; the mean is an
// fp64 sum in worker order.  Optional per-worker packed codes.
// SKIP: with pass 1's span bounds, a worker's group whose codes are
// provably 0 is not loaded (as in the fused pass, with each worker's own
// sigma); skipping it drops a term fp64(0 kappa_i) = +0 from a sum that is
// never -0, so the mean keeps its bits.  A worker whose kappa_i or
// sigma_i 2^16 is not finite is read whole (0 times inf is NaN).
template <int DT, bool SKIP>
__global__ __launch_bounds__(kThreads) void k_local_mean(const void *__restrict__ x, int64_t n,
                                                         int64_t d, int s, uint64_t seed,
                                                         const float *__restrict__ norms,
                                                         const WorkerParams *__restrict__ params,
                                                         float *__restrict__ mean,
                                                         uint8_t *__restrict__ codes, int W,
                                                         int64_t rbytes,
                                                         const uint16_t *__restrict__ bounds,
                                                         int64_t bstride)
{
    __shared__ alignas(16) uint32_t lds[kTile];
    // reverse of pass 1's order, as in the fused pass
    const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t j0 = tile * kTile + (int64_t)threadIdx.x * kPer;
    const bool vec = (d & 7) == 0;
    const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    // one span per wave; its thresholds exist when the span starts in the row
    const int64_t span = tile * (kTile / kSpan) + (int64_t)(threadIdx.x >> 6);
    const bool wave_in = span * kSpan < d;
    double acc[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t Hl = 0x10000u;
    for (int64_t i = 0; i < n; ++i) {
        if (SKIP && (i & 63) == 0 && wave_in) {
            // lane l: worker i + l's threshold for this span (0x10000: dense)
            const int64_t r = i + (int64_t)(threadIdx.x & 63);
            Hl = 0x10000u;
            if (r < n) {
                const WorkerParams pr = params[r];
                const float sig16 = pr.sigma * 0x1p16f;
                const uint32_t b = bounds[r * bstride + span];
                if (sig16 < INFINITY && isfinite(pr.kappa) && b < 0x7F80u) {
                    const float th = (__uint_as_float(b << 16) * pr.pre) * sig16;
                    if (th < 65536.0f)
                        Hl = (uint32_t)th;
                }
            }
        }
        const uint32_t H = (SKIP && wave_in) ? __builtin_amdgcn_readlane(Hl, (int)(i & 63)) : 0x10000u;
        int code[kPer] = {0, 0, 0, 0, 0, 0, 0, 0};
        const WorkerParams wp = params[i];
        if (j0 < d && norms[i] != 0.0f) {
            const uint4 A = philox10(make_uint4(blo, bhi, (uint32_t)i, 0u), k0, k1);
            if (H > 0xFFFFu || min_half16(A) <= H) {
                QParams q = {};
                q.pre = wp.pre;
                q.sigma = wp.sigma;
                q.top = (float)s;
                q.s = s;
                float v[kPer];
                load_group<DT>(x, i * d, j0, d, vec, v);
                float m[kPer];
                bool tie = false;
                const bool pre = wp.pre != 1.0f;
                if (H <= 0xFFFFu) {
                    if (pre)
                        quant_group_sparse<true>(v, A, q, wp.sigma * 0x1p16f, m, tie);
                    else
                        quant_group_sparse<false>(v, A, q, wp.sigma * 0x1p16f, m, tie);
                } else if (pre) {
                    quant_group<GQ_SCHEME_L, true>(v, A, q, m, tie);
                } else {
                    quant_group<GQ_SCHEME_L, false>(v, A, q, m, tie);
                }
                if (tie) {
                    const uint4 B = philox10(make_uint4(blo, bhi, (uint32_t)i, 1u), k0, k1);
                    if (pre)
                        settle_ties<GQ_SCHEME_L, true>(v, A, B, q, m);
                    else
                        settle_ties<GQ_SCHEME_L, false>(v, A, B, q, m);
                }
#pragma unroll
                for (int k = 0; k < kPer; ++k) {
                    code[k] = (int)copysignf(m[k], v[k]);
                    acc[k] = acc[k] + (double)code[k] * wp.kappa;
                }
            }
        }
        if (codes)
            store_tile_packed(lds, code, W, codes + i * rbytes, tile, rbytes);
    }
    if (j0 < d) {
        float m[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            m[k] = (float)acc[k];
        store_mean8(mean, j0, d, m);
    }
}

// ---------------------------------------------------------------------------
// The pages' own 8-bit exponential-dithering wire format and its re-rounding
// tree reduction.  Code byte: bit 7 sign, bits 0..6 level index k; k = 0 is
// the level 0, k >= 1 the level 2^(1-k) (s = 127).  A tree node is the
// average of its two children, added in fp64 and rounded again at random,
// without bias, onto the same grid; the draws of tree level l at node m use
// Philox counter words (lo32(j/8), hi32(j/8), m, 2 l + draw), level 0 being
// the quantization.  n is a power of two up to kE8MaxN.

constexpr int kE8MaxLevels = 10;
constexpr int64_t kE8MaxN = (int64_t)1 << kE8MaxLevels;

__device__ __forceinline__ double e8_value(uint32_t c)
{
    const uint32_t idx = c & 0x7Fu;
    const uint64_t bits = ((uint64_t)(c & 0x80u) << 56) | ((uint64_t)(1024u - idx) << 52);
    return idx ? __longlong_as_double((long long)bits) : 0.0;
}

// Half the values of the four codes in a word, as fp64 high words (the low
// words are 0): exponent field 1023 - k for index k >= 1, so that a parent is
// the plain fp64 sum of its children's halves.  The level 0 becomes
// +-2^-256 instead of 0: far below half an ulp of every other half value
// (>= 2^-128), it leaves every sum with a nonzero half unchanged, and two of
// them sum to 0 or +-2^-255, which rounds to the level 0 like 0 does.
// Per byte, ((k & 127) + 127) ^ 128 is k - 1, or 255 for k = 0, with no
// carries between bytes, so the exponent field is 1022 minus that byte.
__device__ __forceinline__ void e8_half_hi4(uint32_t w, uint32_t *hi)
{
    const uint32_t g4 = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) ^ 0x80808080u;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        hi[b] = ((1022u - ((g4 >> (8 * b)) & 0xFFu)) << 20) | ((w << (24 - 8 * b)) & 0x80000000u);
}

// The same half values for all 256 code bytes as fp64, one LDS entry per
// thread of a 256-thread block (2 KB), then a block barrier.  Decoding a
// byte through this table takes one address computation instead of the
// byte-parallel arithmetic above (~90 of ~255 VALU instructions of an
// 8-coordinate combine), and a 64-bit entry loads the zero low word with
// the value (16 moves fewer); LDS issue stays far below the VALU time.
__device__ __forceinline__ void e8_fill_half_table(double *tab)
{
    static_assert(kThreads == 256, "one table entry per thread");
    uint32_t hi[4];
    e8_half_hi4(threadIdx.x, hi);
    tab[threadIdx.x] = __hiloint2double((int)hi[0], 0);
    __syncthreads();
}

// Main-path rounding of one coordinate to a code.  X holds the biased
// exponent of the value in bits 16 and up and the top 16 fraction bits
// (F >> 16) below; base - exponent is the index of the lower level.  Adding
// hcomp = 0xFFFF - h (h the 16-bit half of the uniform) carries into bit 16
// iff h < F >> 16, which is the step up to the next level (index - 1).  A
// low half of 0xFFFF after the add is the tie h == F >> 16, settled by the
// second draw.  Indices above 127 are the level 0 (no sign).
__device__ __forceinline__ uint32_t e8_round_fields(uint32_t X, uint32_t base, uint32_t hcomp,
                                                    uint32_t sign, bool &tie)
{
    const uint32_t S = X + hcomp;
    tie |= (S & 0xFFFFu) == 0xFFFFu;
    const uint32_t idx = base - (S >> 16);
    return idx > 127u ? 0u : (sign | idx);
}

__device__ __forceinline__ uint32_t comp16(const uint32_t (&Ac)[kPer / 2], int k)
{
    return (k & 1) ? (Ac[k >> 1] >> 16) : (Ac[k >> 1] & 0xFFFFu);
}

// Rounding fields of a parent value v.  The parent of two codes has |v| <= 1
// and is 0, +-2^-255 (two level-0 halves), +-2^-127 or at least 2^-126 in
// magnitude (the smallest nonzero halves and half-differences of two levels
// >= 2^-126 are 2^-127).
// |v| >= 2^-126: v = 2^e (1 + phi) lies between the codes of 2^e (index
// lo = 1 - e, returned) and 2^(e+1) (index lo - 1), F = the top 32 bits of
// phi.  +-2^-127: lo = 128, standing for the level 0, below 2^-126 (index
// 127), F = 2^31.  0 and +-2^-255: lo = 1024 or 256, F = 0.  Indices above
// 127 are the level 0.
// The code taken is sign | (lo - [u < F]), upper iff u < F.
__device__ __forceinline__ uint32_t e8_pair_fields(double v, uint32_t &sign, uint32_t &F)
{
    const uint32_t vh = (uint32_t)__double2hiint(v), vl = (uint32_t)__double2loint(v);
    const uint32_t ef = (vh >> 20) & 0x7FFu; // biased exponent, e = ef - 1023
    sign = (vh >> 24) & 0x80u;
    F = ef == 896u ? 0x80000000u : __builtin_amdgcn_alignbit(vh, vl, 20);
    return 1024u - ef;
}

__device__ __forceinline__ uint32_t e8_pair_code(uint32_t sign, uint32_t idx)
{
    return idx > 127u ? 0u : (sign | idx);
}

// Quantization to 8-bit codes: Global-E_s with s = 127 in the byte format.
// t = min(fp32(|x| pre sigma), 1), sigma = fp32(1 / (N pre)).
template <bool PRE>
__device__ __forceinline__ void e8_quant_bracket(float xv, const QParams &q, uint32_t &lo,
                                                 uint32_t &hi, uint32_t &F)
{
    float a = fabsf(xv);
    if (PRE)
        a = a * q.pre;
    const float t = fminf(a * q.sigma, 1.0f);
    const uint32_t tb = __float_as_uint(t);
    const uint32_t sign = __float_as_uint(xv) & 0x80000000u ? 0x80u : 0u;
    if (tb >= 0x00800000u) {
        F = tb << 9;
        lo = sign | (128u - (tb >> 23));
        hi = sign | (127u - (tb >> 23));
    } else {
        F = (uint32_t)((t * 0x1p126f) * 0x1p32f);
        lo = 0u;
        hi = sign | 127u;
    }
}

__device__ __forceinline__ uint32_t byte_of(const uint2 &w, int k)
{
    return ((k < 4 ? w.x : w.y) >> (8 * (k & 3))) & 0xFFu;
}

__device__ __forceinline__ uint2 pack_bytes(const uint32_t (&c)[kPer])
{
    return make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24,
                      c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
}

// One custom reduction of 8 coordinates: codes a (left child) and b (right),
// with the same draws and lazy second draw as the quantization.  Main path:
// the parent's fp64 high word gives X (exponent and top fraction bits; for
// +-2^-127, between the level 0 and 2^-126, F >> 16 = 2^15 is set in).
__device__ __forceinline__ uint2 e8_combine(const double *tab, const uint2 &a, const uint2 &b,
                                            uint32_t blo, uint32_t bhi, uint32_t node,
                                            uint32_t level, uint32_t k0, uint32_t k1)
{
    const uint4 A = philox10(make_uint4(blo, bhi, node, 2u * level), k0, k1);
    const uint32_t Ac[kPer / 2] = {~A.x, ~A.y, ~A.z, ~A.w};
    double v[kPer];
    uint32_t c[kPer], S[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        v[k] = tab[byte_of(a, k)] + tab[byte_of(b, k)];
        const uint32_t vh = (uint32_t)__double2hiint(v[k]);
        uint32_t X = (vh >> 4) & 0x7FFFFFFu;
        if (X == (896u << 16))
            X |= 0x8000u;
        S[k] = (k & 1) ? add_half16<1>(X, Ac[k >> 1]) : add_half16<0>(X, Ac[k >> 1]);
        const uint32_t idx = 1024u - (S[k] >> 16);
        c[k] = idx > 127u ? 0u : (((vh >> 24) & 0x80u) | idx);
    }
    // a tie leaves the low half of its sum at 0xFFFF (as in e8_round_fields)
    const uint32_t mx = max3_lo16(S[6], S[7], max3_lo16(S[0], S[1], S[2]));
    const bool tie = ((uint16_t)mx == 0xFFFFu) | ((uint16_t)max3_lo16(S[3], S[4], S[5]) == 0xFFFFu);
    if (tie) {
        const uint4 B = philox10(make_uint4(blo, bhi, node, 2u * level + 1u), k0, k1);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            uint32_t sign, F;
            const uint32_t lo = e8_pair_fields(v[k], sign, F);
            if (half16(A, k) == (F >> 16) && half16(B, k) < (F & 0xFFFFu))
                c[k] = e8_pair_code(sign, lo - 1u);
        }
    }
    return pack_bytes(c);
}

// Binary-counter tree: leaf i enters; while bit l of i is set, it is combined
// with the stored left sibling at level l into their parent (level l + 1,
// node i >> (l + 1)).  The same pairs as the level-by-level tree.  The stack
// lives in LDS, slot l of thread t at stk[l kThreads + t]: each thread reads
// only what it wrote, so no barrier is needed, and the loop keeps a single
// copy of the combine (the stack unrolled in registers took 132-136 VGPRs,
// 3 waves per SIMD).  i is wave-uniform, so the loop is uniform.  Level
// kE8MaxLevels is reached only by the last leaf of a full tree, whose
// result is the root itself, so it needs no slot.
constexpr int kE8StackSlots = kE8MaxLevels * kThreads;

// wb is the global index of leaf 0 (0, or a multiple of the subtree's leaf
// count): the parent at level l + 1 is node (wb + i) >> (l + 1) of the
// whole tree, so a subtree held by one device draws what the whole tree
// draws there.
__device__ __forceinline__ uint2 e8_push(const double *tab, uint2 *stk, uint2 cur, int64_t i,
                                         int64_t wb, uint32_t blo, uint32_t bhi, uint32_t k0,
                                         uint32_t k1)
{
    int l = 0;
    for (; (i >> l) & 1; ++l)
        cur = e8_combine(tab, stk[l * kThreads + threadIdx.x], cur, blo, bhi,
                         (uint32_t)((wb + i) >> (l + 1)), (uint32_t)(l + 1), k0, k1);
    if (l < kE8MaxLevels)
        stk[l * kThreads + threadIdx.x] = cur;
    return cur;
}

__device__ __forceinline__ uint2 load_codes8(const uint8_t *row, int64_t j0, int64_t d)
{
    if (j0 + kPer <= d)
        return *(const uint2 *)(row + j0);
    uint32_t c[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        c[k] = (j0 + k < d) ? row[j0 + k] : 0u;
    return pack_bytes(c);
}

__device__ __forceinline__ void store_codes8(uint8_t *row, int64_t j0, int64_t d, const uint2 &w)
{
    if (j0 + kPer <= d) {
        nt_store(row + j0, w);
        return;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        if (j0 + k < d)
            row[j0 + k] = (uint8_t)byte_of(w, k);
}

// Quantization of 8 coordinates to codes.  Main path: t = min(fp32(|x| pre
// sigma), 1) has exponent field eb and F = its fraction bits << 9, so
// X = bits(t) >> 7 and the lower level's index is 128 - eb; a subnormal t
// (eb = 0) gives index 128, the level 0, below 2^-126 (index 127), with the
// same F as the plain bracket.
template <int DT, bool PRE>
__device__ __forceinline__ uint2 e8_quant8(const void *__restrict__ x, int64_t row_off, int64_t j0,
                                           int64_t d, bool vec, const QParams &q, uint32_t worker,
                                           uint32_t blo, uint32_t bhi, uint32_t k0, uint32_t k1)
{
    float v[kPer];
    load_group<DT>(x, row_off, j0, d, vec, v);
    const uint4 A = philox10(make_uint4(blo, bhi, worker, 0u), k0, k1);
    const uint32_t Ac[kPer / 2] = {~A.x, ~A.y, ~A.z, ~A.w};
    uint32_t c[kPer];
    bool tie = false;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        float a = fabsf(v[k]);
        if (PRE)
            a = a * q.pre;
        const uint32_t X = __float_as_uint(fminf(a * q.sigma, 1.0f)) >> 7;
        c[k] = e8_round_fields(X, 128u, comp16(Ac, k), (__float_as_uint(v[k]) >> 24) & 0x80u, tie);
    }
    if (tie) {
        const uint4 B = philox10(make_uint4(blo, bhi, worker, 1u), k0, k1);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            uint32_t lo, hi, F;
            e8_quant_bracket<PRE>(v[k], q, lo, hi, F);
            if (half16(A, k) == (F >> 16) && half16(B, k) < (F & 0xFFFFu))
                c[k] = hi;
        }
    }
    return pack_bytes(c);
}

// The same codes through the plain bracket: one compare of h with F >> 16.
// The standalone quantization kernel, bound by HBM with its byte writes
// interleaved, measured 4-6% faster with this form than with the carry form
// (which issues fewer VALU instructions); the fused tree path is faster with
// the carry form.
template <int DT, bool PRE>
__device__ __forceinline__ uint2 e8_quant8_plain(const void *__restrict__ x, int64_t row_off,
                                                 int64_t j0, int64_t d, bool vec, const QParams &q,
                                                 uint32_t worker, uint32_t blo, uint32_t bhi,
                                                 uint32_t k0, uint32_t k1)
{
    float v[kPer];
    load_group<DT>(x, row_off, j0, d, vec, v);
    const uint4 A = philox10(make_uint4(blo, bhi, worker, 0u), k0, k1);
    uint32_t c[kPer];
    bool tie = false;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        uint32_t lo, hi, F;
        e8_quant_bracket<PRE>(v[k], q, lo, hi, F);
        const uint32_t h = half16(A, k), Fh = F >> 16;
        c[k] = (h < Fh) ? hi : lo;
        tie |= (h == Fh);
    }
    if (tie) {
        const uint4 B = philox10(make_uint4(blo, bhi, worker, 1u), k0, k1);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            uint32_t lo, hi, F;
            e8_quant_bracket<PRE>(v[k], q, lo, hi, F);
            if (half16(A, k) == (F >> 16) && half16(B, k) < (F & 0xFFFFu))
                c[k] = hi;
        }
    }
    return pack_bytes(c);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_e8_quantize(const void *__restrict__ x, int64_t n,
                                                          int64_t d, uint64_t seed,
                                                          int64_t worker_base,
                                                          const float *__restrict__ norm_dev,
                                                          uint8_t *__restrict__ codes,
                                                          int64_t rbytes, int64_t tiles)
{
    const int64_t i = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int64_t j0 = tile * kTile + (int64_t)threadIdx.x * kPer;
    if (j0 >= d)
        return;
    const QParams q = make_qparams(*norm_dev, n, 127, GQ_SCHEME_E);
    uint2 w = make_uint2(0, 0);
    if (!q.zero) {
        const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
        const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
        const bool vec = (d & 7) == 0;
        const uint32_t wk = (uint32_t)(worker_base + i);
        w = q.prescale ? e8_quant8_plain<DT, true>(x, i * d, j0, d, vec, q, wk, blo, bhi, k0, k1)
                       : e8_quant8_plain<DT, false>(x, i * d, j0, d, vec, q, wk, blo, bhi, k0, k1);
    }
    store_codes8(codes + i * rbytes, j0, d, w);
}

__global__ __launch_bounds__(kThreads) void k_e8_pair(const uint8_t *__restrict__ a,
                                                      const uint8_t *__restrict__ b, int64_t d,
                                                      uint64_t seed, uint32_t level, uint32_t node,
                                                      uint8_t *__restrict__ out)
{
    __shared__ double tab[256];
    e8_fill_half_table(tab);
    const int64_t j0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    if (j0 >= d)
        return;
    const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
    const uint2 r = e8_combine(tab, load_codes8(a, j0, d), load_codes8(b, j0, d), blo, bhi, node,
                               level, (uint32_t)seed, (uint32_t)(seed >> 32));
    store_codes8(out, j0, d, r);
}

__global__ __launch_bounds__(kThreads) void k_e8_tree(const uint8_t *__restrict__ codes, int64_t n,
                                                      int64_t d, int64_t rbytes, uint64_t seed,
                                                      int64_t wb, uint8_t *__restrict__ root)
{
    __shared__ double tab[256];
    __shared__ uint2 stk[kE8StackSlots];
    e8_fill_half_table(tab);
    const int64_t j0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    if (j0 >= d)
        return;
    const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    uint2 cur = make_uint2(0, 0);
    for (int64_t i = 0; i < n; ++i)
        cur = e8_push(tab, stk, load_codes8(codes + i * rbytes, j0, d), i, wb, blo, bhi, k0, k1);
    store_codes8(root, j0, d, cur);
}

__global__ __launch_bounds__(kThreads) void k_e8_dequantize(const uint8_t *__restrict__ root,
                                                            int64_t d,
                                                            const float *__restrict__ norm_dev,
                                                            float *__restrict__ mean)
{
    const int64_t j0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    if (j0 >= d)
        return;
    const double N = (double)*norm_dev;
    const uint2 w = load_codes8(root, j0, d);
    float m[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        m[k] = (float)(N * e8_value(byte_of(w, k)));
    store_mean8<false>(mean, j0, d, m);
}

// Fused: quantize the n workers' coordinates, reduce them through the tree in
// registers, dequantize the root.  Tiles in reverse of pass 1's order.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_e8_compress_mean(const void *__restrict__ x, int64_t n,
                                                               int64_t d, uint64_t seed,
                                                               const float *__restrict__ norm_dev,
                                                               float *__restrict__ mean,
                                                               uint8_t *__restrict__ root)
{
    __shared__ double tab[256];
    __shared__ uint2 stk[kE8StackSlots];
    e8_fill_half_table(tab);
    const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t j0 = tile * kTile + (int64_t)threadIdx.x * kPer;
    if (j0 >= d)
        return;
    const float N = *norm_dev;
    const QParams q = make_qparams(N, n, 127, GQ_SCHEME_E);
    uint2 cur = make_uint2(0, 0);
    if (!q.zero) {
        const uint32_t blo = (uint32_t)((uint64_t)j0 >> 3), bhi = (uint32_t)((uint64_t)j0 >> 35);
        const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
        const bool vec = (d & 7) == 0;
        for (int64_t i = 0; i < n; ++i) {
            const uint2 leaf = q.prescale
                ? e8_quant8<DT, true>(x, i * d, j0, d, vec, q, (uint32_t)i, blo, bhi, k0, k1)
                : e8_quant8<DT, false>(x, i * d, j0, d, vec, q, (uint32_t)i, blo, bhi, k0, k1);
            cur = e8_push(tab, stk, leaf, i, 0, blo, bhi, k0, k1);
        }
    }
    if (root)
        store_codes8(root, j0, d, cur);
    float m[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        m[k] = (float)((double)N * e8_value(byte_of(cur, k)));
    store_mean8(mean, j0, d, m);
}

// ---------------------------------------------------------------------------
// Launch helpers

int32_t check_launch(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(GQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int32_t validate_x(const void *x, int32_t dtype, int64_t n, int64_t d)
{
    if (dtype != GQ_IN_F32 && dtype != GQ_IN_BF16)
        return fail(GQ_ERR_ARG, "dtype %d is not GQ_IN_F32 or GQ_IN_BF16", dtype);
    if (n < 1 || n > 0x7FFFFFFF)
        return fail(GQ_ERR_ARG, "n = %lld must be in [1, 2^31)", (long long)n);
    if (d < 0)
        return fail(GQ_ERR_ARG, "d = %lld is negative", (long long)d);
    if (d > 0 && n > INT64_MAX / 8 / d)
        return fail(GQ_ERR_ARG, "n * d overflows");
    if (!x && d > 0)
        return fail(GQ_ERR_NULL, "x is NULL");
    if (!aligned16(x))
        return fail(GQ_ERR_ALIGN, "x is not 16-byte aligned");
    if ((d + kTile - 1) / kTile > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d = %lld exceeds the launch limit", (long long)d);
    return GQ_OK;
}

int32_t validate_scheme(int32_t s, int32_t scheme)
{
    if (scheme != GQ_SCHEME_L && scheme != GQ_SCHEME_E)
        return fail(GQ_ERR_ARG, "scheme %d is not GQ_SCHEME_L or GQ_SCHEME_E", scheme);
    if (!s_ok(s, scheme))
        return fail(GQ_ERR_ARG, "s = %d out of range for the scheme", s);
    return GQ_OK;
}

int32_t validate_width(int64_t n, int32_t s, int32_t scheme, int32_t W)
{
    const int32_t wmin = min_bits(n, s, scheme);
    if (wmin < 0 || wmin > 32)
        return fail(GQ_ERR_CODE_WIDTH, "sums of %lld codes need %d > 32 bits", (long long)n, wmin);
    if (W < wmin || W > 32)
        return fail(GQ_ERR_CODE_WIDTH, "code_bits %d outside [%d, 32]", W, wmin);
    return GQ_OK;
}

int32_t validate_ws(const void *ws, int64_t ws_bytes, int64_t n, int64_t d)
{
    const WsLayout L = ws_layout(n, d);
    if (!ws)
        return fail(GQ_ERR_NULL, "workspace is NULL");
    if (!aligned16(ws))
        return fail(GQ_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (ws_bytes < L.total)
        return fail(GQ_ERR_WORKSPACE, "workspace of %lld bytes < %lld needed", (long long)ws_bytes,
                    (long long)L.total);
    return GQ_OK;
}

#define GQ_TRY(expr)                  \
    do {                              \
        const int32_t st_ = (expr);   \
        if (st_ != GQ_OK)             \
            return st_;               \
    } while (0)

// Enqueue pass 1 (partials + finalize).  Arguments already validated.
// bounds: if not NULL, pass 1 also stores the span bounds there (u16
// [n][bound_stride(d)]) for the zero-code skip of the fused pass.
int32_t launch_norm(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                    bool local, float *norm_out, void *ws, int s, hipStream_t st,
                    double *term_out = nullptr, uint16_t *bounds = nullptr)
{
    const int64_t bstride = bound_stride(d);
    const NormGeom g = norm_geom(n, d);
    const OneShotGeom o = oneshot_geom(n, d, dtype == GQ_IN_F32 ? 4 : 2);
    const WsLayout L = ws_layout(n, d);
    double *partials = (double *)((char *)ws + L.partials);
    double *mid = (double *)((char *)ws + L.mid);
    double *per_worker = (double *)((char *)ws + L.per_worker);
    WorkerParams *params = (WorkerParams *)((char *)ws + L.params);
    const bool qinf = is_inf_order(q), pinf = is_inf_order(p);
    const int qm = qinf ? 1 : (is_two(q) ? 0 : 2);
    const bool gen = !((qinf || is_two(q)) && (pinf || is_two(p)));
    const double qd = qinf ? 0.0 : (double)q, pd = pinf ? 0.0 : (double)p;
    const double *fin_in = partials;
    int64_t fin_chunks = g.chunks;
    if (o.on) {
        if (n * o.bpr > kMaxGrid || n * o.gpr > kMaxGrid)
            return fail(GQ_ERR_UNSUPPORTED, "norm grid too large");
        const dim3 grid((unsigned)(n * o.bpr)), block(kOsThreads);
#define GQ_ONESHOT(DT, QM) \
    k_norm_oneshot<DT, QM><<<grid, block, 0, st>>>(x, d, o.bpr, o.span, qd, partials, bounds, bstride)
        if (dtype == GQ_IN_F32) {
            if (qm == 0) GQ_ONESHOT(GQ_IN_F32, 0); else if (qm == 1) GQ_ONESHOT(GQ_IN_F32, 1); else GQ_ONESHOT(GQ_IN_F32, 2);
        } else {
            if (qm == 0) GQ_ONESHOT(GQ_IN_BF16, 0); else if (qm == 1) GQ_ONESHOT(GQ_IN_BF16, 1); else GQ_ONESHOT(GQ_IN_BF16, 2);
        }
#undef GQ_ONESHOT
        GQ_TRY(check_launch("k_norm_oneshot"));
        const dim3 mgrid((unsigned)(n * o.gpr)), mblock(kMidThreads);
        if (qinf)
            k_norm_mid<true><<<mgrid, mblock, 0, st>>>(partials, o.bpr, o.gpr, mid);
        else
            k_norm_mid<false><<<mgrid, mblock, 0, st>>>(partials, o.bpr, o.gpr, mid);
        GQ_TRY(check_launch("k_norm_mid"));
        fin_in = mid;
        fin_chunks = o.gpr;
    } else if (g.blocks > 0) {
        if (g.blocks > kMaxGrid)
            return fail(GQ_ERR_UNSUPPORTED, "norm grid too large");
        const dim3 grid((unsigned)g.blocks), block(kThreads);
#define GQ_PARTIAL(DT, QM) \
    k_norm_partial<DT, QM><<<grid, block, 0, st>>>(x, n, d, g.chunks, g.chunk_len, qd, partials, \
                                                   bounds, bstride)
        if (dtype == GQ_IN_F32) {
            if (qm == 0) GQ_PARTIAL(GQ_IN_F32, 0); else if (qm == 1) GQ_PARTIAL(GQ_IN_F32, 1); else GQ_PARTIAL(GQ_IN_F32, 2);
        } else {
            if (qm == 0) GQ_PARTIAL(GQ_IN_BF16, 0); else if (qm == 1) GQ_PARTIAL(GQ_IN_BF16, 1); else GQ_PARTIAL(GQ_IN_BF16, 2);
        }
#undef GQ_PARTIAL
        GQ_TRY(check_launch("k_norm_partial"));
    }
    const dim3 one(1), block(kFinThreads);
#define GQ_FIN(QI, PI, LO, GE) \
    k_norm_finalize<QI, PI, LO, GE><<<one, block, 0, st>>>(fin_in, n, fin_chunks, per_worker, norm_out, s, params, qd, pd, term_out)
    if (local)
        GQ_FIN(false, false, true, false);
    else if (gen) {
        if (qinf && pinf) GQ_FIN(true, true, false, true);
        else if (qinf) GQ_FIN(true, false, false, true);
        else if (pinf) GQ_FIN(false, true, false, true);
        else GQ_FIN(false, false, false, true);
    } else if (qinf && pinf)
        GQ_FIN(true, true, false, false);
    else if (qinf)
        GQ_FIN(true, false, false, false);
    else if (pinf)
        GQ_FIN(false, true, false, false);
    else
        GQ_FIN(false, false, false, false);
#undef GQ_FIN
    return check_launch("k_norm_finalize");
}

// The staged compress step: mean == nullptr launches the pass that writes
// the 1-byte sums, otherwise the kernel that turns them into the mean.
int32_t launch_sums8(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                     int32_t scheme, uint64_t seed, const float *norm_dev, uint8_t *sums8,
                     float *mean, hipStream_t st)
{
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    const dim3 grid((unsigned)tiles), block(kThreads);
    const bool facc = n * top_code(s, scheme) <= ((int64_t)1 << 24);
#define GQ_S8(DT, SCH, ACC)                                                                        \
    do {                                                                                           \
        if (!mean)                                                                                 \
            k_compress_sums8<DT, SCH, ACC><<<grid, block, 0, st>>>(x, n, d, s, seed, norm_dev,     \
                                                                   sums8);                         \
        else                                                                                       \
            k_dequantize_sums8<DT, SCH, ACC><<<grid, block, 0, st>>>(x, n, d, s, seed, norm_dev,   \
                                                                     sums8, mean);                 \
    } while (0)
#define GQ_S8_DT(DT)                                     \
    do {                                                 \
        if (scheme == GQ_SCHEME_L) {                     \
            if (facc)                                    \
                GQ_S8(DT, GQ_SCHEME_L, kAccF32);         \
            else                                         \
                GQ_S8(DT, GQ_SCHEME_L, kAccInt);         \
        } else if (facc)                                 \
            GQ_S8(DT, GQ_SCHEME_E, kAccF32);             \
        else                                             \
            GQ_S8(DT, GQ_SCHEME_E, kAccInt);             \
    } while (0)
    if (dtype == GQ_IN_F32)
        GQ_S8_DT(GQ_IN_F32);
    else
        GQ_S8_DT(GQ_IN_BF16);
#undef GQ_S8_DT
#undef GQ_S8
    return check_launch(mean ? "k_dequantize_sums8" : "k_compress_sums8");
}

// bounds: pass 1's span bounds for the zero-code skip, or NULL.
int32_t launch_compress(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                        int32_t scheme, uint64_t seed, const float *norm_dev, int32_t W,
                        float *mean, void *code_sum, hipStream_t st,
                        const uint16_t *bounds = nullptr)
{
    const int64_t bstride = bound_stride(d);
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    const dim3 grid((unsigned)tiles), block(kThreads);
    uint8_t *cs = (uint8_t *)code_sum;
    // fp32 accumulation is exact while every partial sum stays within 2^24;
    // packed int16 sums for bf16 standard dithering while n s < 2^15
    const int64_t nm = n * top_code(s, scheme);
    const bool facc = nm <= ((int64_t)1 << 24);
    const bool pk16 = dtype == GQ_IN_BF16 && scheme == GQ_SCHEME_L && nm < ((int64_t)1 << 15);
#define GQ_COMPRESS(DT, SCH, ACC)                                                                 \
    do {                                                                                          \
        if (bounds)                                                                               \
            k_compress_mean<DT, SCH, ACC, true><<<grid, block, 0, st>>>(x, n, d, s, seed, norm_dev, \
                                                                        mean, cs, W, bounds, bstride); \
        else                                                                                      \
            k_compress_mean<DT, SCH, ACC, false><<<grid, block, 0, st>>>(x, n, d, s, seed,         \
                                                                         norm_dev, mean, cs, W,   \
                                                                         nullptr, 0);             \
    } while (0)
#define GQ_COMPRESS_DT(DT)                          \
    do {                                            \
        if (scheme == GQ_SCHEME_L) {                \
            if (facc)                               \
                GQ_COMPRESS(DT, GQ_SCHEME_L, kAccF32); \
            else                                    \
                GQ_COMPRESS(DT, GQ_SCHEME_L, kAccInt); \
        } else if (facc)                            \
            GQ_COMPRESS(DT, GQ_SCHEME_E, kAccF32);  \
        else                                        \
            GQ_COMPRESS(DT, GQ_SCHEME_E, kAccInt);  \
    } while (0)
    if (dtype == GQ_IN_F32)
        GQ_COMPRESS_DT(GQ_IN_F32);
    else if (pk16)
        GQ_COMPRESS(GQ_IN_BF16, GQ_SCHEME_L, kAccPk16);
    else
        GQ_COMPRESS_DT(GQ_IN_BF16);
#undef GQ_COMPRESS_DT
#undef GQ_COMPRESS
    return check_launch("k_compress_mean");
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices]; // address of `scratch` on each device, once looked up

// Device address of the current device's copy of `scratch`, looked up on
// the first call on that device.  stream, if not NULL, must belong to it.
int32_t noalloc_scratch(hipStream_t stream, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(GQ_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GQ_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    if (stream) {
        int sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess)
            return fail(GQ_ERR_DEVICE, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(GQ_ERR_ARG, "stream belongs to device %d, the current device is %d",
                        sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(GQ_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return GQ_OK;
}

} // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

int32_t gq_min_code_bits(int64_t n, int32_t s, int32_t scheme) { return min_bits(n, s, scheme); }

int64_t gq_code_row_bytes(int64_t d, int32_t code_bits)
{
    if (d < 0 || code_bits < 1 || code_bits > 32 || d > INT64_MAX / 64)
        return -1;
    return row_bytes(d, code_bits);
}

int64_t gq_workspace_bytes(int64_t n, int64_t d)
{
    if (n < 1 || n > 0x7FFFFFFF || d < 0 || (d > 0 && n > INT64_MAX / 8 / d))
        return -1;
    return ws_layout(n, d).total;
}

int64_t gq_sums8_bytes(int64_t d)
{
    if (d < 0 || d > INT64_MAX / 2)
        return -1;
    return sums8_bytes(d);
}

int64_t gq_compress_workspace_bytes(int64_t n, int64_t d)
{
    if (n < 1 || n > 0x7FFFFFFF || d < 0 || (d > 0 && n > INT64_MAX / 8 / d))
        return -1;
    return ws_layout(n, d).total_compress;
}

const char *gq_status_str(int32_t status)
{
    switch (status) {
    case GQ_OK: return "GQ_OK";
    case GQ_ERR_NULL: return "GQ_ERR_NULL";
    case GQ_ERR_ARG: return "GQ_ERR_ARG";
    case GQ_ERR_UNSUPPORTED: return "GQ_ERR_UNSUPPORTED";
    case GQ_ERR_CODE_WIDTH: return "GQ_ERR_CODE_WIDTH";
    case GQ_ERR_WORKSPACE: return "GQ_ERR_WORKSPACE";
    case GQ_ERR_ALIGN: return "GQ_ERR_ALIGN";
    case GQ_ERR_DEVICE: return "GQ_ERR_DEVICE";
    default: return "GQ_ERR_UNKNOWN";
    }
}

const char *gq_last_error(void) { return g_err; }

int32_t gq_global_norm(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                       float *norm_dev, void *workspace, int64_t workspace_bytes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    if (!norm_dev)
        return fail(GQ_ERR_NULL, "norm_dev is NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    GQ_TRY(validate_ws(workspace, workspace_bytes, n, d));
    return launch_norm(x, dtype, n, d, q, p, false, norm_dev, workspace, 0, (hipStream_t)stream);
}

int32_t gq_norm_term(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                     double *term_dev, void *workspace, int64_t workspace_bytes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    if (!term_dev)
        return fail(GQ_ERR_NULL, "term_dev is NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    GQ_TRY(validate_ws(workspace, workspace_bytes, n, d));
    return launch_norm(x, dtype, n, d, q, p, false, nullptr, workspace, 0, (hipStream_t)stream,
                       term_dev);
}

int32_t gq_norm_term_bounds(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                            double *term_dev, uint16_t *bounds, void *workspace,
                            int64_t workspace_bytes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    if (!term_dev || (!bounds && d > 0))
        return fail(GQ_ERR_NULL, "term_dev or bounds is NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    if (!aligned16(bounds))
        return fail(GQ_ERR_ALIGN, "bounds is not 16-byte aligned");
    GQ_TRY(validate_ws(workspace, workspace_bytes, n, d));
    return launch_norm(x, dtype, n, d, q, p, false, nullptr, workspace, 0, (hipStream_t)stream,
                       term_dev, d > 0 ? bounds : nullptr);
}

int32_t gq_norm_from_term(const double *term_dev, float q, float p, float *norm_dev, void *stream)
{
    if (!term_dev || !norm_dev)
        return fail(GQ_ERR_NULL, "term_dev and norm_dev must not be NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    const bool qinf = is_inf_order(q), pinf = is_inf_order(p);
    const bool gen = !((qinf || is_two(q)) && (pinf || is_two(p)));
    const double pd = pinf ? 0.0 : (double)p;
    hipStream_t st = (hipStream_t)stream;
#define GQ_FROM(QI, PI, GE) k_norm_from_term<QI, PI, GE><<<dim3(1), dim3(64), 0, st>>>(term_dev, pd, norm_dev)
    if (gen) {
        if (pinf) GQ_FROM(false, true, true); else GQ_FROM(false, false, true);
    } else if (qinf && pinf) GQ_FROM(true, true, false);
    else GQ_FROM(false, false, false); // the other {2, inf} pairs: fp32(sqrt(term))
#undef GQ_FROM
    return check_launch("k_norm_from_term");
}

int32_t gq_quantize(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s, int32_t scheme,
                    const float *norm_dev, uint64_t seed, int64_t worker_base, int32_t code_bits,
                    void *codes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || (!codes && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or codes is NULL");
    if (worker_base < 0 || worker_base + n > ((int64_t)1 << 32))
        return fail(GQ_ERR_ARG, "worker indices must lie in [0, 2^32)");
    GQ_TRY(validate_width(n, s, scheme, code_bits));
    if (!aligned16(codes))
        return fail(GQ_ERR_ALIGN, "codes is not 16-byte aligned");
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    if (tiles * n > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "n * tiles exceeds the launch limit");
    const int64_t rb = row_bytes(d, code_bits);
    hipStream_t st = (hipStream_t)stream;
    uint8_t *c = (uint8_t *)codes;
    const bool nt = code_bits != 32; // 32-bit codes: writes dominate, plain stores
    const dim3 block(kThreads);
    const dim3 g1((unsigned)(tiles * n)), g2((unsigned)(((tiles + 1) / 2) * n));
#define GQ_QUANT(DT, SCH)                                                                             \
    do {                                                                                              \
        if (DT == GQ_IN_F32) {                                                                        \
            if (nt)                                                                                   \
                k_quantize<DT, SCH, true><<<g1, block, 0, st>>>(x, n, d, s, seed, worker_base,        \
                                                                norm_dev, c, code_bits, rb, tiles);   \
            else                                                                                      \
                k_quantize<DT, SCH, false><<<g1, block, 0, st>>>(x, n, d, s, seed, worker_base,       \
                                                                 norm_dev, c, code_bits, rb, tiles);  \
        } else {                                                                                      \
            if (nt)                                                                                   \
                k_quantize2<DT, SCH, true><<<g2, block, 0, st>>>(x, n, d, s, seed, worker_base,       \
                                                                 norm_dev, c, code_bits, rb, tiles);  \
            else                                                                                      \
                k_quantize2<DT, SCH, false><<<g2, block, 0, st>>>(x, n, d, s, seed, worker_base,      \
                                                                  norm_dev, c, code_bits, rb, tiles); \
        }                                                                                             \
    } while (0)
    if (dtype == GQ_IN_F32) {
        if (scheme == GQ_SCHEME_L)
            GQ_QUANT(GQ_IN_F32, GQ_SCHEME_L);
        else
            GQ_QUANT(GQ_IN_F32, GQ_SCHEME_E);
    } else {
        if (scheme == GQ_SCHEME_L)
            GQ_QUANT(GQ_IN_BF16, GQ_SCHEME_L);
        else
            GQ_QUANT(GQ_IN_BF16, GQ_SCHEME_E);
    }
#undef GQ_QUANT
    return check_launch("k_quantize");
}

int32_t gq_reduce_codes(const void *codes, int64_t n, int64_t d, int32_t code_bits, void *code_sum,
                        void *stream)
{
    if (n < 1 || n > 0x7FFFFFFF || d < 0)
        return fail(GQ_ERR_ARG, "n must be >= 1 and d >= 0");
    if ((!codes || !code_sum) && d > 0)
        return fail(GQ_ERR_NULL, "codes or code_sum is NULL");
    if (code_bits < 2 || code_bits > 32)
        return fail(GQ_ERR_CODE_WIDTH, "code_bits %d outside [2, 32]", code_bits);
    if (!aligned16(codes) || !aligned16(code_sum))
        return fail(GQ_ERR_ALIGN, "codes or code_sum is not 16-byte aligned");
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    if (tiles > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    k_reduce_codes<<<dim3((unsigned)tiles), dim3(kThreads), 0, (hipStream_t)stream>>>(
        (const uint8_t *)codes, n, code_bits, row_bytes(d, code_bits), (uint8_t *)code_sum);
    return check_launch("k_reduce_codes");
}

int32_t gq_dequantize(const void *code_sum, int64_t n, int64_t d, int32_t s, int32_t scheme,
                      int32_t code_bits, const float *norm_dev, float *mean, void *stream)
{
    if (!norm_dev || ((!code_sum || !mean) && d > 0))
        return fail(GQ_ERR_NULL, "code_sum, norm_dev or mean is NULL");
    if (n < 1 || n > 0x7FFFFFFF || d < 0)
        return fail(GQ_ERR_ARG, "n must be >= 1 and d >= 0");
    GQ_TRY(validate_scheme(s, scheme));
    GQ_TRY(validate_width(n, s, scheme, code_bits));
    if (!aligned16(code_sum) || !aligned16(mean))
        return fail(GQ_ERR_ALIGN, "code_sum or mean is not 16-byte aligned");
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    if (tiles > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    const dim3 grid((unsigned)tiles), block(kThreads);
    hipStream_t st = (hipStream_t)stream;
    if (scheme == GQ_SCHEME_L)
        k_dequantize<GQ_SCHEME_L><<<grid, block, 0, st>>>((const uint8_t *)code_sum, n, d, s, code_bits, norm_dev, mean);
    else
        k_dequantize<GQ_SCHEME_E><<<grid, block, 0, st>>>((const uint8_t *)code_sum, n, d, s, code_bits, norm_dev, mean);
    return check_launch("k_dequantize");
}

int64_t gq_word_row_bytes(int64_t d, int32_t code_bits)
{
    if (d < 0 || code_bits < 2 || code_bits > 32 || d > INT64_MAX / 64)
        return -1;
    const int64_t f = word_fields(code_bits), nw = (d + f - 1) / f;
    return ((nw + 3) / 4) * 16;
}

// One launch of a kernel templated on the fields per word, for every value
// floor(32 / W) takes with W in [2, 32].
#define GQ_FPW_SWITCH(FPW_RUNTIME, LAUNCH)   \
    switch (FPW_RUNTIME) {                   \
    case 16: LAUNCH(16); break;              \
    case 10: LAUNCH(10); break;              \
    case 8: LAUNCH(8); break;                \
    case 6: LAUNCH(6); break;                \
    case 5: LAUNCH(5); break;                \
    case 4: LAUNCH(4); break;                \
    case 3: LAUNCH(3); break;                \
    case 2: LAUNCH(2); break;                \
    default: LAUNCH(1); break;               \
    }

int32_t gq_quantize_words(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                          int32_t scheme, const float *norm_dev, uint64_t seed,
                          int64_t worker_base, int32_t code_bits, void *words, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || (!words && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or words is NULL");
    if (worker_base < 0 || worker_base + n > ((int64_t)1 << 32))
        return fail(GQ_ERR_ARG, "worker indices must lie in [0, 2^32)");
    GQ_TRY(validate_width(n, s, scheme, code_bits));
    if (!aligned16(words))
        return fail(GQ_ERR_ALIGN, "words is not 16-byte aligned");
    const int64_t rwords = gq_word_row_bytes(d, code_bits) / 4;
    const int64_t tiles = (rwords + kWordsPerBlock - 1) / kWordsPerBlock;
    if (tiles == 0)
        return ok();
    if (tiles * n > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "n * tiles exceeds the launch limit");
    const uint32_t M = (uint32_t)top_code(s, scheme);
    const dim3 grid((unsigned)(tiles * n)), block(kThreads);
    hipStream_t st = (hipStream_t)stream;
    uint32_t *wd = (uint32_t *)words;
#define GQ_QW(F)                                                                               \
    do {                                                                                       \
        if (dtype == GQ_IN_F32 && scheme == GQ_SCHEME_L)                                       \
            k_quantize_words<GQ_IN_F32, GQ_SCHEME_L, F><<<grid, block, 0, st>>>(               \
                x, n, d, s, seed, worker_base, norm_dev, wd, code_bits, M, rwords, tiles);     \
        else if (dtype == GQ_IN_F32)                                                           \
            k_quantize_words<GQ_IN_F32, GQ_SCHEME_E, F><<<grid, block, 0, st>>>(               \
                x, n, d, s, seed, worker_base, norm_dev, wd, code_bits, M, rwords, tiles);     \
        else if (scheme == GQ_SCHEME_L && F > 1)                                               \
            k_quantize_words<GQ_IN_BF16, GQ_SCHEME_L, F, (F > 1)><<<grid, block, 0, st>>>(     \
                x, n, d, s, seed, worker_base, norm_dev, wd, code_bits, M, rwords, tiles);     \
        else if (scheme == GQ_SCHEME_L)                                                        \
            k_quantize_words<GQ_IN_BF16, GQ_SCHEME_L, F><<<grid, block, 0, st>>>(              \
                x, n, d, s, seed, worker_base, norm_dev, wd, code_bits, M, rwords, tiles);     \
        else                                                                                   \
            k_quantize_words<GQ_IN_BF16, GQ_SCHEME_E, F><<<grid, block, 0, st>>>(              \
                x, n, d, s, seed, worker_base, norm_dev, wd, code_bits, M, rwords, tiles);     \
    } while (0)
    GQ_FPW_SWITCH(word_fields(code_bits), GQ_QW)
#undef GQ_QW
    return check_launch("k_quantize_words");
}

// The word-layout compress pass; bounds != nullptr takes the zero-code skip.
static int32_t compress_words(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                              int32_t scheme, const float *norm_dev, uint64_t seed,
                              int64_t worker_base, int32_t code_bits, void *word_sum,
                              const uint16_t *bounds, hipStream_t st)
{
    const int64_t rwords = gq_word_row_bytes(d, code_bits) / 4;
    const int64_t tiles = (rwords + kWordsPerBlock - 1) / kWordsPerBlock;
    if (tiles == 0)
        return ok();
    if (tiles > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    const uint32_t bias = (uint32_t)(n * top_code(s, scheme)); // < 2^31 by the width rule
    const dim3 grid((unsigned)tiles);
    uint32_t *out = (uint32_t *)word_sum;
    const int64_t nm = n * top_code(s, scheme);
    const bool facc = nm <= ((int64_t)1 << 24);
    const bool pk16 = dtype == GQ_IN_BF16 && scheme == GQ_SCHEME_L && nm < ((int64_t)1 << 15);
#define GQ_CW(F)                                                                               \
    do {                                                                                       \
        if (dtype == GQ_IN_F32 && scheme == GQ_SCHEME_L)                                       \
            launch_compress_words<GQ_IN_F32, GQ_SCHEME_L, F>(grid, st, pk16, facc, x, n, d, s, \
                seed, worker_base, norm_dev, out, code_bits, bias, rwords, bounds);           \
        else if (dtype == GQ_IN_F32)                                                           \
            launch_compress_words<GQ_IN_F32, GQ_SCHEME_E, F>(grid, st, pk16, facc, x, n, d, s, \
                seed, worker_base, norm_dev, out, code_bits, bias, rwords, bounds);           \
        else if (scheme == GQ_SCHEME_L)                                                        \
            launch_compress_words<GQ_IN_BF16, GQ_SCHEME_L, F>(grid, st, pk16, facc, x, n, d,  \
                s, seed, worker_base, norm_dev, out, code_bits, bias, rwords, bounds);        \
        else                                                                                   \
            launch_compress_words<GQ_IN_BF16, GQ_SCHEME_E, F>(grid, st, pk16, facc, x, n, d,  \
                s, seed, worker_base, norm_dev, out, code_bits, bias, rwords, bounds);        \
    } while (0)
    GQ_FPW_SWITCH(word_fields(code_bits), GQ_CW)
#undef GQ_CW
    return check_launch("k_compress_words");
}

static int32_t validate_words_call(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                                   int32_t scheme, const float *norm_dev, int64_t worker_base,
                                   int32_t code_bits, const void *word_sum)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || (!word_sum && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or word_sum is NULL");
    if (worker_base < 0 || worker_base + n > ((int64_t)1 << 32))
        return fail(GQ_ERR_ARG, "worker indices must lie in [0, 2^32)");
    GQ_TRY(validate_width(n, s, scheme, code_bits));
    if (!aligned16(word_sum))
        return fail(GQ_ERR_ALIGN, "word_sum is not 16-byte aligned");
    return ok();
}

int32_t gq_compress_words_from_norm(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                                   int32_t scheme, const float *norm_dev, uint64_t seed,
                                   int64_t worker_base, int32_t code_bits, void *word_sum,
                                   void *stream)
{
    GQ_TRY(validate_words_call(x, dtype, n, d, s, scheme, norm_dev, worker_base, code_bits,
                               word_sum));
    return compress_words(x, dtype, n, d, s, scheme, norm_dev, seed, worker_base, code_bits,
                          word_sum, nullptr, (hipStream_t)stream);
}

int32_t gq_compress_words_skip(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                               int32_t scheme, const float *norm_dev, const uint16_t *bounds,
                               uint64_t seed, int64_t worker_base, int32_t code_bits,
                               void *word_sum, void *stream)
{
    GQ_TRY(validate_words_call(x, dtype, n, d, s, scheme, norm_dev, worker_base, code_bits,
                               word_sum));
    if (!bounds && d > 0)
        return fail(GQ_ERR_NULL, "bounds is NULL");
    if (!aligned16(bounds))
        return fail(GQ_ERR_ALIGN, "bounds is not 16-byte aligned");
    return compress_words(x, dtype, n, d, s, scheme, norm_dev, seed, worker_base, code_bits,
                          word_sum, d > 0 ? bounds : nullptr, (hipStream_t)stream);
}

int32_t gq_sum_words(const void *words, int64_t n, int64_t d, int32_t code_bits, void *word_sum,
                     void *stream)
{
    if (n < 1 || n > 0x7FFFFFFF || d < 0)
        return fail(GQ_ERR_ARG, "n must be >= 1 and d >= 0");
    if ((!words || !word_sum) && d > 0)
        return fail(GQ_ERR_NULL, "words or word_sum is NULL");
    if (code_bits < 2 || code_bits > 32)
        return fail(GQ_ERR_CODE_WIDTH, "code_bits %d outside [2, 32]", code_bits);
    if (!aligned16(words) || !aligned16(word_sum))
        return fail(GQ_ERR_ALIGN, "words or word_sum is not 16-byte aligned");
    const int64_t rwords = gq_word_row_bytes(d, code_bits) / 4;
    const int64_t blocks = (rwords + kWordsPerBlock - 1) / kWordsPerBlock;
    if (blocks == 0)
        return ok();
    if (blocks > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    k_sum_words<<<dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream>>>(
        (const uint32_t *)words, n, rwords, (uint32_t *)word_sum);
    return check_launch("k_sum_words");
}

int32_t gq_dequantize_words(const void *word_sum, int64_t n, int64_t d, int32_t s, int32_t scheme,
                            int32_t code_bits, const float *norm_dev, float *mean, void *stream)
{
    if (!norm_dev || ((!word_sum || !mean) && d > 0))
        return fail(GQ_ERR_NULL, "word_sum, norm_dev or mean is NULL");
    if (n < 1 || n > 0x7FFFFFFF || d < 0)
        return fail(GQ_ERR_ARG, "n must be >= 1 and d >= 0");
    GQ_TRY(validate_scheme(s, scheme));
    GQ_TRY(validate_width(n, s, scheme, code_bits));
    if (!aligned16(word_sum) || !aligned16(mean))
        return fail(GQ_ERR_ALIGN, "word_sum or mean is not 16-byte aligned");
    const int64_t blocks = (d + kTile - 1) / kTile;
    if (blocks == 0)
        return ok();
    if (blocks > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    const uint32_t M = (uint32_t)top_code(s, scheme);
    const dim3 grid((unsigned)blocks), block(kThreads);
    hipStream_t st = (hipStream_t)stream;
    const uint32_t *ws = (const uint32_t *)word_sum;
    const int fpw = word_fields(code_bits);
    if (fpw == 3 || fpw == 5 || fpw == 6 || fpw == 10) {
        // 3, 5, 6 or 10 fields per word: whole words per thread, stores staged in LDS
        const int64_t rwords = gq_word_row_bytes(d, code_bits) / 4;
        const int64_t nw = (d + fpw - 1) / fpw;
        const dim3 g2((unsigned)((nw + kWordsPerBlock - 1) / kWordsPerBlock));
#define GQ_DWL(F)                                                                               \
    do {                                                                                        \
        if (scheme == GQ_SCHEME_L)                                                              \
            k_dequantize_words_lds<GQ_SCHEME_L, F><<<g2, block, 0, st>>>(                       \
                ws, n, d, s, code_bits, M, rwords, norm_dev, mean);                             \
        else                                                                                    \
            k_dequantize_words_lds<GQ_SCHEME_E, F><<<g2, block, 0, st>>>(                       \
                ws, n, d, s, code_bits, M, rwords, norm_dev, mean);                             \
    } while (0)
        switch (fpw) {
        case 10: GQ_DWL(10); break;
        case 6: GQ_DWL(6); break;
        case 5: GQ_DWL(5); break;
        case 3: GQ_DWL(3); break;
        }
#undef GQ_DWL
        return check_launch("k_dequantize_words_lds");
    }
#define GQ_DW(F)                                                                                \
    do {                                                                                        \
        if (scheme == GQ_SCHEME_L)                                                              \
            k_dequantize_words<GQ_SCHEME_L, F><<<grid, block, 0, st>>>(ws, n, d, s, code_bits,  \
                                                                       M, norm_dev, mean);      \
        else                                                                                    \
            k_dequantize_words<GQ_SCHEME_E, F><<<grid, block, 0, st>>>(ws, n, d, s, code_bits,  \
                                                                       M, norm_dev, mean);      \
    } while (0)
    switch (fpw) {
    case 16: GQ_DW(16); break;
    case 8: GQ_DW(8); break;
    case 4: GQ_DW(4); break;
    case 2: GQ_DW(2); break;
    default: GQ_DW(1); break;
    }
#undef GQ_DW
    return check_launch("k_dequantize_words");
}

int32_t gq_compress_mean_from_norm(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                                   int32_t scheme, uint64_t seed, const float *norm_dev,
                                   int32_t code_bits, float *mean, void *code_sum_or_null,
                                   void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || (!mean && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or mean is NULL");
    if (min_bits(n, s, scheme) > 32)
        return fail(GQ_ERR_CODE_WIDTH, "sums of %lld codes do not fit 32 bits", (long long)n);
    if (code_sum_or_null) {
        GQ_TRY(validate_width(n, s, scheme, code_bits));
        if (!aligned16(code_sum_or_null))
            return fail(GQ_ERR_ALIGN, "code_sum is not 16-byte aligned");
    }
    if (!aligned16(mean))
        return fail(GQ_ERR_ALIGN, "mean is not 16-byte aligned");
    return launch_compress(x, dtype, n, d, s, scheme, seed, norm_dev, code_bits, mean,
                           code_sum_or_null, (hipStream_t)stream);
}

int64_t gq_span_bounds_bytes(int64_t n, int64_t d)
{
    if (n < 1 || d < 0 || d > INT64_MAX / 4 / n)
        return -1;
    return 2 * n * bound_stride(d);
}

int32_t gq_global_norm_bounds(const void *x, int32_t dtype, int64_t n, int64_t d, float q,
                              float p, float *norm_dev, uint16_t *bounds, void *workspace,
                              int64_t workspace_bytes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    if (!norm_dev || (!bounds && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or bounds is NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    if (!aligned16(bounds))
        return fail(GQ_ERR_ALIGN, "bounds is not 16-byte aligned");
    GQ_TRY(validate_ws(workspace, workspace_bytes, n, d));
    return launch_norm(x, dtype, n, d, q, p, false, norm_dev, workspace, 0, (hipStream_t)stream,
                       nullptr, d > 0 ? bounds : nullptr);
}

int32_t gq_compress_mean_skip(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                              int32_t scheme, uint64_t seed, const float *norm_dev,
                              const uint16_t *bounds, int32_t code_bits, float *mean,
                              void *code_sum_or_null, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || ((!mean || !bounds) && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev, bounds or mean is NULL");
    if (!aligned16(bounds))
        return fail(GQ_ERR_ALIGN, "bounds is not 16-byte aligned");
    if (min_bits(n, s, scheme) > 32)
        return fail(GQ_ERR_CODE_WIDTH, "sums of %lld codes do not fit 32 bits", (long long)n);
    if (code_sum_or_null) {
        GQ_TRY(validate_width(n, s, scheme, code_bits));
        if (!aligned16(code_sum_or_null))
            return fail(GQ_ERR_ALIGN, "code_sum is not 16-byte aligned");
    }
    if (!aligned16(mean))
        return fail(GQ_ERR_ALIGN, "mean is not 16-byte aligned");
    return launch_compress(x, dtype, n, d, s, scheme, seed, norm_dev, code_bits, mean,
                           code_sum_or_null, (hipStream_t)stream, d > 0 ? bounds : nullptr);
}

int32_t gq_compress_mean(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s, float q,
                         float p, int32_t scheme, uint64_t seed, int32_t code_bits, float *mean,
                         float *norm_dev, void *code_sum_or_null, void *workspace,
                         int64_t workspace_bytes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || (!mean && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or mean is NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    if (min_bits(n, s, scheme) > 32)
        return fail(GQ_ERR_CODE_WIDTH, "sums of %lld codes do not fit 32 bits", (long long)n);
    if (code_sum_or_null) {
        GQ_TRY(validate_width(n, s, scheme, code_bits));
        if (!aligned16(code_sum_or_null))
            return fail(GQ_ERR_ALIGN, "code_sum is not 16-byte aligned");
    }
    if (!aligned16(mean))
        return fail(GQ_ERR_ALIGN, "mean is not 16-byte aligned");
    GQ_TRY(validate_ws(workspace, workspace_bytes, n, d));
    hipStream_t st = (hipStream_t)stream;
    const WsLayout L = ws_layout(n, d);
    // with room for the span bounds, the fused pass skips provably zero codes
    uint16_t *bounds = (L.total_compress > L.total && workspace_bytes >= L.total_compress)
                           ? (uint16_t *)((char *)workspace + L.bounds)
                           : nullptr;
    GQ_TRY(launch_norm(x, dtype, n, d, q, p, false, norm_dev, workspace, 0, st, nullptr, bounds));
    return launch_compress(x, dtype, n, d, s, scheme, seed, norm_dev, code_bits, mean,
                           code_sum_or_null, st, bounds);
}

int32_t gq_compress_sums8(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                          int32_t scheme, uint64_t seed, const float *norm_dev, void *sums8,
                          void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || (!sums8 && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or sums8 is NULL");
    if (min_bits(n, s, scheme) > 32)
        return fail(GQ_ERR_CODE_WIDTH, "sums of %lld codes do not fit 32 bits", (long long)n);
    if (!aligned16(sums8))
        return fail(GQ_ERR_ALIGN, "sums8 is not 16-byte aligned");
    return launch_sums8(x, dtype, n, d, s, scheme, seed, norm_dev, (uint8_t *)sums8, nullptr,
                        (hipStream_t)stream);
}

int32_t gq_dequantize_sums8(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                            int32_t scheme, uint64_t seed, const float *norm_dev,
                            const void *sums8, float *mean, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || ((!sums8 || !mean) && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev, sums8 or mean is NULL");
    if (min_bits(n, s, scheme) > 32)
        return fail(GQ_ERR_CODE_WIDTH, "sums of %lld codes do not fit 32 bits", (long long)n);
    if (!aligned16(sums8) || !aligned16(mean))
        return fail(GQ_ERR_ALIGN, "sums8 or mean is not 16-byte aligned");
    return launch_sums8(x, dtype, n, d, s, scheme, seed, norm_dev, (uint8_t *)sums8, mean,
                        (hipStream_t)stream);
}

int32_t gq_compress_mean_noalloc(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                                 float q, float p, int32_t scheme, uint64_t seed,
                                 int32_t code_bits, float *mean, float *norm_dev,
                                 void *code_sum_or_null, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, scheme));
    if (!norm_dev || (!mean && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or mean is NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    if (min_bits(n, s, scheme) > 32)
        return fail(GQ_ERR_CODE_WIDTH, "sums of %lld codes do not fit 32 bits", (long long)n);
    if (code_sum_or_null) {
        GQ_TRY(validate_width(n, s, scheme, code_bits));
        if (!aligned16(code_sum_or_null))
            return fail(GQ_ERR_ALIGN, "code_sum is not 16-byte aligned");
    }
    if (!aligned16(mean))
        return fail(GQ_ERR_ALIGN, "mean is not 16-byte aligned");
    const WsLayout L = ws_layout(n, d);
    const int64_t need = L.total;
    if (need > GQ_NOALLOC_SCRATCH_BYTES)
        return fail(GQ_ERR_WORKSPACE,
                    "n = %lld, d = %lld needs %lld bytes of scratch, beyond the %lld the "
                    "no-allocation entry point holds (use gq_compress_mean with a workspace)",
                    (long long)n, (long long)d, (long long)need,
                    (long long)GQ_NOALLOC_SCRATCH_BYTES);
    hipStream_t st = (hipStream_t)stream;
    void *ws = nullptr;
    GQ_TRY(noalloc_scratch(st, &ws));
    // the span bounds when they fit as well (the zero-code skip), else none
    uint16_t *bounds = (L.total_compress > L.total && L.total_compress <= GQ_NOALLOC_SCRATCH_BYTES)
                           ? (uint16_t *)((char *)ws + L.bounds)
                           : nullptr;
    GQ_TRY(launch_norm(x, dtype, n, d, q, p, false, norm_dev, ws, 0, st, nullptr, bounds));
    return launch_compress(x, dtype, n, d, s, scheme, seed, norm_dev, code_bits, mean,
                           code_sum_or_null, st, bounds);
}

int32_t gq_qsgd_local_mean(const void *x, int32_t dtype, int64_t n, int64_t d, int32_t s,
                           uint64_t seed, float *mean, float *norms_dev, void *codes_or_null,
                           int32_t code_bits, void *workspace, int64_t workspace_bytes,
                           void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(validate_scheme(s, GQ_SCHEME_L));
    if (!norms_dev || (!mean && d > 0))
        return fail(GQ_ERR_NULL, "mean or norms_dev is NULL");
    if (codes_or_null) {
        GQ_TRY(validate_width(1, s, GQ_SCHEME_L, code_bits));
        if (!aligned16(codes_or_null))
            return fail(GQ_ERR_ALIGN, "codes is not 16-byte aligned");
    }
    if (!aligned16(mean))
        return fail(GQ_ERR_ALIGN, "mean is not 16-byte aligned");
    GQ_TRY(validate_ws(workspace, workspace_bytes, n, d));
    hipStream_t st = (hipStream_t)stream;
    const WsLayout L = ws_layout(n, d);
    // with room for the span bounds, zero codes are skipped as in the fused pass
    uint16_t *bounds = (L.total_compress > L.total && workspace_bytes >= L.total_compress)
                           ? (uint16_t *)((char *)workspace + L.bounds)
                           : nullptr;
    GQ_TRY(launch_norm(x, dtype, n, d, 2.0f, 2.0f, true, norms_dev, workspace, s, st, nullptr,
                       bounds));
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    const WorkerParams *params = (const WorkerParams *)((const char *)workspace + L.params);
    const int64_t rb = codes_or_null ? row_bytes(d, code_bits) : 0;
    const dim3 grid((unsigned)tiles), block(kThreads);
    const int64_t bstride = bound_stride(d);
#define GQ_LOCAL(DT, SK)                                                                          \
    k_local_mean<DT, SK><<<grid, block, 0, st>>>(x, n, d, s, seed, norms_dev, params, mean,       \
                                                 (uint8_t *)codes_or_null, code_bits, rb, bounds, \
                                                 bstride)
    if (dtype == GQ_IN_F32) {
        if (bounds)
            GQ_LOCAL(GQ_IN_F32, true);
        else
            GQ_LOCAL(GQ_IN_F32, false);
    } else if (bounds) {
        GQ_LOCAL(GQ_IN_BF16, true);
    } else {
        GQ_LOCAL(GQ_IN_BF16, false);
    }
#undef GQ_LOCAL
    return check_launch("k_local_mean");
}

int64_t gq_e8_row_bytes(int64_t d)
{
    if (d < 0 || d > INT64_MAX - 16)
        return -1;
    return ((d + 15) / 16) * 16;
}

static int32_t e8_check_n(int64_t n)
{
    if (n < 1 || n > kE8MaxN || (n & (n - 1)) != 0)
        return fail(GQ_ERR_UNSUPPORTED, "the tree needs n a power of two in [1, %lld], got %lld",
                    (long long)kE8MaxN, (long long)n);
    return GQ_OK;
}

int32_t gq_e8_quantize(const void *x, int32_t dtype, int64_t n, int64_t d, const float *norm_dev,
                       uint64_t seed, int64_t worker_base, void *codes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    if (!norm_dev || (!codes && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or codes is NULL");
    if (worker_base < 0 || worker_base + n > ((int64_t)1 << 32))
        return fail(GQ_ERR_ARG, "worker indices must lie in [0, 2^32)");
    if (!aligned16(codes))
        return fail(GQ_ERR_ALIGN, "codes is not 16-byte aligned");
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    if (tiles * n > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "n * tiles exceeds the launch limit");
    const dim3 grid((unsigned)(tiles * n)), block(kThreads);
    hipStream_t st = (hipStream_t)stream;
    const int64_t rb = gq_e8_row_bytes(d);
    if (dtype == GQ_IN_F32)
        k_e8_quantize<GQ_IN_F32><<<grid, block, 0, st>>>(x, n, d, seed, worker_base, norm_dev, (uint8_t *)codes, rb, tiles);
    else
        k_e8_quantize<GQ_IN_BF16><<<grid, block, 0, st>>>(x, n, d, seed, worker_base, norm_dev, (uint8_t *)codes, rb, tiles);
    return check_launch("k_e8_quantize");
}

int32_t gq_e8_reduce_pair(const void *a, const void *b, int64_t d, uint64_t seed, int32_t level,
                          int64_t node, void *out, void *stream)
{
    if (d < 0)
        return fail(GQ_ERR_ARG, "d is negative");
    if ((!a || !b || !out) && d > 0)
        return fail(GQ_ERR_NULL, "a, b or out is NULL");
    if (level < 1 || level > 0x7FFFFFFF / 2 || node < 0 || node > 0xFFFFFFFFll)
        return fail(GQ_ERR_ARG, "level must be >= 1 and node in [0, 2^32)");
    if (!aligned16(a) || !aligned16(b) || !aligned16(out))
        return fail(GQ_ERR_ALIGN, "a, b or out is not 16-byte aligned");
    const int64_t blocks = (d + kTile - 1) / kTile;
    if (blocks == 0)
        return ok();
    if (blocks > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    k_e8_pair<<<dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream>>>(
        (const uint8_t *)a, (const uint8_t *)b, d, seed, (uint32_t)level, (uint32_t)node, (uint8_t *)out);
    return check_launch("k_e8_pair");
}

int32_t gq_e8_subtree(const void *codes, int64_t n, int64_t d, uint64_t seed, int64_t worker_base,
                      void *root, void *stream)
{
    GQ_TRY(e8_check_n(n));
    if (d < 0)
        return fail(GQ_ERR_ARG, "d is negative");
    if (worker_base < 0 || worker_base % n != 0 || worker_base + n > ((int64_t)1 << 32))
        return fail(GQ_ERR_ARG, "worker_base = %lld must be a multiple of n = %lld in [0, 2^32)",
                    (long long)worker_base, (long long)n);
    if ((!codes || !root) && d > 0)
        return fail(GQ_ERR_NULL, "codes or root is NULL");
    if (!aligned16(codes) || !aligned16(root))
        return fail(GQ_ERR_ALIGN, "codes or root is not 16-byte aligned");
    const int64_t blocks = (d + kTile - 1) / kTile;
    if (blocks == 0)
        return ok();
    if (blocks > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    k_e8_tree<<<dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream>>>(
        (const uint8_t *)codes, n, d, gq_e8_row_bytes(d), seed, worker_base, (uint8_t *)root);
    return check_launch("k_e8_tree");
}

int32_t gq_e8_tree(const void *codes, int64_t n, int64_t d, uint64_t seed, void *root, void *stream)
{
    return gq_e8_subtree(codes, n, d, seed, 0, root, stream);
}

int32_t gq_e8_dequantize(const void *root, int64_t d, const float *norm_dev, float *mean,
                         void *stream)
{
    if (d < 0)
        return fail(GQ_ERR_ARG, "d is negative");
    if (!norm_dev || ((!root || !mean) && d > 0))
        return fail(GQ_ERR_NULL, "root, norm_dev or mean is NULL");
    if (!aligned16(root) || !aligned16(mean))
        return fail(GQ_ERR_ALIGN, "root or mean is not 16-byte aligned");
    const int64_t blocks = (d + kTile - 1) / kTile;
    if (blocks == 0)
        return ok();
    if (blocks > kMaxGrid)
        return fail(GQ_ERR_UNSUPPORTED, "d exceeds the launch limit");
    k_e8_dequantize<<<dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream>>>(
        (const uint8_t *)root, d, norm_dev, mean);
    return check_launch("k_e8_dequantize");
}

int32_t gq_e8_compress_mean(const void *x, int32_t dtype, int64_t n, int64_t d, float q, float p,
                            uint64_t seed, float *mean, float *norm_dev, void *root_or_null,
                            void *workspace, int64_t workspace_bytes, void *stream)
{
    GQ_TRY(validate_x(x, dtype, n, d));
    GQ_TRY(e8_check_n(n));
    if (!norm_dev || (!mean && d > 0))
        return fail(GQ_ERR_NULL, "norm_dev or mean is NULL");
    if (!order_ok(q) || !order_ok(p))
        return fail(GQ_ERR_UNSUPPORTED, "q and p must be reals >= 1 or +inf");
    if (!aligned16(mean) || !aligned16(root_or_null))
        return fail(GQ_ERR_ALIGN, "mean or root is not 16-byte aligned");
    GQ_TRY(validate_ws(workspace, workspace_bytes, n, d));
    hipStream_t st = (hipStream_t)stream;
    GQ_TRY(launch_norm(x, dtype, n, d, q, p, false, norm_dev, workspace, 0, st));
    const int64_t tiles = (d + kTile - 1) / kTile;
    if (tiles == 0)
        return ok();
    const dim3 grid((unsigned)tiles), block(kThreads);
    if (dtype == GQ_IN_F32)
        k_e8_compress_mean<GQ_IN_F32><<<grid, block, 0, st>>>(x, n, d, seed, norm_dev, mean, (uint8_t *)root_or_null);
    else
        k_e8_compress_mean<GQ_IN_BF16><<<grid, block, 0, st>>>(x, n, d, seed, norm_dev, mean, (uint8_t *)root_or_null);
    return check_launch("k_e8_compress_mean");
}

} // extern "C"
