// probe.hip -- measurement kernels for the rooflines of libgq.so (MI355X, gfx950).
//
// Two microbenchmarks whose timings give the ceilings the library's kernels
// are measured against.  They compute nothing of the operator.
//
//   gqp_read  streams a device buffer once and reduces it per block, the
//             pattern of a bandwidth-bound pass with one small output per
//             block.  Several launch shapes are offered; the best one gives
//             the measured HBM read ceiling.
//   gqp_valu  issues a long loop of independent vector-ALU instructions of
//             one kind (eight independent chains per lane, no memory access
//             in the loop), so that its time gives the issue rate of that
//             instruction kind: wave64 instructions per CU per clock.  The
//             kinds are the ones the library's VALU-heavy loops are made of:
//             fp32 fma, u32 add, three-input bit operation, the 32x32->64
//             multiply-add of Philox, and fp64 add and fma.
//
// Both are plain C ABI calls on caller-owned device memory, like libgq.so.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

// ---------------------------------------------------------------------------
// Stream read: block b reads `per_block` bytes starting at b * per_block
// (the last block stops at `bytes`), xor-reduces them and writes one word.
template <int THREADS, int VEC> // VEC: 16-byte loads per thread per block
__global__ __launch_bounds__(THREADS) void k_read(const uint4 *__restrict__ buf, int64_t n16,
                                                  uint32_t *__restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * THREADS * VEC;
    uint4 v[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        const int64_t i = base + (int64_t)k * THREADS + threadIdx.x;
        v[k] = i < n16 ? buf[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < VEC; ++k)
        acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    // wave reduction through LDS-free shuffles, then one word per wave
    for (int off = 32; off > 0; off >>= 1)
        acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0)
        out[(int64_t)blockIdx.x * (THREADS / 64) + threadIdx.x / 64] = acc;
}

// ---------------------------------------------------------------------------
// VALU issue: `iters` iterations of 8 independent instructions of one kind
// per lane; the eight chains are combined and written once per lane.  The
// loop is unrolled 4 times (32 VALU instructions per taken branch), so that
// its scalar counter and branch take a negligible share of the issue slots.
enum { kFmaF32 = 0, kAddU32 = 1, kBitop3 = 2, kMadU64 = 3, kAddF64 = 4, kFmaF64 = 5 };

template <int OP>
__global__ __launch_bounds__(256) void k_valu(int iters, uint32_t seed, uint32_t *__restrict__ out)
{
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    uint32_t r = 0;
    if constexpr (OP == kFmaF32) {
        float a[8], b = __uint_as_float(0x3F800001u ^ (seed & 1u)), c = (float)(t & 7) * 1e-7f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a[k] = (float)(t + k);
#pragma unroll 4
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                a[k] = fmaf(a[k], b, c);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            r ^= __float_as_uint(a[k]);
    } else if constexpr (OP == kAddU32) {
        // one v_add_u32 per chain and step, written out (plain C adds of a
        // loop-invariant value would be folded into fewer instructions)
        uint32_t a[8], b = seed | 1u;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a[k] = t + (uint32_t)k;
        int i = 0;
        for (; i + 4 <= iters; i += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    asm("v_add_u32 %0, %1, %2" : "=v"(a[k]) : "v"(a[k]), "v"(b));
        }
        for (; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                asm("v_add_u32 %0, %1, %2" : "=v"(a[k]) : "v"(a[k]), "v"(b));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            r ^= a[k];
    } else if constexpr (OP == kBitop3) {
        uint32_t a[8], b = seed | 1u, c = t * 0x9E3779B9u;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a[k] = t + (uint32_t)k;
#pragma unroll 4
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                a[k] = __builtin_amdgcn_bitop3_b32(a[k], b, c, 0x96);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            r ^= a[k];
    } else if constexpr (OP == kMadU64) {
        uint64_t a[8];
        const uint32_t m = 0xD2511F53u ^ (seed & 2u);
        const uint64_t c = ((uint64_t)t << 32) | (t * 0x9E3779B9u); // per-lane addend
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a[k] = (uint64_t)(t + (uint32_t)k) << 7;
#pragma unroll 4
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                a[k] = (uint64_t)(uint32_t)a[k] * m + c;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            r ^= (uint32_t)a[k] ^ (uint32_t)(a[k] >> 32);
    } else {
        double a[8], b = 1.0 + 0x1p-40 * (double)(seed & 3u), c = (double)(t & 7) * 1e-13;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a[k] = (double)(t + (uint32_t)k);
#pragma unroll 4
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                a[k] = OP == kAddF64 ? a[k] + c : fma(a[k], b, c);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            r ^= (uint32_t)__double_as_longlong(a[k]) ^ (uint32_t)(__double_as_longlong(a[k]) >> 32);
    }
    out[t] = r;
}

} // namespace

extern "C" {

// Blocks of 16-byte words read per launch shape (threads x loads per thread).
// Shape 0: 512 x 2 (16 KB per block), 1: 256 x 2 (8 KB), 2: 512 x 4 (32 KB),
// 3: 256 x 8 (32 KB), 4: 1024 x 1 (16 KB).
int32_t gqp_read_blocks(int64_t bytes, int32_t shape)
{
    static const int per[5] = {512 * 2, 256 * 2, 512 * 4, 256 * 8, 1024};
    if (shape < 0 || shape > 4 || bytes < 16)
        return -1;
    const int64_t n16 = bytes / 16;
    return (int32_t)((n16 + per[shape] - 1) / per[shape]);
}

// Words of `out` gqp_read writes: one per wave of every block.
int32_t gqp_read_out_words(int64_t bytes, int32_t shape)
{
    static const int waves[5] = {8, 4, 8, 4, 16};
    const int32_t b = gqp_read_blocks(bytes, shape);
    return b < 0 ? -1 : b * waves[shape];
}

// Reads bytes / 16 16-byte words of buf (16-byte aligned) once.  out must hold
// gqp_read_out_words(bytes, shape) words.  Returns 0, or -1 / -2 for bad
// arguments / a failed launch.
int32_t gqp_read(const void *buf, int64_t bytes, int32_t shape, void *out, void *stream)
{
    const int32_t blocks = gqp_read_blocks(bytes, shape);
    if (!buf || !out || blocks < 0 || ((uintptr_t)buf & 15u))
        return -1;
    const int64_t n16 = bytes / 16;
    hipStream_t st = (hipStream_t)stream;
    const uint4 *b = (const uint4 *)buf;
    uint32_t *o = (uint32_t *)out;
    switch (shape) {
    case 0: k_read<512, 2><<<blocks, 512, 0, st>>>(b, n16, o); break;
    case 1: k_read<256, 2><<<blocks, 256, 0, st>>>(b, n16, o); break;
    case 2: k_read<512, 4><<<blocks, 512, 0, st>>>(b, n16, o); break;
    case 3: k_read<256, 8><<<blocks, 256, 0, st>>>(b, n16, o); break;
    default: k_read<1024, 1><<<blocks, 1024, 0, st>>>(b, n16, o); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// `blocks` blocks of 256 threads, each lane running `iters` iterations of 8
// instructions of kind op (0 fp32 fma, 1 u32 add, 2 three-input xor,
// 3 32x32->64 multiply-add, 4 fp64 add, 5 fp64 fma).  out: blocks * 256
// words.  Returns 0, -1 (bad arguments) or -2 (failed launch).
int32_t gqp_valu(int32_t op, int32_t blocks, int32_t iters, uint32_t seed, void *out,
                 void *stream)
{
    if (!out || blocks < 1 || iters < 1 || op < 0 || op > 5)
        return -1;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *o = (uint32_t *)out;
    switch (op) {
    case kFmaF32: k_valu<kFmaF32><<<blocks, 256, 0, st>>>(iters, seed, o); break;
    case kAddU32: k_valu<kAddU32><<<blocks, 256, 0, st>>>(iters, seed, o); break;
    case kBitop3: k_valu<kBitop3><<<blocks, 256, 0, st>>>(iters, seed, o); break;
    case kMadU64: k_valu<kMadU64><<<blocks, 256, 0, st>>>(iters, seed, o); break;
    case kAddF64: k_valu<kAddF64><<<blocks, 256, 0, st>>>(iters, seed, o); break;
    default: k_valu<kFmaF64><<<blocks, 256, 0, st>>>(iters, seed, o); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

} // extern "C"
