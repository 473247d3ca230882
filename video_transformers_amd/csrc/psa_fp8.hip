// Per-head e4m3 quantization of bf16 tensors for the fp8 QK^T reading of the attention (PSA
// paper abstract and the news summary at euno.news, "Practical": the block-tile kernel suits
// FP16 and FP8 arithmetic; the pages fix no recipe, this one keeps one scale per (batch, head)).
//
//   amax = max |x| over the head's level-0 rows (all seq_len of them)
//   s    = amax / 448 rounded to float32 (1 for an all-zero head); 448 = largest finite e4m3
//   code = the e4m3 (OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals, no infinities) value
//          nearest to the exact quotient x / s, ties to even
//
// The codes are exact. For s >= 2^-80 they come from float32 arithmetic: an estimate of x / s
// picks a code, and the neighbouring midpoints are compared with x / s exactly by the sign of
// one fma each (e4m3_mag_code_exact). Below 2^-80 the quotient is formed in float64, which is
// exact too: x (bf16, 8 significant bits) and s (float32, 24) give x / s either equal to an
// e4m3 rounding midpoint (5 significant bits) or about 2^-30 or more away from it in relative
// terms, far above float64's 2^-53. The pooled rows of the same head take the same scale
// (their means never exceed amax).
//
// Three passes: |x| maximum per head (an integer max of the bf16 magnitude bits, which order
// like the values), the scale, then the codes; the amax array and the scale array are the
// same memory (the scale pass rewrites each head's entry in place).
#include <stdint.h>

#include "psa_device.h"
#include "psa_internal.h"

namespace psa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerThread = 4;   // 8-element chunks per thread (code pass)
constexpr int kAmaxBlocksPerHead = 64;

__global__ void __launch_bounds__(kThreads) k_fp8_clear(uint32_t* amax, int n) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) amax[i] = 0u;
}

// Chunk c (8 elements) of head bh: row c / (D / 8), columns 8 (c % (D / 8)) + 0..7.
__device__ __forceinline__ const bf16_bits* chunk_ptr(const bf16_bits* x, int64_t xs0, int64_t xs1,
                                                      int64_t xs2, int Hx, int D, int bh, int64_t c) {
    const int b = bh / Hx, h = bh % Hx;
    const int cpr = D / 8;
    return x + b * xs0 + h * xs1 + (c / cpr) * xs2 + (c % cpr) * 8;
}

// kAmaxBlocksPerHead blocks per head stride over its chunks; one atomic per block (atomics
// to one address serialise: keep them few)
__global__ void __launch_bounds__(kThreads) k_fp8_amax(const bf16_bits* __restrict__ x, int64_t xs0,
                                                       int64_t xs1, int64_t xs2, int Hx, int D,
                                                       int64_t chunks, uint32_t* amax) {
    __shared__ uint32_t red[kThreads / 64];
    const int bh = blockIdx.y;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    uint32_t m = 0;
    for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; c0 < chunks; c0 += 4 * stride) {
        u32x4 w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t c = c0 + i * stride;
            w[i] = c < chunks ? *reinterpret_cast<const u32x4*>(chunk_ptr(x, xs0, xs1, xs2, Hx, D, bh, c))
                              : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) m = max(m, max(w[i][j] & 0x7fffu, (w[i][j] >> 16) & 0x7fffu));
    }
    for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
        if (m != 0u) atomicMax(amax + bh, m);
    }
}

// amax (bf16 magnitude bits) -> scale, in place
__global__ void __launch_bounds__(kThreads) k_fp8_scale(uint32_t* amax_scale, int n) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const float amax = __uint_as_float(amax_scale[i] << 16);
    const float s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
    amax_scale[i] = __float_as_uint(s);
}

// e4m3 code (magnitude) of the value nearest to a >= 0, given a float or double, ties to even.
// In the binade [2^e, 2^(e+1)), e >= -6, the spacing is 2^(e-3); below 2^-6 it is 2^-9
// (subnormals), the spacing of e = -6. With r = rint(a / 2^(e-3)) in [0, 16], the code is
// 8 (e + 6) + r: exponent field e + 7 in bits 3..6 and mantissa r - 8 (r = 16 carries into
// the next exponent; for e = -6, r < 8 is the subnormal mantissa). a <= 464.
__device__ __forceinline__ uint32_t e4m3_mag_code(double a) {
    const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(a));
    const int e = max(static_cast<int>(bits >> 52) - 1023, -6);   // a == 0 -> -1023 -> -6
    const double up = __longlong_as_double(static_cast<long long>(static_cast<uint64_t>(1023 + 3 - e) << 52));
    const uint32_t r = static_cast<uint32_t>(rint(a * up));        // exact scaling by 2^(3-e)
    return r == 0u ? 0u : static_cast<uint32_t>(8 * (e + 6)) + r;
}
__device__ __forceinline__ uint32_t e4m3_mag_code(float a) {
    const uint32_t bits = __float_as_uint(a);
    const int e = max(static_cast<int>(bits >> 23) - 127, -6);
    const float up = __uint_as_float(static_cast<uint32_t>(127 + 3 - e) << 23);
    const uint32_t r = static_cast<uint32_t>(rintf(a * up));
    return r == 0u ? 0u : static_cast<uint32_t>(8 * (e + 6)) + r;
}

// value of magnitude code c (0..126): c < 8: c 2^-9; else (8 + c % 8) 2^(c/8 - 10)
__device__ __forceinline__ float e4m3_mag_value(uint32_t c) {
    return c < 8u ? static_cast<float>(c) * 0x1p-9f
                  : __uint_as_float(((c >> 3) + 120u) << 23 | (c & 7u) << 20);
}

// Exact code of a / s (a = |x| >= 0 a bf16 value, s >= 2^-80 a float): a float estimate
// a * (1/s) picks a code at most one step from the exact one (its relative error, ~2^-23, is
// far below the code spacing, >= 2^-4 relative); then each neighbouring midpoint M is
// compared with a / s exactly through the sign of fma(-M, s, a): the product M s is exact
// inside the fma, and near any midpoint every quantity is a multiple of 2^-113 and at least
// 2^-90 (s >= 2^-80, M >= 2^-10), so a nonzero difference never rounds to zero. A tie goes
// to the even code.
__device__ __forceinline__ uint32_t e4m3_mag_code_exact(float a, float s, float inv) {
    uint32_t c = e4m3_mag_code(fminf(a * inv, 448.f));
    if (c < 126u) {
        const float mu = 0.5f * (e4m3_mag_value(c) + e4m3_mag_value(c + 1u));
        const float d = fmaf(-mu, s, a);
        if (d > 0.f || (d == 0.f && (c & 1u))) return c + 1u;
    }
    if (c > 0u) {
        const float md = 0.5f * (e4m3_mag_value(c - 1u) + e4m3_mag_value(c));
        const float d = fmaf(-md, s, a);
        if (d < 0.f || (d == 0.f && (c & 1u))) return c - 1u;
    }
    return c;
}

// codes of one bf16 value x (bits in the high half of a float): sign | magnitude code
__device__ __forceinline__ uint32_t e4m3_code(float x, float s, float inv, bool wide) {
    const float a = fabsf(x);
    const uint32_t c = wide ? e4m3_mag_code(static_cast<double>(a) / static_cast<double>(s))
                            : e4m3_mag_code_exact(a, s, inv);
    return c | (x < 0.f && c != 0u ? 0x80u : 0u);
}

// codes of rows [0, rows) of head bh of src (strides s0, s1, s2) into dst (contiguous
// [bh][rows][D]); grid.z = 0: level 0, 1: pooled rows. Heads whose scale is below 2^-80 take
// the float64 quotient x / s (exact as well, see the file comment), a uniform branch.
__global__ void __launch_bounds__(kThreads) k_fp8_quant(const bf16_bits* __restrict__ x, int64_t xs0,
                                                        int64_t xs1, int64_t xs2,
                                                        const bf16_bits* __restrict__ xp,
                                                        int64_t prow, int Hx, int N, int D,
                                                        const float* __restrict__ scale,
                                                        uint8_t* __restrict__ x8, uint8_t* __restrict__ xp8) {
    const int bh = blockIdx.y;
    const bool pooled = blockIdx.z == 1;
    const int64_t rows = pooled ? prow : N;
    const int64_t chunks = rows * (D / 8);
    const float s = scale[bh];
    const float inv = 1.f / s;
    const bool wide = !(s >= 0x1p-80f);
    u32x4 w[kChunksPerThread];
    int64_t cs[kChunksPerThread];
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
        cs[i] = (static_cast<int64_t>(blockIdx.x) * kChunksPerThread + i) * kThreads + threadIdx.x;
        if (cs[i] < chunks)
            w[i] = *reinterpret_cast<const u32x4*>(pooled ? chunk_ptr(xp, Hx * prow * D, prow * D, D, Hx, D, bh, cs[i])
                                                          : chunk_ptr(x, xs0, xs1, xs2, Hx, D, bh, cs[i]));
    }
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
        if (cs[i] >= chunks) break;
        u32x2 out;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t pair = e4m3_code(__uint_as_float(w[i][j] << 16), s, inv, wide) |
                                  (e4m3_code(__uint_as_float(w[i][j] & 0xffff0000u), s, inv, wide) << 8);
            if (j & 1)
                out[j >> 1] |= pair << 16;
            else
                out[j >> 1] = pair;
        }
        uint8_t* dst = (pooled ? xp8 : x8) + static_cast<int64_t>(bh) * chunks * 8 + cs[i] * 8;
        *reinterpret_cast<u32x2*>(dst) = out;
    }
}

}  // namespace

hipError_t launch_quantize_fp8(int B, int Hx, int N, int D, const void* x, const int64_t xs[3],
                               const void* xp, uint8_t* x8, uint8_t* xp8, float* scale,
                               hipStream_t st) {
    const int nh = B * Hx;
    if (nh == 0) return hipSuccess;
    uint32_t* amax = reinterpret_cast<uint32_t*>(scale);
    const unsigned hb = static_cast<unsigned>((nh + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_fp8_clear, dim3(hb), dim3(kThreads), 0, st, amax, nh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t chunks = static_cast<int64_t>(N) * (D / 8);
    const bf16_bits* xb = static_cast<const bf16_bits*>(x);
    if (chunks > 0) {
        const int64_t want = (chunks + 4 * kThreads - 1) / (4 * kThreads);
        const unsigned gx = static_cast<unsigned>(want < kAmaxBlocksPerHead ? want : kAmaxBlocksPerHead);
        hipLaunchKernelGGL(k_fp8_amax, dim3(gx, nh), dim3(kThreads), 0, st, xb, xs[0], xs[1], xs[2],
                           Hx, D, chunks, amax);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_fp8_scale, dim3(hb), dim3(kThreads), 0, st, amax, nh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (chunks == 0) return hipSuccess;
    const int64_t prow = static_cast<int64_t>(N) / 8 * 7;
    const int64_t per_block = static_cast<int64_t>(kThreads) * kChunksPerThread;
    const unsigned gx = static_cast<unsigned>((chunks + per_block - 1) / per_block);   // >= pooled
    hipLaunchKernelGGL(k_fp8_quant, dim3(gx, nh, xp != nullptr ? 2 : 1), dim3(kThreads), 0, st, xb,
                       xs[0], xs[1], xs[2], static_cast<const bf16_bits*>(xp), prow, Hx, N, D, scale,
                       x8, xp8);
    return hipGetLastError();
}

}  // namespace psa
