// Per-head e4m3 quantization of bf16 tensors for the fp8 QK^T reading of the attention (PSA
// paper abstract and the news summary at euno.news, "Practical": the block-tile kernel suits
// FP16 and FP8 arithmetic; the pages fix no recipe, this one keeps one scale per (batch, head)).
//
//   amax = max |x| over the head's level-0 rows (all seq_len of them)
//   s    = amax / 448 rounded to float32 (1 for an all-zero head); 448 = largest finite e4m3
//   code = the e4m3 (OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals, no infinities) value
//          nearest to x / s, ties to even; x / s is formed in float64
//
// The float64 quotient makes the rounding exact: x (bf16, 8 significant bits) and s (float32,
// 24) give x / s either equal to an e4m3 rounding midpoint (5 significant bits) or at least
// about 2^-30 away from it in relative terms, far above float64's 2^-53, so rounding the
// float64 quotient to e4m3 equals rounding the exact one. The pooled rows of the same head
// take the same scale (their means never exceed amax).
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
constexpr int kChunksPerThread = 4;   // 8-element chunks per thread per pass

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

__global__ void __launch_bounds__(kThreads) k_fp8_amax(const bf16_bits* __restrict__ x, int64_t xs0,
                                                       int64_t xs1, int64_t xs2, int Hx, int D,
                                                       int64_t chunks, uint32_t* amax) {
    const int bh = blockIdx.y;
    uint32_t m = 0;
    for (int i = 0; i < kChunksPerThread; ++i) {
        const int64_t c = (static_cast<int64_t>(blockIdx.x) * kChunksPerThread + i) * kThreads + threadIdx.x;
        if (c < chunks) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(chunk_ptr(x, xs0, xs1, xs2, Hx, D, bh, c));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                m = max(m, w[j] & 0x7fffu);
                m = max(m, (w[j] >> 16) & 0x7fffu);
            }
        }
    }
    // wave max, then one atomic per wave (max is order-independent: deterministic)
    for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
    if ((threadIdx.x & 63) == 0 && m != 0u) atomicMax(amax + bh, m);
}

// amax (bf16 magnitude bits) -> scale, in place
__global__ void __launch_bounds__(kThreads) k_fp8_scale(uint32_t* amax_scale, int n) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const float amax = __uint_as_float(amax_scale[i] << 16);
    const float s = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.f);
    amax_scale[i] = __float_as_uint(s);
}

// e4m3 code of the value nearest to y (|y| <= 464), ties to even. In the binade [2^e, 2^(e+1)),
// e >= -6, the spacing is 2^(e-3); below 2^-6 it is 2^-9 (subnormals), the spacing of e = -6.
// With r = rint(|y| / 2^(e-3)) in [0, 16], the code is 8 (e + 6) + r: the exponent field
// e + 7 in bits 3..6 and the mantissa r - 8 (r = 16 carries into the next exponent; for
// e = -6, r < 8 is the subnormal mantissa).
__device__ __forceinline__ uint32_t e4m3_code(double y) {
    const double a = fabs(y);
    const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(a));
    const int e = max(static_cast<int>(bits >> 52) - 1023, -6);   // a == 0 -> -1023 -> -6
    const double up = __longlong_as_double(static_cast<long long>(static_cast<uint64_t>(1023 + 3 - e) << 52));
    const uint32_t r = static_cast<uint32_t>(rint(a * up));        // exact scaling by 2^(3-e)
    const uint32_t code = r == 0u ? 0u : static_cast<uint32_t>(8 * (e + 6)) + r;
    return code | (y < 0.0 && code != 0u ? 0x80u : 0u);
}

// codes of rows [0, rows) of head bh of src (strides s0, s1, s2) into dst (contiguous
// [bh][rows][D]); grid.z = 0: level 0, 1: pooled rows
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
    const double s = static_cast<double>(scale[bh]);
    for (int i = 0; i < kChunksPerThread; ++i) {
        const int64_t c = (static_cast<int64_t>(blockIdx.x) * kChunksPerThread + i) * kThreads + threadIdx.x;
        if (c >= chunks) break;
        const bf16_bits* src = pooled ? chunk_ptr(xp, Hx * prow * D, prow * D, D, Hx, D, bh, c)
                                      : chunk_ptr(x, xs0, xs1, xs2, Hx, D, bh, c);
        const u32x4 w = *reinterpret_cast<const u32x4*>(src);
        u32x2 out;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double y0 = static_cast<double>(__uint_as_float(w[j] << 16)) / s;
            const double y1 = static_cast<double>(__uint_as_float(w[j] & 0xffff0000u)) / s;
            const uint32_t pair = e4m3_code(y0) | (e4m3_code(y1) << 8);
            if (j & 1)
                out[j >> 1] |= pair << 16;
            else
                out[j >> 1] = pair;
        }
        uint8_t* dst = (pooled ? xp8 : x8) + static_cast<int64_t>(bh) * chunks * 8 + c * 8;
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
    const int64_t per_block = static_cast<int64_t>(kThreads) * kChunksPerThread;
    const bf16_bits* xb = static_cast<const bf16_bits*>(x);
    if (chunks > 0) {
        const unsigned gx = static_cast<unsigned>((chunks + per_block - 1) / per_block);
        hipLaunchKernelGGL(k_fp8_amax, dim3(gx, nh), dim3(kThreads), 0, st, xb, xs[0], xs[1], xs[2],
                           Hx, D, chunks, amax);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_fp8_scale, dim3(hb), dim3(kThreads), 0, st, amax, nh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (chunks == 0) return hipSuccess;
    const int64_t prow = static_cast<int64_t>(N) / 8 * 7;
    const unsigned gx = static_cast<unsigned>((chunks + per_block - 1) / per_block);   // >= pooled
    hipLaunchKernelGGL(k_fp8_quant, dim3(gx, nh, xp != nullptr ? 2 : 1), dim3(kThreads), 0, st, xb,
                       xs[0], xs[1], xs[2], static_cast<const bf16_bits*>(xp), prow, Hx, N, D, scale,
                       x8, xp8);
    return hipGetLastError();
}

}  // namespace psa
