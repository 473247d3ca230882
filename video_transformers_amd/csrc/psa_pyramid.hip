// KV pyramid: levels 1..3 of K and V by 1D mean pooling over 2, 4 and 8 consecutive tokens
// (PSA summary article at rg.mbintangr.com, "Method": progressive 1D mean pooling; skill
// summary at skillsmp.com, "Implementation": level l pools by 2^l).
//
// One thread owns one 8-token window and 8 consecutive head_dim elements of K or V. It reads
// the 8 rows once (16 B per row for bf16, 32 B for f32), forms level 1 as pairwise means of
// the rows, level 2 as pairwise means of level 1, level 3 as the mean of the two level-2 rows,
// and writes 4 + 2 + 1 output rows. Scaling by 1/2 is exact, so this "progressive" tree gives
// the same bits as the direct mean summed pairwise. The output is either the input dtype
// (bf16 rounded to nearest even) or float32 (the tree's values themselves, for parity runs).
// HBM-bound: it reads K and V once and writes 7/8 of their size (in the output dtype).
// Consecutive threads walk head_dim first, then windows, so each wave reads whole contiguous
// rows.
#include "psa_device.h"
#include "psa_internal.h"

namespace psa {
namespace {

template <typename T>
struct Vec8;

template <>
struct Vec8<bf16_bits> {
    static __device__ __forceinline__ void load(const bf16_bits* p, float* x) {
        u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(r[i] << 16);
            x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16_bits* p, const float* x) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        *reinterpret_cast<u32x4*>(p) = r;
    }
};

template <>
struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float* x) {
        f32x4 a = *reinterpret_cast<const f32x4*>(p);
        f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
    static __device__ __forceinline__ void store(float* p, const float* x) {
        f32x4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = x[i];
            b[i] = x[4 + i];
        }
        *reinterpret_cast<f32x4*>(p) = a;
        *reinterpret_cast<f32x4*>(p + 4) = b;
    }
};

struct PyrArgs {
    const void* src[2];   // K, V
    void* dst[2];         // k_pooled, v_pooled
    int64_t stride[2][3]; // (b, h, token) element strides of K, V
    int Hkv, N, D;
    int64_t pooled_rows;  // 7N/8
    int64_t work;         // windows * chunks per tensor = B*Hkv*(N/8)*(D/8)
};

template <typename T, typename TO>
__global__ void __launch_bounds__(256) k_pyramid(PyrArgs a) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int tensor = blockIdx.y;  // 0 = K, 1 = V
    if (gid >= a.work) return;
    const int chunks = a.D >> 3;
    const int c = static_cast<int>(gid % chunks);
    int64_t rest = gid / chunks;
    const int wins = a.N >> 3;
    const int w = static_cast<int>(rest % wins);
    rest /= wins;
    const int h = static_cast<int>(rest % a.Hkv);
    const int b = static_cast<int>(rest / a.Hkv);

    const T* src = static_cast<const T*>(a.src[tensor]) + b * a.stride[tensor][0] +
                   h * a.stride[tensor][1] + static_cast<int64_t>(w) * 8 * a.stride[tensor][2] +
                   c * 8;
    float x[8][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) Vec8<T>::load(src + t * a.stride[tensor][2], x[t]);

    float l1[4][8], l2[2][8], l3[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) l1[j][e] = (x[2 * j][e] + x[2 * j + 1][e]) * 0.5f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) l2[j][e] = (l1[2 * j][e] + l1[2 * j + 1][e]) * 0.5f;
#pragma unroll
    for (int e = 0; e < 8; ++e) l3[e] = (l2[0][e] + l2[1][e]) * 0.5f;

    TO* dst = static_cast<TO*>(a.dst[tensor]) +
             (static_cast<int64_t>(b) * a.Hkv + h) * a.pooled_rows * a.D + c * 8;
    const int64_t D = a.D;
    const int64_t off2 = a.N >> 1, off3 = (a.N >> 1) + (a.N >> 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) Vec8<TO>::store(dst + (static_cast<int64_t>(w) * 4 + j) * D, l1[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        Vec8<TO>::store(dst + (off2 + static_cast<int64_t>(w) * 2 + j) * D, l2[j]);
    Vec8<TO>::store(dst + (off3 + w) * D, l3);
}

}  // namespace

hipError_t launch_pyramid(const Shape& s, const void* k, const void* v, void* kp, void* vp,
                          int out_dtype, hipStream_t st) {
    PyrArgs a;
    a.src[0] = k;
    a.src[1] = v;
    a.dst[0] = kp;
    a.dst[1] = vp;
    for (int i = 0; i < 3; ++i) {
        a.stride[0][i] = s.ks[i];
        a.stride[1][i] = s.vs[i];
    }
    a.Hkv = s.Hkv;
    a.N = s.N;
    a.D = s.D;
    a.pooled_rows = s.pooled_rows;
    a.work = static_cast<int64_t>(s.B) * s.Hkv * (s.N / 8) * (s.D / 8);
    if (a.work == 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((a.work + 255) / 256), 2);
    if (s.dtype == PSA_BF16 && out_dtype == PSA_BF16)
        hipLaunchKernelGGL((k_pyramid<bf16_bits, bf16_bits>), grid, dim3(256), 0, st, a);
    else if (s.dtype == PSA_BF16 && out_dtype == PSA_F32)
        hipLaunchKernelGGL((k_pyramid<bf16_bits, float>), grid, dim3(256), 0, st, a);
    else if (s.dtype == PSA_F32 && out_dtype == PSA_F32)
        hipLaunchKernelGGL((k_pyramid<float, float>), grid, dim3(256), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace psa
