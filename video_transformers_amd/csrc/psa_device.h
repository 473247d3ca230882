// Device-side helpers shared by the PSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {

typedef uint16_t bf16_bits;

// MFMA operand / accumulator vector types.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 (finite inputs; NaN kept quiet).
__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) {
        return static_cast<bf16_bits>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_bits>(u >> 16);
}

typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two packed bf16 in one dword, low half = a: one v_cvt_pk_bf16_f32
// (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

// acc + lo(x) + hi(x) for a dword holding two bf16 values (one v_dot2c_f32_bf16 with 1.0).
__device__ __forceinline__ float add_bf16x2(uint32_t x, float acc) {
    const bf16x2_hw one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_hw, x), one, acc, false);
}

// max / sum of a value across lane l and lane l^32 of the wave: after v_permlane32_swap of
// (x, x), element 0 holds x[l mod 32] and element 1 holds x[l mod 32 + 32] on every lane, so
// combining them gives the same, bitwise, on both lanes of the pair.
__device__ __forceinline__ float pair32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-wide reductions (wave64) through DPP-free shuffles.
__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// One 1 KB direct load: lane i's 16 bytes at global address sbase + voff go to LDS bytes
// [lds + 16 i, lds + 16 i + 16). Written in asm so the compiler does not treat every later
// LDS read as a possible alias of the in-flight write (it would wait for it); the kernel
// waits for these loads itself (vmcnt(0) before the barrier that publishes a tile). The
// instruction has no destination registers; its address operands are read at issue.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    // every operand but voff is wave-uniform: pin them to SGPRs
    // (readfirstlane returns int: widen each half through uint32_t, never by sign extension)
    const uint64_t b = reinterpret_cast<uint64_t>(sbase);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b & 0xffffffffu)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
    const uint64_t bs = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(bs)
        : "memory");
}

}  // namespace psa
