// LDS tile conventions shared by the bf16 attention kernels (forward and backward) on the
// v_mfma_f32_32x32x16_bf16 operand layouts:
//   A (32 x 16): lane l holds row l % 32, k = 8 * (l / 32) + 0..7
//   B (16 x 32): lane l holds column l % 32, k = 8 * (l / 32) + 0..7
//   C (32 x 32): lane l, register r holds row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32
// A 64-row tile of D bf16 per row sits in LDS row-major with its 16-byte chunks XOR-swizzled
// per row: fk for tiles read by rows (ds_read_b128 of one chunk of one row per lane), fv for
// tiles read transposed (ds_read_b64_tr_b16: a 16-lane group reads 4 rows x 16 columns and
// receives them transposed), fq for tiles read both ways. All keep their reads free of bank
// conflicts.
#pragma once

#include <type_traits>

#include "psa_device.h"

namespace psa {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their no-wait maxima
// (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int kWaitVmcnt0 = 0x0F70;

template <int D>
struct Lay {
    static constexpr int CH = D / 8;                 // 16-byte chunks per row
    static constexpr int RPI = 1024 / (2 * D);       // rows per 1 KB direct-load instruction
    static constexpr int INSTR = 64 * D * 2 / 1024;  // instructions per 64-row tile
    static __device__ __forceinline__ int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int fv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
    // One layout for tiles read both ways. Row reads: the 16 rows a 16-lane group reads at
    // one chunk land on 16 distinct 16-byte bank groups (fq is a bijection of r mod 16 within
    // each 256-byte bank sweep). Transposed reads: the 4 consecutive rows a 32-lane half
    // reads over 4 aligned chunks differ in fq's bits 2..3, so the 16 (row, chunk) pairs land
    // on 16 distinct bank groups.
    static __device__ __forceinline__ int fq(int r) {
        return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    }
};

// The tile row that MFMA A-operand row r reads: bits 2 and 3 of r swapped. With it, the C
// registers 8j..8j+7 of lane l hold rows 16j + 8 * (l / 32) + 0..7: exactly the B-operand
// fragment j of the next product whose contraction runs over those rows.
__device__ __forceinline__ int sigma(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int P>
using IC = std::integral_constant<int, P>;

}  // namespace psa
