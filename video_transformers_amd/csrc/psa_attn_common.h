// Definitions shared by the attention kernels (bf16 and f32).
#pragma once

#include <math.h>

#include "psa_device.h"
#include "psa_internal.h"

namespace psa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNoToken = 0x7fffffff;

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* kp;
    const void* vp;
    void* o;
    float* lse;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    // dispatch order [R] (slot -> row; psa_build_index writes it after the CSR offsets), or
    // null: slot = row
    const int32_t* row_order;
    int H, Hkv, N, Nv, NQB, causal;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
    int64_t pooled_rows;
    float c;  // softmax scale * log2(e)
    // fp8 QK^T reading only (null otherwise): per (batch, head) scales of the e4m3 operands,
    // q_scale [B*H] and k_scale [B*Hkv]; the logit of q8 . k8 is c * q_scale * k_scale times it
    const float* q_scale;
    const float* k_scale;
    // fp8 P V reading only (null otherwise): per (batch, KV head) scale of the e4m3 V [B*Hkv]
    const float* v_scale;
};

// Level-by-level walk over a row's block index. Uniform across the workgroup. Only the
// current level's range is held (scalars), so nothing is indexed dynamically.
struct TileWalk {
    const int32_t* rp;  // row_ptr + row * 4
    int l;              // current level (4 = done)
    int lbase;          // col_idx offset of the current level's list
    int lcount;         // length of the current level's list
    int pos;            // first list entry of the current tile

    __device__ void init(const int32_t* row_ptr, int64_t row) {
        rp = row_ptr + row * 4;
        l = 0;
        pos = 0;
        lbase = rp[0];
        lcount = rp[1] - lbase;
        settle();
    }
    __device__ void settle() {
        while (l < 4 && pos >= lcount) {
            ++l;
            pos = 0;
            if (l < 4) {
                lbase = rp[l];
                lcount = rp[l + 1] - lbase;
            }
        }
    }
    __device__ bool valid() const { return l < 4; }
    __device__ void next() {
        pos += 1 << l;
        settle();
    }
    __device__ int count() const {
        const int c = lcount - pos;
        return c < (1 << l) ? c : (1 << l);
    }
};

// Where tile row `row` (0..63) of the current tile comes from.
struct RowSrc {
    int64_t off;  // element offset of the row start (within K/V or within the pooled tensor)
    int last;     // last full-resolution token the row stands for, kNoToken if absent
    bool pooled;
};

__device__ __forceinline__ RowSrc tile_row(const AttnArgs& a, const TileWalk& tw, int row,
                                           int64_t kv_pooled_base, int D, int64_t tok_stride,
                                           int64_t kv_base) {
    const int l = tw.l;
    const int shift = 6 - l;              // log2(rows per logical block at level l)
    const int slab = row >> shift;
    const int rin = row & ((64 >> l) - 1);
    const int cnt = tw.count();
    const int se = slab < cnt ? slab : cnt - 1;
    const int kb = a.col_idx[tw.lbase + tw.pos + se];
    RowSrc r;
    const int prow = kb * (64 >> l) + rin;  // row inside level l
    r.last = slab < cnt ? ((prow + 1) << l) - 1 : kNoToken;
    if (l == 0) {
        r.off = kv_base + static_cast<int64_t>(prow) * tok_stride;
        r.pooled = false;
    } else {
        const int64_t lvl_off = static_cast<int64_t>(a.N) - (static_cast<int64_t>(a.N) >> (l - 1));
        r.off = kv_pooled_base + (lvl_off + prow) * D;
        r.pooled = true;
    }
    return r;
}


// pack = false: one logical block per hardware tile (the unpacked ablation baseline).
hipError_t launch_attn_bf16(const Shape& s, const AttnArgs& a, bool pack, hipStream_t st);

// Q and K (level 0 and pooled) as e4m3 bytes, contiguous, with a.q_scale / a.k_scale set
// (head_dim 128 only; hipErrorNotSupported otherwise). V, O and the index as in the bf16 path.
hipError_t launch_attn_fp8qk(const Shape& s, const AttnArgs& a, hipStream_t st);

// launch_attn_fp8qk with V (level 0 and pooled) as contiguous e4m3 bytes too (a.v_scale set)
// and P quantized to e4m3 for the P V product.
hipError_t launch_attn_fp8(const Shape& s, const AttnArgs& a, hipStream_t st);

}  // namespace psa
