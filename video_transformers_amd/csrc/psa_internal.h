// Internal interface between the host API (psa_api.cpp) and the kernel translation units.
// Everything here is in the library's private namespace; only include/psa.h is public.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psa.h"

namespace psa {

// Shapes and strides of one problem, already validated by the host API.
struct Shape {
    int B, H, Hkv, N, Nv, D, BQ, BK, causal, dtype;
    int NQB, NKB;
    int64_t qs[3], ks[3], vs[3], os[3];
    int64_t pooled_rows;  // 7N/8
};

struct IndexBufs {
    int32_t* row_ptr;  // [R*5 + 1]: the CSR offsets [R*4 + 1], then the dispatch order [R]
    int32_t* col_idx;  // [R*NKB]
    int32_t* dev_err;  // [1]
};

// ---- launchers (each returns the launch's hipError_t) ----

// out_dtype: the problem's dtype, or PSA_F32 (float32 levels of a bf16 problem)
hipError_t launch_pyramid(const Shape& s, const void* k, const void* v, void* kp, void* vp,
                          int out_dtype, hipStream_t st);

hipError_t launch_build_index(const Shape& s, const int8_t* level_map, const IndexBufs& ib,
                              hipStream_t st);

// XCD ranges per chunk of the block index's dispatch order (1, 2, 4 or 8): the smallest for
// which the K and V rows of all levels of the KV heads in flight fit in half the 256 MB
// last-level cache.
int order_share(const Shape& s);

// pack = false selects the unpacked ablation layout (bf16 only; hipErrorNotSupported for f32)
hipError_t launch_attn_fwd(const Shape& s, float scale, const void* q, const void* k,
                           const void* v, const void* kp, const void* vp,
                           const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                           bool pack, hipStream_t st);

// Forward with Q and K (level 0 and pooled) as contiguous e4m3 bytes and one float scale per
// (batch, head) of each (q_scale [B*H], k_scale [B*Hkv]); V, O as in launch_attn_fwd (bf16).
hipError_t launch_attn_fwd_fp8qk(const Shape& s, float scale, const uint8_t* q8,
                                 const float* q_scale, const uint8_t* k8, const uint8_t* kp8,
                                 const float* k_scale, const void* v, const void* vp,
                                 const int32_t* row_ptr, const int32_t* col_idx, void* o,
                                 float* lse, hipStream_t st);

// launch_attn_fwd_fp8qk with V (level 0 and pooled) as contiguous e4m3 bytes too, one scale per
// (batch, KV head) (v_scale [B*Hkv]), and P quantized to e4m3 for the P V product.
hipError_t launch_attn_fwd_fp8(const Shape& s, float scale, const uint8_t* q8, const float* q_scale,
                               const uint8_t* k8, const uint8_t* kp8, const float* k_scale,
                               const uint8_t* v8, const uint8_t* vp8, const float* v_scale,
                               const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                               hipStream_t st);

// Per-head e4m3 quantization of one bf16 tensor [B, Hx, N, D] (strides xs, elements) and,
// when xp is not null, of its packed pooled rows [B, Hx, 7N/8, D] with the same scale.
// Writes x8 / xp8 contiguous and scale [B*Hx]; see psa_quantize_fp8.
hipError_t launch_quantize_fp8(int B, int Hx, int N, int D, const void* x, const int64_t xs[3],
                               const void* xp, uint8_t* x8, uint8_t* xp8, float* scale,
                               hipStream_t st);

// Backward (bf16 only; hipErrorNotSupported otherwise). `scratch` holds
// attn_bwd_scratch_bytes(s): per-row lse2 and D, and the f32 gradients of every level's rows.
size_t attn_bwd_scratch_bytes(const Shape& s);
hipError_t launch_attn_bwd(const Shape& s, float scale, const void* q, const void* k,
                           const void* v, const void* kp, const void* vp, const int8_t* level_map,
                           const int32_t* row_ptr, const int32_t* col_idx, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* scratch, hipStream_t st);

struct MaskBufs {
    float* block_mass;   // [B,H,NQB,NKB]
    float* block_sim;    // [B,Hkv,NKB] or null
    void* ws;
    size_t ws_bytes;
};

size_t mask_workspace_bytes(const Shape& s, const psa_mask_params& mp);
// LDS of one threshold-assignment workgroup (sort keys, masses, staged log-masses when the
// masses come from log-masses, levels); it must not exceed kAssignMaxLds.
constexpr size_t kAssignMaxLds = 64 * 1024;
size_t assign_lds_bytes(const Shape& s, const psa_mask_params& mp, bool from_log_masses);
// Attention and its backward stage a row's block list (NKB int32) in LDS beside the tiles.
constexpr int kAttnMaxKBlocks = 16384;

hipError_t launch_mask_scores(const Shape& s, const psa_mask_params& mp, const void* q,
                              const void* k, const MaskBufs& mb, hipStream_t st);

// sim64 (nullable): the same similarities in float64
hipError_t launch_block_sim(const Shape& s, const void* k, float* block_sim, double* sim64,
                            hipStream_t st);

// Inside psa_mask's workspace: the float64 similarities (null without the cosine check) and the
// two certification counters (rows flagged for float64 rescoring, rows beyond the capacity).
double* mask_sim64(const Shape& s, const psa_mask_params& mp, const MaskBufs& mb);
int* mask_cert_counters(const Shape& s, const psa_mask_params& mp, void* ws);

// Float64 rescoring and reassignment of the rows the assignment flagged (after
// launch_mask_assign_logmass; the counters must have been cleared before it).
hipError_t launch_mask_certify(const Shape& s, const psa_mask_params& mp, const void* q,
                               const void* k, const MaskBufs& mb, int8_t* level_map, hipStream_t st);

// Mean of each query block's valid rows (qbar [B*H][NQB][D]) and of each KV block's valid keys
// (kbar [B*Hkv][NKB][D]), float32; and the float64 sum of each KV block's valid keys (ksum
// [B*Hkv][NKB][D]), which the certification of block-mean scores reads.
hipError_t launch_block_means(const Shape& s, const void* q, const void* k, float* qbar, float* kbar,
                              double* ksum, hipStream_t st);

// Block-mean scoring, threshold assignment and the attention in one kernel (bf16, block_q 128,
// NKB <= 1792): each workgroup scores its query block's mean against every KV block mean,
// assigns the levels (the same steps as the mask's assignment) and attends over the resulting
// list. qbar / kbar / ksum from launch_block_means; sim (or null) from launch_block_sim; map_out
// and mass_out (or null) receive the level map and block masses.
hipError_t launch_attn_fwd_meankey(const Shape& s, float scale, const psa_mask_params& mp,
                                   const void* q, const void* k, const void* v, const void* kp,
                                   const void* vp, const float* qbar, const float* kbar,
                                   const double* ksum, const float* sim, const double* sim64,
                                   int8_t* map_out, float* mass_out, void* o, float* lse,
                                   hipStream_t st);

hipError_t launch_mask_assign(const Shape& s, const psa_mask_params& mp, const float* block_mass,
                              const float* block_sim, int8_t* level_map, hipStream_t st);

// Assignment from the scoring pass's log-masses in mb.ws; writes mb.block_mass and the map.
hipError_t launch_mask_assign_logmass(const Shape& s, const psa_mask_params& mp, const MaskBufs& mb,
                                      int8_t* level_map, hipStream_t st);

// Clears one int32 on the device with a kernel (no memset node, so the call stays safe to
// capture in a graph).
hipError_t launch_clear_i32(int32_t* p, int n, hipStream_t st);

// Diagnostics: fills the LDS of every CU with `pattern` (see psa_debug_fill_lds).
hipError_t launch_fill_lds(uint32_t pattern, hipStream_t st);

}  // namespace psa
