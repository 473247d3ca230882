// Host side of the C ABI declared in include/psa.h: argument checks (before anything is
// enqueued), workspace layout, and dispatch to the kernel launchers. No exception crosses the
// interface; HIP failures map to PSA_ERR_HIP with the hipError_t kept per thread.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "psa.h"
#include "psa_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return PSA_OK;
    g_last_hip_error = static_cast<int>(e);
    return PSA_ERR_HIP;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks a problem and fills the internal shape. Returns PSA_OK or a negative status.
int check_problem(const psa_problem* p, psa::Shape* s) {
    if (p == nullptr) return PSA_ERR_INVALID_ARG;
    if (p->batch < 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seq_len < 0 ||
        p->seq_valid < 0 || p->head_dim <= 0 || p->block_q <= 0 || p->block_k <= 0)
        return PSA_ERR_INVALID_ARG;
    if (p->heads_q % p->heads_kv != 0) return PSA_ERR_INVALID_ARG;
    if (p->seq_valid > p->seq_len) return PSA_ERR_INVALID_ARG;
    if (p->dtype != PSA_F32 && p->dtype != PSA_BF16) return PSA_ERR_UNSUPPORTED;
    if (p->head_dim != 64 && p->head_dim != 128) return PSA_ERR_UNSUPPORTED;
    if (p->block_k != 64) return PSA_ERR_UNSUPPORTED;
    if (p->block_q != 64 && p->block_q != 128) return PSA_ERR_UNSUPPORTED;
    if (p->seq_len % p->block_q != 0) return PSA_ERR_UNSUPPORTED;
    if ((p->seq_len - p->seq_valid) % 8 != 0) return PSA_ERR_UNSUPPORTED;
    const int64_t* strides[4] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride};
    for (auto st : strides)
        for (int i = 0; i < 3; ++i)
            if (st[i] <= 0 || st[i] % 8 != 0) return PSA_ERR_INVALID_ARG;
    if (p->q_stride[2] < p->head_dim || p->k_stride[2] < p->head_dim ||
        p->v_stride[2] < p->head_dim || p->o_stride[2] < p->head_dim)
        return PSA_ERR_INVALID_ARG;
    // byte offsets inside one (batch, head) of K, V or one pooled level stay below 2^31
    const int64_t elem = p->dtype == PSA_BF16 ? 2 : 4;
    if ((static_cast<int64_t>(p->seq_len) * p->k_stride[2] + p->head_dim) * elem >= (int64_t(1) << 31) ||
        (static_cast<int64_t>(p->seq_len) * p->v_stride[2] + p->head_dim) * elem >= (int64_t(1) << 31) ||
        static_cast<int64_t>(p->seq_len) * p->head_dim * elem >= (int64_t(1) << 31))
        return PSA_ERR_UNSUPPORTED;
    // every index the kernels form per (batch, head) row stays in int32 range
    const int64_t R = static_cast<int64_t>(p->batch) * p->heads_q * (p->seq_len / p->block_q);
    if (R * 5 + 1 > INT32_MAX || R * (p->seq_len / 64) > INT32_MAX) return PSA_ERR_UNSUPPORTED;
    if (s != nullptr) {
        s->B = p->batch;
        s->H = p->heads_q;
        s->Hkv = p->heads_kv;
        s->N = p->seq_len;
        s->Nv = p->seq_valid;
        s->D = p->head_dim;
        s->BQ = p->block_q;
        s->BK = p->block_k;
        s->causal = p->causal != 0;
        s->dtype = p->dtype;
        s->NQB = p->seq_len / p->block_q;
        s->NKB = p->seq_len / p->block_k;
        for (int i = 0; i < 3; ++i) {
            s->qs[i] = p->q_stride[i];
            s->ks[i] = p->k_stride[i];
            s->vs[i] = p->v_stride[i];
            s->os[i] = p->o_stride[i];
        }
        s->pooled_rows = static_cast<int64_t>(p->seq_len) / 8 * 7;
    }
    return PSA_OK;
}

// A problem with no tokens or no batch has no work: every entry point returns PSA_OK for it
// after the shape and parameter checks, without reading its pointers (torch gives empty
// tensors a null data pointer) and without launching anything.
bool no_work(const psa::Shape& s) { return s.B == 0 || s.N == 0; }

int check_mask_params(const psa_problem* p, const psa_mask_params* m) {
    if (m == nullptr) return PSA_ERR_INVALID_ARG;
    if (m->mode != PSA_MASK_SAMPLING && m->mode != PSA_MASK_ANTIDIAG && m->mode != PSA_MASK_MEANKEY)
        return PSA_ERR_INVALID_ARG;
    float prev = 0.f;
    for (int i = 0; i < 4; ++i) {
        const float t = m->thresholds[i];
        if (!std::isfinite(t) || t <= 0.f || t > 1.f || t < prev) return PSA_ERR_INVALID_ARG;
        prev = t;
    }
    if (!std::isfinite(m->cos_sim_min)) return PSA_ERR_INVALID_ARG;
    if (m->force_l0_begin < 0 || m->force_l0_end < 0) return PSA_ERR_INVALID_ARG;
    if (m->force_l0_begin < m->force_l0_end && m->force_l0_end > p->seq_len)
        return PSA_ERR_INVALID_ARG;
    if (m->mode == PSA_MASK_SAMPLING) {
        const int S = m->samples_per_qblock;
        if (S < 1 || S > p->block_q) return PSA_ERR_INVALID_ARG;
        // the sampled rows of one query block are reduced inside one half-wave
        if (S > 32 || (S & (S - 1)) != 0) return PSA_ERR_UNSUPPORTED;
    } else if (m->mode == PSA_MASK_ANTIDIAG) {
        const int S = m->antidiag_stride;
        if (S < 1 || S > 64) return PSA_ERR_INVALID_ARG;
        // a KV block must span whole 8-column groups and a query block's compressed rows
        // must fit one half-wave
        if ((S != 2 && S != 4 && S != 8) || p->block_q / S > 32) return PSA_ERR_UNSUPPORTED;
    }
    return PSA_OK;
}

struct AttnWs {
    int32_t* dev_err;
    int32_t* row_ptr;
    int32_t* col_idx;
    size_t bytes;
};

// The address `off` bytes into a workspace, or null when only the size is being computed
// (base null): no arithmetic on a null pointer.
template <typename T>
T* ws_at(void* base, size_t off) {
    return base == nullptr ? nullptr : reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

AttnWs attn_ws_layout(const psa::Shape& s, void* base) {
    const size_t R = static_cast<size_t>(s.B) * s.H * s.NQB;
    AttnWs w;
    size_t off = 0;
    w.dev_err = ws_at<int32_t>(base, off);
    off += kAlign;
    w.row_ptr = ws_at<int32_t>(base, off);
    off += align_up((R * 5 + 1) * sizeof(int32_t));   // CSR offsets, then the dispatch order
    w.col_idx = ws_at<int32_t>(base, off);
    off += align_up(R * s.NKB * sizeof(int32_t));
    w.bytes = off;
    return w;
}

}  // namespace

extern "C" {

int64_t psa_pooled_rows(const psa_problem* prob) {
    if (check_problem(prob, nullptr) != PSA_OK) return -1;
    return static_cast<int64_t>(prob->seq_len) / 8 * 7;
}

int psa_build_pyramid(const psa_problem* prob, const void* k, const void* v, void* k_pooled,
                      void* v_pooled, int32_t out_dtype, void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (out_dtype != PSA_F32 && out_dtype != PSA_BF16) return PSA_ERR_INVALID_ARG;
    if (out_dtype != s.dtype && out_dtype != PSA_F32) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!k || !v || !k_pooled || !v_pooled) return PSA_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_pooled) || !aligned16(v_pooled))
        return PSA_ERR_INVALID_ARG;
    return hip_status(psa::launch_pyramid(s, k, v, k_pooled, v_pooled, out_dtype,
                                          static_cast<hipStream_t>(stream)));
}

size_t psa_mask_workspace_bytes(const psa_problem* prob, const psa_mask_params* params) {
    psa::Shape s;
    if (check_problem(prob, &s) != PSA_OK || check_mask_params(prob, params) != PSA_OK) return 0;
    return psa::mask_workspace_bytes(s, *params);
}

int psa_mask(const psa_problem* prob, const psa_mask_params* params, const void* q,
             const void* k, int8_t* level_map, float* block_mass, float* block_sim, void* ws,
             size_t ws_bytes, void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if ((rc = check_mask_params(prob, params)) != PSA_OK) return rc;
    if (s.dtype != PSA_BF16) return PSA_ERR_UNSUPPORTED;
    if (psa::assign_lds_bytes(s, *params, true) > psa::kAssignMaxLds) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q || !k || !level_map || !block_mass) return PSA_ERR_INVALID_ARG;
    if (params->cos_sim_min > 0.f && block_sim == nullptr) return PSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k)) return PSA_ERR_INVALID_ARG;
    const size_t need = psa::mask_workspace_bytes(s, *params);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return PSA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    psa::MaskBufs mb{block_mass, block_sim, ws, ws_bytes};
    hipError_t e = psa::launch_clear_i32(psa::mask_cert_counters(s, *params, ws), 2, st);
    if (e != hipSuccess) return hip_status(e);
    if ((e = psa::launch_mask_scores(s, *params, q, k, mb, st)) != hipSuccess) return hip_status(e);
    const bool use_sim = params->cos_sim_min > 0.f;
    if (use_sim) {
        e = psa::launch_block_sim(s, k, block_sim, psa::mask_sim64(s, *params, mb), st);
        if (e != hipSuccess) return hip_status(e);
    }
    if ((e = psa::launch_mask_assign_logmass(s, *params, mb, level_map, st)) != hipSuccess)
        return hip_status(e);
    return hip_status(psa::launch_mask_certify(s, *params, q, k, mb, level_map, st));
}

int psa_mask_certified_rows(const psa_problem* prob, const psa_mask_params* params,
                            const void* ws, int32_t* counts, void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if ((rc = check_mask_params(prob, params)) != PSA_OK) return rc;
    if (counts == nullptr) return PSA_ERR_INVALID_ARG;
    counts[0] = counts[1] = 0;
    if (no_work(s)) return PSA_OK;
    if (ws == nullptr) return PSA_ERR_INVALID_ARG;
    const int* c = psa::mask_cert_counters(s, *params, const_cast<void*>(ws));
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(counts, c, 2 * sizeof(int32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return hip_status(e);
}

int psa_mask_assign(const psa_problem* prob, const psa_mask_params* params,
                    const float* block_mass, const float* block_sim, int8_t* level_map,
                    void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if ((rc = check_mask_params(prob, params)) != PSA_OK) return rc;
    if (psa::assign_lds_bytes(s, *params, false) > psa::kAssignMaxLds) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!block_mass || !level_map) return PSA_ERR_INVALID_ARG;
    const bool use_sim = params->cos_sim_min > 0.f;
    if (use_sim && block_sim == nullptr) return PSA_ERR_INVALID_ARG;
    return hip_status(psa::launch_mask_assign(s, *params, block_mass, use_sim ? block_sim : nullptr,
                                              level_map, static_cast<hipStream_t>(stream)));
}

int psa_build_index(const psa_problem* prob, const int8_t* level_map, int32_t* row_ptr,
                    int32_t* col_idx, int32_t* dev_err, void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (no_work(s)) return PSA_OK;
    if (!level_map || !row_ptr || !col_idx || !dev_err) return PSA_ERR_INVALID_ARG;
    psa::IndexBufs ib{row_ptr, col_idx, dev_err};
    return hip_status(psa::launch_build_index(s, level_map, ib, static_cast<hipStream_t>(stream)));
}

size_t psa_attn_workspace_bytes(const psa_problem* prob) {
    psa::Shape s;
    if (check_problem(prob, &s) != PSA_OK) return 0;
    return attn_ws_layout(s, nullptr).bytes;
}

int psa_attn_fwd(const psa_problem* prob, float softmax_scale, const void* q, const void* k,
                 const void* v, const void* k_pooled, const void* v_pooled,
                 const int8_t* level_map, void* o, float* lse, void* ws, size_t ws_bytes,
                 void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (s.NKB > psa::kAttnMaxKBlocks) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q || !k || !v || !k_pooled || !v_pooled || !level_map || !o) return PSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_pooled) ||
        !aligned16(v_pooled) || !aligned16(o))
        return PSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return PSA_ERR_INVALID_ARG;
    const size_t need = attn_ws_layout(s, nullptr).bytes;
    if (ws == nullptr || ws_bytes < need) return PSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return PSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(s.D));
    hipStream_t st = static_cast<hipStream_t>(stream);
    AttnWs w = attn_ws_layout(s, ws);
    psa::IndexBufs ib{w.row_ptr, w.col_idx, w.dev_err};
    hipError_t e = psa::launch_build_index(s, level_map, ib, st);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(psa::launch_attn_fwd(s, scale, q, k, v, k_pooled, v_pooled, w.row_ptr,
                                           w.col_idx, o, lse, true, st));
}

namespace {

int attn_indexed(const psa_problem* prob, float softmax_scale, const void* q, const void* k,
                 const void* v, const void* k_pooled, const void* v_pooled,
                 const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                 bool pack, void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (s.NKB > psa::kAttnMaxKBlocks) return PSA_ERR_UNSUPPORTED;
    if (!pack && s.dtype != PSA_BF16) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q || !k || !v || !k_pooled || !v_pooled || !row_ptr || !col_idx || !o)
        return PSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_pooled) ||
        !aligned16(v_pooled) || !aligned16(o))
        return PSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return PSA_ERR_INVALID_ARG;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(s.D));
    return hip_status(psa::launch_attn_fwd(s, scale, q, k, v, k_pooled, v_pooled, row_ptr,
                                           col_idx, o, lse, pack, static_cast<hipStream_t>(stream)));
}

}  // namespace

int psa_attn_fwd_indexed(const psa_problem* prob, float softmax_scale, const void* q,
                         const void* k, const void* v, const void* k_pooled,
                         const void* v_pooled, const int32_t* row_ptr, const int32_t* col_idx,
                         void* o, float* lse, void* stream) {
    return attn_indexed(prob, softmax_scale, q, k, v, k_pooled, v_pooled, row_ptr, col_idx, o,
                        lse, true, stream);
}

int psa_attn_fwd_unpacked(const psa_problem* prob, float softmax_scale, const void* q,
                          const void* k, const void* v, const void* k_pooled,
                          const void* v_pooled, const int32_t* row_ptr, const int32_t* col_idx,
                          void* o, float* lse, void* stream) {
    return attn_indexed(prob, softmax_scale, q, k, v, k_pooled, v_pooled, row_ptr, col_idx, o,
                        lse, false, stream);
}

int psa_quantize_fp8(int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                     const void* x, const int64_t* x_stride, const void* x_pooled, uint8_t* x8,
                     uint8_t* x8_pooled, float* scale, void* stream) {
    if (batch < 0 || heads <= 0 || seq_len < 0 || head_dim <= 0 || x_stride == nullptr)
        return PSA_ERR_INVALID_ARG;
    if (head_dim % 8 != 0 || seq_len % 8 != 0) return PSA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(batch) * heads > 65535) return PSA_ERR_UNSUPPORTED;
    for (int i = 0; i < 3; ++i)
        if (x_stride[i] <= 0 || x_stride[i] % 8 != 0) return PSA_ERR_INVALID_ARG;
    if (x_stride[2] < head_dim) return PSA_ERR_INVALID_ARG;
    if (batch == 0) return PSA_OK;
    if (!scale || (reinterpret_cast<uintptr_t>(scale) & 3u) != 0) return PSA_ERR_INVALID_ARG;
    if (seq_len == 0)   // every head is empty: scale 1, nothing to code
        return hip_status(psa::launch_quantize_fp8(batch, heads, 0, head_dim, nullptr, x_stride,
                                                   nullptr, nullptr, nullptr, scale,
                                                   static_cast<hipStream_t>(stream)));
    if (!x || !x8 || (x_pooled == nullptr) != (x8_pooled == nullptr)) return PSA_ERR_INVALID_ARG;
    if (!aligned16(x) || (x_pooled && !aligned16(x_pooled)) ||
        (reinterpret_cast<uintptr_t>(x8) & 7u) != 0 ||
        (x8_pooled && (reinterpret_cast<uintptr_t>(x8_pooled) & 7u) != 0) ||
        (reinterpret_cast<uintptr_t>(scale) & 3u) != 0)
        return PSA_ERR_INVALID_ARG;
    return hip_status(psa::launch_quantize_fp8(batch, heads, seq_len, head_dim, x, x_stride,
                                               x_pooled, x8, x8_pooled, scale,
                                               static_cast<hipStream_t>(stream)));
}

int psa_attn_fwd_fp8qk(const psa_problem* prob, float softmax_scale, const uint8_t* q8,
                       const float* q_scale, const uint8_t* k8, const uint8_t* k8_pooled,
                       const float* k_scale, const void* v, const void* v_pooled,
                       const int8_t* level_map, void* o, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (s.NKB > psa::kAttnMaxKBlocks) return PSA_ERR_UNSUPPORTED;
    if (s.dtype != PSA_BF16 || s.D != 128) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q8 || !q_scale || !k8 || !k8_pooled || !k_scale || !v || !v_pooled || !level_map || !o)
        return PSA_ERR_INVALID_ARG;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(k8_pooled) || !aligned16(v) ||
        !aligned16(v_pooled) || !aligned16(o) || (reinterpret_cast<uintptr_t>(q_scale) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(k_scale) & 3u) != 0)
        return PSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return PSA_ERR_INVALID_ARG;
    const size_t need = attn_ws_layout(s, nullptr).bytes;
    if (ws == nullptr || ws_bytes < need) return PSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return PSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(s.D));
    hipStream_t st = static_cast<hipStream_t>(stream);
    AttnWs w = attn_ws_layout(s, ws);
    psa::IndexBufs ib{w.row_ptr, w.col_idx, w.dev_err};
    hipError_t e = psa::launch_build_index(s, level_map, ib, st);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(psa::launch_attn_fwd_fp8qk(s, scale, q8, q_scale, k8, k8_pooled, k_scale, v,
                                                 v_pooled, w.row_ptr, w.col_idx, o, lse, st));
}

int psa_attn_fwd_fp8(const psa_problem* prob, float softmax_scale, const uint8_t* q8,
                     const float* q_scale, const uint8_t* k8, const uint8_t* k8_pooled,
                     const float* k_scale, const uint8_t* v8, const uint8_t* v8_pooled,
                     const float* v_scale, const int8_t* level_map, void* o, float* lse, void* ws,
                     size_t ws_bytes, void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (s.NKB > psa::kAttnMaxKBlocks) return PSA_ERR_UNSUPPORTED;
    if (s.dtype != PSA_BF16 || s.D != 128) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q8 || !q_scale || !k8 || !k8_pooled || !k_scale || !v8 || !v8_pooled || !v_scale ||
        !level_map || !o)
        return PSA_ERR_INVALID_ARG;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(k8_pooled) || !aligned16(v8) ||
        !aligned16(v8_pooled) || !aligned16(o) || (reinterpret_cast<uintptr_t>(q_scale) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(k_scale) & 3u) != 0 || (reinterpret_cast<uintptr_t>(v_scale) & 3u) != 0)
        return PSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return PSA_ERR_INVALID_ARG;
    const size_t need = attn_ws_layout(s, nullptr).bytes;
    if (ws == nullptr || ws_bytes < need) return PSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return PSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(s.D));
    hipStream_t st = static_cast<hipStream_t>(stream);
    AttnWs w = attn_ws_layout(s, ws);
    psa::IndexBufs ib{w.row_ptr, w.col_idx, w.dev_err};
    hipError_t e = psa::launch_build_index(s, level_map, ib, st);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(psa::launch_attn_fwd_fp8(s, scale, q8, q_scale, k8, k8_pooled, k_scale, v8,
                                               v8_pooled, v_scale, w.row_ptr, w.col_idx, o, lse, st));
}

namespace {

struct MeanKeyWs {
    float* qbar;
    float* kbar;
    double* ksum;
    float* sim;
    double* sim64;
    size_t bytes;
};

MeanKeyWs meankey_ws_layout(const psa::Shape& s, void* base) {
    MeanKeyWs w;
    size_t off = 0;
    w.qbar = ws_at<float>(base, off);
    off += align_up(static_cast<size_t>(s.B) * s.H * s.NQB * s.D * sizeof(float));
    w.kbar = ws_at<float>(base, off);
    off += align_up(static_cast<size_t>(s.B) * s.Hkv * s.NKB * s.D * sizeof(float));
    w.ksum = ws_at<double>(base, off);
    off += align_up(static_cast<size_t>(s.B) * s.Hkv * s.NKB * s.D * sizeof(double));
    w.sim = ws_at<float>(base, off);
    off += align_up(static_cast<size_t>(s.B) * s.Hkv * s.NKB * sizeof(float));
    w.sim64 = ws_at<double>(base, off);
    off += align_up(static_cast<size_t>(s.B) * s.Hkv * s.NKB * sizeof(double));
    w.bytes = off;
    return w;
}

}  // namespace

size_t psa_attn_fwd_meankey_workspace_bytes(const psa_problem* prob) {
    psa::Shape s;
    if (check_problem(prob, &s) != PSA_OK) return 0;
    return meankey_ws_layout(s, nullptr).bytes;
}

int psa_attn_fwd_meankey(const psa_problem* prob, const psa_mask_params* params,
                         float softmax_scale, const void* q, const void* k, const void* v,
                         const void* k_pooled, const void* v_pooled, int8_t* level_map,
                         float* block_mass, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if ((rc = check_mask_params(prob, params)) != PSA_OK) return rc;
    if (params->mode != PSA_MASK_MEANKEY) return PSA_ERR_INVALID_ARG;
    if (s.dtype != PSA_BF16 || s.BQ != 128 || s.NKB > 1792) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q || !k || !v || !k_pooled || !v_pooled || !o) return PSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_pooled) ||
        !aligned16(v_pooled) || !aligned16(o))
        return PSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return PSA_ERR_INVALID_ARG;
    const size_t need = meankey_ws_layout(s, nullptr).bytes;
    if (ws == nullptr || ws_bytes < need) return PSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return PSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(s.D));
    hipStream_t st = static_cast<hipStream_t>(stream);
    MeanKeyWs w = meankey_ws_layout(s, ws);
    hipError_t e = psa::launch_block_means(s, q, k, w.qbar, w.kbar, w.ksum, st);
    if (e != hipSuccess) return hip_status(e);
    if (params->cos_sim_min > 0.f && (e = psa::launch_block_sim(s, k, w.sim, w.sim64, st)) != hipSuccess)
        return hip_status(e);
    return hip_status(psa::launch_attn_fwd_meankey(s, scale, *params, q, k, v, k_pooled, v_pooled,
                                                   w.qbar, w.kbar, w.ksum, w.sim, w.sim64, level_map,
                                                   block_mass, o, lse, st));
}

size_t psa_attn_bwd_workspace_bytes(const psa_problem* prob) {
    psa::Shape s;
    if (check_problem(prob, &s) != PSA_OK) return 0;
    return attn_ws_layout(s, nullptr).bytes + align_up(psa::attn_bwd_scratch_bytes(s));
}

int psa_attn_bwd(const psa_problem* prob, float softmax_scale, const void* q, const void* k,
                 const void* v, const void* k_pooled, const void* v_pooled,
                 const int8_t* level_map, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (s.NKB > psa::kAttnMaxKBlocks) return PSA_ERR_UNSUPPORTED;
    if (s.dtype != PSA_BF16) return PSA_ERR_UNSUPPORTED;
    // the key-side kernel lists (query head, query block) rows in LDS beside its three chunk
    // buffer sets and the P/dS exchange: 12-bit query block index, at most 7680 rows per KV head
    const int g = s.H / s.Hkv;
    if (s.NQB >= 4096 || static_cast<int64_t>(g) * s.NQB > 7680) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q || !k || !v || !k_pooled || !v_pooled || !level_map || !o || !lse || !dout || !dq ||
        !dk || !dv)
        return PSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_pooled) ||
        !aligned16(v_pooled) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return PSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return PSA_ERR_INVALID_ARG;
    const AttnWs w0 = attn_ws_layout(s, nullptr);
    const size_t need = w0.bytes + align_up(psa::attn_bwd_scratch_bytes(s));
    if (ws == nullptr || ws_bytes < need) return PSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return PSA_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(s.D));
    hipStream_t st = static_cast<hipStream_t>(stream);
    AttnWs w = attn_ws_layout(s, ws);
    psa::IndexBufs ib{w.row_ptr, w.col_idx, w.dev_err};
    hipError_t e = psa::launch_build_index(s, level_map, ib, st);
    if (e != hipSuccess) return hip_status(e);
    void* scratch = static_cast<char*>(ws) + w0.bytes;
    return hip_status(psa::launch_attn_bwd(s, scale, q, k, v, k_pooled, v_pooled, level_map,
                                           w.row_ptr, w.col_idx, o, lse, dout, dq, dk, dv,
                                           scratch, st));
}

int psa_check_status(const void* ws, void* stream) {
    if (ws == nullptr) return PSA_ERR_INVALID_ARG;
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e);
    int32_t flag = 0;
    e = hipMemcpy(&flag, ws, sizeof(flag), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    return flag == 0 ? PSA_OK : PSA_ERR_BAD_LEVEL_MAP;
}

const char* psa_status_string(int status) {
    switch (status) {
        case PSA_OK: return "PSA_OK";
        case PSA_ERR_INVALID_ARG: return "PSA_ERR_INVALID_ARG: invalid argument";
        case PSA_ERR_UNSUPPORTED: return "PSA_ERR_UNSUPPORTED: outside the supported domain";
        case PSA_ERR_WORKSPACE: return "PSA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case PSA_ERR_HIP: return "PSA_ERR_HIP: HIP runtime or launch failure";
        case PSA_ERR_BAD_LEVEL_MAP: return "PSA_ERR_BAD_LEVEL_MAP: level map entry outside {-1,0,1,2,3}";
        case PSA_ERR_SCRATCH:
            return "PSA_ERR_SCRATCH: block index larger than the allocation-free call's fixed scratch";
        default: return "unknown psa status";
    }
}

int psa_last_hip_error(void) { return g_last_hip_error; }

int psa_debug_fill_lds(uint32_t pattern, void* stream) {
    return hip_status(psa::launch_fill_lds(pattern, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Allocation-free attention: psa_attn_fwd with its block index (row_ptr, col_idx) in a
// file-scope device array instead of a caller workspace. Each GPU holds its own copy of the
// array from the library's load until the process ends; its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that address is passed
// to kernels. Every call on one GPU shares the array: calls that overlap on one GPU race.
// ---------------------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;   // 128 MiB per GPU
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use on that device).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t psa_attn_fwd_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int psa_attn_fwd_noalloc(const psa_problem* prob, float softmax_scale, const void* q, const void* k,
                         const void* v, const void* k_pooled, const void* v_pooled,
                         const int8_t* level_map, void* o, float* lse, int32_t* dev_err,
                         void* stream) {
    psa::Shape s;
    int rc = check_problem(prob, &s);
    if (rc != PSA_OK) return rc;
    if (s.NKB > psa::kAttnMaxKBlocks) return PSA_ERR_UNSUPPORTED;
    if (no_work(s)) return PSA_OK;
    if (!q || !k || !v || !k_pooled || !v_pooled || !level_map || !o || !dev_err)
        return PSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_pooled) ||
        !aligned16(v_pooled) || !aligned16(o))
        return PSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return PSA_ERR_INVALID_ARG;
    // the index: row_ptr [R*5 + 1] then col_idx [R*NKB], as in the workspace of psa_attn_fwd
    const size_t R = static_cast<size_t>(s.B) * s.H * s.NQB;
    const size_t rp_bytes = align_up((R * 5 + 1) * sizeof(int32_t));
    const size_t need = rp_bytes + align_up(R * s.NKB * sizeof(int32_t));
    if (need > kNoAllocScratchBytes) return PSA_ERR_SCRATCH;
    void* base = nullptr;
    hipError_t e = scratch_address(&base);
    if (e != hipSuccess) return hip_status(e);
    int32_t* row_ptr = static_cast<int32_t*>(base);
    int32_t* col_idx = reinterpret_cast<int32_t*>(static_cast<char*>(base) + rp_bytes);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(s.D));
    hipStream_t st = static_cast<hipStream_t>(stream);
    psa::IndexBufs ib{row_ptr, col_idx, dev_err};
    if ((e = psa::launch_build_index(s, level_map, ib, st)) != hipSuccess) return hip_status(e);
    return hip_status(psa::launch_attn_fwd(s, scale, q, k, v, k_pooled, v_pooled, row_ptr, col_idx,
                                           o, lse, true, st));
}

}  // extern "C"
