/*
 * psa.h - C ABI of libpsa: the Pyramid Sparse Attention (PSA) path, written in HIP
 * for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * PSA (arXiv 2512.04025; summary article at rg.mbintangr.com, section "Method") replaces the
 * keep/drop decision of block-sparse attention with a level per (query block, KV block) pair:
 * level 0 reads the block's full-resolution keys/values, levels 1/2/3 read them 1D mean-pooled
 * by 2/4/8, and the least important pairs are skipped. The path has three calls:
 *   psa_build_pyramid  - the mean-pooled levels 1..3 of K and V;
 *   psa_mask           - block importance (sampling or antidiagonal scoring, optional
 *                        intra-block cosine check) and threshold assignment of levels;
 *   psa_attn_fwd       - the level-weighted flash-style attention;
 *   psa_attn_bwd       - its backward (dq, dk, dv through every pyramid level).
 * plus psa_mask_assign and psa_build_index, the mask's and the attention's integer stages,
 * exported on their own, psa_quantize_fp8 / psa_attn_fwd_fp8qk / psa_attn_fwd_fp8, the
 * forward with its q . k products (and its P V product) on e4m3 operands, and
 * psa_attn_fwd_meankey, block-mean scoring fused into the attention.
 *
 * Conventions shared by every call
 *  - Pointers named q, k, v, o, k_pooled, v_pooled, level_map, block_mass, block_sim, lse,
 *    row_ptr, col_idx, dev_err, dout, dq, dk, dv, x, x_pooled, q8, k8, k8_pooled, v8,
 *    v8_pooled, x8, x8_pooled, scale, q_scale, k_scale, v_scale and ws are DEVICE pointers owned by the
 *    caller; the library never allocates or frees device memory and keeps no state between
 *    calls. psa_problem, psa_mask_params and x_stride are HOST pointers, read during the call
 *    only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is only
 *    enqueued: no call synchronises except psa_check_status.
 *  - Arguments are checked on the host before anything is enqueued. A failed check returns a
 *    negative psa_status and enqueues nothing. No C++ exception crosses this interface.
 *  - A problem with batch 0 or seq_len 0 has no work: after the shape and parameter checks
 *    every call returns PSA_OK without reading its device pointers (they may be null) or
 *    enqueueing anything (psa_quantize_fp8 with seq_len 0 still writes scale = 1 per head).
 *  - All calls are reentrant; calls on different streams may run concurrently provided their
 *    output and workspace buffers do not overlap.
 *
 * Tensor layouts (element counts, row-major):
 *   Q, O      [batch, heads_q,  seq_len, head_dim]  with strides q_stride / o_stride
 *   K, V      [batch, heads_kv, seq_len, head_dim]  with strides k_stride / v_stride
 *   k_pooled, v_pooled  [batch, heads_kv, 7*seq_len/8, head_dim], contiguous, same dtype as K:
 *             level l (1..3) occupies rows [seq_len - 2*seq_len/2^l, seq_len - seq_len/2^l),
 *             i.e. level 1 at row 0, level 2 at seq_len/2, level 3 at 3*seq_len/4.
 *   level_map [batch, heads_q, seq_len/block_q, seq_len/block_k] int8, contiguous;
 *             0..3 = level, -1 = skip.
 *   block_mass [batch, heads_q, NQB, NKB] float32; block_sim [batch, heads_kv, NKB] float32.
 *   lse       [batch, heads_q, seq_len] float32 (natural-log logsumexp of the logits).
 * Strides are in elements for the (batch, head, token) axes; head_dim is contiguous. Strides
 * must be positive multiples of 8 and base pointers 16-byte aligned.
 * GQA: query head h reads KV head h / (heads_q / heads_kv).
 *
 * Supported domain (anything else returns PSA_ERR_UNSUPPORTED): dtype f32 or bf16;
 * head_dim 64 or 128; block_k 64; block_q 64 or 128; seq_len a multiple of block_q;
 * 0 <= seq_valid <= seq_len with (seq_len - seq_valid) a multiple of 8 (so that every pooled
 * token is either wholly valid or wholly padding). The attention calls (forward, fp8,
 * backward) need seq_len/64 <= 16384: a row's block list is staged in LDS. psa_mask and
 * psa_mask_assign need one row's assignment to fit 64 KB of LDS: 8*P + 5*NKB bytes, plus
 * 4*NKB*RQ when scoring (P = NKB rounded up to a power of two, NKB = seq_len/64, RQ = the
 * scoring rows per query block: samples_per_qblock, block_q/antidiag_stride, or 1 for block
 * means), e.g. NKB <= 1328 with 8 samples, NKB <= 831 with antidiagonal stride 8 and block_q
 * 128. Checked on the host before anything is enqueued.
 */
#ifndef PSA_H_
#define PSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define PSA_OK 0
#define PSA_ERR_INVALID_ARG (-1)   /* null pointer, negative size, inconsistent shape/stride */
#define PSA_ERR_UNSUPPORTED (-2)   /* valid request outside the supported domain above */
#define PSA_ERR_WORKSPACE (-3)     /* workspace null or smaller than the *_workspace_bytes query */
#define PSA_ERR_HIP (-4)           /* a HIP runtime call or kernel launch failed; see psa_last_hip_error */
#define PSA_ERR_BAD_LEVEL_MAP (-5) /* a level map entry outside {-1,0,1,2,3} was seen on the device */
#define PSA_ERR_SCRATCH (-6)       /* the allocation-free call's fixed scratch cannot hold the index */

/* Element types. */
#define PSA_F32 0
#define PSA_BF16 1

#define PSA_SKIP (-1)
#define PSA_NUM_LEVELS 4

/* Mask generator modes (summary article, "Method": sampling-based for generation, antidiagonal
 * scoring with an intra-block similarity check for understanding). */
#define PSA_MASK_SAMPLING 0
#define PSA_MASK_ANTIDIAG 1
/* Block-mean scoring (skill summary at skillsmp.com, "Implementation": a query against each KV
 * block's mean key): the cheapest estimator, one score per (query block, KV block). */
#define PSA_MASK_MEANKEY 2

typedef struct psa_problem {
    int32_t batch, heads_q, heads_kv;
    int32_t seq_len;    /* padded length N */
    int32_t seq_valid;  /* valid tokens Nv; keys >= Nv are never attended, queries >= Nv give 0 */
    int32_t head_dim;
    int32_t block_q, block_k;
    int32_t causal;     /* nonzero: query i sees full-resolution key j iff j <= i */
    int32_t dtype;      /* PSA_F32 or PSA_BF16, for Q, K, V, O and the pooled levels */
    int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
} psa_problem;

typedef struct psa_mask_params {
    int32_t mode;                 /* PSA_MASK_SAMPLING, PSA_MASK_ANTIDIAG or PSA_MASK_MEANKEY */
    float thresholds[4];          /* cumulative-mass thresholds t0 <= t1 <= t2 <= t3, in (0, 1] */
    int32_t samples_per_qblock;   /* sampling mode: rows per query block; 1, 2, 4, .., 32 */
    int32_t antidiag_stride;      /* antidiagonal mode: stride S in {2, 4, 8}, block_q/S <= 32 */
    float cos_sim_min;            /* pooled levels need block similarity >= this; <= 0 disables */
    int32_t force_diag_l0;        /* nonzero: blocks overlapping the query block's tokens are L0 */
    int32_t force_l0_begin;       /* token span [begin, end) forced to L0 in both directions; */
    int32_t force_l0_end;         /* empty if begin >= end */
} psa_mask_params;

/* Rows per (batch, KV head) of the packed pooled tensors: 7*seq_len/8; -1 on a bad problem. */
int64_t psa_pooled_rows(const psa_problem* prob);

/*
 * Levels 1..3 of K and V (summary article, "Method": a pyramid built by progressive 1D mean
 * pooling; skill summary at skillsmp.com, "Implementation": level l pools by 2^l).
 * k_pooled/v_pooled row j of level l = mean of full-resolution rows [j*2^l, (j+1)*2^l).
 * Accumulation is a pairwise float32 tree (each level is the pairwise mean of the one
 * below), which equals the direct mean up to one rounding per addition.
 * out_dtype: the problem's dtype (bf16 outputs are the tree's float32 values rounded to
 * nearest even; this is what the attention calls read), or PSA_F32 for float32 levels of a
 * bf16 problem (parity runs: the tree's values before rounding). A float32 problem with a
 * bf16 out_dtype returns PSA_ERR_UNSUPPORTED; any other value PSA_ERR_INVALID_ARG.
 * k_pooled/v_pooled: [batch][heads_kv][7*seq_len/8][head_dim] contiguous, in out_dtype,
 * 16-byte aligned, caller-owned. Level 0 is not copied: the attention reads K and V directly.
 */
int psa_build_pyramid(const psa_problem* prob, const void* k, const void* v,
                      void* k_pooled, void* v_pooled, int32_t out_dtype, void* stream);

/* Device workspace psa_mask needs for `params`; 0 on a bad argument. */
size_t psa_mask_workspace_bytes(const psa_problem* prob, const psa_mask_params* params);

/*
 * Multi-level mask generator (summary article, "Method" and "Results").
 *  Sampling mode: for each query block, S = samples_per_qblock rows r_s = floor(s*R/S) of its
 *   R valid rows are scored against every valid level-0 key of its KV head (softmax of
 *   q.k/sqrt(d), keys >= seq_valid masked, causal keys after the row masked);
 *   block_mass[qb][kb] = mean over the S rows of the probability mass of KV block kb.
 *  Antidiagonal mode, stride S: compressed logits
 *   A[r][c] = (1/sqrt(d)) * sum_{t<S} q[r*S+S-1-t] . k[c*S+t], softmax over valid c
 *   (causal: c <= r), block_mass[qb][kb] = mass of kb's columns averaged over qb's valid rows.
 *  Block-mean mode: q_bar = mean of the query block's valid rows, k_bar = mean of the KV
 *   block's n valid keys, block_mass[qb][kb] = softmax over the candidate blocks of
 *   q_bar.k_bar/sqrt(d) + ln(n) (causal: blocks up to the last one overlapping the query
 *   block); samples_per_qblock and antidiag_stride are ignored.
 *  If cos_sim_min > 0, block_sim[b][hkv][kb] = mean cosine similarity over ordered pairs of
 *   distinct valid level-0 keys of the block (written; block_sim must then be non-null).
 *  Then psa_mask_assign's rule turns block_mass (and block_sim) into level_map.
 * block_mass is required (it is an output). Workspace: psa_mask_workspace_bytes.
 * Scoring runs bf16 MFMA: psa_mask needs dtype PSA_BF16 (PSA_ERR_UNSUPPORTED otherwise);
 * psa_mask_assign takes masses of any origin.
 */
int psa_mask(const psa_problem* prob, const psa_mask_params* params, const void* q,
             const void* k, int8_t* level_map, float* block_mass, float* block_sim,
             void* ws, size_t ws_bytes, void* stream);

/*
 * Certification inside psa_mask (the level map's threshold decisions are discontinuous in the
 * masses, so float32 scores could flip a decision that sits at their rounding level). The
 * scores and the assignment run in float32 (the assignment's running sum in float64); a row
 * with a decision within a margin of a threshold, or with two sorted masses within the margin
 * (relative) of each other on either side of a level change, is rescored in float64 on the
 * device (logits as float64 dots of the bf16 inputs, float64 softmax and block masses; in
 * block-mean mode float64 means) and reassigned in float64 (margins, from the float32 masses'
 * largest errors measured against float64 at full size: 4e-6 absolute and 8e-6 relative for
 * sampling and block-mean scores, 5e-6 and 3.3e-5 for antidiagonal scores); its block_mass
 * row then holds those masses
 * rounded to float. The similarity check compares the float64 similarity (block_sim holds it
 * rounded to float). At most a workspace-bounded number of rows per call (all rows of the
 * usual shapes; at least 16) are rescored; rows beyond it keep the float32 decisions.
 * psa_mask_certified_rows reads the counters of the last psa_mask call on `ws`:
 * counts[0] = rows flagged, counts[1] = flagged rows left uncertified (beyond the capacity).
 * It synchronizes `stream` (the stream psa_mask ran on). counts: host memory, 2 int32.
 */
int psa_mask_certified_rows(const psa_problem* prob, const psa_mask_params* params,
                            const void* ws, int32_t* counts, void* stream);

/*
 * Threshold assignment (summary article, "Results": threshold-based levels with a cosine
 * constraint on pooling). Per (batch, head, query block) row, over the candidate blocks
 * (all; causal: those overlapping tokens <= the block's last token):
 *   sort by block_mass descending (ties: lower kb first); exclusive running sum c in float64
 *   in that order; level = min{l : c < thresholds[l]}, otherwise skip.
 * Then: causal non-candidates -> skip; forced L0 (force_diag_l0: blocks overlapping the query
 * block's tokens; the forced span in either direction) -> 0; a pooled level on a block with
 * block_sim < cos_sim_min (when cos_sim_min > 0) -> 0. A query block with no valid query row is
 * all skip. block_sim may be null when cos_sim_min <= 0. Integer output, deterministic.
 */
int psa_mask_assign(const psa_problem* prob, const psa_mask_params* params,
                    const float* block_mass, const float* block_sim, int8_t* level_map,
                    void* stream);

/*
 * Block index: a CSR over (row, level) keys, rows r = (b*heads_q + h)*NQB + qb.
 * row_ptr[R*5+1] int32: col_idx[row_ptr[r*4+l] .. row_ptr[r*4+l+1]) lists, in ascending
 * order, the kb with level_map == l; then row_ptr[R*4+1 + p], p < R, is the row the attention
 * runs in dispatch slot p (a permutation of the rows: slot p runs on XCD p / ceil(R/8)). The
 * rows are grouped by KV head, r / (NQB*heads_q/heads_kv), groups in ascending order, each
 * group listed by its rows' count of 64-row tiles, sum over l of ceil(n_l / 2^l), largest
 * first (a stable counting sort over 32 buckets of the group's span of counts, exact when that
 * span is at most 32). That list is laid over chunks of f consecutive XCD ranges, f the
 * smallest of 1, 2, 4, 8 with (8/f) * 2 * (N + 7N/8) * d * sizeof(element) <= 128 MB (1 when
 * B*heads_kv == 1): inside a chunk, position j goes to range (first + j mod f), slot j/f of that
 * range, while every range of the chunk has slots left, the chunk's tail to the remaining slots
 * in order. For f < 8 each range is sorted on its own where it cuts a group; for f = 8 whole
 * groups are sorted. col_idx needs capacity R*NKB int32; its entries past
 * row_ptr[R*4] are unspecified (the call parks scan partial sums there). Entries outside
 * {-1..3} are treated as skip and set *dev_err (device int32) to PSA_ERR_BAD_LEVEL_MAP;
 * the call clears *dev_err first.
 */
int psa_build_index(const psa_problem* prob, const int8_t* level_map, int32_t* row_ptr,
                    int32_t* col_idx, int32_t* dev_err, void* stream);

/* Device workspace psa_attn_fwd needs; 0 on a bad problem. */
size_t psa_attn_workspace_bytes(const psa_problem* prob);

/*
 * Adaptive Pyramid Attention forward (summary article, "Method": each KV block is fetched at
 * its level and a scaling factor keeps the probabilities consistent; news summary at
 * euno.news, "Methodology" item 4: equivalent to upsampling the pooled block and running
 * standard scaled dot-product attention). For every valid query i of query block qb:
 *   z_j = softmax_scale * q_i . Kbar_j + l_j * ln 2
 * over the pooled rows j of every block listed for (b, h, qb) at its level l_j (weight 2^l_j
 * per pooled token), a pooled token being visible iff its last full-resolution token is
 * < seq_valid and (causal) <= i; o_i = sum_j softmax(z)_j Vbar_j, lse_i = logsumexp_j z_j.
 * A query with no visible key, and every query >= seq_valid, gets o = 0 and lse = -inf.
 * softmax_scale <= 0 selects 1/sqrt(head_dim). lse may be null. k_pooled/v_pooled come from
 * psa_build_pyramid on the same K, V. The block index is built inside the call (into ws).
 * bf16 runs MFMA in bf16 with float32 accumulation and softmax; f32 runs float32 MFMA.
 */
int psa_attn_fwd(const psa_problem* prob, float softmax_scale, const void* q, const void* k,
                 const void* v, const void* k_pooled, const void* v_pooled,
                 const int8_t* level_map, void* o, float* lse, void* ws, size_t ws_bytes,
                 void* stream);

/*
 * psa_attn_fwd on a block index already built by psa_build_index (row_ptr, col_idx) for the
 * same problem, e.g. a map reused across layers or denoising steps. Same math and outputs;
 * no workspace. The index must describe a map of this problem's shape.
 */
int psa_attn_fwd_indexed(const psa_problem* prob, float softmax_scale, const void* q,
                         const void* k, const void* v, const void* k_pooled,
                         const void* v_pooled, const int32_t* row_ptr, const int32_t* col_idx,
                         void* o, float* lse, void* stream);

/*
 * psa_attn_fwd_indexed without the decoupled block-tile packing (summary article, "Results":
 * the block-tile kernel against a naive implementation): every 64-row hardware tile holds ONE
 * logical block, so a level-l tile carries 64/2^l pooled rows and masks the rest. Same math
 * and outputs as psa_attn_fwd_indexed; it exists as the ablation baseline that the packed
 * kernel is measured against. dtype PSA_BF16 only (PSA_ERR_UNSUPPORTED otherwise).
 */
int psa_attn_fwd_unpacked(const psa_problem* prob, float softmax_scale, const void* q,
                          const void* k, const void* v, const void* k_pooled,
                          const void* v_pooled, const int32_t* row_ptr, const int32_t* col_idx,
                          void* o, float* lse, void* stream);

/*
 * Per-head e4m3 quantization for the fp8 QK^T reading (PSA paper abstract and the news summary
 * at euno.news, "Practical": the block-tile kernel suits FP16 and FP8 arithmetic; the pages fix
 * no quantization recipe, this one keeps one scale per (batch, head)). For each of the
 * batch*heads heads of x (bf16 [batch, heads, seq_len, head_dim], element strides x_stride[3]
 * for the batch, head and token axes, head_dim contiguous):
 *   amax  = max |x| over the head's seq_len rows;
 *   scale[b*heads + h] = amax / 448 rounded to float32 (448 = the largest finite e4m3), or 1
 *           when amax = 0;
 *   x8    = the e4m3 (OCP FP8 E4M3, bias 7, with subnormals) code nearest to the exact
 *           quotient x / scale, ties to even, written contiguous [batch, heads, seq_len,
 *           head_dim] bytes; the code stands for value(code) * scale.
 * With x_pooled (bf16 [batch, heads, 7*seq_len/8, head_dim], contiguous, the layout of
 * psa_build_pyramid's outputs) the pooled rows are quantized with the same scale into
 * x8_pooled (contiguous, same shape, bytes); x_pooled and x8_pooled are both null or both set.
 * x must be finite. seq_len and head_dim multiples of 8, batch*heads <= 65535; x, x_pooled
 * 16-byte aligned, x8, x8_pooled 8-byte aligned. All pointers are device pointers; x_stride
 * is a host array.
 */
int psa_quantize_fp8(int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                     const void* x, const int64_t* x_stride, const void* x_pooled, uint8_t* x8,
                     uint8_t* x8_pooled, float* scale, void* stream);

/*
 * psa_attn_fwd with the q . k products taken on e4m3 operands (paper abstract and news
 * summary, "Practical": FP8 arithmetic on the block-tile kernel): q8 (scale q_scale), k8 and
 * k8_pooled (one scale k_scale per KV head, shared by the pooled levels) as written by
 * psa_quantize_fp8 from Q, K and psa_build_pyramid's k_pooled. The logits are
 *   z_j = softmax_scale * q_scale[b,h] * k_scale[b,hkv] * (q8_i . k8bar_j) + l_j ln 2
 * with the products exact and summed in float32 (v_mfma_f32_32x32x64_f8f6f4); everything else
 * (levels, masking, softmax, P V in bf16, o, lse, the workspace and its status) is as in
 * psa_attn_fwd. q8 [batch, heads_q, seq_len, 128], k8 [batch, heads_kv, seq_len, 128] and
 * k8_pooled [batch, heads_kv, 7*seq_len/8, 128] are contiguous bytes (prob->q_stride and
 * prob->k_stride are not used); q_scale [batch*heads_q], k_scale [batch*heads_kv] float32.
 * v, v_pooled, o follow the problem (dtype PSA_BF16). head_dim 128 only; anything else returns
 * PSA_ERR_UNSUPPORTED. Workspace: psa_attn_workspace_bytes.
 */
int psa_attn_fwd_fp8qk(const psa_problem* prob, float softmax_scale, const uint8_t* q8,
                       const float* q_scale, const uint8_t* k8, const uint8_t* k8_pooled,
                       const float* k_scale, const void* v, const void* v_pooled,
                       const int8_t* level_map, void* o, float* lse, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * psa_attn_fwd_fp8qk with the P V product on e4m3 operands as well (paper abstract and news
 * summary, "Practical"): v8 and v8_pooled are psa_quantize_fp8's codes of V and of
 * psa_build_pyramid's v_pooled (one scale v_scale per KV head), contiguous like k8 and
 * k8_pooled. For each valid query, in log2 units t_j = z_j / ln 2 (z_j as in
 * psa_attn_fwd_fp8qk), with M an integer no less than max_j t_j - 8 (the kernel's running
 * maximum, rounded up to an integer):
 *   P8_j = e4m3(2^(t_j - M)) (round to nearest even),
 *   o = v_scale * sum_j P8_j v8_j / sum_j P8_j,   lse = (M + log2 sum_j P8_j) ln 2.
 * e4m3 rounding commutes with the power-of-two change of M except for values in e4m3's
 * subnormal range, so the result depends on the running maximum only at that level. Both
 * products run on v_mfma_f32_32x32x64_f8f6f4 with float32 accumulation (the sum of P8 by a
 * ones-row product). head_dim 128, dtype PSA_BF16 (o) only; anything else returns
 * PSA_ERR_UNSUPPORTED. Workspace: psa_attn_workspace_bytes.
 */
int psa_attn_fwd_fp8(const psa_problem* prob, float softmax_scale, const uint8_t* q8,
                     const float* q_scale, const uint8_t* k8, const uint8_t* k8_pooled,
                     const float* k_scale, const uint8_t* v8, const uint8_t* v8_pooled,
                     const float* v_scale, const int8_t* level_map, void* o, float* lse, void* ws,
                     size_t ws_bytes, void* stream);

/* Device workspace psa_attn_fwd_meankey needs; 0 on a bad problem. */
size_t psa_attn_fwd_meankey_workspace_bytes(const psa_problem* prob);

/*
 * Block-mean scoring fused into the attention (skill summary at skillsmp.com,
 * "Implementation": a query against each KV block's mean key, the cheapest estimator; scored
 * inside the attention's prologue, no separate mask pass or block index). params->mode must
 * be PSA_MASK_MEANKEY (else PSA_ERR_INVALID_ARG). Computes exactly what psa_mask (block-mean
 * mode, same params) followed by psa_attn_fwd computes - the same level map bit for bit, the
 * same outputs - but each attention workgroup scores its own query block's mean against every
 * KV block mean (float64 dots), assigns the levels with the same steps as psa_mask_assign and
 * attends over the resulting list. level_map and block_mass (layouts as in psa_mask) receive
 * the map and the masses when not null. The cosine check runs when cos_sim_min > 0.
 * dtype PSA_BF16, block_q 128 and seq_len/64 <= 1792 only (PSA_ERR_UNSUPPORTED otherwise).
 * Workspace: psa_attn_fwd_meankey_workspace_bytes (the block means, the float64 key sums of each
 * KV block and the similarities).
 */
int psa_attn_fwd_meankey(const psa_problem* prob, const psa_mask_params* params,
                         float softmax_scale, const void* q, const void* k, const void* v,
                         const void* k_pooled, const void* v_pooled, int8_t* level_map,
                         float* block_mass, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/* Device workspace psa_attn_bwd needs; 0 on a bad problem. */
size_t psa_attn_bwd_workspace_bytes(const psa_problem* prob);

/*
 * Backward of psa_attn_fwd (news summary at euno.news, "Methodology" item 4: pooling is
 * deterministic, so gradients flow through every pyramid level and the layer trains end to
 * end). Given the forward's o and lse for the same problem, map and softmax_scale, and the
 * output gradient dout, writes
 *   dq = dL/dq,  dk = dL/dk,  dv = dL/dv   (L with dL/do = dout)
 * for the level-0 q, k, v: with P the forward's softmax weights over the gathered pooled rows,
 * dVbar = P^T dO, dS = P * (dO Vbar^T - rowsum(dO * o)), dq = s dS Kbar, dKbar = s dS^T q, and a
 * pooled row of level l hands 2^-l of its gradient to each of its 2^l tokens. A KV head's
 * gradient sums over the query heads that share it. Pad query rows and rows with no visible
 * key contribute nothing and get dq = 0; pad tokens get dk = dv = 0.
 * Layouts: dout and o use o_stride, dq uses q_stride, dk uses k_stride, dv uses v_stride (all
 * in the problem's dtype); lse is the forward's [batch, heads_q, seq_len] float32 output (not
 * null). The block index is built inside the call (into ws); invalid map entries are
 * recorded for psa_check_status as in psa_attn_fwd.
 * dtype PSA_BF16 only (bf16 MFMA, f32 accumulation; P and dS enter the products rounded to
 * bf16); seq_len/block_q < 4096 and (heads_q/heads_kv) * seq_len/block_q <= 7680.
 * Anything else returns PSA_ERR_UNSUPPORTED.
 */
int psa_attn_bwd(const psa_problem* prob, float softmax_scale, const void* q, const void* k,
                 const void* v, const void* k_pooled, const void* v_pooled,
                 const int8_t* level_map, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * Waits for `stream`, then reports device-side errors recorded in `ws` by the last
 * psa_attn_fwd or psa_attn_bwd that used it: PSA_OK or PSA_ERR_BAD_LEVEL_MAP (or PSA_ERR_HIP).
 */
int psa_check_status(const void* ws, void* stream);

/* Static string for a status code. */
const char* psa_status_string(int status);

/*
 * Allocation-free psa_attn_fwd, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation). Same math, kernels
 * and outputs as psa_attn_fwd; the block index it builds lives in a file-scope device array of
 * psa_attn_fwd_noalloc_max_bytes() bytes (128 MiB) that each GPU holds from the library's load
 * until the process ends, instead of a caller workspace. The call allocates and frees nothing.
 * Needs 4*(R*5 + 1) + 4*R*NKB bytes (rounded up to 256 each; R = batch*heads_q*NQB) of it,
 * else returns PSA_ERR_SCRATCH with nothing enqueued. dev_err: caller-owned device int32,
 * cleared by the call and set to PSA_ERR_BAD_LEVEL_MAP on an invalid map entry (read it after
 * the stream completes). Calls on one GPU share the array: calls that overlap on one GPU (two
 * streams, two host threads) race; serialize them.
 */
int psa_attn_fwd_noalloc(const psa_problem* prob, float softmax_scale, const void* q, const void* k,
                         const void* v, const void* k_pooled, const void* v_pooled,
                         const int8_t* level_map, void* o, float* lse, int32_t* dev_err,
                         void* stream);

/* Size in bytes of psa_attn_fwd_noalloc's per-GPU scratch array. */
size_t psa_attn_fwd_noalloc_max_bytes(void);

/*
 * Diagnostics (no part of the path): enqueues workgroups that fill the LDS of every CU with
 * the 32-bit `pattern` (e.g. a NaN), so that the kernels enqueued next start on LDS holding
 * it. A kernel that read LDS it had not written would then show the pattern in its outputs;
 * the tests run the path after such a fill and require outputs bit-identical to a run
 * without it.
 */
int psa_debug_fill_lds(uint32_t pattern, void* stream);

/* The hipError_t of the last PSA_ERR_HIP returned on this thread (0 if none). */
int psa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PSA_H_ */
