// Adaptive Pyramid Attention forward: the float32 kernel and the dispatch for both dtypes
// (the bf16 kernel, the fast path, lives in psa_attn_bf16.hip).
//
// Math (PSA summary article at rg.mbintangr.com, "Method"): for query i and the pooled rows j
// of the listed blocks, z_j = scale * q_i . Kbar_j + l_j * ln2, i.e. weight 2^l per pooled
// token (news summary at euno.news, "Methodology" item 4: the same as upsampling the pooled
// block and running standard attention). In the exp2 domain the level term is exactly +l.
//
// The f32 kernel: one workgroup per (batch, head, query block) row, 32 queries per wave,
// S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x2f32 with K and V row-major in LDS (one
// fp32 value per lane per operand needs no transposition), register double buffering of the
// next tile, online softmax in the exp2 domain. It serves float32 problems (parity-grade
// accuracy), not the bf16 fast path.
#include <math.h>

#include "psa_attn_common.h"

namespace psa {
namespace {

// ---------------------------------------------------------------------------------------
// f32 kernel (v_mfma_f32_32x32x2f32): same walk, K and V row-major in LDS.
// ---------------------------------------------------------------------------------------
template <int D, int BQ>
struct F32Cfg {
    static constexpr int NW = BQ / 32;
    static constexpr int NT = 64 * NW;
    static constexpr int KSTR = D + 2;   // even row shift: keys on even banks, hi on odd
    static constexpr int VSTR = D + 8;   // 4 rows apart = 32 banks
    static constexpr int KCH = 64 * (D / 4) / NT;  // 16-byte chunks per thread (K and V each)
    static_assert(KCH >= 1, "tile too small for the workgroup");
};

template <int D, int BQ>
__global__ void __launch_bounds__(2 * BQ)
    k_attn_fwd_f32(AttnArgs a) {
    using C = F32Cfg<D, BQ>;
    __shared__ __attribute__((aligned(16))) float Ks[64 * C::KSTR];
    __shared__ __attribute__((aligned(16))) float Vs[64 * C::VSTR];
    __shared__ int lastk[64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int64_t row = blockIdx.x;
    const int qb = static_cast<int>(row % a.NQB);
    const int bh = static_cast<int>(row / a.NQB);
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);

    const float* __restrict__ Q = static_cast<const float*>(a.q);
    const float* __restrict__ K = static_cast<const float*>(a.k);
    const float* __restrict__ V = static_cast<const float*>(a.v);
    const float* __restrict__ KP = static_cast<const float*>(a.kp);
    const float* __restrict__ VP = static_cast<const float*>(a.vp);

    const int q_tok = qb * BQ + wave * 32 + l32;
    const int limit = a.causal ? (q_tok < a.Nv - 1 ? q_tok : a.Nv - 1) : a.Nv - 1;
    const int blk_first = qb * BQ;
    const int min_limit = a.causal ? (blk_first < a.Nv - 1 ? blk_first : a.Nv - 1) : a.Nv - 1;

    float qf[D / 2];
    {
        const float* qp = Q + b * a.qs0 + h * a.qs1 + static_cast<int64_t>(q_tok) * a.qs2;
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) qf[kk] = qp[kk * 2 + hi];
    }
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    TileWalk tw;
    tw.init(a.row_ptr, row);
    const bool any_valid_query = blk_first < a.Nv;
    const int64_t kbase = b * a.ks0 + hk * a.ks1;
    const int64_t vbase = b * a.vs0 + hk * a.vs1;
    const int64_t pbase = (static_cast<int64_t>(b) * a.Hkv + hk) * a.pooled_rows * D;

    f32x4 kreg[C::KCH], vreg[C::KCH];
    int lastreg = kNoToken;
    auto load_tile = [&](const TileWalk& t) {
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
            const int c = tid + i * C::NT;
            const int r = c / (D / 4);
            const int col = (c % (D / 4)) * 4;
            RowSrc s = tile_row(a, t, r, pbase, D, a.ks2, kbase);
            kreg[i] = *reinterpret_cast<const f32x4*>((s.pooled ? KP : K) + s.off + col);
            RowSrc sv = tile_row(a, t, r, pbase, D, a.vs2, vbase);
            vreg[i] = *reinterpret_cast<const f32x4*>((sv.pooled ? VP : V) + sv.off + col);
        }
        if (tid < 64) lastreg = tile_row(a, t, tid, pbase, D, a.ks2, kbase).last;
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
            const int c = tid + i * C::NT;
            const int r = c / (D / 4);
            const int col = (c % (D / 4)) * 4;
            float* kd = &Ks[r * C::KSTR + col];
            kd[0] = kreg[i][0];
            kd[1] = kreg[i][1];
            kd[2] = kreg[i][2];
            kd[3] = kreg[i][3];
            *reinterpret_cast<f32x4*>(&Vs[r * C::VSTR + col]) = vreg[i];
        }
        if (tid < 64) lastk[tid] = lastreg;
    };

    if (any_valid_query && tw.valid()) load_tile(tw);
    while (any_valid_query && tw.valid()) {
        const int lvl = tw.l;
        const int cnt = tw.count();
        const int kb_max = a.col_idx[tw.lbase + tw.pos + cnt - 1];
        const bool need_mask = (cnt < (1 << lvl)) || ((kb_max + 1) * 64 - 1 > min_limit);
        __syncthreads();
        store_tile();
        __syncthreads();
        TileWalk nxt = tw;
        nxt.next();
        if (nxt.valid()) load_tile(nxt);

        f32x16 sacc[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kh][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const float ka = Ks[(kh * 32 + l32) * C::KSTR + kk * 2 + hi];
                sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, qf[kk], sacc[kh], 0, 0, 0);
            }
        if (need_mask) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int kr = kh * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
                    if (lastk[kr] > limit) sacc[kh][e] = -INFINITY;
                }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kh][e]);
        mt = pair32_max(mt);
        const float flvl = static_cast<float>(lvl);
        const float m_new = fmaxf(m_run, fmaf(mt, a.c, flvl));
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_ref);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
        const float off = flvl - m_ref;
        float psum = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = exp2f(fmaf(sacc[kh][e], a.c, off));
                sacc[kh][e] = p;
                psum += p;
            }
        l_run += psum;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = kh * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
#pragma unroll
                for (int dblk = 0; dblk < D / 32; ++dblk) {
                    const float va = Vs[key * C::VSTR + dblk * 32 + l32];
                    oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, sacc[kh][e], oacc[dblk], 0, 0, 0);
                }
            }
        tw = nxt;
    }

    const float l_tot = pair32_sum(l_run);
    const bool valid_q = q_tok < a.Nv && l_tot > 0.f;
    const float inv = valid_q ? 1.f / l_tot : 0.f;
    float* O = static_cast<float*>(a.o) + b * a.os0 + h * a.os1 + static_cast<int64_t>(q_tok) * a.os2;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = oacc[dblk][4 * g + e] * inv;
            *reinterpret_cast<f32x4*>(O + dblk * 32 + g * 8 + hi * 4) = w;
        }
    if (a.lse != nullptr && hi == 0) {
        const float lse = valid_q ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        a.lse[(static_cast<int64_t>(b) * a.H + h) * a.N + q_tok] = lse;
    }
}

template <typename Kern>
hipError_t launch(Kern kern, int threads, const AttnArgs& a, int64_t rows, hipStream_t st) {
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(rows)), dim3(threads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

namespace {

AttnArgs make_args(const Shape& s, float scale, const void* q, const void* k, const void* v,
                   const void* kp, const void* vp, const int32_t* row_ptr,
                   const int32_t* col_idx, void* o, float* lse) {
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.kp = kp;
    a.vp = vp;
    a.o = o;
    a.lse = lse;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.row_order = row_ptr != nullptr ? row_ptr + static_cast<int64_t>(s.B) * s.H * s.NQB * 4 + 1 : nullptr;
    a.H = s.H;
    a.Hkv = s.Hkv;
    a.N = s.N;
    a.Nv = s.Nv;
    a.NQB = s.NQB;
    a.causal = s.causal;
    a.qs0 = s.qs[0]; a.qs1 = s.qs[1]; a.qs2 = s.qs[2];
    a.ks0 = s.ks[0]; a.ks1 = s.ks[1]; a.ks2 = s.ks[2];
    a.vs0 = s.vs[0]; a.vs1 = s.vs[1]; a.vs2 = s.vs[2];
    a.os0 = s.os[0]; a.os1 = s.os[1]; a.os2 = s.os[2];
    a.pooled_rows = s.pooled_rows;
    a.c = scale * kLog2e;
    a.q_scale = nullptr;
    a.k_scale = nullptr;
    a.v_scale = nullptr;
    return a;
}

}  // namespace

hipError_t launch_attn_fwd(const Shape& s, float scale, const void* q, const void* k,
                           const void* v, const void* kp, const void* vp,
                           const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                           bool pack, hipStream_t st) {
    const AttnArgs a = make_args(s, scale, q, k, v, kp, vp, row_ptr, col_idx, o, lse);
    const int64_t rows = static_cast<int64_t>(s.B) * s.H * s.NQB;
    if (rows == 0) return hipSuccess;
    if (s.dtype == PSA_BF16) {
        return launch_attn_bf16(s, a, pack, st);
    } else {
        if (!pack) return hipErrorNotSupported;
        if (s.D == 128 && s.BQ == 128) return launch(k_attn_fwd_f32<128, 128>, 256, a, rows, st);
        if (s.D == 128 && s.BQ == 64) return launch(k_attn_fwd_f32<128, 64>, 128, a, rows, st);
        if (s.D == 64 && s.BQ == 128) return launch(k_attn_fwd_f32<64, 128>, 256, a, rows, st);
        if (s.D == 64 && s.BQ == 64) return launch(k_attn_fwd_f32<64, 64>, 128, a, rows, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_fp8qk(const Shape& s, float scale, const uint8_t* q8,
                                 const float* q_scale, const uint8_t* k8, const uint8_t* kp8,
                                 const float* k_scale, const void* v, const void* vp,
                                 const int32_t* row_ptr, const int32_t* col_idx, void* o,
                                 float* lse, hipStream_t st) {
    if (s.dtype != PSA_BF16) return hipErrorNotSupported;
    AttnArgs a = make_args(s, scale, q8, k8, v, kp8, vp, row_ptr, col_idx, o, lse);
    // the e4m3 operands are contiguous [batch, head, token, head_dim] bytes
    const int64_t nd = static_cast<int64_t>(s.N) * s.D;
    a.qs0 = s.H * nd; a.qs1 = nd; a.qs2 = s.D;
    a.ks0 = s.Hkv * nd; a.ks1 = nd; a.ks2 = s.D;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    return launch_attn_fp8qk(s, a, st);
}

hipError_t launch_attn_fwd_fp8(const Shape& s, float scale, const uint8_t* q8, const float* q_scale,
                               const uint8_t* k8, const uint8_t* kp8, const float* k_scale,
                               const uint8_t* v8, const uint8_t* vp8, const float* v_scale,
                               const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                               hipStream_t st) {
    if (s.dtype != PSA_BF16) return hipErrorNotSupported;
    AttnArgs a = make_args(s, scale, q8, k8, v8, kp8, vp8, row_ptr, col_idx, o, lse);
    // every e4m3 operand is contiguous [batch, head, token, head_dim] bytes
    const int64_t nd = static_cast<int64_t>(s.N) * s.D;
    a.qs0 = s.H * nd; a.qs1 = nd; a.qs2 = s.D;
    a.ks0 = s.Hkv * nd; a.ks1 = nd; a.ks2 = s.D;
    a.vs0 = s.Hkv * nd; a.vs1 = nd; a.vs2 = s.D;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return launch_attn_fp8(s, a, st);
}

}  // namespace psa
