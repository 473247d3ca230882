// Adaptive Pyramid Attention forward on gfx950 (PSA summary article at rg.mbintangr.com,
// "Method": every KV block is fetched at its assigned pyramid level and a scaling factor keeps
// the probabilities consistent; the kernel separates the logical block size from the hardware
// tile size and is flash-attention compatible).
//
// Math. For query i and the pooled rows j of the listed blocks,
//   z_j = scale * q_i . Kbar_j + l_j * ln2,
// i.e. weight 2^l per pooled token (it stands for 2^l tokens: nearest-neighbour upsampling
// followed by standard attention, news summary at euno.news, "Methodology" item 4, gives the
// same result). In the exp2 domain the level term is exactly +l, so it folds into the
// per-row offset of the exp2 argument: p = exp2(s * c + (l - m)), c = scale * log2(e).
//
// Work decomposition. One workgroup owns one (batch, head, query block) row. It walks the
// row's block index level by level; a 64-row hardware tile at level l packs 2^l logical
// pooled blocks (64 / 2^l rows each), gathered from the level's contiguous rows, so every
// tile is full-height whatever the level (the decoupled block-tile idea, rebuilt for a
// 64-wide wavefront and the 32x32 MFMA). Skipped blocks are never loaded. A partial last
// tile of a level is padded by repeating its first block and masking the absent rows.
//
// Per wave: 32 query rows. S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, queries on
// N), so every lane holds one query and 16 keys per 32x32 accumulator: the row max and sum
// are in-lane plus one v_permlane32_swap. P^T stays in registers and feeds O^T = V^T * P^T
// directly as the B operand; the matching key order is produced by reading V^T from LDS.
// Q lives in registers for the whole row. Global loads of the next tile are issued before the
// current tile's math (register double buffering); LDS holds one K tile and one V^T tile.
//
// f32 inputs run the same schedule on v_mfma_f32_32x32x2f32 with K and V row-major in LDS.
#include <math.h>

#include "psa_device.h"
#include "psa_internal.h"

namespace psa {
namespace {

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
    int H, Hkv, N, Nv, NQB, causal;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
    int64_t pooled_rows;
    float c;  // softmax scale * log2(e)
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

// ---------------------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------------------
template <int D, int BQ>
struct Bf16Cfg {
    static constexpr int NW = BQ / 32;        // waves
    static constexpr int NT = 64 * NW;        // threads
    static constexpr int KSTR = D + 8;        // K tile row stride (elements)
    static constexpr int VSTR = 64 + 4;       // V^T tile row stride (elements)
    static constexpr int KCH = 64 * (D / 8) / NT;   // 16-byte K chunks per thread
    static constexpr int VUN = 64 * D / 16 / NT;    // 4x4 V units per thread
    static_assert(KCH >= 1 && VUN >= 1, "tile too small for the workgroup");
};

template <int D, int BQ>
__global__ void __launch_bounds__(2 * BQ)
    k_attn_fwd_bf16(AttnArgs a) {
    using C = Bf16Cfg<D, BQ>;
    __shared__ __attribute__((aligned(16))) bf16_bits Ks[64 * C::KSTR];
    __shared__ __attribute__((aligned(16))) bf16_bits Vt[D * C::VSTR];
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

    const bf16_bits* __restrict__ Q = static_cast<const bf16_bits*>(a.q);
    const bf16_bits* __restrict__ K = static_cast<const bf16_bits*>(a.k);
    const bf16_bits* __restrict__ V = static_cast<const bf16_bits*>(a.v);
    const bf16_bits* __restrict__ KP = static_cast<const bf16_bits*>(a.kp);
    const bf16_bits* __restrict__ VP = static_cast<const bf16_bits*>(a.vp);

    const int q_tok = qb * BQ + wave * 32 + l32;  // this lane's query
    const int limit = a.causal ? (q_tok < a.Nv - 1 ? q_tok : a.Nv - 1) : a.Nv - 1;
    const int blk_first = qb * BQ;
    const int min_limit = a.causal ? (blk_first < a.Nv - 1 ? blk_first : a.Nv - 1) : a.Nv - 1;

    // Q fragments (B operand of S^T = K Q^T): query l32, head-dim slice hi*8 of each 16-chunk.
    bf16x8 qf[D / 16];
    {
        const bf16_bits* qp = Q + b * a.qs0 + h * a.qs1 + static_cast<int64_t>(q_tok) * a.qs2;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hi * 8);
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

    // register staging of the next tile
    u32x4 kreg[C::KCH];
    u32x2 vreg[C::VUN][4];
    int lastreg = kNoToken;

    auto load_tile = [&](const TileWalk& t) {
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
            const int c = tid + i * C::NT;
            const int r = c / (D / 8);
            const int col = (c % (D / 8)) * 8;
            RowSrc s = tile_row(a, t, r, pbase, D, a.ks2, kbase);
            const bf16_bits* p = (s.pooled ? KP : K) + s.off + col;
            kreg[i] = *reinterpret_cast<const u32x4*>(p);
        }
#pragma unroll
        for (int i = 0; i < C::VUN; ++i) {
            const int u = tid + i * C::NT;
            const int kq = u / (D / 4);
            const int dq = (u % (D / 4)) * 4;
            RowSrc s = tile_row(a, t, kq * 4, pbase, D, a.vs2, vbase);
            const bf16_bits* p = (s.pooled ? VP : V) + s.off + dq;
            const int64_t rs = s.pooled ? D : a.vs2;
#pragma unroll
            for (int j = 0; j < 4; ++j) vreg[i][j] = *reinterpret_cast<const u32x2*>(p + j * rs);
        }
        if (tid < 64) lastreg = tile_row(a, t, tid, pbase, D, a.ks2, kbase).last;
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
            const int c = tid + i * C::NT;
            const int r = c / (D / 8);
            const int col = (c % (D / 8)) * 8;
            *reinterpret_cast<u32x4*>(&Ks[r * C::KSTR + col]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < C::VUN; ++i) {
            const int u = tid + i * C::NT;
            const int kq = u / (D / 4);
            const int dq = (u % (D / 4)) * 4;
            // vreg[i][j] holds V[key 4kq+j][dq..dq+3]; write V^T[dq+e][4kq..4kq+3].
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int w = e >> 1;
                const int sh = (e & 1) * 16;
                const uint32_t x0 = (vreg[i][0][w] >> sh) & 0xffffu;
                const uint32_t x1 = (vreg[i][1][w] >> sh) & 0xffffu;
                const uint32_t x2 = (vreg[i][2][w] >> sh) & 0xffffu;
                const uint32_t x3 = (vreg[i][3][w] >> sh) & 0xffffu;
                u32x2 t2;
                t2[0] = x0 | (x1 << 16);
                t2[1] = x2 | (x3 << 16);
                *reinterpret_cast<u32x2*>(&Vt[(dq + e) * C::VSTR + kq * 4]) = t2;
            }
        }
        if (tid < 64) lastk[tid] = lastreg;
    };

    if (any_valid_query && tw.valid()) load_tile(tw);

    while (any_valid_query && tw.valid()) {
        const int lvl = tw.l;
        const int cnt = tw.count();
        const int kb_max = a.col_idx[tw.lbase + tw.pos + cnt - 1];
        const bool need_mask = (cnt < (1 << lvl)) || ((kb_max + 1) * 64 - 1 > min_limit);

        __syncthreads();  // previous tile's LDS reads are done
        store_tile();
        __syncthreads();

        TileWalk nxt = tw;
        nxt.next();
        if (nxt.valid()) load_tile(nxt);

        // ---- S^T = K Q^T ----
        f32x16 sacc[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kh][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                    &Ks[(kh * 32 + l32) * C::KSTR + kk * 16 + hi * 8]);
                sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sacc[kh], 0, 0, 0);
            }
        }

        // ---- mask, online softmax ----
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
        const float alpha = fast_exp2(m_run - m_ref);
        m_run = m_new;
        if (__ballot(alpha != 1.f) != 0ull) {
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
        }
        const float off = flvl - m_ref;
        float psum = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = fast_exp2(fmaf(sacc[kh][e], a.c, off));
                sacc[kh][e] = p;
                psum += p;
            }
        l_run += psum;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kh = j >> 1;
            const int e0 = (j & 1) * 8;
            union {
                bf16x8 v;
                uint32_t u[4];
            } pb;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                pb.u[t] = pack_bf16x2(sacc[kh][e0 + 2 * t], sacc[kh][e0 + 2 * t + 1]);
            const int kb0 = 32 * kh + 16 * (j & 1) + hi * 4;
#pragma unroll
            for (int dblk = 0; dblk < D / 32; ++dblk) {
                const bf16_bits* vr = &Vt[(dblk * 32 + l32) * C::VSTR + kb0];
                union {
                    bf16x8 v;
                    u32x2 h[2];
                } va;
                va.h[0] = *reinterpret_cast<const u32x2*>(vr);
                va.h[1] = *reinterpret_cast<const u32x2*>(vr + 8);
                oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va.v, pb.v, oacc[dblk], 0, 0, 0);
            }
        }
        tw = nxt;
    }

    // ---- epilogue ----
    const float l_tot = pair32_sum(l_run);
    const bool valid_q = q_tok < a.Nv && l_tot > 0.f;
    const float inv = valid_q ? 1.f / l_tot : 0.f;
    bf16_bits* O = static_cast<bf16_bits*>(a.o) + b * a.os0 + h * a.os1 +
                   static_cast<int64_t>(q_tok) * a.os2;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[dblk][4 * g] * inv, oacc[dblk][4 * g + 1] * inv);
            w[1] = pack_bf16x2(oacc[dblk][4 * g + 2] * inv, oacc[dblk][4 * g + 3] * inv);
            *reinterpret_cast<u32x2*>(O + dblk * 32 + g * 8 + hi * 4) = w;
        }
    if (a.lse != nullptr && hi == 0) {
        const float lse = valid_q ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        a.lse[(static_cast<int64_t>(b) * a.H + h) * a.N + q_tok] = lse;
    }
}

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

hipError_t launch_attn_fwd(const Shape& s, float scale, const void* q, const void* k,
                           const void* v, const void* kp, const void* vp,
                           const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                           hipStream_t st) {
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
    const int64_t rows = static_cast<int64_t>(s.B) * s.H * s.NQB;
    if (rows == 0) return hipSuccess;
    if (s.dtype == PSA_BF16) {
        if (s.D == 128 && s.BQ == 128) return launch(k_attn_fwd_bf16<128, 128>, 256, a, rows, st);
        if (s.D == 128 && s.BQ == 64) return launch(k_attn_fwd_bf16<128, 64>, 128, a, rows, st);
        if (s.D == 64 && s.BQ == 128) return launch(k_attn_fwd_bf16<64, 128>, 256, a, rows, st);
        if (s.D == 64 && s.BQ == 64) return launch(k_attn_fwd_bf16<64, 64>, 128, a, rows, st);
    } else {
        if (s.D == 128 && s.BQ == 128) return launch(k_attn_fwd_f32<128, 128>, 256, a, rows, st);
        if (s.D == 128 && s.BQ == 64) return launch(k_attn_fwd_f32<128, 64>, 128, a, rows, st);
        if (s.D == 64 && s.BQ == 128) return launch(k_attn_fwd_f32<64, 128>, 256, a, rows, st);
        if (s.D == 64 && s.BQ == 64) return launch(k_attn_fwd_f32<64, 64>, 128, a, rows, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace psa
