// Backward of the Adaptive Pyramid Attention, bf16 on gfx950 (news summary at euno.news,
// "Methodology" item 4: pooling is deterministic, so gradients flow through every level and
// the layer trains end to end).
//
// With P_ij = exp(z_ij - lse_i) recomputed from the forward's lse (z as in the forward:
// softmax scale * q_i . Kbar_j + l_j ln 2 over the row's listed pooled rows):
//   dVbar = P^T dO,  dP = dO Vbar^T,  D_i = dO_i . o_i,  dS = P * (dP - D),
//   dq = s dS Kbar,  dKbar = s dS^T q,
// and a pooled row of level l (the mean of 2^l tokens) hands 2^-l of its gradient to each
// of its tokens. A KV head's gradient is the sum over the query heads that share it.
//
// Kernels (in launch order):
//  k_bwd_rowdot  D_i = dO_i . o_i and lse2_i = lse_i log2 e per query row (f32); rows that
//                are padding or see no key get lse2 = +inf, so their P is exactly 0.
//  k_bwd_dq      one workgroup per (batch, head, query block) row, walking the row's block
//                index in packed tiles like the forward: S^T = Kbar Q^T, dP^T = Vbar dO^T,
//                dQ^T += Kbar^T dS^T. 32 queries per wave; each wave owns its queries' dq.
//  k_bwd_dkv     one workgroup per (batch, KV head, level, 64-row pooled tile; the tiles are
//                claimed per XCD range with spill-over to the next ranges): scans the
//                level map for the (query head, query block) rows that list one of the
//                tile's blocks at that level (ordered, so the sums are deterministic), then
//                per listed row and 64-query chunk: S = Q Kbar^T, dP = dO Vbar^T,
//                dVbar^T += dO^T P, dKbar^T += Q^T dS. Eight waves: four producers (S, dP,
//                P, dS; each owns 32 keys and half of the chunk's queries) hand P and dS
//                through LDS to four consumers (the dV / dK products and accumulators), one
//                chunk behind; a producer and its consumer share a SIMD. Three chunk buffer
//                sets (producers' chunk, consumers' chunk, the next one loading) by direct
//                loads, Q and dO staged once each in the fq layout. The loop holds no load the
//                compiler tracks (a compiler-placed wait would also drain the direct loads in
//                flight). The tile's pooled-row gradients go to an f32 workspace (every row
//                written, zeros included: no clearing pass).
//  k_bwd_pool    dK[t] = sum_l 2^-l dKbar_l[t >> l] (and dV), in the input dtype.
//
// All products run on v_mfma_f32_32x32x16_bf16 with f32 accumulation; P and dS enter the
// products rounded to bf16. Operand tiles are staged in LDS by direct loads
// (global_load_lds_dwordx4), in the swizzled layouts of psa_bf16_tile.h: in the dq kernel K
// once in the fq layout (read by rows for S and transposed for dQ) and V in fk; in the dkv
// kernel Q and dO once each in the fq layout, read both ways.
#include <limits.h>
#include <math.h>

#include "psa_attn_common.h"
#include "psa_bf16_tile.h"

namespace psa {
namespace {

struct BwdArgs {
    const bf16_bits* q;
    const bf16_bits* k;
    const bf16_bits* v;
    const bf16_bits* kp;
    const bf16_bits* vp;
    const bf16_bits* o;
    const bf16_bits* dout;
    const float* lse;
    const int8_t* map;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    float* lse2;   // [B*H*N]
    float* dd;     // [B*H*N]
    float* gk;     // [B*Hkv][N + 7N/8][D]: level 0 rows, then the pooled levels' rows
    float* gv;
    bf16_bits* dq;
    bf16_bits* dk;
    bf16_bits* dv;
    int* claim;    // [8] next unclaimed pooled tile of each XCD's range (k_bwd_dkv), zeroed per call
    int share;        // k_bwd_dkv's XCD ranges per chunk of tiles (1, 2, 4, 8), as the index's order
    int B, H, Hkv, N, Nv, NQB, NKB, BQ, causal;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
    int64_t pooled_rows;   // 7N/8
    float c;               // softmax scale * log2 e
    float scale;
};

// Row of pooled level l (1..3) inside the packed pooled tensor; level 0 rows are the tokens.
__device__ __forceinline__ int64_t level_row_offset(int N, int l) {
    return l == 0 ? 0 : static_cast<int64_t>(N) - (static_cast<int64_t>(N) >> (l - 1));
}

// ---------------------------------------------------------------------------------------
// D_i = dO_i . o_i, lse2_i = lse_i log2 e. 16 lanes per row (16-byte chunks), 16 rows per
// 256-thread workgroup.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) k_bwd_rowdot(BwdArgs a) {
    constexpr int CH = D / 8;                       // chunks per row
    constexpr int RPW = 256 / 16;                   // rows per workgroup
    const int tid = threadIdx.x;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPW + tid / 16;
    const int sub = tid % 16;
    const int64_t rows = static_cast<int64_t>(a.B) * a.H * a.N;
    if (row >= rows) return;   // whole 16-lane groups leave together
    const int i = static_cast<int>(row % a.N);
    const int64_t bh = row / a.N;
    const int h = static_cast<int>(bh % a.H);
    const int b = static_cast<int>(bh / a.H);
    const bf16_bits* op = a.o + b * a.os0 + h * a.os1 + static_cast<int64_t>(i) * a.os2;
    const bf16_bits* gp = a.dout + b * a.os0 + h * a.os1 + static_cast<int64_t>(i) * a.os2;
    float s = 0.f;
    for (int c = sub; c < CH; c += 16) {
        const u32x4 ov = *reinterpret_cast<const u32x4*>(op + c * 8);
        const u32x4 gv = *reinterpret_cast<const u32x4*>(gp + c * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            s = fmaf(__uint_as_float(ov[w] << 16), __uint_as_float(gv[w] << 16), s);
            s = fmaf(__uint_as_float(ov[w] & 0xffff0000u), __uint_as_float(gv[w] & 0xffff0000u), s);
        }
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 16);
    if (sub == 0) {
        const float l = a.lse[row];
        const bool live = i < a.Nv && l > -INFINITY;
        a.dd[row] = live ? s : 0.f;
        a.lse2[row] = live ? l * kLog2e : INFINITY;
    }
}

// ---------------------------------------------------------------------------------------
// Direct loads of 64 consecutive tile rows into a swizzled LDS tile. Tile row t comes from
// `src_row(t)` (an element pointer to its first element; rows RPI-aligned runs are
// consecutive with byte stride `stride`). Each of the workgroup's NW waves issues
// IPW = INSTR / NW instructions; instruction m covers tile rows [m*RPI, (m+1)*RPI).
// ---------------------------------------------------------------------------------------
// tile layouts of psa_bf16_tile.h
enum { kLayK = 0, kLayV = 1, kLayQ = 2 };
template <int D, int LAY>
__device__ __forceinline__ int swz(int r) {
    return LAY == kLayK ? Lay<D>::fk(r) : LAY == kLayV ? Lay<D>::fv(r) : Lay<D>::fq(r);
}

template <int D, int NW, int LAY, typename RunBase>
__device__ __forceinline__ void load_tile(uint32_t lds, int wave, int lane, uint32_t stride,
                                          RunBase&& run_base) {
    using LY = Lay<D>;
    constexpr int IPW = LY::INSTR / NW;
    const int rr = lane / LY::CH;
    const int p = lane % LY::CH;
#pragma unroll
    for (int mi = 0; mi < IPW; ++mi) {
        const int m = wave * IPW + mi;
        const int trow = m * LY::RPI + rr;
        const int f = swz<D, LAY>(trow);
        const uint32_t voff = rr * stride + static_cast<uint32_t>((p ^ f) << 4);
        dma16(run_base(m * LY::RPI), voff, lds + static_cast<uint32_t>(m) * 1024u);
    }
}

// Per-lane LDS byte address of the A-operand row reads (rows row0 + sigma(l % 32)) of a tile
// in layout LAY: the address of k-step kk is the result XOR 32 kk.
template <int D, int LAY>
__device__ __forceinline__ uint32_t row_read_base(uint32_t lds, int lane, int row0) {
    const int r = row0 + sigma(lane & 31);
    const int hi = lane >> 5;
    const int f = swz<D, LAY>(r);
    return lds + static_cast<uint32_t>(r * D * 2 + 16 * ((hi ^ f) & 1) + 16 * (f & ~1));
}

// Per-lane LDS byte address of the transposed A-operand reads of 32-wide d block dblk, for
// contraction rows row0 + 8 (grp / 2) + jj / 4 + 4 s (s = 0, 1: the two halves of a
// fragment), in layout LAY. Fragment j adds 16 rows (j * 16 * D * 2 bytes), which leaves
// every layout's swizzle unchanged; so does a row0 that is a multiple of 16.
template <int D, int LAY>
__device__ __forceinline__ uint32_t tr_read_base(uint32_t lds, int lane, int dblk, int row0, int s) {
    const int grp = lane >> 4;
    const int jj = lane & 15;
    const int d = dblk * 32 + 16 * (grp & 1) + 4 * (jj & 3);
    const int c = d >> 3;
    const int half = d & 7;
    const int r = row0 + 8 * (grp >> 1) + (jj >> 2) + 4 * s;
    return lds + static_cast<uint32_t>((r * D + ((c ^ swz<D, LAY>(r)) << 3) + half) * 2);
}

__device__ __forceinline__ bf16x8 read_row(uint32_t base, int kk) {
    return *(const lds_bf16x8*)(uintptr_t)(base ^ static_cast<uint32_t>(32 * kk));
}

// fragment j of a transposed read: the halves at bases b0 (rows + 0) and b1 (rows + 4)
template <int D>
__device__ __forceinline__ bf16x8 read_tr(uint32_t b0, uint32_t b1, int j) {
    union {
        bf16x8 v;
        v4i16 h[2];
    } x;
    x.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(b0 + static_cast<uint32_t>(j * 16 * D * 2)));
    x.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(b1 + static_cast<uint32_t>(j * 16 * D * 2)));
    return x.v;
}

// ---------------------------------------------------------------------------------------
// dq: one workgroup per (batch, head, query block).
// ---------------------------------------------------------------------------------------
template <int D, int BQ>
__global__ void __launch_bounds__(2 * BQ, 2) k_bwd_dq(BwdArgs a, int total_rows) {
    using LY = Lay<D>;
    constexpr int NW = BQ / 32;
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(1024))) bf16_bits Kr[64 * D];   // K, read both ways (fq)
    __shared__ __attribute__((aligned(1024))) bf16_bits Vr[64 * D];   // V rows (fk)
    extern __shared__ int cols[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // XCD-aware row order: XCD x = i % 8 takes a contiguous range of rows in the index's
    // dispatch order (grouped by KV head, largest first), as the forward does
    const int nper = (total_rows + 7) >> 3;
    const int slot = (blockIdx.x & 7) * nper + (blockIdx.x >> 3);
    if (slot >= total_rows) return;
    const int row = a.row_ptr[static_cast<int64_t>(total_rows) * 4 + 1 + slot];
    const int qb = row % a.NQB;
    const int bh = row / a.NQB;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);

    const int32_t* rp = a.row_ptr + static_cast<int64_t>(row) * 4;
    const int r0 = rp[0];
    const int lb1 = rp[1] - r0, lb2 = rp[2] - r0, lb3 = rp[3] - r0, lb4 = rp[4] - r0;
    auto lb = [&](int l) { return l <= 0 ? 0 : l == 1 ? lb1 : l == 2 ? lb2 : l == 3 ? lb3 : lb4; };
    for (int i = tid; i < lb4; i += 2 * BQ) cols[i] = a.col_idx[r0 + i];

    const int qt = qb * BQ + wave * 32 + l32;   // this lane's query
    const int64_t qrow = (static_cast<int64_t>(b) * a.H + h) * a.N + qt;
    const float lse2 = a.lse2[qrow];
    const float dd = a.dd[qrow];

    bf16x8 qf[KK], gf[KK];
    {
        const bf16_bits* qp = a.q + b * a.qs0 + h * a.qs1 + static_cast<int64_t>(qt) * a.qs2;
        const bf16_bits* gp = a.dout + b * a.os0 + h * a.os1 + static_cast<int64_t>(qt) * a.os2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hi * 8);
            gf[kk] = *reinterpret_cast<const bf16x8*>(gp + kk * 16 + hi * 8);
        }
    }
    f32x16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

    const char* kl0 = reinterpret_cast<const char*>(a.k + b * a.ks0 + hk * a.ks1);
    const char* vl0 = reinterpret_cast<const char*>(a.v + b * a.vs0 + hk * a.vs1);
    const int64_t pbase = (static_cast<int64_t>(b) * a.Hkv + hk) * a.pooled_rows * D;
    const char* kpl = reinterpret_cast<const char*>(a.kp + pbase);
    const char* vpl = reinterpret_cast<const char*>(a.vp + pbase);
    const uint32_t lds_kr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Kr[0]));
    const uint32_t lds_vr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Vr[0]));
    const uint32_t kr_base = row_read_base<D, kLayQ>(lds_kr, lane, 0);   // + 32 rows: fq unchanged
    const uint32_t vr_base = row_read_base<D, kLayK>(lds_vr, lane, 0);
    uint32_t kt_base[2][DB];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dblk = 0; dblk < DB; ++dblk) kt_base[s2][dblk] = tr_read_base<D, kLayQ>(lds_kr, lane, dblk, 0, s2);
    __syncthreads();   // cols[] visible

    for (int l = 0; l < 4; ++l) {
        const int lbeg = lb(l), lend = lb(l + 1);
        const int sh = 6 - l;
        const int rs = 1 << sh;   // rows per logical block
        const int64_t lvl = level_row_offset(a.N, l);
        const uint32_t kst = static_cast<uint32_t>(l == 0 ? a.ks2 : D) * 2u;
        const uint32_t vst = static_cast<uint32_t>(l == 0 ? a.vs2 : D) * 2u;
        const char* kb0 = l == 0 ? kl0 : kpl + lvl * D * 2;
        const char* vb0 = l == 0 ? vl0 : vpl + lvl * D * 2;
        for (int base = lbeg; base < lend; base += 1 << l) {
            const int cnt = min(lend - base, 1 << l);
            // tile row t -> its block (absent blocks of a partial tile repeat the last one)
            auto src_row = [&](int t) {
                const int s = min(t >> sh, cnt - 1);
                return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(cols[base + s]) * rs + (t & (rs - 1)));
            };
            __syncthreads();   // the previous tile's reads are done
            load_tile<D, NW, kLayQ>(lds_kr, wave, lane, kst, [&](int t) { return kb0 + static_cast<uint64_t>(src_row(t)) * kst; });
            load_tile<D, NW, kLayK>(lds_vr, wave, lane, vst, [&](int t) { return vb0 + static_cast<uint64_t>(src_row(t)) * vst; });
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();

#pragma unroll 1
            for (int hh = 0; hh < 2; ++hh) {
                f32x16 s, dp;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    s[e] = 0.f;
                    dp[e] = 0.f;
                }
                const uint32_t hoff = static_cast<uint32_t>(hh * 32 * D * 2);
                bf16x8 ka[KK], va[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    ka[kk] = read_row(kr_base + hoff, kk);
                    va[kk] = read_row(vr_base + hoff, kk);
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk], gf[kk], dp, 0, 0, 0);
                }
                // P and dS of the 16 keys this lane holds: tile key t = 32 hh + 16 j + 8 hi + u
                // (j = r / 8, u = r % 8); a run of 8 aligned keys lies in one logical block
                uint32_t dsk[8];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int t0 = 32 * hh + 16 * j + 8 * hi;
                    const int sblk = t0 >> sh;
                    const bool present = sblk < cnt;
                    const int kb = cols[base + (present ? sblk : 0)];
                    const int last0 = ((kb * rs + (t0 & (rs - 1)) + 1) << l) - 1;   // key t0's last token
                    // key t0 + x is visible iff its last token <= lim (absent blocks: never)
                    const int lim = present ? (a.causal ? min(qt, a.Nv - 1) : a.Nv - 1) : -1;
#pragma unroll
                    for (int u = 0; u < 8; u += 2) {
                        float ds2[2];
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const int e = 8 * j + u + w;
                            const bool vis = last0 + ((u + w) << l) <= lim;
                            // branch-free: an invisible key's exponent is -inf, its P exactly 0
                            const float p = fast_exp2(vis ? fmaf(s[e], a.c, static_cast<float>(l) - lse2) : -INFINITY);
                            ds2[w] = p * (dp[e] - dd);
                        }
                        dsk[(8 * j + u) >> 1] = pack_bf16x2(ds2[0], ds2[1]);
                    }
                }
                // dQ^T += Kbar^T dS^T over the 32 keys of this half (two 16-key fragments)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const bf16x8 df = __builtin_bit_cast(bf16x8, u32x4{dsk[4 * j], dsk[4 * j + 1], dsk[4 * j + 2], dsk[4 * j + 3]});
                    bf16x8 kt[DB];
#pragma unroll
                    for (int dblk = 0; dblk < DB; ++dblk) kt[dblk] = read_tr<D>(kt_base[0][dblk] + hoff, kt_base[1][dblk] + hoff, j);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int dblk = 0; dblk < DB; ++dblk)
                        acc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[dblk], df, acc[dblk], 0, 0, 0);
                }
            }
        }
    }

    // dq rows: this lane's query, d = 32 dblk + 8 gg + 4 hi + 0..3
    bf16_bits* out = a.dq + b * a.qs0 + h * a.qs1 + static_cast<int64_t>(qt) * a.qs2;
#pragma unroll
    for (int dblk = 0; dblk < DB; ++dblk)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[dblk][4 * gg] * a.scale, acc[dblk][4 * gg + 1] * a.scale);
            w[1] = pack_bf16x2(acc[dblk][4 * gg + 2] * a.scale, acc[dblk][4 * gg + 3] * a.scale);
            *reinterpret_cast<u32x2*>(out + dblk * 32 + gg * 8 + hi * 4) = w;
        }
}

// ---------------------------------------------------------------------------------------
// dKbar, dVbar: one workgroup of 8 waves per (batch, KV head, level, 64-row pooled tile).
// Waves 0..3 produce: wave p owns tile keys 32 (p & 1) + 0..31 and queries 32 (p >> 1) + 0..31
// of each 64-query chunk of a listed query block; it computes S = Q Kbar^T, dP = dO Vbar^T,
// P and dS and hands P, dS to LDS. Wave p + 4 consumes them one chunk later: dVbar^T +=
// dO^T P, dKbar^T += Q^T dS for the same keys and queries. A producer and its consumer share a
// SIMD, so one's softmax work runs beside the other's MFMAs. Chunks are staged once each (the
// fq layout serves the row reads and the transposed reads) in three buffer sets: the chunk
// the producers work on, the one the consumers work on, and the next one loading.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(512, 1) k_bwd_dkv(BwdArgs a, int total_tiles, int tiles_per_bh,
                                                   int t1, int t2, int t3) {
    using LY = Lay<D>;
    constexpr int NW = 8;
    constexpr int KK = D / 16;
    constexpr int DB = D / 32;
    constexpr int NSET = 3;
    constexpr uint32_t kTileBytes = 64u * D * 2u;
    __shared__ __attribute__((aligned(1024))) bf16_bits Xs[NSET][2][64 * D];   // [set][Q, dO]
    __shared__ __attribute__((aligned(16))) float Ls[NSET][64];
    __shared__ __attribute__((aligned(16))) float Ds[NSET][64];
    __shared__ __attribute__((aligned(16))) u32x4 Xch[2][4][2][2][64];   // [buf][producer][j][P, dS][lane]
    __shared__ int wsum[NW + 1];
    extern __shared__ int ent[];   // listed rows: (query head in group << 20) | (qb << 8) | blocks

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int pw = wave & 3;      // producer / consumer pair index
    const int kh = pw & 1;
    const int qh = pw >> 1;

    // Tile claim. Workgroup i runs on XCD x = i % 8; it takes the next unclaimed tile of XCD
    // x's range of tiles and, once that range is exhausted, the next tile of the first
    // following range that has one left, so an XCD whose tiles happen to be cheap takes over
    // tiles of a busier one. The tiles are cut in chunks of f nper (f = the block index's XCD
    // ranges per chunk: the KV heads in flight fit in half the last-level cache), and range x
    // of its chunk is every f-th tile from the chunk's start + (x mod f): with f = 1 the
    // contiguous tiles [x nper, (x + 1) nper) (neighbouring tiles of a KV head share that
    // XCD's L2), with f = 8 the tiles x, x + 8, ... (the XCDs work through one KV head at a
    // time). The grid has
    // one workgroup per tile: every claim succeeds and every tile is processed once. (The
    // tiles are independent, so the assignment does not change any result.)
    const int nper = (total_tiles + 7) >> 3;
    __shared__ int claimed;
    if (tid == 0) {
        int t = -1;
        for (int d = 0; d < 8 && t < 0; ++d) {
            const int x = (static_cast<int>(blockIdx.x & 7) + d) & 7;
            const int f = a.share;
            const int x0 = x - x % f;                                // the chunk's first range
            const int lo = x0 * nper + (x - x0);                     // range x's first tile
            const int end = min((x0 + f) * nper, total_tiles);       // the chunk's end
            if (lo >= end) continue;
            const int c = atomicAdd(&a.claim[x], 1);
            if (lo + c * f < end) t = lo + c * f;
        }
        claimed = t;
    }
    __syncthreads();
    const int tile = claimed;
    if (tile < 0) return;
    const int bhk = tile / tiles_per_bh;
    int m = tile % tiles_per_bh;
    const int l = m < t1 ? 0 : m < t2 ? 1 : m < t3 ? 2 : 3;
    m -= l == 0 ? 0 : l == 1 ? t1 : l == 2 ? t2 : t3;
    const int hk = bhk % a.Hkv;
    const int b = bhk / a.Hkv;
    const int g = a.H / a.Hkv;
    const int nb = 1 << l;             // logical blocks per tile
    const int sh = 6 - l;

    // ---- the rows (query head, query block) that list one of the tile's blocks at level l,
    //      in ascending order ----
    int count = 0;
    const int cand = g * a.NQB;
    for (int c0 = 0; c0 < cand; c0 += 64 * NW) {
        const int e = c0 + tid;
        int bits = 0;
        if (e < cand) {
            const int hl = e / a.NQB;
            const int qb = e % a.NQB;
            const int8_t* mrow = a.map + ((static_cast<int64_t>(b) * a.H + hk * g + hl) * a.NQB + qb) * a.NKB;
            for (int s = 0; s < nb; ++s) {
                const int kb = m * nb + s;
                if (kb < a.NKB && mrow[kb] == l) bits |= 1 << s;
            }
        }
        const uint64_t ball = __ballot(bits != 0);
        if (lane == 0) wsum[wave] = __popcll(ball);
        __syncthreads();
        int before = count;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        const int mine = __popcll(ball & ((1ull << lane) - 1ull));
        if (bits != 0) ent[before + mine] = ((e / a.NQB) << 20) | ((e % a.NQB) << 8) | bits;
        int tot = 0;
        for (int w = 0; w < NW; ++w) tot += wsum[w];
        count += tot;
        __syncthreads();
    }

    // items: (listed row, 64-query chunk); item it is entry it >> csh, chunk it & csh
    const int csh = a.BQ == 128 ? 1 : 0;
    const int items = count << csh;
    auto item_entry = [&](int it) { return __builtin_amdgcn_readfirstlane(ent[it >> csh]); };
    auto item_q0 = [&](int en, int it) { return ((en >> 8) & 0xfff) * a.BQ + ((it & csh) << 6); };

    // ---- direct loads of a chunk: Q's 64 rows by waves 0..3, dO's by waves 4..7 (IPW
    //      instructions each); lse2 and D by wave 0 (16 lanes x 16 bytes) ----
    constexpr int IPW = LY::INSTR / 4;
    const bool ld_q = wave < 4;
    const int m0 = (wave & 3) * IPW;            // the wave's first instruction of its tensor
    const uint32_t stride = static_cast<uint32_t>(ld_q ? a.qs2 : a.os2) * 2u;
    uint32_t lo[IPW];
    {
        const int rr = lane / LY::CH;
        const int p = lane % LY::CH;
#pragma unroll
        for (int mi = 0; mi < IPW; ++mi) {
            const int trow = (m0 + mi) * LY::RPI + rr;
            lo[mi] = static_cast<uint32_t>(mi * LY::RPI + rr) * stride + static_cast<uint32_t>((p ^ LY::fq(trow)) << 4);
        }
    }
    const uint32_t xs0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Xs[0][0][0]));
    const uint32_t ls0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Ls[0][0]));
    const uint32_t ds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Ds[0][0]));
    auto issue = [&](int it, int set) {
        const int en = item_entry(it);
        const int h = hk * g + (en >> 20);
        const int q0 = item_q0(en, it);
        const int64_t r0 = static_cast<int64_t>(q0 + m0 * LY::RPI);
        const char* src = ld_q ? reinterpret_cast<const char*>(a.q + b * a.qs0 + h * a.qs1 + r0 * a.qs2)
                               : reinterpret_cast<const char*>(a.dout + b * a.os0 + h * a.os1 + r0 * a.os2);
        const uint32_t l0 = xs0 + static_cast<uint32_t>(set) * 2u * kTileBytes + (ld_q ? 0u : kTileBytes) +
                            static_cast<uint32_t>(m0) * 1024u;
#pragma unroll
        for (int mi = 0; mi < IPW; ++mi) dma16(src, lo[mi], l0 + static_cast<uint32_t>(mi) * 1024u);
        if (wave == 0 && lane < 16) {
            const int64_t r = (static_cast<int64_t>(b) * a.H + h) * a.N + q0;
            dma16(a.lse2 + r, static_cast<uint32_t>(lane) * 16u, ls0 + static_cast<uint32_t>(set) * 256u);
            dma16(a.dd + r, static_cast<uint32_t>(lane) * 16u, ds0 + static_cast<uint32_t>(set) * 256u);
        }
    };
    if (items > 0) issue(0, 0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // per-lane LDS read addresses in set 0 (other sets: + set * 2 * kTileBytes)
    auto fq_row_base = [&](uint32_t lds) { return row_read_base<D, kLayQ>(lds, lane, 32 * qh); };
    auto fq_tr_base = [&](uint32_t lds, int dblk, int s2) { return tr_read_base<D, kLayQ>(lds, lane, dblk, 32 * qh, s2); };
    const uint32_t xch0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Xch[0][0][0][0][0]));

    if (wave < 4) {
        // ================= producer =================
        const int jrow = 64 * m + 32 * kh + l32;          // pooled row of level l
        const bool in_level = jrow < (a.N >> l);
        const int jr = in_level ? jrow : 0;
        const int klast = ((jr + 1) << l) - 1;             // last token the key stands for
        const bool key_ok = in_level && klast < a.Nv;
        const int ksub = (32 * kh + l32) >> sh;            // its block inside the tile
        bf16x8 kf[KK], vf[KK];
        {
            const int64_t pbase = (static_cast<int64_t>(b) * a.Hkv + hk) * a.pooled_rows * D;
            const bf16_bits* kp = l == 0 ? a.k + b * a.ks0 + hk * a.ks1 + static_cast<int64_t>(jr) * a.ks2
                                         : a.kp + pbase + (level_row_offset(a.N, l) + jr) * D;
            const bf16_bits* vp = l == 0 ? a.v + b * a.vs0 + hk * a.vs1 + static_cast<int64_t>(jr) * a.vs2
                                         : a.vp + pbase + (level_row_offset(a.N, l) + jr) * D;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                kf[kk] = *reinterpret_cast<const bf16x8*>(kp + kk * 16 + hi * 8);
                vf[kk] = *reinterpret_cast<const bf16x8*>(vp + kk * 16 + hi * 8);
            }
        }
        const uint32_t q_rows = fq_row_base(xs0);
        const uint32_t g_rows = fq_row_base(xs0 + kTileBytes);
        const uint32_t xw = xch0 + static_cast<uint32_t>(pw) * (2u * 2u * 64u * 16u) + static_cast<uint32_t>(lane) * 16u;
        int set = 0;
        for (int k = 0; k <= items; ++k) {
            if (k + 1 < items) issue(k + 1, set == 2 ? 0 : set + 1);
            if (k < items) {
                const int en = item_entry(k);
                const int q0 = item_q0(en, k);
                const int bits = en & 0xff;
                // query q sees this lane's key iff q >= kmin (an unlisted or invalid key: never)
                const bool sub_ok = key_ok && ((bits >> ksub) & 1);
                const int kmin = sub_ok ? (a.causal ? klast : INT_MIN) : INT_MAX;
                const uint32_t soff = static_cast<uint32_t>(set) * 2u * kTileBytes;
                bf16x8 qa[KK], ga[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    qa[kk] = read_row(q_rows + soff, kk);
                    ga[kk] = read_row(g_rows + soff, kk);
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
                f32x16 s, dp;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    s[e] = 0.f;
                    dp[e] = 0.f;
                }
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], kf[kk], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[kk], vf[kk], dp, 0, 0, 0);
                }
                // register e holds chunk query 32 qh + 16 (e / 8) + 8 hi + e % 8, this lane's key
                const uint32_t xb = xw + static_cast<uint32_t>(k & 1) * (4u * 2u * 2u * 64u * 16u);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int qi0 = 32 * qh + 16 * j + 8 * hi;   // 8 consecutive chunk queries
                    const f32x4 la = *reinterpret_cast<const f32x4*>(&Ls[set][qi0]);
                    const f32x4 lb2 = *reinterpret_cast<const f32x4*>(&Ls[set][qi0 + 4]);
                    const f32x4 da = *reinterpret_cast<const f32x4*>(&Ds[set][qi0]);
                    const f32x4 db = *reinterpret_cast<const f32x4*>(&Ds[set][qi0 + 4]);
                    u32x4 pk, dk4;
#pragma unroll
                    for (int u = 0; u < 8; u += 2) {
                        float pp[2], ds2[2];
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const int e = 8 * j + u + w;
                            const int x = u + w;
                            const float lq = static_cast<float>(l) - (x < 4 ? la[x] : lb2[x - 4]);
                            const float dq = x < 4 ? da[x] : db[x - 4];
                            const bool vis = q0 + qi0 + x >= kmin;
                            const float p = fast_exp2(vis ? fmaf(s[e], a.c, lq) : -INFINITY);
                            pp[w] = p;
                            ds2[w] = p * (dp[e] - dq);
                        }
                        pk[u >> 1] = pack_bf16x2(pp[0], pp[1]);
                        dk4[u >> 1] = pack_bf16x2(ds2[0], ds2[1]);
                    }
                    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(xb + static_cast<uint32_t>(j) * (2u * 64u * 16u)) = pk;
                    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(xb + static_cast<uint32_t>(j) * (2u * 64u * 16u) + 64u * 16u) = dk4;
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            set = set == 2 ? 0 : set + 1;
        }
        __syncthreads();   // the consumers' reduction (two barriers, as on their side)
        __syncthreads();
    } else {
        // ================= consumer =================
        f32x16 dka[DB], dva[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                dka[i][e] = 0.f;
                dva[i][e] = 0.f;
            }
        uint32_t qt_base[2][DB], gt_base[2][DB];
#pragma unroll
        for (int sh2 = 0; sh2 < 2; ++sh2)
#pragma unroll
            for (int dblk = 0; dblk < DB; ++dblk) {
                qt_base[sh2][dblk] = fq_tr_base(xs0, dblk, sh2);
                gt_base[sh2][dblk] = fq_tr_base(xs0 + kTileBytes, dblk, sh2);
            }
        const uint32_t xr = xch0 + static_cast<uint32_t>(pw) * (2u * 2u * 64u * 16u) + static_cast<uint32_t>(lane) * 16u;
        int set = 0;        // set of item k
        int pset = 2;       // set of item k - 1
        for (int k = 0; k <= items; ++k) {
            if (k + 1 < items) issue(k + 1, set == 2 ? 0 : set + 1);
            if (k >= 1) {
                const uint32_t soff = static_cast<uint32_t>(pset) * 2u * kTileBytes;
                const uint32_t xb = xr + static_cast<uint32_t>((k - 1) & 1) * (4u * 2u * 2u * 64u * 16u);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x4 pk = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(xb + static_cast<uint32_t>(j) * (2u * 64u * 16u));
                    const u32x4 dk4 = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(xb + static_cast<uint32_t>(j) * (2u * 64u * 16u) + 64u * 16u);
                    bf16x8 gtr[DB], qtr[DB];
#pragma unroll
                    for (int dblk = 0; dblk < DB; ++dblk) {
                        gtr[dblk] = read_tr<D>(gt_base[0][dblk] + soff, gt_base[1][dblk] + soff, j);
                        qtr[dblk] = read_tr<D>(qt_base[0][dblk] + soff, qt_base[1][dblk] + soff, j);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
                    const bf16x8 df = __builtin_bit_cast(bf16x8, dk4);
#pragma unroll
                    for (int dblk = 0; dblk < DB; ++dblk) {
                        dva[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gtr[dblk], pf, dva[dblk], 0, 0, 0);
                        dka[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtr[dblk], df, dka[dblk], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            pset = set;
            set = set == 2 ? 0 : set + 1;
        }

        // ---- add the two query halves (consumers 2, 3 hand theirs to 0, 1), then write ----
        float* red = reinterpret_cast<float*>(&Xs[0][0][0]);   // [kh][2][DB][16][64] floats
        __syncthreads();
        if (qh == 1) {
#pragma unroll
            for (int dblk = 0; dblk < DB; ++dblk)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    red[(((kh * 2 + 0) * DB + dblk) * 16 + e) * 64 + lane] = dka[dblk][e];
                    red[(((kh * 2 + 1) * DB + dblk) * 16 + e) * 64 + lane] = dva[dblk][e];
                }
        }
        __syncthreads();
        const int jrow = 64 * m + 32 * kh + l32;
        if (qh == 0 && jrow < (a.N >> l)) {
            const int64_t rows15 = static_cast<int64_t>(a.N) + a.pooled_rows;
            const int64_t grow = (static_cast<int64_t>(b) * a.Hkv + hk) * rows15 +
                                 (l == 0 ? 0 : a.N + level_row_offset(a.N, l)) + jrow;
            float* gkp = a.gk + grow * D;
            float* gvp = a.gv + grow * D;
#pragma unroll
            for (int dblk = 0; dblk < DB; ++dblk)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    f32x4 wk, wv;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int e = 4 * gg + u;
                        wk[u] = (dka[dblk][e] + red[(((kh * 2 + 0) * DB + dblk) * 16 + e) * 64 + lane]) * a.scale;
                        wv[u] = dva[dblk][e] + red[(((kh * 2 + 1) * DB + dblk) * 16 + e) * 64 + lane];
                    }
                    *reinterpret_cast<f32x4*>(gkp + dblk * 32 + gg * 8 + hi * 4) = wk;
                    *reinterpret_cast<f32x4*>(gvp + dblk * 32 + gg * 8 + hi * 4) = wv;
                }
        }
    }
}

// ---------------------------------------------------------------------------------------
// dK[t] = sum_l 2^-l dKbar_l[t >> l] (and dV). One thread per (row, 4 values).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) k_bwd_pool(BwdArgs a) {
    constexpr int C4 = D / 4;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = static_cast<int64_t>(a.B) * a.Hkv * a.N * C4;
    if (idx >= total) return;
    const int c = static_cast<int>(idx % C4);
    const int64_t rowg = idx / C4;
    const int t = static_cast<int>(rowg % a.N);
    const int64_t bhk = rowg / a.N;
    const int hk = static_cast<int>(bhk % a.Hkv);
    const int b = static_cast<int>(bhk / a.Hkv);
    const int64_t rows15 = static_cast<int64_t>(a.N) + a.pooled_rows;
    const float* gk = a.gk + bhk * rows15 * D + c * 4;
    const float* gv = a.gv + bhk * rows15 * D + c * 4;
    f32x4 sk = *reinterpret_cast<const f32x4*>(gk + static_cast<int64_t>(t) * D);
    f32x4 sv = *reinterpret_cast<const f32x4*>(gv + static_cast<int64_t>(t) * D);
#pragma unroll
    for (int l = 1; l < 4; ++l) {
        const int64_t r = a.N + level_row_offset(a.N, l) + (t >> l);
        const float w = 1.0f / static_cast<float>(1 << l);
        const f32x4 xk = *reinterpret_cast<const f32x4*>(gk + r * D);
        const f32x4 xv = *reinterpret_cast<const f32x4*>(gv + r * D);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sk[u] = fmaf(xk[u], w, sk[u]);
            sv[u] = fmaf(xv[u], w, sv[u]);
        }
    }
    u32x2 wk, wv;
    wk[0] = pack_bf16x2(sk[0], sk[1]);
    wk[1] = pack_bf16x2(sk[2], sk[3]);
    wv[0] = pack_bf16x2(sv[0], sv[1]);
    wv[1] = pack_bf16x2(sv[2], sv[3]);
    *reinterpret_cast<u32x2*>(a.dk + b * a.ks0 + hk * a.ks1 + static_cast<int64_t>(t) * a.ks2 + c * 4) = wk;
    *reinterpret_cast<u32x2*>(a.dv + b * a.vs0 + hk * a.vs1 + static_cast<int64_t>(t) * a.vs2 + c * 4) = wv;
}

template <int D>
hipError_t launch_d(const Shape& s, const BwdArgs& a, hipStream_t st) {
    const int64_t rows = static_cast<int64_t>(s.B) * s.H * s.N;
    hipError_t e = launch_clear_i32(a.claim, 8, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_rowdot<D>, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int qrows = s.B * s.H * s.NQB;
    const int nper = (qrows + 7) / 8;
    const size_t dyn = static_cast<size_t>(s.NKB) * sizeof(int);
    if (s.BQ == 128)
        hipLaunchKernelGGL((k_bwd_dq<D, 128>), dim3(8 * nper), dim3(256), dyn, st, a, qrows);
    else
        hipLaunchKernelGGL((k_bwd_dq<D, 64>), dim3(8 * nper), dim3(128), dyn, st, a, qrows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // pooled tiles of 64 rows per level: level l has N >> l rows
    int tl[4];
    for (int l = 0; l < 4; ++l) tl[l] = ((s.N >> l) + 63) / 64;
    const int tiles_per_bh = tl[0] + tl[1] + tl[2] + tl[3];
    const int tiles = s.B * s.Hkv * tiles_per_bh;
    const size_t edyn = static_cast<size_t>(s.H / s.Hkv) * s.NQB * sizeof(int);
    hipLaunchKernelGGL(k_bwd_dkv<D>, dim3(tiles), dim3(512), edyn, st, a, tiles, tiles_per_bh,
                       tl[0], tl[0] + tl[1], tl[0] + tl[1] + tl[2]);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int64_t pool_threads = static_cast<int64_t>(s.B) * s.Hkv * s.N * (D / 4);
    hipLaunchKernelGGL(k_bwd_pool<D>, dim3(static_cast<unsigned>((pool_threads + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

size_t attn_bwd_scratch_bytes(const Shape& s) {
    const size_t rows = static_cast<size_t>(s.B) * s.H * s.N;
    const size_t grows = static_cast<size_t>(s.B) * s.Hkv * (static_cast<size_t>(s.N) + s.pooled_rows);
    return 2 * rows * sizeof(float) + 2 * grows * s.D * sizeof(float) + 8 * sizeof(int);
}

hipError_t launch_attn_bwd(const Shape& s, float scale, const void* q, const void* k,
                           const void* v, const void* kp, const void* vp, const int8_t* level_map,
                           const int32_t* row_ptr, const int32_t* col_idx, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* scratch, hipStream_t st) {
    if (s.dtype != PSA_BF16) return hipErrorNotSupported;
    BwdArgs a;
    a.q = static_cast<const bf16_bits*>(q);
    a.k = static_cast<const bf16_bits*>(k);
    a.v = static_cast<const bf16_bits*>(v);
    a.kp = static_cast<const bf16_bits*>(kp);
    a.vp = static_cast<const bf16_bits*>(vp);
    a.o = static_cast<const bf16_bits*>(o);
    a.dout = static_cast<const bf16_bits*>(dout);
    a.lse = lse;
    a.map = level_map;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    const size_t rows = static_cast<size_t>(s.B) * s.H * s.N;
    const size_t grows = static_cast<size_t>(s.B) * s.Hkv * (static_cast<size_t>(s.N) + s.pooled_rows);
    float* f = static_cast<float*>(scratch);
    a.lse2 = f;
    a.dd = f + rows;
    a.gk = f + 2 * rows;
    a.gv = a.gk + grows * s.D;
    a.claim = reinterpret_cast<int*>(a.gv + grows * s.D);
    a.share = order_share(s);
    a.dq = static_cast<bf16_bits*>(dq);
    a.dk = static_cast<bf16_bits*>(dk);
    a.dv = static_cast<bf16_bits*>(dv);
    a.B = s.B;
    a.H = s.H;
    a.Hkv = s.Hkv;
    a.N = s.N;
    a.Nv = s.Nv;
    a.NQB = s.NQB;
    a.NKB = s.NKB;
    a.BQ = s.BQ;
    a.causal = s.causal;
    a.qs0 = s.qs[0];
    a.qs1 = s.qs[1];
    a.qs2 = s.qs[2];
    a.ks0 = s.ks[0];
    a.ks1 = s.ks[1];
    a.ks2 = s.ks[2];
    a.vs0 = s.vs[0];
    a.vs1 = s.vs[1];
    a.vs2 = s.vs[2];
    a.os0 = s.os[0];
    a.os1 = s.os[1];
    a.os2 = s.os[2];
    a.pooled_rows = s.pooled_rows;
    a.scale = scale;
    a.c = scale * kLog2e;
    return s.D == 128 ? launch_d<128>(s, a, st) : launch_d<64>(s, a, st);
}

}  // namespace psa
