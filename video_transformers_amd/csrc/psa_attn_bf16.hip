// Adaptive Pyramid Attention forward, bf16 fast path for gfx950 (PSA summary article at
// rg.mbintangr.com, "Method": each KV block is fetched at its assigned pyramid level, a scaling
// factor keeps the probabilities consistent, and the kernel decouples the logical block size
// from the hardware tile size while staying flash-attention compatible).
//
// Work decomposition
//  * One workgroup per (batch, head, query block) row; 64 queries per wave (block_q / 64
//    waves). Workgroups are remapped so that each XCD walks a contiguous range of rows (one
//    head's K/V stays in that XCD's L2).
//  * The row's block list (its slice of the CSR) is copied to LDS once; the walk visits level
//    0 tiles first, then 1, 2, 3. A 64-row hardware tile at level l packs 2^l logical pooled
//    blocks of 64 / 2^l rows (decoupled block-tile); a level's partial last tile repeats its
//    first block and masks the absent rows. Skipped blocks are never loaded.
//  * K and V tiles travel HBM/L2 -> LDS with global_load_lds_dwordx4 (no VGPR staging), two
//    LDS buffers per tensor: the loads of tile t+1 are in flight while tile t is computed; one
//    barrier per tile.
//
// Math per wave (queries on the MFMA N axis, so each lane owns one query):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q (registers, whole
//    row). A-operand row r reads the tile key sigma(r) (bits 2 and 3 of r swapped); then the 16
//    accumulator values a lane holds for MFMA j of the P V product are 8 consecutive keys,
//    16j + 8*(lane/32) + e, so P needs no shuffling. K and V sit in LDS in natural key order,
//    so every 1 KB direct load covers consecutive keys of one logical block: its block offset
//    is wave-uniform (an SGPR base) and each lane's offset inside it is fixed per kernel.
//  * Online softmax in the exp2 domain, per lane (one query) plus one v_permlane32_swap; the
//    level term folds into the exp2 offset: p = exp2(s*c + (l - m)). The running max is
//    refreshed lazily: the accumulators are rescaled only when a tile's max exceeds the one in
//    use by more than 8 (p <= 2^8 otherwise, exact after the final 1/l).
//  * O^T = V^T P^T: A = V^T read from the row-major V tile with ds_read_b64_tr_b16 (each
//    16-lane group reads a 4x16 block and receives it transposed), B = P^T from registers.
//    Both query groups of a wave share every K and V operand read (64 FLOP per LDS byte).
//  * LDS tiles are XOR-swizzled per row at 16-byte granularity so the operand reads are free of
//    bank conflicts.
#include <stdlib.h>

#include "psa_attn_common.h"

namespace psa {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_cvoid;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr float kLazyRescale = 8.0f;  // log2-domain headroom before the accumulators rescale
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their no-wait maxima
// (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int kWaitVmcnt0 = 0x0F70;

template <int D>
struct Lay {
    static constexpr int CH = D / 8;                 // 16-byte chunks per row
    static constexpr int RPI = 1024 / (2 * D);       // rows per 1 KB direct-load instruction
    static constexpr int INSTR = 64 * D * 2 / 1024;  // instructions per 64-row tile
    // chunk swizzles (conflict-free operand reads, see the header)
    static __device__ __forceinline__ int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int fv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

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

// The K tile row that MFMA A-operand row r reads: bits 2 and 3 of r swapped.
__device__ __forceinline__ int sigma(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

struct Tile {
    int l;     // level (4 = walk finished)
    int base;  // offset of the tile's first block in the row's list
    int lend;  // end of the current level's list
    int cnt;   // blocks present in the tile (<= 2^l)
};

// G: query groups of 32 per wave (1 or 2). G = 2 shares every LDS operand read between two
// groups at one wave per SIMD; G = 1 halves the registers so two waves share each SIMD.
template <int D, int BQ, int G>
__global__ void __launch_bounds__(2 * BQ / G, 3 - G) k_attn_fwd_bf16(AttnArgs a, int total_rows) {
    constexpr int NW = BQ / (32 * G);
    using LY = Lay<D>;
    constexpr int IPW = LY::INSTR / NW;  // direct-load instructions per wave per tensor
    __shared__ __attribute__((aligned(1024))) bf16_bits Kt[2][64 * D];
    __shared__ __attribute__((aligned(1024))) bf16_bits Vt[2][64 * D];
    extern __shared__ int cols[];   // the row's block list (LDS reads do not wait on vmcnt)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps tile math scalar
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // XCD-aware row order: workgroup i runs on XCD i % 8; give each XCD a contiguous range.
    const int nper = (total_rows + 7) >> 3;
    const int row = (blockIdx.x & 7) * nper + (blockIdx.x >> 3);
    if (row >= total_rows) return;
    const int qb = row % a.NQB;
    const int bh = row / a.NQB;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);

    const bf16_bits* __restrict__ Q = static_cast<const bf16_bits*>(a.q);
    const bf16_bits* __restrict__ K = static_cast<const bf16_bits*>(a.k);
    const bf16_bits* __restrict__ V = static_cast<const bf16_bits*>(a.v);
    const bf16_bits* __restrict__ KP = static_cast<const bf16_bits*>(a.kp);
    const bf16_bits* __restrict__ VP = static_cast<const bf16_bits*>(a.vp);

    // ---- the row's block list -> LDS ----
    const int32_t* rp = a.row_ptr + static_cast<int64_t>(row) * 4;
    const int r0 = rp[0];
    const int lb1 = rp[1] - r0, lb2 = rp[2] - r0, lb3 = rp[3] - r0, lb4 = rp[4] - r0;
    // list offset of level l (l = 0..4), by selects: nothing is indexed dynamically
    auto lb = [&](int l) { return l <= 0 ? 0 : l == 1 ? lb1 : l == 2 ? lb2 : l == 3 ? lb3 : lb4; };
    for (int i = tid; i < lb4; i += BQ) cols[i] = a.col_idx[r0 + i];

    const int blk_first = qb * BQ;
    const int qbase = blk_first + wave * 32 * G;
    const int min_limit = a.causal ? min(blk_first, a.Nv - 1) : a.Nv - 1;
    const bool any_valid_query = blk_first < a.Nv;

    // ---- Q fragments: two groups of 32 queries ----
    bf16x8 qf[G][D / 16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const bf16_bits* qp = Q + b * a.qs0 + h * a.qs1 +
                              static_cast<int64_t>(qbase + g * 32 + l32) * a.qs2;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[g][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hi * 8);
    }
    int limit[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int qt = qbase + g * 32 + l32;
        limit[g] = a.causal ? min(qt, a.Nv - 1) : a.Nv - 1;
    }

    f32x16 oacc[G][D / 32];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[g][i][e] = 0.f;
    float m_use[G], l_run[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_use[g] = -INFINITY;
        l_run[g] = 0.f;
    }

    const int64_t kbase = b * a.ks0 + hk * a.ks1;
    const int64_t vbase = b * a.vs0 + hk * a.vs1;
    const int64_t pbase = (static_cast<int64_t>(b) * a.Hkv + hk) * a.pooled_rows * D;

    // walk state (uniform): first tile, then next() per tile; level changes are rare
    auto enter_level = [&](Tile& t) {   // t.l set, list position at the level's start
        while (t.l < 4 && lb(t.l + 1) == lb(t.l)) ++t.l;
        if (t.l < 4) {
            t.base = lb(t.l);
            t.lend = lb(t.l + 1);
        }
    };
    auto set_cnt = [&](Tile& t) {
        if (t.l < 4) t.cnt = min(t.lend - t.base, 1 << t.l);
    };
    auto next_tile = [&](const Tile& t) {
        Tile n = t;
        n.base += 1 << t.l;
        if (n.base >= n.lend) {
            ++n.l;
            enter_level(n);
        }
        set_cnt(n);
        return n;
    };

    // Issue the direct loads of tile t into buffer `buf`. Instruction m fills LDS rows
    // [m*RPI, (m+1)*RPI): consecutive keys of one logical block, so its block offset is
    // uniform and folds into the SGPR base; the lane offsets (row inside the instruction,
    // swizzled chunk) depend only on the row stride (level 0 or pooled) and, for K, on m.
    constexpr int KVAR = D == 128 ? 4 : 2;   // distinct K chunk swizzles across instructions
    static_assert(IPW % KVAR == 0, "instruction m and its index inside the wave agree mod KVAR");
    uint32_t lpk[2][KVAR], lpv[2];
    {
        const uint32_t st[2] = {static_cast<uint32_t>(a.ks2) * 2u, static_cast<uint32_t>(D) * 2u};
        const uint32_t sv[2] = {static_cast<uint32_t>(a.vs2) * 2u, static_cast<uint32_t>(D) * 2u};
        const int rr = lane / LY::CH;   // row inside the instruction
        const int p = lane % LY::CH;    // LDS chunk position
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < KVAR; ++q)
                lpk[i][q] = rr * st[i] + static_cast<uint32_t>((p ^ LY::fk(q * LY::RPI + rr)) << 4);
            lpv[i] = rr * sv[i] + static_cast<uint32_t>((p ^ LY::fv(rr)) << 4);
        }
    }
    // LDS byte offsets of the tile buffers (32-bit local-address-space pointers)
    const uint32_t lds_k0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Kt[0][0]));
    const uint32_t lds_v0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Vt[0][0]));
    constexpr uint32_t kBufBytes = 64 * D * 2;
    auto issue = [&](const Tile& t, int buf) {
        const int l = t.l;
        const int rs = 64 >> l;
        const int sh = 6 - l;
        const int pooled = l > 0 ? 1 : 0;
        const int64_t lvl_off = static_cast<int64_t>(a.N) - (static_cast<int64_t>(a.N) >> (l > 0 ? l - 1 : 0));
        const char* kb_base = reinterpret_cast<const char*>(l == 0 ? K + kbase : KP + pbase + lvl_off * D);
        const char* vb_base = reinterpret_cast<const char*>(l == 0 ? V + vbase : VP + pbase + lvl_off * D);
        // byte offsets inside one (batch, head) of one level fit 32 bits (checked on the host)
        const uint32_t kstride = static_cast<uint32_t>(l == 0 ? a.ks2 : D) * 2u;  // bytes per row
        const uint32_t vstride = static_cast<uint32_t>(l == 0 ? a.vs2 : D) * 2u;
        const uint32_t kblk = kstride * static_cast<uint32_t>(rs);  // bytes per logical block
        const uint32_t vblk = vstride * static_cast<uint32_t>(rs);
        const int clast = t.cnt - 1;
        const uint32_t lk = lds_k0 + (buf ? kBufBytes : 0u);
        const uint32_t lv = lds_v0 + (buf ? kBufBytes : 0u);
        uint32_t lk_lane[KVAR];
#pragma unroll
        for (int q = 0; q < KVAR; ++q) lk_lane[q] = pooled ? lpk[1][q] : lpk[0][q];
        const uint32_t lv_lane = pooled ? lpv[1] : lpv[0];
        // every block index first (LDS reads + readfirstlane), then the loads
        int kbs[IPW];
#pragma unroll
        for (int mi = 0; mi < IPW; ++mi) {
            const int key0 = (wave * IPW + mi) * LY::RPI;   // first tile key of the instruction
            const int s = min(key0 >> sh, clast);           // its logical block (absent -> last)
            kbs[mi] = __builtin_amdgcn_readfirstlane(cols[t.base + s]);
        }
#pragma unroll
        for (int mi = 0; mi < IPW; ++mi) {
            const int m = wave * IPW + mi;
            const uint32_t rin = static_cast<uint32_t>((m * LY::RPI) & (rs - 1));
            const uint32_t kb = static_cast<uint32_t>(kbs[mi]);
            dma16(kb_base + (kb * kblk + rin * kstride), lk_lane[mi % KVAR], lk + m * 1024);
            dma16(vb_base + (kb * vblk + rin * vstride), lv_lane, lv + m * 1024);
        }
    };

    __syncthreads();  // cols[] visible

    Tile cur{0, 0, 0, 0};
    enter_level(cur);
    set_cnt(cur);
    if (!any_valid_query) cur.l = 4;
    if (cur.l < 4) issue(cur, 0);

    int buf = 0;
    while (cur.l < 4) {
        const Tile nxt = next_tile(cur);
        const int lvl = cur.l;
        const int kb_max = cols[cur.base + cur.cnt - 1];
        const bool need_mask = (cur.cnt < (1 << lvl)) || ((kb_max + 1) * 64 - 1 > min_limit);

        // tile `cur` landed in `buf`: each wave waits for its own direct loads (vmcnt), then
        // the barrier publishes them and retires every wave's reads of the other buffer
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (nxt.l < 4) issue(nxt, buf ^ 1);

        const bf16_bits* Kb = Kt[buf];
        const bf16_bits* Vb = Vt[buf];

        // ---- S^T = K Q^T for both query groups ----
        f32x16 sacc[G][2];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[g][kh][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const int r = sigma(kh * 32 + l32);
                const int pos = (2 * kk + hi) ^ LY::fk(r);
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kb[r * D + pos * 8]);
#pragma unroll
                for (int g = 0; g < G; ++g)
                    sacc[g][kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[g][kk], sacc[g][kh], 0, 0, 0);
            }
        }

        // ---- mask (partial tiles, padding, causal diagonal) ----
        // A lane's 32 accumulator slots per query group are 8 runs of 4 consecutive tile keys
        // tk0 + i; a run lies inside one logical block (>= 8 rows), so one list read per run.
        if (need_mask) {
            const int rs = 64 >> lvl;
            const int sh = 6 - lvl;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    const int tk0 = kh * 32 + 16 * (gi >> 1) + 8 * hi + 4 * (gi & 1);
                    const int s = tk0 >> sh;
                    const int kb = cols[cur.base + (s < cur.cnt ? s : 0)];
                    const int last0 = s < cur.cnt ? ((kb * rs + (tk0 & (rs - 1)) + 1) << lvl) - 1
                                                  : 0x7fffffff - (3 << 3);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int last = last0 + (i << lvl);
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            if (last > limit[g]) sacc[g][kh][gi * 4 + i] = -INFINITY;
                    }
                }
        }

        // ---- online softmax (exp2 domain, lazy rescale) ----
        const float flvl = static_cast<float>(lvl);
        float mt[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float x = sacc[g][0][0];
#pragma unroll
            for (int e = 1; e < 31; e += 2)
                x = fmaxf(x, fmaxf(sacc[g][e >> 4][e & 15], sacc[g][(e + 1) >> 4][(e + 1) & 15]));
            x = fmaxf(x, sacc[g][1][15]);
            mt[g] = fmaf(pair32_max(x), a.c, flvl);   // tile max of z in log2 units
        }
        bool grow = false;
#pragma unroll
        for (int g = 0; g < G; ++g) grow |= mt[g] > m_use[g] + kLazyRescale;
        if (__builtin_expect(__ballot(grow) != 0ull, 0)) {
            // rare (lazy max): the accumulators leave the AGPRs only here
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float m_new = fmaxf(m_use[g], mt[g]);
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_use[g] - m_new);
                m_use[g] = m_new;
                l_run[g] *= alpha;
#pragma unroll
                for (int i = 0; i < D / 32; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[g][i][e] *= alpha;
            }
        }
        float off[G], psum[G];
#pragma unroll
        for (int g = 0; g < G; ++g) psum[g] = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) off[g] = flvl - (m_use[g] == -INFINITY ? 0.f : m_use[g]);

        // ---- O^T += V^T P^T; P for 16 keys is formed just before its MFMAs ----
        const int grp = lane >> 4;   // 16-lane group: d half (grp & 1), key half (grp >> 1)
        const int jj = lane & 15;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 pf[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                union {
                    bf16x8 v;
                    uint32_t u[4];
                } pk;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float p0 = fast_exp2(fmaf(sacc[g][j >> 1][(j & 1) * 8 + 2 * t], a.c, off[g]));
                    const float p1 = fast_exp2(fmaf(sacc[g][j >> 1][(j & 1) * 8 + 2 * t + 1], a.c, off[g]));
                    pk.u[t] = pack_bf16x2(p0, p1);
                    psum[g] = add_bf16x2(pk.u[t], psum[g]);
                }
                pf[g] = pk.v;
            }
#pragma unroll
            for (int dblk = 0; dblk < D / 32; ++dblk) {
                const int d = dblk * 32 + 16 * (grp & 1) + 4 * (jj & 3);
                const int c = d >> 3;
                const int half = (d & 7);  // 0 or 4 elements
                const int rA = 16 * j + 8 * (grp >> 1) + (jj >> 2);
                const int rB = rA + 4;
                const bf16_bits* pA = &Vb[rA * D + ((c ^ LY::fv(rA)) << 3) + half];
                const bf16_bits* pB = &Vb[rB * D + ((c ^ LY::fv(rB)) << 3) + half];
                union {
                    bf16x8 v;
                    v4i16 h[2];
                } va;
                va.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)pA);
                va.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)pB);
#pragma unroll
                for (int g = 0; g < G; ++g)
                    oacc[g][dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va.v, pf[g], oacc[g][dblk], 0, 0, 0);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) l_run[g] += psum[g];
        cur = nxt;
        buf ^= 1;
    }

    // ---- epilogue ----
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int qt = qbase + g * 32 + l32;
        const float l_tot = pair32_sum(l_run[g]);
        const bool valid_q = qt < a.Nv && l_tot > 0.f;
        const float inv = valid_q ? 1.f / l_tot : 0.f;
        bf16_bits* O = static_cast<bf16_bits*>(a.o) + b * a.os0 + h * a.os1 +
                       static_cast<int64_t>(qt) * a.os2;
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[g][dblk][4 * gg] * inv, oacc[g][dblk][4 * gg + 1] * inv);
                w[1] = pack_bf16x2(oacc[g][dblk][4 * gg + 2] * inv, oacc[g][dblk][4 * gg + 3] * inv);
                *reinterpret_cast<u32x2*>(O + dblk * 32 + gg * 8 + hi * 4) = w;
            }
        if (a.lse != nullptr && hi == 0) {
            const float lse = valid_q ? (m_use[g] + log2f(l_tot)) * kLn2 : -INFINITY;
            a.lse[(static_cast<int64_t>(b) * a.H + h) * a.N + qt] = lse;
        }
    }
}

template <int D, int BQ, int G>
hipError_t launch_one(const Shape& s, const AttnArgs& a, hipStream_t st) {
    const int rows = s.B * s.H * s.NQB;
    const int nper = (rows + 7) / 8;
    const size_t dyn = static_cast<size_t>(s.NKB) * sizeof(int);
    hipLaunchKernelGGL((k_attn_fwd_bf16<D, BQ, G>), dim3(8 * nper), dim3(2 * BQ / G), dyn, st, a, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Shape& s, const AttnArgs& a, hipStream_t st) {
    // query groups per wave: PSA_ATTN_GROUPS=1|2 overrides the default (tuning runs)
    static const int groups = [] {
        const char* e = getenv("PSA_ATTN_GROUPS");
        return (e != nullptr && e[0] == '2') ? 2 : 1;
    }();
    if (groups == 1) {
        if (s.D == 128 && s.BQ == 128) return launch_one<128, 128, 1>(s, a, st);
        if (s.D == 128 && s.BQ == 64) return launch_one<128, 64, 1>(s, a, st);
        if (s.D == 64 && s.BQ == 128) return launch_one<64, 128, 1>(s, a, st);
        if (s.D == 64 && s.BQ == 64) return launch_one<64, 64, 1>(s, a, st);
    } else {
        if (s.D == 128 && s.BQ == 128) return launch_one<128, 128, 2>(s, a, st);
        if (s.D == 128 && s.BQ == 64) return launch_one<128, 64, 2>(s, a, st);
        if (s.D == 64 && s.BQ == 128) return launch_one<64, 128, 2>(s, a, st);
        if (s.D == 64 && s.BQ == 64) return launch_one<64, 64, 2>(s, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace psa
