// Adaptive Pyramid Attention forward, bf16 fast path for gfx950 (PSA summary article at
// rg.mbintangr.com, "Method": each KV block is fetched at its assigned pyramid level, a scaling
// factor keeps the probabilities consistent, and the kernel decouples the logical block size
// from the hardware tile size while staying flash-attention compatible).
//
// Work decomposition
//  * One workgroup per (batch, head, query block) row, 32 queries per wave (block_q / 32
//    waves), two workgroups per CU (two waves per SIMD). Workgroups are remapped so that each
//    XCD walks a contiguous range of rows.
//  * The row's block list (its slice of the CSR) is copied to LDS once; the walk visits level
//    0 tiles first, then 1, 2, 3. A 64-row hardware tile at level l packs 2^l logical pooled
//    blocks of 64 / 2^l rows (decoupled block-tile); a level's partial last tile repeats its
//    first block and masks the absent rows. Skipped blocks are never loaded.
//  * K and V tiles travel HBM/L2 -> LDS with global_load_lds_dwordx4 (no VGPR staging). K:
//    two 64-row buffers. V: a ring of four 32-row slots (half tile u lives in slot u mod 4),
//    because the O product of a half runs one half behind its S product. One barrier per
//    tile; the next tile's direct loads are issued from inside the first step's MFMA stream.
//    The tile loop has one body per buffer parity, so LDS operand addresses are loop
//    invariants plus instruction immediates.
//
// Software pipeline (per wave), in steps of 32 keys (half tiles u = 2t + h):
//    S(u) = K(u) Q^T                       8 MFMAs (d = 128), K reads three MFMAs ahead
//    P(u-1) = exp2(S(u-1) - m) -> bf16      VALU, one slice after each S MFMA
//    O += V(u-1)^T P(u-1)                  8 MFMAs, interleaved with the second half of S(u)
//    row max of S(u)                       VALU, beside the last O MFMAs
//    (tiles that need it) mask, max again; lazy rescale check
//  A scheduling barrier after every MFMA keeps this issue order.
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
//  * LDS tiles are XOR-swizzled per row at 16-byte granularity so the operand reads are free of
//    bank conflicts.
#include <stdlib.h>

#include <cmath>

#include <type_traits>

#include "psa_assign.h"
#include "psa_attn_common.h"
#include "psa_bf16_tile.h"

namespace psa {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2-domain headroom before the accumulators rescale

// Block-mean scoring fused into the prologue (MK): the query block means, KV block means, the
// assignment's parameters and where the map and masses go (either may be null).
struct MkArgs {
    const float* qbar;   // [B*H][NQB][D]
    const float* kbar;   // [B*Hkv][NKB][D]
    const double* ksum;  // [B*Hkv][NKB][D] float64 key sums (the certification)
    float* mass_out;     // [B*H*NQB][NKB] or null
    int8_t* map_out;     // [B*H*NQB][NKB] or null
    AssignArgs asg;      // RQ = 1, sampling counting, sim set when the cosine check is on
    double c;            // (1 / sqrt(d)) * log2(e), the scorer's logit scale
    double scale;        // 1 / sqrt(d), the certification's (natural-log) logit scale
    int share;           // XCD ranges per chunk of the row order (1, 2, 4, 8)
};

struct Tile {
    int l;     // level (4 = walk finished)
    int base;  // offset of the tile's first block in the row's list
    int lend;  // end of the current level's list
    int cnt;   // blocks present in the tile (<= 2^l)
};

// CONTIG: K and V rows are D elements apart (level 0 and the pooled levels share the lane
// offsets of the direct loads).
// PACK: a tile packs 2^l logical blocks of level l (the decoupled block-tile). Without it
// every tile holds one logical block and its other rows are masked: the naive layout, kept
// as the ablation baseline the packing is measured against.
// FP8 >= 1: Q and K (level 0 and pooled) are e4m3 bytes with one scale per (batch, head); S
// comes from v_mfma_f32_32x32x64_f8f6f4 (A: lane l holds row l % 32, bytes 32 * (l / 32) + 0..31
// of the 64-wide k-step; B likewise per column; C as in the bf16 product). A K row of D bytes
// has the byte layout of a bf16 row of D / 2 elements and travels with that layout's direct
// loads and swizzle.
// FP8 == 2: V is e4m3 too (one scale per (batch, KV head)) and P is quantized to e4m3 for an
// fp8 P V product over whole 64-key tiles (see the fp8 P V pipeline below). Otherwise P, V and
// O stay bf16.
// MK: the row's block list comes from block-mean scoring and the threshold assignment run in
// the prologue (block_q 128: the assignment's 256 threads), instead of the CSR index.
template <int D, int BQ, bool CONTIG, bool PACK, int FP8, bool MK = false>
__global__ void __launch_bounds__(2 * BQ, 2) k_attn_fwd_bf16(AttnArgs a, int total_rows, MkArgs mk) {
    constexpr bool F8 = FP8 >= 1;
    constexpr bool PV8 = FP8 == 2;
    constexpr int NW = BQ / 32;
    using LY = Lay<D>;                   // bf16 V tiles (and K tiles in bf16)
    using KL = Lay<F8 ? D / 2 : D>;      // K tiles
    using VL = Lay<PV8 ? D / 2 : D>;     // V tiles
    constexpr int EK = F8 ? 1 : 2;       // bytes per K element
    constexpr int EV = PV8 ? 1 : 2;      // bytes per V element
    constexpr int RBK = D * EK;          // bytes per K row
    constexpr int RBV = D * EV;          // bytes per V row
    constexpr int KK = D / 16;           // pipeline slots per step (k-steps of the bf16 S product)
    constexpr int KS = F8 ? D / 64 : KK; // k-steps of the S product
    constexpr int KSL = KK / KS;         // slots per k-step
    constexpr int DB = D / 32;           // 32-wide d blocks of the O product
    using KT = std::conditional_t<F8, uint8_t, bf16_bits>;
    using VT = std::conditional_t<PV8, uint8_t, bf16_bits>;
    using KOp = std::conditional_t<F8, i32x8, bf16x8>;   // one lane's S operand of a k-step
    static_assert(!F8 || D == 128, "fp8 K rows of 128 bytes");
    __shared__ __attribute__((aligned(1024))) uint8_t Kt[2][64 * RBK];
    // bf16: a ring of four 32-row V slots; fp8 P V: three 64-row V tiles
    __shared__ __attribute__((aligned(1024))) uint8_t Vt[PV8 ? 3 * 64 * RBV : 2 * 64 * RBV];
    extern __shared__ int cols[];   // the row's block list (LDS reads do not wait on vmcnt)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps tile math scalar
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // XCD-aware row order: workgroup i runs on XCD i % 8; give each XCD a contiguous range of
    // rows, taken in the index's dispatch order (largest first) when it has one.
    const int nper = (total_rows + 7) >> 3;
    int row;
    if constexpr (MK) {
        // No block index (the map is made in the prologue), so no sort by tile count: rows in
        // natural order (a KV head's query heads are consecutive), laid over the XCDs in chunks
        // of f ranges as the index's dispatch order is: range x of its chunk takes every f-th
        // row from the chunk's start + (x mod f), so the f XCDs of a chunk work through one KV
        // head together. Each XCD's slots cover at most nper rows; every row is taken once.
        const int x = blockIdx.x & 7;
        const int f = mk.share;
        const int x0 = x - x % f;
        const int pos = x0 * nper + (x - x0) + static_cast<int>(blockIdx.x >> 3) * f;
        if (pos >= min((x0 + f) * nper, total_rows)) return;
        row = pos;
    } else {
        const int slot = (blockIdx.x & 7) * nper + (blockIdx.x >> 3);
        if (slot >= total_rows) return;
        row = a.row_order != nullptr ? a.row_order[slot] : slot;
    }
    const int qb = row % a.NQB;
    const int bh = row / a.NQB;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);

    const KT* __restrict__ Q = static_cast<const KT*>(a.q);
    const KT* __restrict__ K = static_cast<const KT*>(a.k);
    const VT* __restrict__ V = static_cast<const VT*>(a.v);
    const KT* __restrict__ KP = static_cast<const KT*>(a.kp);
    const VT* __restrict__ VP = static_cast<const VT*>(a.vp);

    // ---- the row's block list -> LDS ----
    int lb1, lb2, lb3, lb4;
    if constexpr (MK) {
        static_assert(!MK || (BQ == 128 && !F8), "fused block-mean scoring: bf16, block_q 128");
        // Scratch aliased on the tile buffers, which the first tile's loads only fill after the
        // list is built: the query block mean, the log-masses, masses and levels in Kt, the
        // sort keys in Vt.
        const int NKB = mk.asg.NKB;
        float* qs = reinterpret_cast<float*>(&Kt[0][0]);
        float* Ls = qs + D;
        float* Ms = Ls + NKB;
        int8_t* lvl = reinterpret_cast<int8_t*>(Ms + NKB);
        uint64_t* keys = reinterpret_cast<uint64_t*>(&Vt[0]);
        __shared__ int lcnt[4];
        __shared__ int wtot[2][4][4];   // [chunk parity][level][wave]
        for (int i = tid; i < D; i += 256) qs[i] = mk.qbar[static_cast<int64_t>(row) * D + i];
        if (tid < 4) lcnt[tid] = 0;
        __syncthreads();
        // log2-masses exactly as the block-mean scorer writes them (float64 dot in d order)
        const float* kh_bar = mk.kbar + static_cast<int64_t>(b * a.Hkv + hk) * NKB * D;
        const int qlo = qb * BQ;
        const int lastk = a.causal ? min((qlo + BQ - 1) / 64, NKB - 1) : NKB - 1;
        for (int kb = tid; kb < NKB; kb += 256) {
            const int nv = min(max(a.Nv - kb * 64, 0), 64);
            const float* kr = kh_bar + static_cast<int64_t>(kb) * D;
            double dot = 0.0;
            for (int e = 0; e < D; ++e) dot += static_cast<double>(kr[e]) * static_cast<double>(qs[e]);
            Ls[kb] = (qlo < a.Nv && nv > 0 && kb <= lastk)
                         ? static_cast<float>(dot * mk.c + log2(static_cast<double>(nv)))
                         : -INFINITY;
        }
        __shared__ int cflag;
        if (tid == 0) cflag = 0;
        __syncthreads();
        assign_masses(mk.asg, qb, Ls, Ms, mk.mass_out != nullptr ? mk.mass_out + static_cast<int64_t>(row) * NKB : nullptr, tid);
        assign_levels(mk.asg, qb, b, hk, Ms, keys, lvl, tid, &cflag);
        if (cflag) {
            // Certification, as psa_mask does it: a decision within the margins of the float32
            // assignment is redone from float64 block-mean scores (same functions, same order as
            // psa_mask's rescoring). Scratch: the float64 log-masses and then the sort keys in
            // place of the float32 keys; q_bar and the sort's kb column after the levels when
            // they fit in the K buffers, else over the dead float32 log-masses and masses.
            char* kt = reinterpret_cast<char*>(&Kt[0][0]);
            const int used = (4 * D + 9 * NKB + 7) & ~7;
            const int need = 8 * D + 2 * mk.asg.P;
            char* scr = used + need <= static_cast<int>(sizeof(Kt)) ? kt + used : reinterpret_cast<char*>(Ls);
            double* qbar64 = reinterpret_cast<double*>(scr);
            uint16_t* idx = reinterpret_cast<uint16_t*>(scr + 8 * D);
            double* Ld = reinterpret_cast<double*>(keys);
            cert_qbar_f64(Q + b * a.qs0 + h * a.qs1, a.qs2, qb, BQ, a.Nv, D, qbar64, tid);
            __syncthreads();
            const double* ks = mk.ksum + static_cast<int64_t>(b * a.Hkv + hk) * NKB * D;
            for (int kb = tid; kb < NKB; kb += 256)
                Ld[kb] = cert_meankey_logmass(ks, qbar64, D, kb, a.Nv, qlo < a.Nv && kb <= lastk, mk.scale);
            __syncthreads();
            __shared__ double clse[32], cwm[4][32], cws[4][32];
            cert_lse(Ld, 1, NKB, clse, cwm, cws, tid);
            const int den = cert_den(mk.asg, qb);
            for (int kb = tid; kb < NKB; kb += 256) {
                const double mass = cert_mass(Ld, clse, 1, NKB, kb, den);
                if (mk.mass_out != nullptr) mk.mass_out[static_cast<int64_t>(row) * NKB + kb] = static_cast<float>(mass);
                if (kb <= lastk) {
                    keys[kb] = ~double_order(mass);
                    idx[kb] = static_cast<uint16_t>(kb);
                }
            }
            __syncthreads();
            assign_levels_f64(mk.asg, qb, b, hk, keys, idx, lvl, tid);
        }
        if (mk.map_out != nullptr)
            for (int kb = tid; kb < NKB; kb += 256) mk.map_out[static_cast<int64_t>(row) * NKB + kb] = lvl[kb];
        // the list: level 0, 1, 2, 3, ascending kb within a level (an ordered compaction)
        {
            int cnt[4] = {0, 0, 0, 0};
            for (int kb = tid; kb < NKB; kb += 256) {
                const int L = lvl[kb];
                if (L >= 0) ++cnt[L];
            }
#pragma unroll
            for (int l = 0; l < 4; ++l)
                if (cnt[l]) atomicAdd(&lcnt[l], cnt[l]);
        }
        __syncthreads();
        lb1 = __builtin_amdgcn_readfirstlane(lcnt[0]);
        lb2 = lb1 + __builtin_amdgcn_readfirstlane(lcnt[1]);
        lb3 = lb2 + __builtin_amdgcn_readfirstlane(lcnt[2]);
        lb4 = lb3 + __builtin_amdgcn_readfirstlane(lcnt[3]);
        {
            int run0 = 0, run1 = 0, run2 = 0, run3 = 0;   // entries placed so far per level
            int par = 0;
            const uint64_t below = (1ull << lane) - 1ull;
            for (int c0 = 0; c0 < NKB; c0 += 256) {
                const int kb = c0 + tid;
                const int L = kb < NKB ? lvl[kb] : -1;
                uint64_t bal[4];
#pragma unroll
                for (int l = 0; l < 4; ++l) bal[l] = __ballot(L == l);
                if (lane == 0)
#pragma unroll
                    for (int l = 0; l < 4; ++l) wtot[par][l][wave] = __popcll(bal[l]);
                __syncthreads();
                int pre[4], tot[4];
#pragma unroll
                for (int l = 0; l < 4; ++l) {
                    pre[l] = 0;
                    tot[l] = 0;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const int t = wtot[par][l][w];
                        tot[l] += t;
                        if (w < wave) pre[l] += t;
                    }
                }
                if (L >= 0) {
                    const int base = L == 0 ? run0 : L == 1 ? lb1 + run1 : L == 2 ? lb2 + run2 : lb3 + run3;
                    const int pl = L == 0 ? pre[0] : L == 1 ? pre[1] : L == 2 ? pre[2] : pre[3];
                    const uint64_t bl = L == 0 ? bal[0] : L == 1 ? bal[1] : L == 2 ? bal[2] : bal[3];
                    cols[base + pl + __popcll(bl & below)] = kb;
                }
                run0 += tot[0];
                run1 += tot[1];
                run2 += tot[2];
                run3 += tot[3];
                par ^= 1;
            }
        }
    } else {
        const int32_t* rp = a.row_ptr + static_cast<int64_t>(row) * 4;
        const int r0 = rp[0];
        lb1 = rp[1] - r0;
        lb2 = rp[2] - r0;
        lb3 = rp[3] - r0;
        lb4 = rp[4] - r0;
        for (int i = tid; i < lb4; i += BQ * 2) cols[i] = a.col_idx[r0 + i];
    }
    // list offset of level l (l = 0..4), by selects: nothing is indexed dynamically
    auto lb = [&](int l) { return l <= 0 ? 0 : l == 1 ? lb1 : l == 2 ? lb2 : l == 3 ? lb3 : lb4; };

    const int blk_first = qb * BQ;
    const int qt = blk_first + wave * 32 + l32;   // this lane's query
    const int min_limit = a.causal ? min(blk_first, a.Nv - 1) : a.Nv - 1;
    const bool any_valid_query = blk_first < a.Nv;
    const int limit = a.causal ? min(qt, a.Nv - 1) : a.Nv - 1;

    // ---- Q fragments (B operand of S^T = K Q^T): 16 bytes (bf16) or 32 bytes (fp8) per k-step ----
    KOp qf[KS];
    {
        const KT* qp = Q + b * a.qs0 + h * a.qs1 + static_cast<int64_t>(qt) * a.qs2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *reinterpret_cast<const KOp*>(qp + (ks * 2 + hi) * (sizeof(KOp) / sizeof(KT)));
    }
    // logit scale in log2 units (fp8: times the two operand scales)
    const float cs = F8 ? a.c * a.q_scale[b * a.H + h] * a.k_scale[b * a.Hkv + hk] : a.c;

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
    float m_use = -INFINITY, l_run = 0.f;
    // fp8 P V only: the row sums of the quantized P, from a ones-row MFMA (every register of a
    // lane holds its query's sum), and the fp32 P of a tile's first half, kept until the tile's
    // P V product
    f32x16 lacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) lacc[e] = 0.f;
    float pAf[16];

    const int64_t kbase = b * a.ks0 + hk * a.ks1;
    const int64_t vbase = b * a.vs0 + hk * a.vs1;
    const int64_t pbase = (static_cast<int64_t>(b) * a.Hkv + hk) * a.pooled_rows * D;  // elements

    // walk state (uniform): first tile, then next_tile() per tile; level changes are rare
    auto enter_level = [&](Tile& t) {   // t.l set, list position at the level's start
        while (t.l < 4 && lb(t.l + 1) == lb(t.l)) ++t.l;
        if (t.l < 4) {
            t.base = lb(t.l);
            t.lend = lb(t.l + 1);
        }
    };
    auto set_cnt = [&](Tile& t) {
        if (t.l < 4) t.cnt = min(t.lend - t.base, PACK ? 1 << t.l : 1);
    };
    auto next_tile = [&](const Tile& t) {
        Tile n = t;
        n.base += PACK ? 1 << t.l : 1;
        if (n.base >= n.lend) {
            ++n.l;
            enter_level(n);
        }
        set_cnt(n);
        return n;
    };

    // V tile chunk swizzle. bf16: fv, for the 16-bit transposed reads. fp8: 2 ((r >> 1) & 3):
    // a 16-lane 8-bit transposed read covers 8 aligned rows x 16 bytes (two chunk columns), and
    // with this swizzle the 32 lanes of a read pass (8 rows x 2 chunks x 2 halves) land on 64
    // distinct banks. Within a direct-load instruction (8 rows) it depends on the row only
    // through r mod 8.
    auto vswz = [](int r) { return PV8 ? 2 * ((r >> 1) & 3) : LY::fv(r); };
    // Direct loads of one tensor of tile t. Instruction m of the tile covers RPI consecutive
    // tile rows; a wave issues ipw consecutive instructions. Logical blocks hold 8 rows or
    // more, so every run of 8 rows (an aligned group of 8 / RPI instructions) lies in one
    // block: group j of the wave reads from SGPR base b[j], which points at the group's
    // first row minus the rows of the instructions before it. Instruction mi's lane offsets
    // (row inside the instruction, swizzled 16-byte chunk, plus mi instructions of rows) are
    // then loop invariants, and no per-instruction address work remains but the LDS
    // destination in M0. K and V differ in rows per instruction (KL, LY) when K is fp8.
    constexpr int KVAR = KL::CH == 16 ? 4 : 2;   // distinct K chunk swizzles across instructions
    constexpr int VROWS = PV8 ? 64 : 32;          // rows per V load: a whole tile (fp8) or a half
    constexpr int IPWK = 64 / KL::RPI / NW;       // K instructions per wave per tile
    constexpr int IPWV = VROWS / VL::RPI / NW;    // V instructions per wave per V load
    constexpr int IPGK = 8 / KL::RPI;             // instructions per 8-row group (K)
    constexpr int IPGV = 8 / VL::RPI;             // instructions per 8-row group (V)
    static_assert(IPWK % KVAR == 0, "instruction m and its index inside the wave agree mod KVAR");
    static_assert(IPGK >= 1 && IPWK % IPGK == 0 && IPWV % IPGV == 0 && IPWK / IPGK <= 4, "direct-load groups");
    constexpr int NSTR = CONTIG ? 1 : 2;          // lane offset sets: pooled stride (and level 0)
    uint32_t lok[NSTR][IPWK], lov[NSTR][IPWV];
    {
        const int rk = lane / KL::CH;   // row inside the instruction
        const int pk = lane % KL::CH;   // LDS chunk position
        const int rv = lane / VL::CH;
        const int pv = lane % VL::CH;
#pragma unroll
        for (int i = 0; i < NSTR; ++i) {
            const uint32_t sk = (i == 1 ? static_cast<uint32_t>(a.ks2) : static_cast<uint32_t>(D)) * EK;
            const uint32_t sv = (i == 1 ? static_cast<uint32_t>(a.vs2) : static_cast<uint32_t>(D)) * EV;
#pragma unroll
            for (int mi = 0; mi < IPWK; ++mi)
                lok[i][mi] = (rk + mi * KL::RPI) * sk + static_cast<uint32_t>((pk ^ KL::fk((mi % KVAR) * KL::RPI + rk)) << 4);
#pragma unroll
            for (int mi = 0; mi < IPWV; ++mi)
                lov[i][mi] = (rv + mi * VL::RPI) * sv + static_cast<uint32_t>((pv ^ vswz(rv)) << 4);
        }
    }
    // LDS byte offsets of the tile buffers (32-bit local-address-space pointers)
    const uint32_t lds_k0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Kt[0][0]));
    const uint32_t lds_v0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&Vt[0]));
    constexpr uint32_t kBufBytes = 64 * RBK;   // one K buffer
    struct Dma {
        uint64_t b[4];   // SGPR bases of the wave's 8-row groups
        uint32_t lds;    // LDS byte address of the wave's first instruction
    };
    // the list entries (logical blocks) of the wave's groups: LDS reads, issued one pipeline
    // slot before their values are used
    struct Pend {
        int c[4];
    };
    // A wave's share of NR tile rows from R0 on: NR / NW rows, in groups of 8.
    auto pend = [&](const Tile& t, auto R0, auto NR) {
        constexpr int rpw = decltype(NR)::value / NW;
        const int sh = 6 - t.l;
        const int clast = t.cnt - 1;
        const int key0 = decltype(R0)::value + wave * rpw;
        // an absent block of a level's partial last tile is replaced by the last one (masked)
        Pend pd;
#pragma unroll
        for (int j = 0; j < rpw / 8; ++j) pd.c[j] = cols[t.base + min((key0 + 8 * j) >> sh, clast)];
        return pd;
    };
    auto resolve = [&](const Tile& t, const Pend& pd, uint32_t lds_dst, bool is_v, auto R0, auto NR) {
        constexpr int rpw = decltype(NR)::value / NW;
        const uint32_t rb = static_cast<uint32_t>(is_v ? RBV : RBK);   // bytes per row
        const int l = t.l;
        const int sh = 6 - l;
        const int rsm1 = (1 << sh) - 1;   // rows per logical block - 1
        // pooled level l starts at row N - N / 2^(l-1) (0 for l = 1 and, by the same formula
        // with shift 0, for l = 0); the level-0 / pooled tensor choice is a mask, not a branch
        const uint32_t lvl_off = static_cast<uint32_t>(a.N - (a.N >> max(l - 1, 0)));
        const uint64_t l0 = is_v ? reinterpret_cast<uint64_t>(V + vbase) : reinterpret_cast<uint64_t>(K + kbase);
        const uint64_t pl = is_v ? reinterpret_cast<uint64_t>(VP + pbase) : reinterpret_cast<uint64_t>(KP + pbase);
        const uint64_t m0 = 0ull - static_cast<uint64_t>(l == 0);
        const uint64_t base = ((l0 & m0) | (pl & ~m0)) + static_cast<uint64_t>(lvl_off * rb);
        // byte offsets inside one (batch, head) of one level fit 32 bits (checked on the host)
        const uint32_t stride = static_cast<uint32_t>(l == 0 && !CONTIG ? (is_v ? a.vs2 : a.ks2) : D) * (is_v ? EV : EK);
        const int key0 = decltype(R0)::value + wave * rpw;
        Dma d;
#pragma unroll
        for (int j = 0; j < rpw / 8; ++j) {
            const uint32_t r = (static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(pd.c[j])) << sh) +
                               static_cast<uint32_t>((key0 + 8 * j) & rsm1);
            d.b[j] = base + static_cast<uint64_t>(r * stride) - static_cast<uint64_t>(8 * j * stride);
        }
        d.lds = lds_dst + static_cast<uint32_t>(wave * rpw) * rb;
        return d;
    };
    // instruction mi of the wave (level-0 / pooled lane offsets by `pooled`)
    auto fire = [&](const Dma& d, bool is_v, int pooled, int mi) {
        const int s = CONTIG ? 0 : (pooled ? 0 : 1);
        const uint32_t lo = is_v ? lov[s][mi] : lok[s][mi];
        dma16(reinterpret_cast<const void*>(d.b[mi / (is_v ? IPGV : IPGK)]), lo, d.lds + static_cast<uint32_t>(mi) * 1024u);
    };
    auto issue = [&](const Tile& t, uint32_t lds_dst, auto ISV, auto R0, auto NR) {
        constexpr bool is_v = decltype(ISV)::value != 0;
        constexpr int ipw = decltype(NR)::value / (is_v ? VL::RPI : KL::RPI) / NW;
        const Dma d = resolve(t, pend(t, R0, NR), lds_dst, is_v, R0, NR);
#pragma unroll
        for (int mi = 0; mi < ipw; ++mi) fire(d, is_v, t.l > 0, mi);
    };
    constexpr uint32_t kSlotBytes = 32 * D * 2;   // one 32-row V slot
    auto issue_k = [&](const Tile& t, int buf) {
        issue(t, lds_k0 + (buf ? kBufBytes : 0u), IC<0>{}, IC<0>{}, IC<64>{});
    };
    auto issue_vh = [&](const Tile& t, int half, int slot) {
        if (half == 0)
            issue(t, lds_v0 + slot * kSlotBytes, IC<1>{}, IC<0>{}, IC<32>{});
        else
            issue(t, lds_v0 + slot * kSlotBytes, IC<1>{}, IC<32>{}, IC<32>{});
    };

    // Loop-invariant per-lane LDS byte addresses of the operand reads (buffer 0; buffer 1 and
    // the kh / j steps are instruction immediates).
    // K, bf16: chunk (2kk + hi) ^ fk(r) -> byte address ka_base ^ (32 kk): the row start and
    // the hi / low-swizzle chunk bit occupy other bits than 32 kk (rows are D*2 >= 128 bytes).
    // K, fp8: chunks (4ks + 2hi + e) ^ fk(r), e = 0, 1 -> ka_base[e] ^ (64 ks), for the same
    // reason (rows of 128 bytes; 2hi + e and fk(r) < 8 stay below bit 6).
    uint32_t ka_base[F8 ? 2 : 1];
    {
        const int r = sigma(l32);          // kh = 1 adds 32 rows: an immediate
        const int f = KL::fk(r);
        if constexpr (F8) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                ka_base[e] = lds_k0 + static_cast<uint32_t>(r * RBK + 16 * ((2 * hi + e) ^ f));
        } else {
            ka_base[0] = lds_k0 + static_cast<uint32_t>(r * D * 2 + 16 * ((hi ^ f) & 1) + 16 * (f & ~1));
        }
    }
    const int grp = lane >> 4;   // 16-lane group: d half (grp & 1), key half (grp >> 1)
    const int jj = lane & 15;
    uint32_t va_addr[DB];
#pragma unroll
    for (int dblk = 0; dblk < DB; ++dblk) {
        const int d = dblk * 32 + 16 * (grp & 1) + 4 * (jj & 3);
        const int c = d >> 3;
        const int half = d & 7;  // 0 or 4 elements
        const int rA = 8 * (grp >> 1) + (jj >> 2);   // j adds 16 rows, B adds 4: immediates
        va_addr[dblk] = lds_v0 + static_cast<uint32_t>((rA * D + ((c ^ LY::fv(rA)) << 3) + half) * 2);
    }

    f32x16 sacc[2];   // S of two consecutive 32-key half tiles (index: the half)
    float psum0 = 0.f, psum1 = 0.f;

    // K operand address of k-step ks: a loop-invariant register per k-step (and fp8 half)
    // plus an immediate (buffer and half); every operand read of the loop then takes its
    // offset from the instruction
    constexpr int KX = F8 ? 2 : 1;
    uint32_t kx[KS][KX];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < KX; ++e) kx[ks][e] = ka_base[e] ^ static_cast<uint32_t>((F8 ? 64 : 32) * ks);
    auto read_kx = [&](int ks, uint32_t off) -> KOp {
        if constexpr (F8) {
            union {
                i32x8 v;
                u32x4 h[2];
            } r;
            r.h[0] = *(const lds_u32x4*)(uintptr_t)(kx[ks][0] + off);
            r.h[1] = *(const lds_u32x4*)(uintptr_t)(kx[ks][1] + off);
            return r.v;
        } else {
            return *(const lds_bf16x8*)(uintptr_t)(kx[ks][0] + off);
        }
    };
    auto mfma_s = [&](const KOp& ka, int ks, const f32x16& acc) {
        if constexpr (F8)
            return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qf[ks], acc, 0, 0, 0, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], acc, 0, 0, 0);
    };
    // S^T of half H of the K tile at LDS byte offset kbuf (0 or one buffer) into sacc[H]
    auto compute_s = [&](auto H, uint32_t kbuf) {
        constexpr int hh = decltype(H)::value;
        const uint32_t off = kbuf + hh * 32 * RBK;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[hh][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc[hh] = mfma_s(read_kx(ks, off), ks, sacc[hh]);
    };
    // P fragment j (0/1) of sacc[H]: 16 keys 16j + 8*hi + e of that half; exp2 offset `off`
    auto make_p = [&](auto H, int j, float off) {
        constexpr int hh = decltype(H)::value;
        union {
            bf16x8 v;
            uint32_t u[4];
        } pk;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float p0 = fast_exp2(fmaf(sacc[hh][j * 8 + 2 * t], cs, off));
            const float p1 = fast_exp2(fmaf(sacc[hh][j * 8 + 2 * t + 1], cs, off));
            pk.u[t] = pack_bf16x2(p0, p1);
            if (t & 1)
                psum1 = add_bf16x2(pk.u[t], psum1);
            else
                psum0 = add_bf16x2(pk.u[t], psum0);
        }
        return pk.v;
    };
    // O^T += V^T(j) P^T(j) for the 16 keys j (0/1) of the V slot at LDS byte offset vslot
    auto pv = [&](uint32_t vslot, int j, const bf16x8& pf) {
#pragma unroll
        for (int dblk = 0; dblk < DB; ++dblk) {
            const uint32_t pa = va_addr[dblk] + vslot + j * 16 * D * 2;
            union {
                bf16x8 v;
                v4i16 h[2];
            } va;
            va.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)pa);
            va.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(pa + 4 * D * 2));
            oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va.v, pf, oacc[dblk], 0, 0, 0);
        }
    };
    // mask (partial tiles, padding, causal diagonal) of half H of tile t in sacc[H]
    auto apply_mask = [&](auto H, const Tile& t) {
        constexpr int hh = decltype(H)::value;
        const int lvl = t.l;
        // A lane's 16 accumulator slots are 4 runs of 4 consecutive tile keys tk0 + i; a run
        // lies inside one logical block (>= 8 rows), so one list read per run.
        const int rs = 64 >> lvl;
        const int sh = 6 - lvl;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int tk0 = hh * 32 + 16 * (gi >> 1) + 8 * hi + 4 * (gi & 1);
            const int s = tk0 >> sh;
            const int kb = cols[t.base + (s < t.cnt ? s : 0)];
            const int last0 = s < t.cnt ? ((kb * rs + (tk0 & (rs - 1)) + 1) << lvl) - 1
                                        : 0x7fffffff - (3 << 3);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int last = last0 + (i << lvl);
                if (last > limit) sacc[hh][gi * 4 + i] = -INFINITY;
            }
        }
    };
    // max over the 8 values of part `part` of sacc[H]: a chain of three max3 and one max
    auto half_max_part = [&](auto H, int part) {
        constexpr int hh = decltype(H)::value;
        const int e0 = part * 8;
        float m = __builtin_fmaxf(__builtin_fmaxf(sacc[hh][e0], sacc[hh][e0 + 1]), sacc[hh][e0 + 2]);
        asm volatile("" : "+v"(m));
        m = __builtin_fmaxf(__builtin_fmaxf(m, sacc[hh][e0 + 3]), sacc[hh][e0 + 4]);
        asm volatile("" : "+v"(m));
        m = __builtin_fmaxf(__builtin_fmaxf(m, sacc[hh][e0 + 5]), sacc[hh][e0 + 6]);
        return __builtin_fmaxf(m, sacc[hh][e0 + 7]);
    };
    // this lane's max over its half of the step's keys (the other half of each query's keys
    // sits in lane l ^ 32; the two are combined only when the max in use is raised), log2 units
    auto half_max = [&](float x0, float x1, int lvl) {
        return fmaf(fmaxf(x0, x1), cs, static_cast<float>(lvl));
    };
    // lazy running max: rescale the O accumulators and row sums only when the max in use is
    // exceeded by more than kLazyRescale (after the O products issued so far)
    // fp8 P V: the max in use is an integer (the ceiling) and is raised as soon as the row max
    // exceeds it by more than 1, so it stays within [M - 1, M] of the final M = ceil(row max);
    // P is quantized as 2^(t - m_use + 7) <= 2^8, i.e. relative to 2^(m_use - 7) in
    // [2^(M - 8), 2^(M - 7)]: every weight down to 2^-13 of the largest stays in e4m3's normal
    // range, where rounding commutes with the power-of-two rescales. P held in fp32 for a
    // pending product (`pending`) is rescaled with the accumulators.
    constexpr float kRescale = PV8 ? 1.0f : kLazyRescale;
    auto update_max = [&](float mt, bool pending = false) {
        // mt is this lane's half of the query's keys: the query's max exceeds the bound iff
        // one of its two lanes' does, and the new max is taken over both
        if (__builtin_expect(__ballot(mt > m_use + kRescale) != 0ull, 0)) {
            const float mt_all = pair32_max(mt);
            const float m_new = fmaxf(m_use, PV8 ? ceilf(mt_all) : mt_all);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_use - m_new);
            m_use = m_new;
            if constexpr (PV8) {
                lacc[0] *= alpha;
                if (pending)
#pragma unroll
                    for (int e = 0; e < 16; ++e) pAf[e] *= alpha;
            } else {
                psum0 *= alpha;
                psum1 *= alpha;
            }
#pragma unroll
            for (int i = 0; i < DB; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
        }
    };
    auto tile_needs_mask = [&](const Tile& t) {
        const int kb_max = cols[t.base + t.cnt - 1];
        return (t.cnt < (1 << t.l)) || ((kb_max + 1) * 64 - 1 > min_limit);
    };
    auto exp_off = [&](int lvl) {
        return static_cast<float>(lvl + (PV8 ? 7 : 0)) - (m_use == -INFINITY ? 0.f : m_use);
    };
    auto wait_publish = [&]() {
        // this wave's direct loads landed (vmcnt), then the barrier publishes every wave's and
        // retires every wave's reads of the buffers about to be refilled
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    };
    // exp chunk c (of KK) of the P fragments of sacc[H]: 8 / KK * 4 ... pairs of keys
    constexpr int PAIRS = 8 / KK;   // key pairs per chunk (1 for D = 128, 2 for D = 64)
    auto exp_a = [&](auto H, int c, float off, float (&ef)[2 * PAIRS]) {
        constexpr int hh = decltype(H)::value;
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int pr = c * PAIRS + q;
            ef[2 * q] = fast_exp2(fmaf(sacc[hh][2 * pr], cs, off));
            ef[2 * q + 1] = fast_exp2(fmaf(sacc[hh][2 * pr + 1], cs, off));
        }
    };
    auto exp_b = [&](int c, const float (&ef)[2 * PAIRS], uint32_t (&pk)[8]) {
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int pr = c * PAIRS + q;
            pk[pr] = pack_bf16x2(ef[2 * q], ef[2 * q + 1]);
            if (pr & 1)
                psum1 = add_bf16x2(pk[pr], psum1);
            else
                psum0 = add_bf16x2(pk[pr], psum0);
        }
    };
    auto read_v = [&](uint32_t vslot, int j, int dblk) {
        const uint32_t pa = va_addr[dblk] + vslot + j * 16 * D * 2;
        union {
            bf16x8 v;
            v4i16 h[2];
        } va;
        va.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)pa);
        va.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(pa + 4 * D * 2));
        return va.v;
    };
    // One pipeline step of KK slots, in a fixed issue order (a scheduling barrier after each
    // MFMA). The exp work is software-pipelined: slot kk issues the fma and exp2 of chunk kk and
    // the bf16 packing and row sums of chunk kk-1, whose exp2 results arrived meanwhile. The
    // wave raises its issue priority for the MFMA-dense second half of the step (S and O
    // MFMAs per slot) and drops it for the exp-heavy first half, so that the two waves sharing
    // a SIMD tend to alternate between the two kinds of work.
    //   S(h) MFMAs: bf16 one per slot, K reads three MFMAs ahead; fp8 one per KSL slots, K
    //   reads all at the start. In each slot 1/KK of the exp work of the previous half
    //   (sacc[H^1], level lvl_p); from slot KK/2 on, the O MFMAs of its first 16 keys; then the
    //   O MFMAs of its last 16 keys, alongside the row max of S(h).
    // Returns the half's unmasked max (log2 units).
    auto step = [&](auto H, uint32_t kbuf, uint32_t vslot, int lvl_p, int lvl_h, auto&& dma) {
        constexpr int hh = decltype(H)::value;
        constexpr int KPRE = F8 ? KS : 3;   // K reads issued before the first slot
        const float off = exp_off(lvl_p);
        const uint32_t koff = kbuf + hh * 32 * RBK;   // an immediate: no carry into the XORed bits
        uint32_t pk[8];
        float ef[2][2 * PAIRS];   // exp results of chunks kk and kk - 1
        KOp kr[KS];
        bf16x8 vr0[DB], vr1[DB];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < KPRE && i < KS; ++i) kr[i] = read_kx(i, koff);
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[hh][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (!F8 && kk + KPRE < KS) kr[kk + KPRE] = read_kx(kk + KPRE, koff);
            if (kk == 0)
#pragma unroll
                for (int d = 0; d < DB; ++d) vr0[d] = read_v(vslot, 0, d);
            if (kk == KK / 2) {
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int d = 0; d < DB; ++d) vr1[d] = read_v(vslot, 1, d);
            }
            if (kk % KSL == 0) sacc[hh] = mfma_s(kr[kk / KSL], kk / KSL, sacc[hh]);
            if (kk > 0) exp_b(kk - 1, ef[(kk - 1) & 1], pk);
            exp_a(IC<hh ^ 1>{}, kk, off, ef[kk & 1]);
            dma(kk);   // the next tiles' direct loads ride along with the MFMAs
            if (kk >= KK / 2) {
                const int d = kk - KK / 2;
                const bf16x8 p0 = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
                oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr0[d], p0, oacc[d], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        exp_b(KK - 1, ef[(KK - 1) & 1], pk);
        float x0 = -INFINITY, x1 = -INFINITY;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
            const bf16x8 p1 = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr1[d], p1, oacc[d], 0, 0, 0);
            // (the empty asm pins each partial max to its slot; the compiler would sink it)
            if (d == 0) {
                x0 = half_max_part(H, 0);
                asm volatile("" : "+v"(x0));
            }
            if (d == (DB > 1 ? 1 : 0)) {
                x1 = half_max_part(H, 1);
                asm volatile("" : "+v"(x1));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        return half_max(x0, x1, lvl_h);
    };
    // step, then (tiles that need it) the mask and the max again, then the lazy max update
    auto step_max = [&](auto H, bool need, uint32_t kbuf, uint32_t vslot, int lvl_p, const Tile& t,
                        auto&& dma) {
        float mt = step(H, kbuf, vslot, lvl_p, t.l, dma);
        if (need) {
            apply_mask(H, t);
            mt = half_max(half_max_part(H, 0), half_max_part(H, 1), t.l);
        }
        update_max(mt);
    };

    // ---- fp8 P V pipeline pieces ----
    // O^T += V^T P^T on v_mfma_f32_32x32x64_f8f6f4 over a whole 64-key tile. B = P^T: lane l holds
    // query l % 32 and the 32 bytes kappa = 16 h + 8 j + e (h = the tile's half, j, e as in the
    // S accumulators: C registers 8j + e of half h hold tile key 32 h + 16 j + 8 (l / 32) + e),
    // i.e. [P8 of half 0, P8 of half 1] in register order. A = V^T: lane l holds column
    // d = 32 dblk + l % 32 and the same 32 keys, which four 8-bit transposed reads deliver: a
    // 16-lane group names 8 aligned rows x 16 bytes (lanes 2m and 2m+1: row m's two 8-byte
    // halves) and lane i receives byte i of each of the 8 rows, in row order. Read (h, j) of
    // lane l covers rows 32 h + 16 j + 8 (l / 32) + 0..7 at columns 32 dblk + 16 ((l / 16) & 1)
    // + 0..15; the swizzle term 2 ((r >> 1) & 3) of those rows depends only on the lane, so
    // each dblk has one loop-invariant address and (h, j) is an immediate.
    uint32_t va8[DB];
#pragma unroll
    for (int dblk = 0; dblk < DB; ++dblk)
        va8[dblk] = lds_v0 + static_cast<uint32_t>((8 * hi + (jj >> 1)) * RBV +
                                                   16 * ((2 * dblk + (grp & 1)) ^ (2 * ((jj >> 2) & 3))) +
                                                   8 * (jj & 1));
    auto read_v8 = [&](uint32_t vbuf, int dblk) {
        union {
            i32x8 v;
            i32x2 h[4];
        } r;
#pragma unroll
        for (int hj = 0; hj < 4; ++hj)
            r.h[hj] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)(uintptr_t)(va8[dblk] + vbuf + static_cast<uint32_t>((32 * (hj >> 1) + 16 * (hj & 1)) * RBV)));
        return r.v;
    };
    // exp chunk c of sacc[H], kept in fp32 (a tile's first half) or packed to e4m3 (its second
    // half): pair pr = registers 2pr, 2pr + 1 -> bytes 2pr, 2pr + 1 (v_cvt_pk_fp8_f32 rounds to
    // nearest even, with subnormals; src0 goes to the lower byte)
    auto exp_f = [&](auto H, int c, float off) {
        constexpr int hh = decltype(H)::value;
        constexpr int PAIRS = 8 / KK;
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int pr = c * PAIRS + q;
            pAf[2 * pr] = fast_exp2(fmaf(sacc[hh][2 * pr], cs, off));
            pAf[2 * pr + 1] = fast_exp2(fmaf(sacc[hh][2 * pr + 1], cs, off));
        }
    };
    auto exp_q = [&](auto H, int c, float off, uint32_t (&pq)[4]) {
        constexpr int hh = decltype(H)::value;
        constexpr int PAIRS = 8 / KK;
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int pr = c * PAIRS + q;
            const float p0 = fast_exp2(fmaf(sacc[hh][2 * pr], cs, off));
            const float p1 = fast_exp2(fmaf(sacc[hh][2 * pr + 1], cs, off));
            const int old = static_cast<int>(pq[pr >> 1]);   // (the word select must be a constant)
            pq[pr >> 1] = static_cast<uint32_t>((pr & 1) ? __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, old, true)
                                                         : __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, old, false));
        }
    };
    // the tile's P V product and its row sums (A = all ones: e4m3 1.0 is 0x38)
    auto pv8 = [&](const i32x8 (&vf)[DB], const uint32_t (&pq)[4]) {
        uint32_t qa[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            qa[w] = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(pAf[4 * w], pAf[4 * w + 1], 0, false));
            qa[w] = static_cast<uint32_t>(
                __builtin_amdgcn_cvt_pk_fp8_f32(pAf[4 * w + 2], pAf[4 * w + 3], static_cast<int>(qa[w]), true));
        }
        const i32x8 pf = {static_cast<int>(qa[0]), static_cast<int>(qa[1]), static_cast<int>(qa[2]),
                          static_cast<int>(qa[3]), static_cast<int>(pq[0]), static_cast<int>(pq[1]),
                          static_cast<int>(pq[2]), static_cast<int>(pq[3])};
        const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                            0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
        for (int dblk = 0; dblk < DB; ++dblk) {
            oacc[dblk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[dblk], pf, oacc[dblk], 0, 0, 0, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 0, 0, 0);
    };
    // One step of the fp8 P V pipeline (KK slots, a scheduling barrier after each):
    //   S(h) on the fp8 MFMA in slots 0 and KSL (K reads at the start); in each slot 1/KK of
    //   the exp work of the other half: H = 0 exponentiates the previous tile's second half
    //   (to e4m3) and then runs that tile's P V product (V tile reads issued from the middle
    //   slot, buffer `vprev`); H = 1 exponentiates this tile's first half into pAf (fp32).
    // Returns the half's unmasked max (log2 units).
    auto step8 = [&](auto H, uint32_t kbuf, int lvl_p, int lvl_h, auto&& dma, uint32_t vprev) {
        constexpr int hh = decltype(H)::value;
        const float off = exp_off(lvl_p);
        const uint32_t koff = kbuf + hh * 32 * RBK;
        KOp kr[KS];
        uint32_t pq[4] = {0u, 0u, 0u, 0u};
        i32x8 vf[DB];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < KS; ++i) kr[i] = read_kx(i, koff);
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[hh][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (hh == 0 && kk == KK / 2)
#pragma unroll
                for (int d = 0; d < DB; ++d) vf[d] = read_v8(vprev, d);
            if (kk % KSL == 0) sacc[hh] = mfma_s(kr[kk / KSL], kk / KSL, sacc[hh]);
            if constexpr (hh == 0)
                exp_q(IC<1>{}, kk, off, pq);
            else
                exp_f(IC<0>{}, kk, off);
            dma(kk);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (hh == 0) pv8(vf, pq);
        float x0 = half_max_part(H, 0);
        float x1 = half_max_part(H, 1);
        return half_max(x0, x1, lvl_h);
    };
    auto step8_max = [&](auto H, bool need, uint32_t kbuf, int lvl_p, const Tile& t, auto&& dma,
                         uint32_t vprev) {
        constexpr int hh = decltype(H)::value;
        float mt = step8(H, kbuf, lvl_p, t.l, dma, vprev);
        if (need) {
            apply_mask(H, t);
            mt = half_max(half_max_part(H, 0), half_max_part(H, 1), t.l);
        }
        update_max(mt, hh == 1);   // after H = 1 the first half's P waits in pAf
    };

    __syncthreads();  // cols[] visible

    Tile cur{0, 0, 0, 0};
    enter_level(cur);
    set_cnt(cur);
    if (!any_valid_query) cur.l = 4;

    if constexpr (PV8) {
        // ---- fp8 P V: K(t) in buffer t & 1, V(t) (a whole tile) in buffer t mod 3 ----
        // Tile t's P V product runs at the end of tile t+1's first step, once its second half
        // is exponentiated; V(t)'s buffer is refilled (with V(t+3)) only after tile t+2's
        // barrier. K(t+1) and V(t+1) are loaded during tile t's first step, sharing one list
        // lookup (both tiles' rows are split over the waves alike).
        constexpr uint32_t kVTile = 64 * RBV;
        if (cur.l < 4) {
            issue_k(cur, 0);
            issue(cur, lds_v0, IC<1>{}, IC<0>{}, IC<64>{});
            Tile nxt = next_tile(cur);
            wait_publish();
            if (nxt.l < 4) {
                issue_k(nxt, 1);
                issue(nxt, lds_v0 + kVTile, IC<1>{}, IC<0>{}, IC<64>{});
            }
            const bool nm = tile_needs_mask(cur);
            compute_s(IC<0>{}, 0u);
            if (nm) apply_mask(IC<0>{}, cur);
            update_max(half_max(half_max_part(IC<0>{}, 0), half_max_part(IC<0>{}, 1), cur.l));
            step8_max(IC<1>{}, nm, 0u, cur.l, cur, [](int) {}, 0u);
            int lvl_prev = cur.l;
            cur = nxt;
            int vb = 1;   // V buffer of tile `cur`
            auto tile_body8 = [&](auto TT) -> bool {   // false after the row's last tile
                constexpr int T = decltype(TT)::value;
                const Tile nx = next_tile(cur);
                wait_publish();
                const bool has_nx = nx.l < 4;
                const bool need = tile_needs_mask(cur);
                const uint32_t kbuf = T ? kBufBytes : 0u;
                const Tile nsrc = has_nx ? nx : cur;
                const uint32_t vprev = static_cast<uint32_t>(vb == 0 ? 2 : vb - 1) * kVTile;
                const uint32_t vnext = static_cast<uint32_t>(vb == 2 ? 0 : vb + 1) * kVTile;
                Pend pd{};
                Dma dk{}, dv{};
                auto dma = [&](int sl) {
                    if (sl == 0) {
                        pd = pend(nsrc, IC<0>{}, IC<64>{});
                    } else if (sl == 1) {
                        dk = resolve(nsrc, pd, lds_k0 + (T ? 0u : kBufBytes), false, IC<0>{}, IC<64>{});
                        dv = resolve(nsrc, pd, lds_v0 + vnext, true, IC<0>{}, IC<64>{});
                    } else {
#pragma unroll
                        for (int i = 0; i < IPWK + IPWV; ++i)
                            if (i % (KK - 2) == sl - 2) {
                                if (i < IPWK)
                                    fire(dk, false, nsrc.l > 0, i);
                                else
                                    fire(dv, true, nsrc.l > 0, i - IPWK);
                            }
                    }
                };
                step8_max(IC<0>{}, need, kbuf, lvl_prev, cur, dma, vprev);
                step8_max(IC<1>{}, need, kbuf, cur.l, cur, [](int) {}, 0u);
                lvl_prev = cur.l;
                cur = nx;
                vb = vb == 2 ? 0 : vb + 1;
                return cur.l < 4;
            };
            if (cur.l < 4) {
                for (;;) {
                    if (!tile_body8(IC<1>{})) break;
                    if (!tile_body8(IC<0>{})) break;
                }
            }
            // ---- after the last tile: its second half's P, then its P V product ----
            wait_publish();
            {
                const float off = exp_off(lvl_prev);
                uint32_t pq[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int c = 0; c < KK; ++c) exp_q(IC<1>{}, c, off, pq);
                const uint32_t vlast = static_cast<uint32_t>(vb == 0 ? 2 : vb - 1) * kVTile;
                i32x8 vf[DB];
#pragma unroll
                for (int d = 0; d < DB; ++d) vf[d] = read_v8(vlast, d);
                pv8(vf, pq);
            }
        }
    } else if (cur.l < 4) {
        // ---- tile 0: K(0) and V half 0 first; S of half 0 alone, then step(half 1) ----
        issue_k(cur, 0);
        issue_vh(cur, 0, 0);
        Tile nxt = next_tile(cur);
        wait_publish();
        if (nxt.l < 4) issue_k(nxt, 1);
        issue_vh(cur, 1, 1);
        if (nxt.l < 4) issue_vh(nxt, 0, 2);
        bool nm = tile_needs_mask(cur);
        compute_s(IC<0>{}, 0u);
        if (nm) apply_mask(IC<0>{}, cur);
        update_max(half_max(half_max_part(IC<0>{}, 0), half_max_part(IC<0>{}, 1), cur.l));
        step_max(IC<1>{}, nm, 0u, 0u, cur.l, cur, [](int) {});
        int lvl_prev = cur.l;
        cur = nxt;
        int last_parity = 0;   // parity of the row's last tile

        // ---- tile t >= 1 (T = t & 1): K(t) in buffer T; V half u = 2t + h in slot u & 3 ----
        // Two copies of the body, one per parity, so that every buffer and slot offset is an
        // instruction immediate.
        auto tile_body = [&](auto TT) -> bool {   // false after the row's last tile
            constexpr int T = decltype(TT)::value;
            const Tile nx = next_tile(cur);
            wait_publish();
            const bool has_nx = nx.l < 4;
            const bool need = tile_needs_mask(cur);
            const uint32_t kbuf = T ? kBufBytes : 0u;
            // All of the next direct loads ride along with the first step, so each has about
            // one and a half steps to land before the barrier that publishes it: K(t+1) into
            // the other K buffer, V halves 2t+1 and 2t+2 into ring slots whose previous halves
            // (2t-3, 2t-2) were consumed before this tile's barrier. Slot 0 reads the list
            // entries, slot 1 resolves the addresses, slot s >= 2 fires the instructions i
            // (K, then V half 2t+1, then V half 2t+2) with i % (KK - 2) == s - 2.
            // After the row's last tile the "next" loads repeat the current tile into buffers
            // that are never read again: no branches inside the steps.
            const Tile nsrc = has_nx ? nx : cur;
            Pend pk{}, pv1{}, pv0{};
            Dma dk{}, dv1{}, dv0{};
            auto dma = [&](int sl) {
                if (sl == 0) {
                    pk = pend(nsrc, IC<0>{}, IC<64>{});
                    pv1 = pend(cur, IC<32>{}, IC<32>{});
                    pv0 = pend(nsrc, IC<0>{}, IC<32>{});
                } else if (sl == 1) {
                    dk = resolve(nsrc, pk, lds_k0 + (T ? 0u : kBufBytes), false, IC<0>{}, IC<64>{});
                    dv1 = resolve(cur, pv1, lds_v0 + static_cast<uint32_t>(2 * T + 1) * kSlotBytes, true, IC<32>{}, IC<32>{});
                    dv0 = resolve(nsrc, pv0, lds_v0 + static_cast<uint32_t>((2 * T + 2) & 3) * kSlotBytes, true, IC<0>{}, IC<32>{});
                } else {
#pragma unroll
                    for (int i = 0; i < IPWK + 2 * IPWV; ++i)
                        if (i % (KK - 2) == sl - 2) {
                            if (i < IPWK)
                                fire(dk, false, nsrc.l > 0, i);
                            else if (i < IPWK + IPWV)
                                fire(dv1, true, cur.l > 0, i - IPWK);
                            else
                                fire(dv0, true, nsrc.l > 0, i - IPWK - IPWV);
                        }
                }
            };
            // half 0: P of the previous tile's half 1 (slot 2t-1 = 2T+3 mod 4)
            step_max(IC<0>{}, need, kbuf, static_cast<uint32_t>((2 * T + 3) & 3) * kSlotBytes, lvl_prev, cur, dma);
            // half 1: P of this tile's half 0 (slot 2T)
            step_max(IC<1>{}, need, kbuf, static_cast<uint32_t>(2 * T) * kSlotBytes, cur.l, cur, [](int) {});
            lvl_prev = cur.l;
            cur = nx;
            return cur.l < 4;
        };
        if (cur.l < 4) {
            for (;;) {
                if (!tile_body(IC<1>{})) {
                    last_parity = 1;
                    break;
                }
                if (!tile_body(IC<0>{})) break;
            }
        }
        // ---- after the last tile (parity P): P and O of its half 1 (slot 2P+1) ----
        wait_publish();
        {
            const float off = exp_off(lvl_prev);
            const bf16x8 p0 = make_p(IC<1>{}, 0, off);
            const bf16x8 p1 = make_p(IC<1>{}, 1, off);
            const uint32_t vslot = static_cast<uint32_t>(2 * last_parity + 1) * kSlotBytes;
            pv(vslot, 0, p0);
            pv(vslot, 1, p1);
        }
    }
    l_run += psum0 + psum1;

    // ---- epilogue ----
    const float l_tot = PV8 ? lacc[0] : pair32_sum(l_run);
    const bool valid_q = qt < a.Nv && l_tot > 0.f;
    float inv = valid_q ? 1.f / l_tot : 0.f;
    if constexpr (PV8) inv *= a.v_scale[b * a.Hkv + hk];
    bf16_bits* O = static_cast<bf16_bits*>(a.o) + b * a.os0 + h * a.os1 + static_cast<int64_t>(qt) * a.os2;
#pragma unroll
    for (int dblk = 0; dblk < DB; ++dblk)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[dblk][4 * gg] * inv, oacc[dblk][4 * gg + 1] * inv);
            w[1] = pack_bf16x2(oacc[dblk][4 * gg + 2] * inv, oacc[dblk][4 * gg + 3] * inv);
            *reinterpret_cast<u32x2*>(O + dblk * 32 + gg * 8 + hi * 4) = w;
        }
    if (a.lse != nullptr && hi == 0) {
        const float lse = valid_q ? (m_use - (PV8 ? 7.f : 0.f) + log2f(l_tot)) * kLn2 : -INFINITY;
        a.lse[(static_cast<int64_t>(b) * a.H + h) * a.N + qt] = lse;
    }
}

template <int D, int BQ, bool PACK, int FP8 = 0, bool MK = false>
hipError_t launch_one(const Shape& s, const AttnArgs& a, hipStream_t st, const MkArgs& mk = MkArgs{}) {
    const int rows = s.B * s.H * s.NQB;
    const int nper = (rows + 7) / 8;
    const size_t dyn = static_cast<size_t>(s.NKB) * sizeof(int);
    if (a.ks2 == D && a.vs2 == D)
        hipLaunchKernelGGL((k_attn_fwd_bf16<D, BQ, true, PACK, FP8, MK>), dim3(8 * nper), dim3(2 * BQ), dyn, st, a, rows, mk);
    else
        hipLaunchKernelGGL((k_attn_fwd_bf16<D, BQ, false, PACK, FP8, MK>), dim3(8 * nper), dim3(2 * BQ), dyn, st, a, rows, mk);
    return hipGetLastError();
}

template <bool PACK>
hipError_t launch_packed(const Shape& s, const AttnArgs& a, hipStream_t st) {
    if (s.D == 128 && s.BQ == 128) return launch_one<128, 128, PACK>(s, a, st);
    if (s.D == 128 && s.BQ == 64) return launch_one<128, 64, PACK>(s, a, st);
    if (s.D == 64 && s.BQ == 128) return launch_one<64, 128, PACK>(s, a, st);
    if (s.D == 64 && s.BQ == 64) return launch_one<64, 64, PACK>(s, a, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_bf16(const Shape& s, const AttnArgs& a, bool pack, hipStream_t st) {
    return pack ? launch_packed<true>(s, a, st) : launch_packed<false>(s, a, st);
}

hipError_t launch_attn_fp8qk(const Shape& s, const AttnArgs& a, hipStream_t st) {
    if (s.B * s.H * s.NQB == 0) return hipSuccess;
    if (a.q_scale == nullptr || a.k_scale == nullptr) return hipErrorInvalidValue;
    if (s.D == 128 && s.BQ == 128) return launch_one<128, 128, true, 1>(s, a, st);
    if (s.D == 128 && s.BQ == 64) return launch_one<128, 64, true, 1>(s, a, st);
    return hipErrorNotSupported;
}

hipError_t launch_attn_fwd_meankey(const Shape& s, float scale, const psa_mask_params& mp,
                                   const void* q, const void* k, const void* v, const void* kp,
                                   const void* vp, const float* qbar, const float* kbar,
                                   const double* ksum, const float* sim, const double* sim64,
                                   int8_t* map_out, float* mass_out, void* o, float* lse,
                                   hipStream_t st) {
    if (s.dtype != PSA_BF16 || s.BQ != 128 || s.BK != 64 || s.NKB > 1792) return hipErrorNotSupported;
    if (s.B * s.H * s.NQB == 0) return hipSuccess;
    AttnArgs a{};
    a.q = q; a.k = k; a.v = v; a.kp = kp; a.vp = vp; a.o = o; a.lse = lse;
    a.row_ptr = nullptr;
    a.col_idx = nullptr;
    a.H = s.H; a.Hkv = s.Hkv; a.N = s.N; a.Nv = s.Nv; a.NQB = s.NQB; a.causal = s.causal;
    a.qs0 = s.qs[0]; a.qs1 = s.qs[1]; a.qs2 = s.qs[2];
    a.ks0 = s.ks[0]; a.ks1 = s.ks[1]; a.ks2 = s.ks[2];
    a.vs0 = s.vs[0]; a.vs1 = s.vs[1]; a.vs2 = s.vs[2];
    a.os0 = s.os[0]; a.os1 = s.os[1]; a.os2 = s.os[2];
    a.pooled_rows = s.pooled_rows;
    a.c = scale * kLog2e;
    MkArgs mk;
    mk.qbar = qbar;
    mk.kbar = kbar;
    mk.ksum = ksum;
    mk.mass_out = mass_out;
    mk.map_out = map_out;
    mk.asg = assign_args_of(s, mp);
    mk.asg.sim = mp.cos_sim_min > 0.f ? sim : nullptr;
    mk.asg.sim64 = mp.cos_sim_min > 0.f ? sim64 : nullptr;
    mk.asg.RQ = 1;
    mk.asg.rows_per_head = s.NQB;
    mk.asg.sampling = 1;   // one scoring row per query block, counted like a sampled row
    mk.asg.S = 1;
    mk.c = (1.0 / std::sqrt(static_cast<double>(s.D))) * 1.4426950408889634;
    mk.scale = 1.0 / std::sqrt(static_cast<double>(s.D));
    mk.share = order_share(s);
    if (s.D == 128) return launch_one<128, 128, true, 0, true>(s, a, st, mk);
    if (s.D == 64) return launch_one<64, 128, true, 0, true>(s, a, st, mk);
    return hipErrorNotSupported;
}

hipError_t launch_attn_fp8(const Shape& s, const AttnArgs& a, hipStream_t st) {
    if (s.B * s.H * s.NQB == 0) return hipSuccess;
    if (a.q_scale == nullptr || a.k_scale == nullptr || a.v_scale == nullptr) return hipErrorInvalidValue;
    // the e4m3 K and V are contiguous: only the CONTIG instantiation is used
    if (a.ks2 != s.D || a.vs2 != s.D) return hipErrorInvalidValue;
    if (s.D == 128 && s.BQ == 128) return launch_one<128, 128, true, 2>(s, a, st);
    if (s.D == 128 && s.BQ == 64) return launch_one<128, 64, true, 2>(s, a, st);
    return hipErrorNotSupported;
}

}  // namespace psa
