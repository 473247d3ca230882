// Multi-level mask generator (PSA summary article at rg.mbintangr.com, "Method": block
// importance from a sampling-based strategy for generation, antidiagonal scoring with an
// intra-block similarity check for understanding; "Results": threshold-based assignment and a
// cosine-similarity constraint on pooling).
//
// k_mask_logmass per scoring row and KV block, the log2 of the row's unnormalised softmax
//                mass on the block: L = m + log2(sum_t exp2(z_t c - m)), m the block's max of
//                z c (z the logits, c = scale * log2 e). Rows of the scoring GEMM are either
//                sampled query rows (sampling mode, S rows per query block) or compressed query
//                rows (antidiagonal mode, stride S: row r pairs q[rS+S-1-t] with k[cS+t], t < S,
//                summed). One workgroup owns 128 rows of one (batch, head) and a range of
//                64-column key tiles; logits come from v_mfma_f32_32x32x16_bf16 as in the
//                attention kernel (keys on M, rows on N). One pass, no cross-workgroup state:
//                the normalisation is left to the assignment.
// k_block_sim    mean pairwise cosine similarity of each KV block's valid keys, via
//                sum_{i!=j} khat_i.khat_j = |sum khat|^2 - sum |khat|^2, in float64.
// k_mask_assign  one workgroup per (batch, head, query block) row. From log-masses: each
//                scoring row's logsumexp over the KV blocks, block_mass[kb] = the mean over the
//                query block's valid rows of exp2(L - lse) (written out). Then a bitonic sort of
//                (mass desc, kb asc) in LDS, a float64 exclusive block scan of the sorted
//                masses (equal to a left-to-right float64 sum up to float64 rounding) gives
//                each block its level, then the overrides. psa_mask_assign enters with given
//                masses.
#include <math.h>

#include <algorithm>

#include "psa_device.h"
#include "psa_internal.h"
#include "psa_assign.h"

namespace psa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kScoreWaves = 4;
constexpr int kScoreThreads = 64 * kScoreWaves;

struct ScoreArgs {
    const bf16_bits* q;
    const bf16_bits* k;
    float* L;           // [B*H][NKB][rows_per_head] log2 masses
    int B, H, Hkv, N, Nv, BQ, NQB, NKB, causal;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2;
    int rows_per_head;  // sampling: NQB*S; antidiag: N/S
    int RQ;             // rows per query block: sampling S, antidiag BQ/S
    int wg_per_head;    // row groups of 128 per (batch, head)
    int nsplit;         // key-tile ranges per row group
    int tiles_per_split;
    float c;            // scale * log2(e)
};

// MODE 0: sampling with S samples per query block; MODE 1: antidiagonal with stride S.
// Workgroup = 128 rows x one range of key tiles; grid = B*H*wg_per_head*nsplit. In MODE 1 each
// chunk t (d products of one query row and one key row) accumulates from zero and is then added
// to the logit, so the running float32 sum is rounded S times instead of once per MFMA.
template <int MODE, int D, int S>
__global__ void __launch_bounds__(kScoreThreads) k_mask_logmass(ScoreArgs a) {
    constexpr int SI = MODE == 1 ? S : 1;          // inner chunks of D
    constexpr int CPK = MODE == 1 ? 64 / S : 64;   // columns per KV block
    constexpr int KT = 64 / CPK;                   // KV blocks per 64-column tile
    constexpr int KSTR = D + 8;
    constexpr int KCH = 64 * (D / 8) / kScoreThreads;
    static_assert(KCH >= 1, "tile");
    static_assert(CPK >= 8, "a KV block's columns are whole runs of 4 in each lane half");
    __shared__ __attribute__((aligned(16))) bf16_bits Ks[64 * KSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int split = blockIdx.x % a.nsplit;
    const int rg = blockIdx.x / a.nsplit;      // row group over all (batch, head)
    const int bh = rg / a.wg_per_head;
    const int wg = rg % a.wg_per_head;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);

    const int r = wg * 128 + wave * 32 + l32;  // 128 rows per workgroup
    const int r_last = wg * 128 + 127;
    bool row_ok;
    int tok = 0;  // sampling: the sampled token
    if (MODE == 0) {
        const int qb = r / S;
        const int s = r % S;
        const int rv = qb < a.NQB ? min(max(a.Nv - qb * a.BQ, 0), a.BQ) : 0;
        row_ok = rv > 0;
        tok = rv > 0 ? qb * a.BQ + (s * rv) / S : 0;
    } else {
        row_ok = r < a.rows_per_head && (r * S + S - 1) < a.Nv;
    }
    const bool row_in = r < a.rows_per_head;
    // log-mass of (row r, block kb) lives at Lh[kb * rows_per_head + r]: the 32 rows of a wave
    // store one contiguous 128-byte run per block
    float* Lh = a.L + static_cast<int64_t>(bh) * a.NKB * a.rows_per_head;

    const bf16_bits* qbase = a.q + b * a.qs0 + h * a.qs1;
    const bf16_bits* kbase = a.k + b * a.ks0 + hk * a.ks1;

    bf16x8 qf[D / 16];
    auto load_q = [&](int t) {
        const int qt = MODE == 0 ? tok : (row_ok ? r * S + S - 1 - t : 0);
        const bf16_bits* qp = qbase + static_cast<int64_t>(qt) * a.qs2;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hi * 8);
    };
    if (MODE == 0) load_q(0);

    // 64-column tiles; in antidiagonal mode the last one may be partial (N/S not a multiple
    // of 64): its columns past ncols read no key and are masked like padding
    const int ncols = MODE == 0 ? a.N : a.N / S;
    const int ntiles = (ncols + 63) / 64;
    // tiles past the causal frontier of the workgroup's rows are fully masked
    int tiles_needed = ntiles;
    if (MODE == 1 && a.causal) tiles_needed = min(ntiles, r_last / 64 + 1);
    if (MODE == 0 && a.causal) {
        const int qb_last = min(r_last / S, a.NQB - 1);
        tiles_needed = min(ntiles, (qb_last * a.BQ + a.BQ - 1) / 64 + 1);
    }
    const int j_lo = split * a.tiles_per_split;
    const int j_hi = min(ntiles, j_lo + a.tiles_per_split);
    const int j_end = min(j_hi, tiles_needed);   // tiles [j_lo, j_end) are computed

    u32x4 kreg[KCH];
    auto load_k = [&](int j, int t) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int cidx = tid + i * kScoreThreads;
            const int row = cidx / (D / 8);
            const int col = (cidx % (D / 8)) * 8;
            const int64_t key = MODE == 0 ? static_cast<int64_t>(j) * 64 + row
                                          : (static_cast<int64_t>(j) * 64 + row) * S + t;
            if (MODE == 1 && j * 64 + row >= ncols)
                kreg[i] = u32x4{0u, 0u, 0u, 0u};
            else
                kreg[i] = *reinterpret_cast<const u32x4*>(kbase + key * a.ks2 + col);
        }
    };
    auto store_k = [&]() {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int cidx = tid + i * kScoreThreads;
            const int row = cidx / (D / 8);
            const int col = (cidx % (D / 8)) * 8;
            *reinterpret_cast<u32x4*>(&Ks[row * KSTR + col]) = kreg[i];
        }
    };

    if (j_lo < j_end) load_k(j_lo, 0);
    for (int j = j_lo; j < j_end; ++j) {
        f32x16 sacc[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kh][e] = 0.f;
        for (int t = 0; t < SI; ++t) {
            __syncthreads();
            store_k();
            __syncthreads();
            {   // prefetch the next (tile, chunk) step
                int nj = j, nt = t + 1;
                if (nt == SI) {
                    nt = 0;
                    ++nj;
                }
                if (nj < j_end) load_k(nj, nt);
            }
            if (MODE == 1) load_q(t);
            f32x16 cacc[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) cacc[kh][e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                        &Ks[(kh * 32 + l32) * KSTR + kk * 16 + hi * 8]);
                    cacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], cacc[kh], 0, 0, 0);
                }
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) sacc[kh] += cacc[kh];
        }
        // mask: lane value e of half kh is column j*64 + kh*32 + (e/4)*8 + hi*4 + e%4
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int cc = j * 64 + kh * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
                bool ok;
                if (MODE == 0)
                    ok = row_ok && cc < a.Nv && (!a.causal || cc <= tok);
                else
                    ok = row_ok && (cc * S + S - 1) < a.Nv && (!a.causal || cc <= r);
                if (!ok) sacc[kh][e] = -INFINITY;
            }
        // per KV block of the tile: max, then the sum of exp2 relative to it (the block's
        // columns are whole 8-column groups, half in each lane of a lane pair)
        float Lk[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            constexpr int G8 = CPK / 8;   // 8-column groups per block
            float m = -INFINITY;
#pragma unroll
            for (int g = 0; g < G8; ++g) {
                const int gg = kt * G8 + g;   // group 0..7 of the tile: half gg/4, e = (gg%4)*4 + i
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, sacc[gg >> 2][(gg & 3) * 4 + i]);
            }
            m = pair32_max(m);
            const float mc = m * a.c;
            float sum = 0.f;
            if (m != -INFINITY) {
#pragma unroll
                for (int g = 0; g < G8; ++g) {
                    const int gg = kt * G8 + g;
#pragma unroll
                    for (int i = 0; i < 4; ++i) sum += fast_exp2(fmaf(sacc[gg >> 2][(gg & 3) * 4 + i], a.c, -mc));
                }
            }
            sum = pair32_sum(sum);
            Lk[kt] = sum > 0.f ? mc + __builtin_amdgcn_logf(sum) : -INFINITY;
        }
        if (hi == 0 && row_in) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                if (j * KT + kt < a.NKB) Lh[static_cast<int64_t>(j * KT + kt) * a.rows_per_head + r] = Lk[kt];
        }
    }
    // tiles of this range past the causal frontier: no mass
    if (hi == 0 && row_in)
        for (int j = max(j_lo, j_end); j < j_hi; ++j)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                if (j * KT + kt < a.NKB) Lh[static_cast<int64_t>(j * KT + kt) * a.rows_per_head + r] = -INFINITY;
}

// Sampling mode, the fast path: 64 rows per wave (two groups of 32 sharing every K operand
// read), 256 rows per workgroup; K tiles move HBM/L2 -> LDS with direct loads into two
// XOR-swizzled buffers (no VGPR staging), one barrier per tile. Same outputs as
// k_mask_logmass<0, D, S>.
constexpr int kSampRows = 256;

template <int D, int S>
__global__ void __launch_bounds__(kScoreThreads) k_mask_logmass_sampling(ScoreArgs a) {
    constexpr int KK = D / 16;
    constexpr int CH = D / 8;                 // 16-byte chunks per K row
    constexpr int RPI = 1024 / (2 * D);       // K rows per 1 KB direct load
    constexpr int IPW = 64 / RPI / kScoreWaves;   // direct loads per wave per tile
    constexpr int KVAR = D == 128 ? 4 : 2;    // distinct chunk swizzles across instructions
    static_assert(IPW % KVAR == 0, "instruction and its index inside the wave agree mod KVAR");
    constexpr uint32_t kBuf = 64 * D * 2;
    __shared__ __attribute__((aligned(1024))) bf16_bits Kt[2][64 * D];
    auto fk = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    // XCD-aware order: workgroup i runs on XCD i % 8; each XCD takes a contiguous range of
    // (head, key range, row group) items, row group fastest, so the workgroups resident on an
    // XCD read the same K tiles (one head's key ranges) from its L2.
    const int total = a.B * a.H * a.wg_per_head * a.nsplit;
    const int nper = (total + 7) >> 3;
    const int item = (blockIdx.x & 7) * nper + (blockIdx.x >> 3);
    if (item >= total) return;
    const int wg = item % a.wg_per_head;
    const int split = (item / a.wg_per_head) % a.nsplit;
    const int bh = item / (a.wg_per_head * a.nsplit);
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);

    const int r0 = wg * kSampRows + wave * 64;   // group g holds rows r0 + 32 g + l32
    int tok[2];
    bool row_ok[2], row_in[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int r = r0 + 32 * g + l32;
        const int qb = r / S;
        const int rv = qb < a.NQB ? min(max(a.Nv - qb * a.BQ, 0), a.BQ) : 0;
        row_ok[g] = rv > 0;
        row_in[g] = r < a.rows_per_head;
        tok[g] = rv > 0 ? qb * a.BQ + ((r % S) * rv) / S : 0;
    }
    float* Lh = a.L + static_cast<int64_t>(bh) * a.NKB * a.rows_per_head;

    bf16x8 qf[2][KK];
    {
        const bf16_bits* qbase = a.q + b * a.qs0 + h * a.qs1;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const bf16_bits* qp = qbase + static_cast<int64_t>(tok[g]) * a.qs2;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) qf[g][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hi * 8);
        }
    }

    const int ntiles = a.N / 64;
    int tiles_needed = ntiles;
    const int r_last = min(wg * kSampRows + kSampRows, a.rows_per_head) - 1;
    if (a.causal) {
        const int qb_last = min(r_last / S, a.NQB - 1);
        tiles_needed = min(ntiles, (qb_last * a.BQ + a.BQ - 1) / 64 + 1);
    }
    const int j_lo = split * a.tiles_per_split;
    const int j_hi = min(ntiles, j_lo + a.tiles_per_split);
    const int j_end = min(j_hi, tiles_needed);
    // the smallest sampled token of the workgroup: tiles entirely at or below it and below Nv
    // need no mask
    const int tok_min = (wg * kSampRows / S) * a.BQ;

    // direct-load lane offsets: row inside the instruction, swizzled source chunk
    const bf16_bits* kbase = a.k + b * a.ks0 + hk * a.ks1;
    const uint32_t kstride = static_cast<uint32_t>(a.ks2) * 2u;
    uint32_t lpk[KVAR];
    {
        const int rr = lane / CH;
        const int p = lane % CH;
#pragma unroll
        for (int q = 0; q < KVAR; ++q)
            lpk[q] = rr * kstride + static_cast<uint32_t>((p ^ fk(q * RPI + rr)) << 4);
    }
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)&Kt[0][0]));
    auto issue = [&](int j, int buf) {
        // tile j = keys [64 j, 64 j + 64); instruction m covers rows [m RPI, m RPI + RPI)
        const char* tb = reinterpret_cast<const char*>(kbase) + static_cast<uint32_t>(j * 64) * kstride;
#pragma unroll
        for (int mi = 0; mi < IPW; ++mi) {
            const int m = wave * IPW + mi;
            dma16(tb + static_cast<uint32_t>(m * RPI) * kstride, lpk[mi % KVAR], lds0 + buf * kBuf + m * 1024);
        }
    };
    // A-operand address of row kh*32 + l32, chunk 2kk + hi: base ^ (32 kk) (see the attention
    // kernel: the XOR only touches the chunk bits)
    uint32_t ka_base;
    {
        const int r = l32;
        const int f = fk(r);
        ka_base = lds0 + static_cast<uint32_t>(r * D * 2 + 16 * ((hi ^ f) & 1) + 16 * (f & ~1));
    }

    if (j_lo < j_end) issue(j_lo, 0);
    int buf = 0;
    for (int j = j_lo; j < j_end; ++j) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of tile j landed
        __syncthreads();                       // everyone's landed; buffer buf^1 free
        if (j + 1 < j_end) issue(j + 1, buf ^ 1);
        f32x16 sacc[2][2];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[g][kh][e] = 0.f;
        const uint32_t kb0 = ka_base + (buf ? kBuf : 0u);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint32_t ad = kb0 ^ static_cast<uint32_t>(32 * kk);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x8 ka = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(ad + kh * 32 * D * 2);
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    sacc[g][kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[g][kk], sacc[g][kh], 0, 0, 0);
            }
        }
        // lane value e of half kh is key 64 j + 32 kh + (e / 4) * 8 + 4 hi + e % 4
        const bool need_mask = (j * 64 + 63 >= a.Nv) || (a.causal && j * 64 + 63 > tok_min);
        if (need_mask) {
            asm volatile("");   // keeps the branch: if-converted, the mask would run on every tile
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int cc = j * 64 + kh * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
                        if (!(cc < a.Nv && (!a.causal || cc <= tok[g]))) sacc[g][kh][e] = -INFINITY;
                    }
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            // two max chains and four partial sums: short dependency chains
            float m0 = fmaxf(sacc[g][0][0], sacc[g][0][1]), m1 = fmaxf(sacc[g][1][0], sacc[g][1][1]);
#pragma unroll
            for (int e = 2; e < 16; e += 2) {
                m0 = fmaxf(fmaxf(m0, sacc[g][0][e]), sacc[g][0][e + 1]);
                m1 = fmaxf(fmaxf(m1, sacc[g][1][e]), sacc[g][1][e + 1]);
            }
            const float m = pair32_max(fmaxf(m0, m1));
            const float mc = m * a.c;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
            if (m != -INFINITY) {
#pragma unroll
                for (int e = 0; e < 32; ++e) s4[e & 3] += fast_exp2(fmaf(sacc[g][e >> 4][e & 15], a.c, -mc));
            }
            const float sum = pair32_sum((s4[0] + s4[1]) + (s4[2] + s4[3]));
            const float Lv = (row_ok[g] && sum > 0.f) ? mc + __builtin_amdgcn_logf(sum) : -INFINITY;
            if (hi == 0 && row_in[g]) Lh[static_cast<int64_t>(j) * a.rows_per_head + r0 + 32 * g + l32] = Lv;
        }
        buf ^= 1;
    }
    // tiles of this range past the causal frontier: no mass
#pragma unroll
    for (int g = 0; g < 2; ++g)
        if (hi == 0 && row_in[g])
            for (int j = max(j_lo, j_end); j < j_hi; ++j)
                Lh[static_cast<int64_t>(j) * a.rows_per_head + r0 + 32 * g + l32] = -INFINITY;
}

// Antidiagonal mode, the fast path. The compressed logit A[r][c] = sum_t q[rS+S-1-t].k[cS+t]
// is a GEMM with contraction S*D. A workgroup owns 128 compressed rows (32 per wave) and a
// range of 128-column tiles; per (tile, chunk t) step the K chunk (keys cS+t of the tile's
// columns) moves HBM/L2 -> LDS by direct loads into two XOR-swizzled buffers while each wave's
// Q chunk (q[rS+S-1-t] of its rows) is prefetched into registers one step ahead. Each chunk's
// products accumulate from zero and are added to the tile's running logits (the running
// float32 sum is rounded S times, not once per MFMA: on a 32k-token causal layer the float32
// block masses then stay within 6e-6 relative of float64 instead of 1.7e-5). After the S
// chunks of a tile the per-block log-masses of its columns are reduced and stored. Same
// outputs as k_mask_logmass<1, D, S>.
constexpr int kAdCols = 128;

template <int D, int S>
__global__ void __launch_bounds__(kScoreThreads) k_mask_logmass_antidiag(ScoreArgs a) {
    constexpr int KK = D / 16;
    constexpr int CH = D / 8;
    constexpr int RPI = 1024 / (2 * D);          // columns per 1 KB direct load
    constexpr int IPW = kAdCols / RPI / kScoreWaves;
    constexpr int KVAR = D == 128 ? 4 : 2;
    static_assert(IPW % KVAR == 0, "instruction and its index inside the wave agree mod KVAR");
    constexpr uint32_t kBuf = kAdCols * D * 2;
    constexpr int CPK = 64 / S;                  // compressed columns per KV block
    constexpr int KT = kAdCols / CPK;            // KV blocks per column tile
    static_assert(CPK >= 8, "a KV block's columns are whole runs of 4 in each lane half");
    __shared__ __attribute__((aligned(1024))) bf16_bits Kt[2][kAdCols * D];
    auto fk = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    // XCD-aware order as in the sampling kernel: row group fastest within a key range
    const int total = a.B * a.H * a.wg_per_head * a.nsplit;
    const int nper = (total + 7) >> 3;
    const int item = (blockIdx.x & 7) * nper + (blockIdx.x >> 3);
    if (item >= total) return;
    const int wg = item % a.wg_per_head;
    const int split = (item / a.wg_per_head) % a.nsplit;
    const int bh = item / (a.wg_per_head * a.nsplit);
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);

    const int r = wg * 128 + wave * 32 + l32;
    const bool row_in = r < a.rows_per_head;
    const bool row_ok = row_in && (r * S + S - 1) < a.Nv;
    float* Lh = a.L + static_cast<int64_t>(bh) * a.NKB * a.rows_per_head;

    const int ncols = a.N / S;
    const int ntiles = ncols / kAdCols;
    int tiles_needed = ntiles;
    if (a.causal) tiles_needed = min(ntiles, (min(wg * 128 + 127, a.rows_per_head - 1)) / kAdCols + 1);
    const int j_lo = split * a.tiles_per_split;
    const int j_hi = min(ntiles, j_lo + a.tiles_per_split);
    const int j_end = min(j_hi, tiles_needed);

    const bf16_bits* kbase = a.k + b * a.ks0 + hk * a.ks1;
    // the row's last token; chunk t reads S-1-t rows before it (rows without a valid token
    // read tokens 0..S-1, in bounds, and are masked)
    const bf16_bits* qrow = a.q + b * a.qs0 + h * a.qs1 + static_cast<int64_t>(row_ok ? r * S + S - 1 : S - 1) * a.qs2;
    const uint32_t kstride = static_cast<uint32_t>(a.ks2) * 2u;
    uint32_t lpk[KVAR];
    {
        const int rr = lane / CH;
        const int p = lane % CH;
#pragma unroll
        for (int q = 0; q < KVAR; ++q)
            lpk[q] = rr * (S * kstride) + static_cast<uint32_t>((p ^ fk(q * RPI + rr)) << 4);
    }
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)&Kt[0][0]));
    // step u = (tile j_lo + u / S, chunk t = u % S)
    auto issue = [&](int u, int buf) {
        const int j = j_lo + u / S;
        const int t = u % S;
        const char* tb = reinterpret_cast<const char*>(kbase) +
                         static_cast<uint32_t>(j * kAdCols * S + t) * kstride;
#pragma unroll
        for (int mi = 0; mi < IPW; ++mi) {
            const int m = wave * IPW + mi;
            dma16(tb + static_cast<uint32_t>(m * RPI * S) * kstride, lpk[mi % KVAR], lds0 + buf * kBuf + m * 1024);
        }
    };
    bf16x8 qf[KK], qn[KK];
    auto load_q = [&](int u, bf16x8 (&dst)[KK]) {
        const int t = u % S;
        const bf16_bits* qp = qrow - static_cast<int64_t>(t) * a.qs2;   // q[rS + S-1-t]
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) dst[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hi * 8);
    };
    uint32_t ka_base;
    {
        const int f = fk(l32);
        ka_base = lds0 + static_cast<uint32_t>(l32 * D * 2 + 16 * ((hi ^ f) & 1) + 16 * (f & ~1));
    }

    const int steps = (j_end - j_lo) * S;
    f32x16 sacc[4], cacc[4];
#pragma unroll
    for (int kh = 0; kh < 4; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kh][e] = 0.f;
    if (steps > 0) {
        issue(0, 0);
        load_q(0, qf);
    }
    int buf = 0;
    for (int u = 0; u < steps; ++u) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's K loads and Q chunk landed
        __syncthreads();                       // everyone's landed; buffer buf^1 free
        if (u + 1 < steps) {
            issue(u + 1, buf ^ 1);
            load_q(u + 1, qn);
        }
        const uint32_t kb0 = ka_base + (buf ? kBuf : 0u);
#pragma unroll
        for (int kh = 0; kh < 4; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) cacc[kh][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint32_t ad = kb0 ^ static_cast<uint32_t>(32 * kk);
#pragma unroll
            for (int kh = 0; kh < 4; ++kh) {
                const bf16x8 ka = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(ad + kh * 32 * D * 2);
                cacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], cacc[kh], 0, 0, 0);
            }
        }
#pragma unroll
        for (int kh = 0; kh < 4; ++kh) sacc[kh] += cacc[kh];
        if (u % S == S - 1) {
            // tile complete: lane value e of group kh is column 128 j + 32 kh + (e/4)*8 + 4 hi + e%4
            const int j = j_lo + u / S;
            const bool need_mask = !row_ok || ((j * kAdCols + kAdCols - 1) * S + S - 1 >= a.Nv) ||
                                   (a.causal && j * kAdCols + kAdCols - 1 > wg * 128);
            if (need_mask) {
                asm volatile("");   // keeps the branch (see the sampling kernel)
#pragma unroll
                for (int kh = 0; kh < 4; ++kh)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int cc = j * kAdCols + kh * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
                        if (!(row_ok && (cc * S + S - 1) < a.Nv && (!a.causal || cc <= r))) sacc[kh][e] = -INFINITY;
                    }
            }
            float Lk[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                constexpr int G8 = CPK / 8;
                float m = -INFINITY;
#pragma unroll
                for (int g = 0; g < G8; ++g) {
                    const int gg = kt * G8 + g;   // 8-column group of the tile: kh = gg / 4, e = (gg % 4) * 4 + i
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, sacc[gg >> 2][(gg & 3) * 4 + i]);
                }
                m = pair32_max(m);
                const float mc = m * a.c;
                float sum = 0.f;
                if (m != -INFINITY) {
#pragma unroll
                    for (int g = 0; g < G8; ++g) {
                        const int gg = kt * G8 + g;
#pragma unroll
                        for (int i = 0; i < 4; ++i) sum += fast_exp2(fmaf(sacc[gg >> 2][(gg & 3) * 4 + i], a.c, -mc));
                    }
                }
                sum = pair32_sum(sum);
                Lk[kt] = sum > 0.f ? mc + __builtin_amdgcn_logf(sum) : -INFINITY;
            }
            if (hi == 0 && row_in) {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) Lh[static_cast<int64_t>(j * KT + kt) * a.rows_per_head + r] = Lk[kt];
            }
#pragma unroll
            for (int kh = 0; kh < 4; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kh][e] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = qn[kk];
        buf ^= 1;
    }
    // tiles of this range past the causal frontier: no mass
    if (hi == 0 && row_in)
        for (int j = max(j_lo, j_end); j < j_hi; ++j)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) Lh[static_cast<int64_t>(j * KT + kt) * a.rows_per_head + r] = -INFINITY;
}

// ---------------------------------------------------------------------------------------
// Block-mean scoring: k_block_means writes the mean of each query block's valid rows and of
// each KV block's valid keys (float32); k_meankey_logmass scores 16 query blocks of one
// (batch, head) per workgroup against every KV block mean (float64 dots) and writes the
// log-masses z*log2(e) + log2(n) for the assignment (one scoring row per query block).
// ---------------------------------------------------------------------------------------
struct MeanArgs {
    const bf16_bits* q;
    const bf16_bits* k;
    float* qbar;   // [B*H][NQB][D]
    float* kbar;   // [B*Hkv][NKB][D]
    double* ksum;  // [B*Hkv][NKB][D] float64 sums of each KV block's valid keys (certification)
    int B, H, Hkv, N, Nv, D, BQ, BK, NQB, NKB;
    int64_t qs0, qs1, qs2, ks0, ks1, ks2;
};

__global__ void __launch_bounds__(256) k_block_means(MeanArgs a) {
    // 16-byte loads: thread t reads 8 columns (t % (D/8)) of rows t / (D/8), t / (D/8) + 256/(D/8), ..
    __shared__ float part[256 * 8];
    __shared__ double part64[256 * 8];
    const int64_t nq = static_cast<int64_t>(a.B) * a.H * a.NQB;
    const int64_t item = blockIdx.x;
    const bool is_q = item < nq;
    int b, h, blk, len;
    if (is_q) {
        blk = static_cast<int>(item % a.NQB);
        const int bh = static_cast<int>(item / a.NQB);
        h = bh % a.H;
        b = bh / a.H;
        len = a.BQ;
    } else {
        const int64_t it = item - nq;
        blk = static_cast<int>(it % a.NKB);
        const int bh = static_cast<int>(it / a.NKB);
        h = bh % a.Hkv;
        b = bh / a.Hkv;
        len = a.BK;
    }
    const int lo = blk * len;
    const int rows = min(max(a.Nv - lo, 0), len);
    const bf16_bits* src = is_q ? a.q + b * a.qs0 + h * a.qs1 + static_cast<int64_t>(lo) * a.qs2
                                : a.k + b * a.ks0 + h * a.ks1 + static_cast<int64_t>(lo) * a.ks2;
    const int64_t rs = is_q ? a.qs2 : a.ks2;
    const int cpr = a.D / 8;                 // 16-byte chunks per row
    const int phases = 256 / cpr;
    const int ch = threadIdx.x % cpr;
    const int ph = threadIdx.x / cpr;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // KV blocks: the certification's float64 key sums beside the float32 means (64 bf16 values
    // sum exactly in float64 unless their exponents span more than about 45 bits)
    double acc64[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int r = ph; r < rows; r += phases) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(r) * rs + ch * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += __uint_as_float(w[i] << 16);
            acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
            if (!is_q) {
                acc64[2 * i] += static_cast<double>(__uint_as_float(w[i] << 16));
                acc64[2 * i + 1] += static_cast<double>(__uint_as_float(w[i] & 0xffff0000u));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[threadIdx.x * 8 + i] = acc[i];
    if (!is_q) {
#pragma unroll
        for (int i = 0; i < 8; ++i) part64[threadIdx.x * 8 + i] = acc64[i];
    }
    __syncthreads();
    if (threadIdx.x < a.D) {
        const int e = threadIdx.x;
        float sum = 0.f;
        for (int p = 0; p < phases; ++p) sum += part[(p * cpr + e / 8) * 8 + e % 8];
        const float mean = rows > 0 ? sum / static_cast<float>(rows) : 0.f;
        float* dst = is_q ? a.qbar + item * a.D : a.kbar + (item - nq) * a.D;
        dst[e] = mean;
        if (!is_q) {
            double s64 = 0.0;
            for (int p = 0; p < phases; ++p) s64 += part64[(p * cpr + e / 8) * 8 + e % 8];
            a.ksum[(item - nq) * a.D + e] = s64;
        }
    }
}

struct MeanKeyArgs {
    const float* qbar;
    const float* kbar;
    float* L;        // [B*H][NKB][NQB]
    int H, Hkv, N, Nv, D, BQ, BK, NQB, NKB, causal;
    double c;        // scale * log2(e)
};

constexpr int kMeanRows = 16;   // query blocks per workgroup
constexpr int kMeanCols = 64;   // KV blocks per workgroup

__global__ void __launch_bounds__(256) k_meankey_logmass(MeanKeyArgs a) {
    // 16 query blocks x 64 KV blocks of one (batch, head): both sets of means staged in LDS,
    // thread t takes KV block t % 64 against query blocks t / 64 + 4 i (float64 dots)
    extern __shared__ float sm[];
    const int ksd = a.D + 1;                 // padded row: the 64 lanes read 64 rows at once
    float* qs = sm;                          // [kMeanRows][D]
    float* ks = sm + kMeanRows * a.D;        // [kMeanCols][D + 1]
    const int rchunks = (a.NQB + kMeanRows - 1) / kMeanRows;
    const int cchunks = (a.NKB + kMeanCols - 1) / kMeanCols;
    const int per_bh = rchunks * cchunks;
    const int bh = blockIdx.x / per_bh;
    const int qb0 = ((blockIdx.x % per_bh) / cchunks) * kMeanRows;
    const int kb0 = (blockIdx.x % cchunks) * kMeanCols;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);
    const int nr = min(kMeanRows, a.NQB - qb0);
    const int nc = min(kMeanCols, a.NKB - kb0);
    for (int i = threadIdx.x; i < nr * a.D; i += 256)
        qs[i] = a.qbar[(static_cast<int64_t>(bh) * a.NQB + qb0) * a.D + i];
    for (int i = threadIdx.x; i < nc * a.D; i += 256)
        ks[(i / a.D) * ksd + i % a.D] = a.kbar[(static_cast<int64_t>(b * a.Hkv + hk) * a.NKB + kb0) * a.D + i];
    __syncthreads();
    float* Lh = a.L + static_cast<int64_t>(bh) * a.NKB * a.NQB;
    const int c = threadIdx.x % kMeanCols;
    const int r0 = threadIdx.x / kMeanCols;   // 0..3
    if (c >= nc) return;
    const int kb = kb0 + c;
    const int nv = min(max(a.Nv - kb * a.BK, 0), a.BK);
    const float* kr = ks + c * ksd;
    for (int i = r0; i < nr; i += 256 / kMeanCols) {
        const float* qr = qs + i * a.D;
        double dot = 0.0;
        for (int e = 0; e < a.D; ++e) dot += static_cast<double>(kr[e]) * static_cast<double>(qr[e]);
        const int qb = qb0 + i;
        const int qlo = qb * a.BQ;
        const int last = a.causal ? min((qlo + a.BQ - 1) / a.BK, a.NKB - 1) : a.NKB - 1;
        float L = -INFINITY;
        if (qlo < a.Nv && nv > 0 && kb <= last) L = static_cast<float>(dot * a.c + log2(static_cast<double>(nv)));
        Lh[static_cast<int64_t>(kb) * a.NQB + qb] = L;
    }
}

// ---------------------------------------------------------------------------------------
// Intra-block key similarity, one wave per (batch, KV head, KV block).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
    k_block_sim(const bf16_bits* __restrict__ k, int64_t ks0, int64_t ks1, int64_t ks2, int Hkv,
                int NKB, int Nv, int64_t items, float* __restrict__ sim, double* __restrict__ sim64) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= items) return;
    const int kb = static_cast<int>(item % NKB);
    const int bh = static_cast<int>(item / NKB);
    const int h = bh % Hkv;
    const int b = bh / Hkv;
    const int lo = kb * 64;
    const int nv = min(max(Nv - lo, 0), 64);
    if (nv < 2) {
        if (lane == 0) {
            sim[item] = 1.f;
            if (sim64 != nullptr) sim64[item] = 1.0;
        }
        return;
    }
    // lane t owns key lo + t: its norm, then every lane accumulates head-dim slices of the
    // normalised sum. Keys >= nv contribute nothing.
    const bf16_bits* kp = k + b * ks0 + h * ks1;
    double nrm2 = 0.0;
    if (lane < nv) {
        const bf16_bits* row = kp + static_cast<int64_t>(lo + lane) * ks2;
        for (int e = 0; e < D; ++e) {
            const double x = bf16_to_f32(row[e]);
            nrm2 += x * x;
        }
    }
    const double inv = (lane < nv && nrm2 > 0.0) ? 1.0 / sqrt(nrm2) : 0.0;
    const double self = (lane < nv && nrm2 > 0.0) ? nrm2 * inv * inv : 0.0;
    const double self_sum = wave_sum_f64(self);
    // |sum_i khat_i|^2, head-dim element e handled by lane e % 64 over keys
    double sq = 0.0;
    for (int e = lane; e < D; e += 64) {
        double s = 0.0;
        for (int t = 0; t < nv; ++t) {
            const double it = __shfl(inv, t, 64);
            s += static_cast<double>(bf16_to_f32(kp[static_cast<int64_t>(lo + t) * ks2 + e])) * it;
        }
        sq += s * s;
    }
    sq = wave_sum_f64(sq);
    const double sv = (sq - self_sum) / (static_cast<double>(nv) * (nv - 1));
    if (lane == 0) {
        sim[item] = static_cast<float>(sv);
        if (sim64 != nullptr) sim64[item] = sv;
    }
}

// ---------------------------------------------------------------------------------------
// Threshold assignment, one workgroup per (batch, head, query block) row (psa_assign.h holds
// the per-row steps, shared with the attention kernel that scores block means in its prologue).
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(kAssignThreads) k_mask_assign(AssignArgs a) {
    // P sort keys, NKB masses, (log-mass path) NKB * RQ staged log-masses, NKB int8 levels
    extern __shared__ uint64_t keys[];
    float* Ms = reinterpret_cast<float*>(keys + a.P);
    float* Ls = Ms + a.NKB;
    int8_t* lvl = reinterpret_cast<int8_t*>(Ls + (a.L != nullptr ? a.NKB * a.RQ : 0));
    const int64_t row = blockIdx.x;
    const int qb = static_cast<int>(row % a.NQB);
    const int bh = static_cast<int>(row / a.NQB);
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int hk = h / (a.H / a.Hkv);
    const int tid = threadIdx.x;

    if (a.L != nullptr) {
        // The RQ rows of one block are contiguous in the workspace: the block's values are
        // staged in LDS (Ls[kb * RQ + i]) with independent loads, thread t taking row
        // i = t % RQ of blocks t / RQ + k * (256 / RQ).
        const int RQ = a.RQ;
        const int i = tid & (RQ - 1);
        const int kstep = kAssignThreads / RQ;
        const float* Lh = a.L + static_cast<int64_t>(bh) * a.NKB * a.rows_per_head + qb * RQ + i;
#pragma unroll 8
        for (int kb = tid / RQ; kb < a.NKB; kb += kstep)
            Ls[kb * RQ + i] = Lh[static_cast<int64_t>(kb) * a.rows_per_head];
        __syncthreads();
        assign_masses(a, qb, Ls, Ms, a.M_out + row * a.NKB, tid);
    } else {
        const float* Mrow = a.M + row * a.NKB;
        for (int kb = tid; kb < a.NKB; kb += kAssignThreads) Ms[kb] = Mrow[kb];
    }
    __shared__ int cflag;
    if (tid == 0) cflag = 0;
    __syncthreads();
    assign_levels(a, qb, b, hk, Ms, keys, lvl, tid, a.cert != nullptr ? &cflag : nullptr);
    int8_t* out = a.map + row * a.NKB;
    for (int kb = tid; kb < a.NKB; kb += kAssignThreads) out[kb] = lvl[kb];
    if (a.cert != nullptr && tid == 0 && cflag) {
        const int slot = atomicAdd(&a.cert[0], 1);
        if (slot < a.cert_cap)
            a.cert_rows[slot] = static_cast<int>(row);
        else
            atomicAdd(&a.cert[1], 1);
    }
}

// ---------------------------------------------------------------------------------------
// Certification: float64 rescoring of the rows the float32 assignment flagged (a decision
// within the mode's margin of a threshold, or a tie within it across a level change). Each
// rescoring kernel walks (flagged row, column chunk) items over a fixed grid and writes, per
// scoring row i of the query block and KV block kb, the natural log of the row's
// unnormalised softmax mass on the block in float64 (logits are float64 dots of the bf16
// inputs). k_cert_assign then forms the block masses in float64 (each scoring row normalised
// by its logsumexp, averaged over the valid rows), runs the float64 assignment and overwrites
// the row's levels and masses. Rows beyond the capacity keep the float32 decisions and are
// counted in cert[1].
// ---------------------------------------------------------------------------------------
struct CertArgs {
    const bf16_bits* q;
    const bf16_bits* k;
    int H, Hkv, N, Nv, BQ, NQB, NKB, causal;
    int S;        // samples per query block (sampling) or stride (antidiagonal)
    int RQ;       // scoring rows per query block
    int64_t qs0, qs1, qs2, ks0, ks1, ks2;
    double scale; // 1 / sqrt(d)
    const int* cert;
    const int* rows;
    double* Lg;   // [cap][RQ][NKB]
    const double* ksum;   // block-mean mode: float64 key sums per KV block [B*Hkv][NKB][D]
    int cap;
    int nchunks;  // column chunks per row
};

// log of sum_t exp(z_t) over the lanes of a group of G consecutive lanes (a power of two
// <= 64); -inf when every z is -inf. Every lane of the group gets the value.
template <int G>
__device__ __forceinline__ double group_logsumexp(double z) {
    double m = z;
#pragma unroll
    for (int o = 1; o < G; o <<= 1) m = fmax(m, __shfl_xor(m, o, 64));
    double e = m == -INFINITY ? 0.0 : exp(z - m);
#pragma unroll
    for (int o = 1; o < G; o <<= 1) e += __shfl_xor(e, o, 64);
    return m == -INFINITY ? -INFINITY : m + log(e);
}

struct RowIds {
    int qb, h, b, hk;
};

__device__ __forceinline__ RowIds row_ids(int row, int NQB, int H, int Hkv) {
    RowIds r;
    r.qb = row % NQB;
    const int bh = row / NQB;
    r.h = bh % H;
    r.b = bh / H;
    r.hk = r.h / (H / Hkv);
    return r;
}

// Sampling mode: items (flagged row, chunk of 256 * KPT keys); thread = KPT keys (256 apart),
// every sampled row of the query block against each (float64 dots over d); the sampled rows sit
// in LDS as float64, [e][s], read two at a time. For key group j one wave covers one KV block.
template <int D, int S>
__global__ void __launch_bounds__(256) k_cert_sampling(CertArgs a) {
    constexpr int KPT = S <= 8 ? 4 : (S == 16 ? 2 : 1);   // keys per thread (KPT * S <= 32 sums)
    constexpr int SP = S < 2 ? 2 : S;                      // LDS row of one e: even length
    __shared__ __attribute__((aligned(16))) double qs[D * SP];
    const int tid = threadIdx.x;
    const int nrows = min(a.cert[0], a.cap);
    const int64_t items = static_cast<int64_t>(nrows) * a.nchunks;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int slot = static_cast<int>(it / a.nchunks);
        const int chunk = static_cast<int>(it % a.nchunks);
        const RowIds r = row_ids(a.rows[slot], a.NQB, a.H, a.Hkv);
        const int rv = min(max(a.Nv - r.qb * a.BQ, 0), a.BQ);
        __syncthreads();   // the previous item's reads of qs are done
        const bf16_bits* qh = a.q + r.b * a.qs0 + r.h * a.qs1;
        for (int i = tid; i < D * SP; i += 256) {
            const int e = i / SP, si = i % SP;
            const int qrow = r.qb * a.BQ + (si * rv) / S;
            qs[i] = (rv > 0 && si < S) ? static_cast<double>(bf16_to_f32(qh[static_cast<int64_t>(qrow) * a.qs2 + e])) : 0.0;
        }
        __syncthreads();
        const int t0 = chunk * 256 * KPT + tid;
        double acc[KPT][S];
#pragma unroll
        for (int j = 0; j < KPT; ++j)
#pragma unroll
            for (int si = 0; si < S; ++si) acc[j][si] = 0.0;
        const bf16_bits* kh = a.k + r.b * a.ks0 + r.hk * a.ks1;
        if (rv > 0 && t0 < a.Nv) {
            for (int e0 = 0; e0 < D; e0 += 8) {
                double kv[KPT][8];
#pragma unroll
                for (int j = 0; j < KPT; ++j) {
                    const int t = t0 + 256 * j;
                    u32x4 w = u32x4{0u, 0u, 0u, 0u};
                    if (t < a.Nv) w = *reinterpret_cast<const u32x4*>(kh + static_cast<int64_t>(t) * a.ks2 + e0);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        kv[j][2 * x] = static_cast<double>(__uint_as_float(w[x] << 16));
                        kv[j][2 * x + 1] = static_cast<double>(__uint_as_float(w[x] & 0xffff0000u));
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double* qe = &qs[(e0 + e) * SP];
#pragma unroll
                    for (int si = 0; si < S; si += 2) {
                        const double2 q2 = *reinterpret_cast<const double2*>(qe + si);
#pragma unroll
                        for (int j = 0; j < KPT; ++j) {
                            acc[j][si] = fma(q2.x, kv[j][e], acc[j][si]);
                            if (si + 1 < S) acc[j][si + 1] = fma(q2.y, kv[j][e], acc[j][si + 1]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int t = t0 + 256 * j;
            const int kb = t >> 6;
#pragma unroll
            for (int si = 0; si < S; ++si) {
                const int qrow = r.qb * a.BQ + (si * rv) / S;
                const bool vis = rv > 0 && t < a.Nv && (!a.causal || t <= qrow);
                const double L = group_logsumexp<64>(vis ? acc[j][si] * a.scale : -INFINITY);
                if ((tid & 63) == 0 && kb < a.NKB)
                    a.Lg[(static_cast<int64_t>(slot) * a.RQ + si) * a.NKB + kb] = L;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Sampling mode on float64 MFMA (v_mfma_f64_16x16x4_f64): the flagged rows are first grouped
// by KV head into batches of 16 / S rows (k_cert_batches), so that the 16 MFMA rows hold the
// S sampled queries of every row of a batch and one K read serves them all. Operand layouts
// of the instruction (16x16x4, one double per lane): A[i][k] in lane i + 16k, B[k][j] in lane
// j + 16k; the result D[4r + (l >> 4)][l & 15] in lane l, register r. The contraction index
// k of k-step ks maps to head dimension (D / 4) * k + ks, so a lane's operands are D / 4
// consecutive dimensions of one query (A) or one key (B).
// ---------------------------------------------------------------------------------------
constexpr int kBatchThreads = 1024;
constexpr int kBatchSortMax = 16384;   // flagged rows sorted in LDS; beyond, one row per batch

struct BatchArgs {
    int* cert;         // cert[0] flagged rows, cert[2] <- batches
    const int* rows;   // [cap] the flagged rows, in the order they were flagged
    int* bat;          // [cap][16] slots of each batch (-1: none)
    int cap, unit, BR; // unit: rows per KV head (NQB * heads_q / heads_kv); BR: rows per batch
};

// exclusive sum over the workgroup of one value per thread (kBatchThreads threads)
__device__ int batch_exclusive_sum(int v, int* wsum) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    __syncthreads();
    return before + x - v;
}

__global__ void __launch_bounds__(kBatchThreads) k_cert_batches(BatchArgs b) {
    extern __shared__ uint64_t skeys[];   // (KV head << 32) | slot, sorted
    __shared__ int wsum[kBatchThreads / 64];
    const int tid = threadIdx.x;
    const int n = min(b.cert[0], b.cap);
    if (n > kBatchSortMax) {   // (uniform) no grouping: one row per batch
        for (int i = tid; i < n; i += kBatchThreads)
            for (int j = 0; j < 16; ++j) b.bat[i * 16 + j] = j == 0 ? i : -1;
        if (tid == 0) b.cert[2] = n;
        return;
    }
    int P = 1;
    while (P < n) P <<= 1;
    for (int i = tid; i < P; i += kBatchThreads)
        skeys[i] = i < n ? (static_cast<uint64_t>(b.rows[i] / b.unit) << 32) | static_cast<uint32_t>(i) : ~0ull;
    __syncthreads();
    // bitonic sort, ascending
    for (int size = 2; size <= P; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P; i += kBatchThreads) {
                const int jx = i ^ stride;
                if (jx > i) {
                    const bool up = (i & size) == 0;
                    const uint64_t x = skeys[i], y = skeys[jx];
                    if ((x > y) == up) {
                        skeys[i] = y;
                        skeys[jx] = x;
                    }
                }
            }
            __syncthreads();
        }
    // batch heads: every BR-th position of each KV head's run (the run's start by binary search);
    // thread t takes the positions [t per, (t + 1) per), per = ceil(n / threads) <= 16
    const int per = (n + kBatchThreads - 1) / kBatchThreads;
    uint32_t heads = 0;   // bit e: position t per + e starts a batch
    int cnt = 0;
    for (int e = 0; e < per; ++e) {
        const int p = tid * per + e;
        if (p < n) {
            const uint32_t key = static_cast<uint32_t>(skeys[p] >> 32);
            int lo = 0, hi = p;   // first position with this key
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (static_cast<uint32_t>(skeys[mid] >> 32) < key) lo = mid + 1; else hi = mid;
            }
            if ((p - lo) % b.BR == 0) {
                heads |= 1u << e;
                ++cnt;
            }
        }
    }
    int bidx = batch_exclusive_sum(cnt, wsum);
    for (int e = 0; e < per; ++e) {
        if ((heads >> e) & 1u) {
            const int p = tid * per + e;
            const uint32_t key = static_cast<uint32_t>(skeys[p] >> 32);
            for (int j = 0; j < 16; ++j) {
                const int q = p + j;
                const bool in = j < b.BR && q < n && static_cast<uint32_t>(skeys[q] >> 32) == key;
                b.bat[bidx * 16 + j] = in ? static_cast<int>(skeys[q] & 0xffffffffu) : -1;
            }
            ++bidx;
        }
    }
    if (tid == kBatchThreads - 1) b.cert[2] = bidx;   // the last thread ends past every head
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// items (batch, 4 KV blocks); wave w of the workgroup takes KV block 4 * (item % ceil(NKB/4)) + w:
// 4 column tiles of 16 keys, D / 4 k-steps each, then per sampled query the block's log-mass.
template <int D, int S>
__global__ void __launch_bounds__(256) k_cert_sampling_mfma(CertArgs a, const int* bat) {
    constexpr int BR = 16 / S;
    constexpr int KST = D / 4;   // k-steps; a lane's D / 4 consecutive dimensions
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int nb = a.cert[2];
    const int nkb4 = (a.NKB + 3) / 4;
    const int64_t items = static_cast<int64_t>(nb) * nkb4;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int batch = static_cast<int>(it / nkb4);
        const int kb = static_cast<int>(it % nkb4) * 4 + wave;
        if (kb >= a.NKB) continue;   // wave-uniform
        const int* bs = bat + static_cast<int64_t>(batch) * 16;
        const RowIds r0 = row_ids(a.rows[bs[0]], a.NQB, a.H, a.Hkv);   // the batch's KV head
        // A operand: sampled query j (batch row j / S, sample j % S), dimensions g*KST ...
        double av[KST];
        {
            const int slot = bs[j / S];
            const int si = j % S;
            bool ok = slot >= 0 && j / S < BR;
            int qrow = 0;
            const bf16_bits* qh = a.q;
            if (ok) {
                const RowIds r = row_ids(a.rows[slot], a.NQB, a.H, a.Hkv);
                const int rv = min(max(a.Nv - r.qb * a.BQ, 0), a.BQ);
                ok = rv > 0;
                qrow = r.qb * a.BQ + (si * rv) / S;
                qh = a.q + r.b * a.qs0 + r.h * a.qs1 + static_cast<int64_t>(qrow) * a.qs2 + g * KST;
            }
#pragma unroll
            for (int c = 0; c < KST / 8; ++c) {
                u32x4 w = u32x4{0u, 0u, 0u, 0u};
                if (ok) w = *reinterpret_cast<const u32x4*>(qh + 8 * c);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    av[8 * c + 2 * x] = static_cast<double>(__uint_as_float(w[x] << 16));
                    av[8 * c + 2 * x + 1] = static_cast<double>(__uint_as_float(w[x] & 0xffff0000u));
                }
            }
        }
        // the sampled queries of this lane's results: m = 4 rr + g
        int mslot[4], msi[4], mqrow[4];
        bool mok[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = 4 * rr + g;
            mslot[rr] = bs[m / S];
            msi[rr] = m % S;
            mok[rr] = false;
            mqrow[rr] = 0;
            if (mslot[rr] >= 0) {
                const RowIds r = row_ids(a.rows[mslot[rr]], a.NQB, a.H, a.Hkv);
                const int rv = min(max(a.Nv - r.qb * a.BQ, 0), a.BQ);
                mok[rr] = rv > 0;
                mqrow[rr] = r.qb * a.BQ + (msi[rr] * rv) / S;
            }
        }
        const bf16_bits* kh = a.k + r0.b * a.ks0 + r0.hk * a.ks1 + g * KST;
        double mx[4], zt[4][4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mx[rr] = -INFINITY;
#pragma unroll
        for (int tile = 0; tile < 4; ++tile) {
            const int t = kb * 64 + tile * 16 + j;   // this lane's key (B operand and results)
            u32x4 kw[KST / 8];
#pragma unroll
            for (int c = 0; c < KST / 8; ++c) {
                kw[c] = u32x4{0u, 0u, 0u, 0u};
                if (t < a.Nv) kw[c] = *reinterpret_cast<const u32x4*>(kh + static_cast<int64_t>(t) * a.ks2 + 8 * c);
            }
            f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int ks = 0; ks < KST; ++ks) {
                const uint32_t w = kw[ks / 8][(ks % 8) / 2];
                const double bv = static_cast<double>(__uint_as_float((ks & 1) ? (w & 0xffff0000u) : (w << 16)));
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ks], bv, acc, 0, 0, 0);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const bool vis = mok[rr] && t < a.Nv && (!a.causal || t <= mqrow[rr]);
                zt[rr][tile] = vis ? acc[rr] * a.scale : -INFINITY;
                mx[rr] = fmax(mx[rr], zt[rr][tile]);
            }
        }
        // each sampled query's log-mass on the block: logsumexp over 4 tiles x 16 lanes
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            double m = mx[rr];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmax(m, __shfl_xor(m, o, 64));
            double e = 0.0;
            if (m != -INFINITY)
#pragma unroll
                for (int tile = 0; tile < 4; ++tile) e += exp(zt[rr][tile] - m);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) e += __shfl_xor(e, o, 64);
            const double L = m == -INFINITY ? -INFINITY : m + log(e);
            if (j == 0 && mslot[rr] >= 0)
                a.Lg[(static_cast<int64_t>(mslot[rr]) * a.RQ + msi[rr]) * a.NKB + kb] = L;
        }
    }
}

// Antidiagonal mode on float64 MFMA, RQ = 16 compressed rows per query block (the 16 MFMA
// rows): items (256 compressed columns, flagged row), column-chunk major; wave w takes columns
// 64 w .. 64 w + 63 of the item as 4 column tiles of 16. The contraction runs over kdim = t * D + d (t < S, d < D):
// A[i][kdim] = q[(qb * RQ + i) * S + S - 1 - t][d], B[kdim][c] = k[c * S + t][d]; lane group
// g = lane / 16 holds kdims g * (S * D / 4) + ks, streamed in chunks of 32 (64 bytes of one
// query row and one key row per lane). Column tiles that lie wholly past the block's last
// compressed row (causal) or past the valid keys are skipped.
template <int D, int S>
__global__ void __launch_bounds__(256, 2) k_cert_antidiag_mfma(CertArgs a) {
    constexpr int RQ = 16;
    constexpr int G = 64 / S;            // compressed columns per KV block
    constexpr int KSP = S * D / 4;       // k-steps; lane group g holds kdims g * KSP + ks
    constexpr int CH = 16;               // k-steps per chunk (32 bytes of one row)
    static_assert(KSP % (2 * CH) == 0 && D % CH == 0, "chunks inside one row, in pairs");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int ncols = a.N / S;
    const int nrows = min(a.cert[0], a.cap);
    const int nchunk = (ncols + 255) / 256;
    const int64_t items = static_cast<int64_t>(nrows) * nchunk;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        // column-chunk major: the workgroups in flight share one chunk's keys in L2
        const int slot = static_cast<int>(it % nrows);
        const int c0 = static_cast<int>(it / nrows) * 256 + wave * 64;
        const RowIds r = row_ids(a.rows[slot], a.NQB, a.H, a.Hkv);
        const int rlast = r.qb * RQ + RQ - 1;   // last compressed row of the query block
        // the wave's column tiles that hold a visible column at all (wave-uniform); the others
        // are not computed, and their log-masses are written as -inf below like any invisible one
        const int cvis_end = min(ncols, (a.causal ? rlast + 1 : ncols));
        const int ntiles = (c0 >= cvis_end || c0 * S >= a.Nv) ? 0 : min(4, (cvis_end - c0 + 15) / 16);
        const bf16_bits* qh = a.q + r.b * a.qs0 + r.h * a.qs1;
        const bf16_bits* kh = a.k + r.b * a.ks0 + r.hk * a.ks1;
        f64x4 acc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[nt] = f64x4{0.0, 0.0, 0.0, 0.0};
        // a chunk's operands: A = 32 bytes of one query row, B = 32 bytes of one key row per
        // live tile (a column past the last is clamped to it; its results are not used); the
        // next chunk's loads are issued before the current chunk's MFMAs
        auto load = [&](int kc, u32x4 (&qa)[CH / 8], u32x4 (&kb)[4][CH / 8]) {
            const int kd = g * KSP + kc;   // first kdim of the chunk
            const int t = kd / D;
            const int d0 = kd % D;
            const int qrow = (r.qb * RQ + j) * S + S - 1 - t;
#pragma unroll
            for (int x = 0; x < CH / 8; ++x)
                qa[x] = *reinterpret_cast<const u32x4*>(qh + static_cast<int64_t>(qrow) * a.qs2 + d0 + 8 * x);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                if (nt >= ntiles) break;   // wave-uniform
                const int c = min(c0 + nt * 16 + j, ncols - 1);
#pragma unroll
                for (int x = 0; x < CH / 8; ++x)
                    kb[nt][x] = *reinterpret_cast<const u32x4*>(kh + static_cast<int64_t>(c * S + t) * a.ks2 + d0 + 8 * x);
            }
        };
        auto mul = [&](const u32x4 (&qa)[CH / 8], const u32x4 (&kb)[4][CH / 8]) {
            double av[CH];   // converted once, used by every tile
#pragma unroll
            for (int ks = 0; ks < CH; ++ks) {
                const uint32_t wa = qa[ks / 8][(ks % 8) / 2];
                av[ks] = static_cast<double>(__uint_as_float((ks & 1) ? (wa & 0xffff0000u) : (wa << 16)));
            }
            auto bval = [&](int nt, int ks) {
                const uint32_t wb = kb[nt][ks / 8][(ks % 8) / 2];
                return static_cast<double>(__uint_as_float((ks & 1) ? (wb & 0xffff0000u) : (wb << 16)));
            };
            if (ntiles == 4) {
                // the four tiles' accumulation chains interleaved: consecutive MFMAs are
                // independent
#pragma unroll
                for (int ks = 0; ks < CH; ++ks) {
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ks], bval(nt, ks), acc[nt], 0, 0, 0);
                    // (keeps each conversion next to its MFMA: hoisted, they exhaust the VGPRs)
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (nt >= ntiles) break;   // wave-uniform
#pragma unroll
                    for (int ks = 0; ks < CH; ++ks) {
                        acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ks], bval(nt, ks), acc[nt], 0, 0, 0);
                        if (ks % 4 == 3) __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        };
        if (ntiles > 0) {
            u32x4 qa0[CH / 8], qa1[CH / 8], kb0[4][CH / 8], kb1[4][CH / 8];
            load(0, qa0, kb0);
            for (int kc = 0; kc < KSP; kc += 2 * CH) {
                load(kc + CH, qa1, kb1);
                mul(qa0, kb0);
                if (kc + 2 * CH < KSP) load(kc + 2 * CH, qa0, kb0);
                mul(qa1, kb1);
            }
        }
        // results: D[4 rr + g][j] of tile nt = compressed row 4 rr + g, column c0 + 16 nt + j;
        // each KV block is G = 8 consecutive columns, i.e. 8 lanes of one tile
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int c = c0 + nt * 16 + j;
            const bool col_ok = c < ncols && c * S + S - 1 < a.Nv;
            const int kb = c / G;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = 4 * rr + g;
                const int rg = r.qb * RQ + i;
                const bool row_ok = rg * S + S - 1 < a.Nv;
                const bool vis = nt < ntiles && col_ok && row_ok && (!a.causal || c <= rg);
                const double z = vis ? acc[nt][rr] * a.scale : -INFINITY;
                double m = z;
#pragma unroll
                for (int o = 1; o < G; o <<= 1) m = fmax(m, __shfl_xor(m, o, 64));
                double e = m == -INFINITY ? 0.0 : exp(z - m);
#pragma unroll
                for (int o = 1; o < G; o <<= 1) e += __shfl_xor(e, o, 64);
                const double L = m == -INFINITY ? -INFINITY : m + log(e);
                if ((j % G) == 0 && c < ncols)
                    a.Lg[(static_cast<int64_t>(slot) * RQ + i) * a.NKB + kb] = L;
            }
        }
    }
}

// Antidiagonal mode, stride S: items (flagged row, chunk of 512 compressed columns); thread =
// columns c and c + 256, every compressed row i < RQ of the query block against each: the
// float64 sum over t < S of q[(qb*RQ + i)*S + S-1-t] . k[c*S + t]. The query block's rows sit
// in LDS as float32 (exact for bf16 values), [t][e][i], read four at a time. A KV block is
// 64/S consecutive columns.
template <int D, int S, int RQ>
__global__ void __launch_bounds__(256) k_cert_antidiag(CertArgs a) {
    constexpr int G = 64 / S;                 // columns per KV block
    constexpr int CPT = 2;                    // columns per thread
    __shared__ __attribute__((aligned(16))) float qs[S * D * RQ];   // qs[(t*D + e)*RQ + i]
    const int tid = threadIdx.x;
    const int ncols = a.N / S;
    const int nrows = min(a.cert[0], a.cap);
    const int64_t items = static_cast<int64_t>(nrows) * a.nchunks;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int slot = static_cast<int>(it / a.nchunks);
        const int chunk = static_cast<int>(it % a.nchunks);
        const RowIds r = row_ids(a.rows[slot], a.NQB, a.H, a.Hkv);
        __syncthreads();
        const bf16_bits* qh = a.q + r.b * a.qs0 + r.h * a.qs1;
        for (int x = tid; x < S * D * RQ; x += 256) {
            const int i = x % RQ, te = x / RQ, e = te % D, t = te / D;
            qs[x] = bf16_to_f32(qh[static_cast<int64_t>(r.qb * a.BQ + i * S + S - 1 - t) * a.qs2 + e]);
        }
        __syncthreads();
        const int c0 = chunk * 256 * CPT + tid;
        const int rlast = r.qb * RQ + RQ - 1;   // last compressed row of the query block
        double acc[CPT][RQ];
#pragma unroll
        for (int j = 0; j < CPT; ++j)
#pragma unroll
            for (int i = 0; i < RQ; ++i) acc[j][i] = 0.0;
        bool any = false;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = c0 + 256 * j;
            any = any || (c < ncols && c * S + S - 1 < a.Nv && (!a.causal || c <= rlast));
        }
        if (any) {
            const bf16_bits* kh = a.k + r.b * a.ks0 + r.hk * a.ks1;
            for (int t = 0; t < S; ++t) {
                for (int e0 = 0; e0 < D; e0 += 8) {
                    double kv[CPT][8];
#pragma unroll
                    for (int j = 0; j < CPT; ++j) {
                        const int c = c0 + 256 * j;
                        u32x4 w = u32x4{0u, 0u, 0u, 0u};
                        if (c < ncols) w = *reinterpret_cast<const u32x4*>(kh + static_cast<int64_t>(c * S + t) * a.ks2 + e0);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            kv[j][2 * x] = static_cast<double>(__uint_as_float(w[x] << 16));
                            kv[j][2 * x + 1] = static_cast<double>(__uint_as_float(w[x] & 0xffff0000u));
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float* qe = &qs[(t * D + e0 + e) * RQ];
#pragma unroll
                        for (int i = 0; i < RQ; i += 4) {
                            const f32x4 q4 = *reinterpret_cast<const f32x4*>(qe + i);
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const double qd = static_cast<double>(q4[u]);
#pragma unroll
                                for (int j = 0; j < CPT; ++j) acc[j][i + u] = fma(qd, kv[j][e], acc[j][i + u]);
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = c0 + 256 * j;
            const bool col_ok = c < ncols && c * S + S - 1 < a.Nv;
            const int kb = c / G;
#pragma unroll
            for (int i = 0; i < RQ; ++i) {
                const int rg = r.qb * RQ + i;
                const bool row_ok = rg * S + S - 1 < a.Nv;
                const bool vis = col_ok && row_ok && (!a.causal || c <= rg);
                const double L = group_logsumexp<G>(vis ? acc[j][i] * a.scale : -INFINITY);
                if ((tid % G) == 0 && c < ncols)
                    a.Lg[(static_cast<int64_t>(slot) * RQ + i) * a.NKB + kb] = L;
            }
        }
    }
}

// Block-mean mode: one workgroup per flagged row: q_bar and each KV block's log-mass in
// float64 (the same functions as the fused prologue).
template <int D>
__global__ void __launch_bounds__(256) k_cert_meankey(CertArgs a) {
    __shared__ double qbar[D];
    const int tid = threadIdx.x;
    const int nrows = min(a.cert[0], a.cap);
    for (int slot = blockIdx.x; slot < nrows; slot += gridDim.x) {
        const RowIds r = row_ids(a.rows[slot], a.NQB, a.H, a.Hkv);
        __syncthreads();
        cert_qbar_f64(a.q + r.b * a.qs0 + r.h * a.qs1, a.qs2, r.qb, a.BQ, a.Nv, D, qbar, tid);
        __syncthreads();
        const bool anyq = r.qb * a.BQ < a.Nv;
        const int last = a.causal ? min((r.qb * a.BQ + a.BQ - 1) / 64, a.NKB - 1) : a.NKB - 1;
        const double* ks = a.ksum + static_cast<int64_t>(r.b * a.Hkv + r.hk) * a.NKB * D;
        for (int kb = tid; kb < a.NKB; kb += 256)
            a.Lg[static_cast<int64_t>(slot) * a.NKB + kb] =
                cert_meankey_logmass(ks, qbar, D, kb, a.Nv, anyq && kb <= last, a.scale);
    }
}

// One workgroup per flagged row: the float64 masses from Lg, the float64 assignment, then the
// row's levels and masses (as float) overwrite the float32 ones.
__global__ void __launch_bounds__(kAssignThreads) k_cert_assign(AssignArgs a, CertArgs c) {
    extern __shared__ uint64_t ckeys[];               // a.P
    uint16_t* idx = reinterpret_cast<uint16_t*>(ckeys + a.P);   // a.P
    int8_t* lvl = reinterpret_cast<int8_t*>(idx + a.P);         // NKB
    __shared__ double lse[32];
    __shared__ double wm[kAssignThreads / 64][32], wsum[kAssignThreads / 64][32];
    const int tid = threadIdx.x;
    const int nrows = min(c.cert[0], c.cap);
    for (int slot = blockIdx.x; slot < nrows; slot += gridDim.x) {
        const int row = c.rows[slot];
        const RowIds r = row_ids(row, a.NQB, a.H, a.Hkv);
        const double* L = c.Lg + static_cast<int64_t>(slot) * a.RQ * a.NKB;
        __syncthreads();
        cert_lse(L, a.RQ, a.NKB, lse, wm, wsum, tid);
        const int den = cert_den(a, r.qb);
        const int last = a.causal ? min((r.qb * a.BQ + a.BQ - 1) / a.BK, a.NKB - 1) : a.NKB - 1;
        for (int kb = tid; kb < a.NKB; kb += kAssignThreads) {
            const double mass = cert_mass(L, lse, a.RQ, a.NKB, kb, den);
            if (a.M_out != nullptr) a.M_out[static_cast<int64_t>(row) * a.NKB + kb] = static_cast<float>(mass);
            if (kb <= last) {
                ckeys[kb] = ~double_order(mass);
                idx[kb] = static_cast<uint16_t>(kb);
            }
        }
        __syncthreads();
        assign_levels_f64(a, r.qb, r.b, r.hk, ckeys, idx, lvl, tid);
        int8_t* out = a.map + static_cast<int64_t>(row) * a.NKB;
        for (int kb = tid; kb < a.NKB; kb += kAssignThreads) out[kb] = lvl[kb];
    }
}

template <int MODE, int S>
hipError_t launch_scores_d(const ScoreArgs& a, int D, int blocks, hipStream_t st) {
    if (D == 128)
        hipLaunchKernelGGL((k_mask_logmass<MODE, 128, S>), dim3(blocks), dim3(kScoreThreads), 0, st, a);
    else
        hipLaunchKernelGGL((k_mask_logmass<MODE, 64, S>), dim3(blocks), dim3(kScoreThreads), 0, st, a);
    return hipGetLastError();
}

template <int S>
hipError_t launch_sampling(const ScoreArgs& a, int D, int blocks, hipStream_t st) {
    if (D == 128)
        hipLaunchKernelGGL((k_mask_logmass_sampling<128, S>), dim3(blocks), dim3(kScoreThreads), 0, st, a);
    else
        hipLaunchKernelGGL((k_mask_logmass_sampling<64, S>), dim3(blocks), dim3(kScoreThreads), 0, st, a);
    return hipGetLastError();
}

// The antidiagonal fast path needs whole 128-column tiles of compressed columns.
bool antidiag_fast(const Shape& s, int S) { return (s.N / S) % kAdCols == 0 && 64 / S >= 8; }

template <int S>
hipError_t launch_antidiag(const ScoreArgs& a, int D, int blocks, hipStream_t st) {
    if (D == 128)
        hipLaunchKernelGGL((k_mask_logmass_antidiag<128, S>), dim3(blocks), dim3(kScoreThreads), 0, st, a);
    else
        hipLaunchKernelGGL((k_mask_logmass_antidiag<64, S>), dim3(blocks), dim3(kScoreThreads), 0, st, a);
    return hipGetLastError();
}

// Row groups, key-tile ranges and the log-mass workspace for a problem.
struct ScoreGeom {
    int S, rows_per_head, RQ, rows_per_wg, wg_per_head, ntiles, nsplit, tiles_per_split;
    size_t ws_bytes;
    size_t qbar_off = 0, kbar_off = 0, ksum_off = 0;   // block-mean mode: means, float64 key sums
    // certification: counters, flagged row list, batches (16 slots each), float64
    // similarities, float64 log-masses
    size_t cert_off = 0, rows_off = 0, bat_off = 0, sim64_off = 0, lg_off = 0;
    int cap = 0;
};

// Float64 log-masses of the flagged rows take at most this much workspace; the rows that fit
// (at least 16, at most all) are the certification capacity.
constexpr size_t kCertLgBytes = size_t(64) << 20;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

ScoreGeom score_geom_base(const Shape& s, const psa_mask_params& mp);

ScoreGeom score_geom(const Shape& s, const psa_mask_params& mp) {
    ScoreGeom g = score_geom_base(s, mp);
    const int64_t R = static_cast<int64_t>(s.B) * s.H * s.NQB;
    const size_t per_row = static_cast<size_t>(g.RQ) * s.NKB * sizeof(double);
    const int64_t fit = per_row > 0 ? static_cast<int64_t>(kCertLgBytes / per_row) : R;
    g.cap = static_cast<int>(std::min<int64_t>(R, std::max<int64_t>(16, fit)));
    size_t off = align256(g.ws_bytes);
    g.cert_off = off;
    off += 256;
    g.rows_off = off;
    off = align256(off + static_cast<size_t>(g.cap) * sizeof(int));
    g.bat_off = off;
    off = align256(off + static_cast<size_t>(g.cap) * 16 * sizeof(int));
    g.sim64_off = off;
    if (mp.cos_sim_min > 0.f) off = align256(off + static_cast<size_t>(s.B) * s.Hkv * s.NKB * sizeof(double));
    g.lg_off = off;
    off += static_cast<size_t>(g.cap) * per_row;
    g.ws_bytes = off;
    return g;
}

ScoreGeom score_geom_base(const Shape& s, const psa_mask_params& mp) {
    ScoreGeom g;
    if (mp.mode == PSA_MASK_MEANKEY) {
        // one scoring row per query block; workspace: log-masses, query and key block means
        g.S = 1;
        g.rows_per_head = s.NQB;
        g.RQ = 1;
        g.rows_per_wg = kMeanRows;
        g.wg_per_head = (s.NQB + kMeanRows - 1) / kMeanRows;
        g.ntiles = 0;
        g.nsplit = 1;
        g.tiles_per_split = 0;
        g.ws_bytes = static_cast<size_t>(s.B) * s.H * s.NKB * s.NQB * sizeof(float);
        g.ws_bytes = (g.ws_bytes + 255) & ~static_cast<size_t>(255);
        g.qbar_off = g.ws_bytes;
        g.ws_bytes += static_cast<size_t>(s.B) * s.H * s.NQB * s.D * sizeof(float);
        g.ws_bytes = (g.ws_bytes + 255) & ~static_cast<size_t>(255);
        g.kbar_off = g.ws_bytes;
        g.ws_bytes += static_cast<size_t>(s.B) * s.Hkv * s.NKB * s.D * sizeof(float);
        g.ws_bytes = (g.ws_bytes + 255) & ~static_cast<size_t>(255);
        g.ksum_off = g.ws_bytes;
        g.ws_bytes += static_cast<size_t>(s.B) * s.Hkv * s.NKB * s.D * sizeof(double);
        return g;
    }
    const bool sampling = mp.mode == PSA_MASK_SAMPLING;
    g.S = sampling ? mp.samples_per_qblock : mp.antidiag_stride;
    g.rows_per_head = sampling ? s.NQB * g.S : s.N / g.S;
    g.RQ = sampling ? g.S : s.BQ / g.S;
    g.rows_per_wg = sampling ? kSampRows : 128;
    g.wg_per_head = (g.rows_per_head + g.rows_per_wg - 1) / g.rows_per_wg;
    // column tiles: 64 columns (sampling), 128 compressed columns (antidiagonal fast path)
    // (the general antidiagonal path ends in a partial tile when N/S is not a multiple of 64)
    g.ntiles = sampling ? s.N / 64
                        : antidiag_fast(s, g.S) ? (s.N / g.S) / kAdCols : (s.N / g.S + 63) / 64;
    // enough workgroups to fill the chip several times over; at least 4 tiles per range
    const int64_t groups = static_cast<int64_t>(s.B) * s.H * g.wg_per_head;
    int64_t want = groups > 0 ? (2048 + groups - 1) / groups : 1;
    want = std::max<int64_t>(1, std::min<int64_t>(want, std::max(1, g.ntiles / 4)));
    g.tiles_per_split = (g.ntiles + static_cast<int>(want) - 1) / static_cast<int>(want);
    g.nsplit = g.tiles_per_split > 0 ? (g.ntiles + g.tiles_per_split - 1) / g.tiles_per_split : 1;
    g.ws_bytes = static_cast<size_t>(s.B) * s.H * s.NKB * g.rows_per_head * sizeof(float);
    return g;
}

AssignArgs assign_args(const Shape& s, const psa_mask_params& mp) { return assign_args_of(s, mp); }

// sort keys, masses, (log-mass path) the staged log-masses, levels
size_t assign_bytes(const Shape& s, int P, int RQ, bool from_log_masses) {
    return static_cast<size_t>(P) * sizeof(uint64_t) + static_cast<size_t>(s.NKB) * sizeof(float) +
           (from_log_masses ? static_cast<size_t>(s.NKB) * RQ * sizeof(float) : 0) +
           static_cast<size_t>(s.NKB);
}

hipError_t launch_assign(const Shape& s, const AssignArgs& a, hipStream_t st) {
    const int64_t rows = static_cast<int64_t>(s.B) * s.H * s.NQB;
    if (rows == 0) return hipSuccess;
    const size_t lds = assign_bytes(s, a.P, a.RQ, a.L != nullptr);
    if (lds > kAssignMaxLds) return hipErrorNotSupported;
    hipLaunchKernelGGL(k_mask_assign, dim3(static_cast<unsigned>(rows)), dim3(kAssignThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

size_t mask_workspace_bytes(const Shape& s, const psa_mask_params& mp) {
    return score_geom(s, mp).ws_bytes;
}

size_t assign_lds_bytes(const Shape& s, const psa_mask_params& mp, bool from_log_masses) {
    return assign_bytes(s, assign_args_of(s, mp).P, score_geom(s, mp).RQ, from_log_masses);
}

hipError_t launch_mask_scores(const Shape& s, const psa_mask_params& mp, const void* q,
                              const void* k, const MaskBufs& mb, hipStream_t st) {
    if (s.dtype != PSA_BF16) return hipErrorNotSupported;
    ScoreArgs a;
    a.q = static_cast<const bf16_bits*>(q);
    a.k = static_cast<const bf16_bits*>(k);
    a.B = s.B;
    a.H = s.H;
    a.Hkv = s.Hkv;
    a.N = s.N;
    a.Nv = s.Nv;
    a.BQ = s.BQ;
    a.NQB = s.NQB;
    a.NKB = s.NKB;
    a.causal = s.causal;
    a.qs0 = s.qs[0]; a.qs1 = s.qs[1]; a.qs2 = s.qs[2];
    a.ks0 = s.ks[0]; a.ks1 = s.ks[1]; a.ks2 = s.ks[2];
    a.c = (1.0f / sqrtf(static_cast<float>(s.D))) * kLog2e;
    const ScoreGeom g = score_geom(s, mp);
    if (mb.ws == nullptr || mb.ws_bytes < g.ws_bytes) return hipErrorInvalidValue;
    if (mp.mode == PSA_MASK_MEANKEY) {
        char* ws = static_cast<char*>(mb.ws);
        float* qbar = reinterpret_cast<float*>(ws + g.qbar_off);
        float* kbar = reinterpret_cast<float*>(ws + g.kbar_off);
        double* ksum = reinterpret_cast<double*>(ws + g.ksum_off);
        if (static_cast<int64_t>(s.B) * (s.H * s.NQB + s.Hkv * s.NKB) == 0) return hipSuccess;
        hipError_t e = launch_block_means(s, q, k, qbar, kbar, ksum, st);
        if (e != hipSuccess) return e;
        MeanKeyArgs k;
        k.qbar = qbar;
        k.kbar = kbar;
        k.L = static_cast<float*>(mb.ws);
        k.H = s.H; k.Hkv = s.Hkv; k.N = s.N; k.Nv = s.Nv; k.D = s.D; k.BQ = s.BQ; k.BK = s.BK;
        k.NQB = s.NQB; k.NKB = s.NKB; k.causal = s.causal;
        k.c = (1.0 / std::sqrt(static_cast<double>(s.D))) * 1.4426950408889634;
        const int blocks = s.B * s.H * g.wg_per_head * ((s.NKB + kMeanCols - 1) / kMeanCols);
        hipLaunchKernelGGL(k_meankey_logmass, dim3(blocks), dim3(256),
                           (static_cast<size_t>(kMeanRows) * s.D + static_cast<size_t>(kMeanCols) * (s.D + 1)) *
                               sizeof(float), st, k);
        return hipGetLastError();
    }
    a.L = static_cast<float*>(mb.ws);
    a.rows_per_head = g.rows_per_head;
    a.RQ = g.RQ;
    a.wg_per_head = g.wg_per_head;
    a.nsplit = g.nsplit;
    a.tiles_per_split = g.tiles_per_split;
    const int blocks = s.B * s.H * a.wg_per_head * a.nsplit;
    if (blocks == 0) return hipSuccess;
    if (mp.mode == PSA_MASK_SAMPLING) {
        const int grid = 8 * ((blocks + 7) / 8);   // the kernel remaps blocks XCD-wise
        // direct loads: K rows 16-byte aligned (the host checks strides), 32-bit offsets
        switch (g.S) {
            case 1: return launch_sampling<1>(a, s.D, grid, st);
            case 2: return launch_sampling<2>(a, s.D, grid, st);
            case 4: return launch_sampling<4>(a, s.D, grid, st);
            case 8: return launch_sampling<8>(a, s.D, grid, st);
            case 16: return launch_sampling<16>(a, s.D, grid, st);
            case 32: return launch_sampling<32>(a, s.D, grid, st);
            default: return hipErrorNotSupported;
        }
    }
    if (a.RQ > 32 || a.RQ < 1) return hipErrorNotSupported;
    if (antidiag_fast(s, g.S)) {
        const int grid = 8 * ((blocks + 7) / 8);   // the kernel remaps blocks XCD-wise
        switch (g.S) {
            case 2: return launch_antidiag<2>(a, s.D, grid, st);
            case 4: return launch_antidiag<4>(a, s.D, grid, st);
            case 8: return launch_antidiag<8>(a, s.D, grid, st);
            default: return hipErrorNotSupported;
        }
    }
    switch (g.S) {
        case 2: return launch_scores_d<1, 2>(a, s.D, blocks, st);
        case 4: return launch_scores_d<1, 4>(a, s.D, blocks, st);
        case 8: return launch_scores_d<1, 8>(a, s.D, blocks, st);
        default: return hipErrorNotSupported;
    }
}

hipError_t launch_mask_assign_logmass(const Shape& s, const psa_mask_params& mp, const MaskBufs& mb,
                                      int8_t* level_map, hipStream_t st) {
    const ScoreGeom g = score_geom(s, mp);
    if (mb.ws == nullptr || mb.ws_bytes < g.ws_bytes) return hipErrorInvalidValue;
    AssignArgs a = assign_args(s, mp);
    a.L = static_cast<const float*>(mb.ws);
    a.M_out = mb.block_mass;
    a.sim = mp.cos_sim_min > 0.f ? mb.block_sim : nullptr;
    a.sim64 = mask_sim64(s, mp, mb);
    a.map = level_map;
    a.cert = reinterpret_cast<int*>(static_cast<char*>(mb.ws) + g.cert_off);
    a.cert_rows = reinterpret_cast<int*>(static_cast<char*>(mb.ws) + g.rows_off);
    a.cert_cap = g.cap;
    a.RQ = g.RQ;
    a.rows_per_head = g.rows_per_head;
    // block-mean mode: one row per query block, counted like a sampled row
    a.sampling = mp.mode != PSA_MASK_ANTIDIAG;
    a.S = g.S;
    return launch_assign(s, a, st);
}

hipError_t launch_block_means(const Shape& s, const void* q, const void* k, float* qbar, float* kbar,
                              double* ksum, hipStream_t st) {
    MeanArgs m;
    m.q = static_cast<const bf16_bits*>(q);
    m.k = static_cast<const bf16_bits*>(k);
    m.qbar = qbar;
    m.kbar = kbar;
    m.ksum = ksum;
    m.B = s.B; m.H = s.H; m.Hkv = s.Hkv; m.N = s.N; m.Nv = s.Nv; m.D = s.D;
    m.BQ = s.BQ; m.BK = s.BK; m.NQB = s.NQB; m.NKB = s.NKB;
    m.qs0 = s.qs[0]; m.qs1 = s.qs[1]; m.qs2 = s.qs[2];
    m.ks0 = s.ks[0]; m.ks1 = s.ks[1]; m.ks2 = s.ks[2];
    const int64_t items = static_cast<int64_t>(s.B) * (s.H * s.NQB + s.Hkv * s.NKB);
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(k_block_means, dim3(static_cast<unsigned>(items)), dim3(256), 0, st, m);
    return hipGetLastError();
}

hipError_t launch_block_sim(const Shape& s, const void* k, float* block_sim, double* sim64,
                            hipStream_t st) {
    if (s.dtype != PSA_BF16) return hipErrorNotSupported;
    const int64_t items = static_cast<int64_t>(s.B) * s.Hkv * s.NKB;
    if (items == 0) return hipSuccess;
    const unsigned blocks = static_cast<unsigned>((items + 3) / 4);
    if (s.D == 128)
        hipLaunchKernelGGL(k_block_sim<128>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const bf16_bits*>(k), s.ks[0], s.ks[1], s.ks[2], s.Hkv,
                           s.NKB, s.Nv, items, block_sim, sim64);
    else
        hipLaunchKernelGGL(k_block_sim<64>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const bf16_bits*>(k), s.ks[0], s.ks[1], s.ks[2], s.Hkv,
                           s.NKB, s.Nv, items, block_sim, sim64);
    return hipGetLastError();
}

double* mask_sim64(const Shape& s, const psa_mask_params& mp, const MaskBufs& mb) {
    if (mp.cos_sim_min <= 0.f) return nullptr;
    return reinterpret_cast<double*>(static_cast<char*>(mb.ws) + score_geom(s, mp).sim64_off);
}

int* mask_cert_counters(const Shape& s, const psa_mask_params& mp, void* ws) {
    return reinterpret_cast<int*>(static_cast<char*>(ws) + score_geom(s, mp).cert_off);
}

hipError_t launch_mask_certify(const Shape& s, const psa_mask_params& mp, const void* q,
                               const void* k, const MaskBufs& mb, int8_t* level_map, hipStream_t st) {
    const ScoreGeom g = score_geom(s, mp);
    char* ws = static_cast<char*>(mb.ws);
    CertArgs c;
    c.q = static_cast<const bf16_bits*>(q);
    c.k = static_cast<const bf16_bits*>(k);
    c.H = s.H; c.Hkv = s.Hkv; c.N = s.N; c.Nv = s.Nv; c.BQ = s.BQ; c.NQB = s.NQB; c.NKB = s.NKB;
    c.causal = s.causal;
    c.S = g.S;
    c.RQ = g.RQ;
    c.qs0 = s.qs[0]; c.qs1 = s.qs[1]; c.qs2 = s.qs[2];
    c.ks0 = s.ks[0]; c.ks1 = s.ks[1]; c.ks2 = s.ks[2];
    c.scale = 1.0 / std::sqrt(static_cast<double>(s.D));
    c.cert = reinterpret_cast<const int*>(ws + g.cert_off);
    c.rows = reinterpret_cast<const int*>(ws + g.rows_off);
    c.Lg = reinterpret_cast<double*>(ws + g.lg_off);
    c.ksum = mp.mode == PSA_MASK_MEANKEY ? reinterpret_cast<const double*>(ws + g.ksum_off) : nullptr;
    c.cap = g.cap;
    if (c.cap == 0) return hipSuccess;
    // fixed grids walking the device-side count of flagged rows
    const bool sampling = mp.mode == PSA_MASK_SAMPLING, antidiag = mp.mode == PSA_MASK_ANTIDIAG;
    const int ncols = sampling ? s.N : antidiag ? s.N / g.S : 0;
    const int per_item = sampling ? 256 * (g.S <= 8 ? 4 : (g.S == 16 ? 2 : 1)) : 512;
    c.nchunks = (ncols + per_item - 1) / per_item;
    const unsigned score_grid = static_cast<unsigned>(
        std::min<int64_t>(2048, std::max<int64_t>(1, static_cast<int64_t>(c.cap) * std::max(1, c.nchunks))));
    hipError_t e = hipSuccess;
    const int D = s.D;
#define PSA_CERT_SAMP(DD, SS) hipLaunchKernelGGL((k_cert_sampling<DD, SS>), dim3(score_grid), dim3(256), 0, st, c)
#define PSA_CERT_AD(DD, SS, RR) hipLaunchKernelGGL((k_cert_antidiag<DD, SS, RR>), dim3(score_grid), dim3(256), 0, st, c)
    if (sampling && g.S <= 16) {
        // group the flagged rows by KV head into batches, then rescore on float64 MFMA
        BatchArgs b;
        b.cert = reinterpret_cast<int*>(ws + g.cert_off);
        b.rows = c.rows;
        b.bat = reinterpret_cast<int*>(ws + g.bat_off);
        b.cap = c.cap;
        b.unit = s.NQB * (s.H / s.Hkv);
        b.BR = 16 / g.S;
        int P = 1;
        while (P < std::min(c.cap, kBatchSortMax)) P <<= 1;
        hipLaunchKernelGGL(k_cert_batches, dim3(1), dim3(kBatchThreads), static_cast<size_t>(P) * sizeof(uint64_t),
                           st, b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int nkb4 = (s.NKB + 3) / 4;
        const unsigned grid = static_cast<unsigned>(
            std::min<int64_t>(4096, std::max<int64_t>(1, static_cast<int64_t>(c.cap) * nkb4)));
        const int* bat = b.bat;
#define PSA_CERT_SM(DD, SS) hipLaunchKernelGGL((k_cert_sampling_mfma<DD, SS>), dim3(grid), dim3(256), 0, st, c, bat)
        switch (g.S) {
            case 1: if (D == 128) PSA_CERT_SM(128, 1); else PSA_CERT_SM(64, 1); break;
            case 2: if (D == 128) PSA_CERT_SM(128, 2); else PSA_CERT_SM(64, 2); break;
            case 4: if (D == 128) PSA_CERT_SM(128, 4); else PSA_CERT_SM(64, 4); break;
            case 8: if (D == 128) PSA_CERT_SM(128, 8); else PSA_CERT_SM(64, 8); break;
            case 16: if (D == 128) PSA_CERT_SM(128, 16); else PSA_CERT_SM(64, 16); break;
            default: return hipErrorNotSupported;
        }
#undef PSA_CERT_SM
    } else if (sampling) {
        switch (g.S) {
            case 1: if (D == 128) PSA_CERT_SAMP(128, 1); else PSA_CERT_SAMP(64, 1); break;
            case 2: if (D == 128) PSA_CERT_SAMP(128, 2); else PSA_CERT_SAMP(64, 2); break;
            case 4: if (D == 128) PSA_CERT_SAMP(128, 4); else PSA_CERT_SAMP(64, 4); break;
            case 8: if (D == 128) PSA_CERT_SAMP(128, 8); else PSA_CERT_SAMP(64, 8); break;
            case 16: if (D == 128) PSA_CERT_SAMP(128, 16); else PSA_CERT_SAMP(64, 16); break;
            case 32: if (D == 128) PSA_CERT_SAMP(128, 32); else PSA_CERT_SAMP(64, 32); break;
            default: return hipErrorNotSupported;
        }
    } else if (antidiag && g.RQ == 16 && (g.S == 8 || g.S == 4)) {
        // float64 MFMA: the query block's 16 compressed rows are the 16 MFMA rows
        const int nchunk = (s.N / g.S + 255) / 256;
        const unsigned grid = static_cast<unsigned>(
            std::min<int64_t>(4096, std::max<int64_t>(1, static_cast<int64_t>(c.cap) * nchunk)));
        if (g.S == 8) {
            if (D == 128) hipLaunchKernelGGL((k_cert_antidiag_mfma<128, 8>), dim3(grid), dim3(256), 0, st, c);
            else hipLaunchKernelGGL((k_cert_antidiag_mfma<64, 8>), dim3(grid), dim3(256), 0, st, c);
        } else {
            if (D == 128) hipLaunchKernelGGL((k_cert_antidiag_mfma<128, 4>), dim3(grid), dim3(256), 0, st, c);
            else hipLaunchKernelGGL((k_cert_antidiag_mfma<64, 4>), dim3(grid), dim3(256), 0, st, c);
        }
    } else if (antidiag) {
        const int key = g.S * 100 + g.RQ;
        switch (key) {
            case 232: if (D == 128) PSA_CERT_AD(128, 2, 32); else PSA_CERT_AD(64, 2, 32); break;
            case 416: if (D == 128) PSA_CERT_AD(128, 4, 16); else PSA_CERT_AD(64, 4, 16); break;
            case 432: if (D == 128) PSA_CERT_AD(128, 4, 32); else PSA_CERT_AD(64, 4, 32); break;
            case 808: if (D == 128) PSA_CERT_AD(128, 8, 8); else PSA_CERT_AD(64, 8, 8); break;
            case 816: if (D == 128) PSA_CERT_AD(128, 8, 16); else PSA_CERT_AD(64, 8, 16); break;
            default: return hipErrorNotSupported;
        }
    } else {
        const unsigned grid = static_cast<unsigned>(std::min(c.cap, 1024));
        if (D == 128)
            hipLaunchKernelGGL(k_cert_meankey<128>, dim3(grid), dim3(256), 0, st, c);
        else
            hipLaunchKernelGGL(k_cert_meankey<64>, dim3(grid), dim3(256), 0, st, c);
    }
#undef PSA_CERT_SAMP
#undef PSA_CERT_AD
    if ((e = hipGetLastError()) != hipSuccess) return e;
    AssignArgs a = assign_args(s, mp);
    a.M_out = mb.block_mass;
    a.sim = mp.cos_sim_min > 0.f ? mb.block_sim : nullptr;
    a.sim64 = mask_sim64(s, mp, mb);
    a.map = level_map;
    a.RQ = g.RQ;
    a.rows_per_head = g.rows_per_head;
    a.sampling = mp.mode != PSA_MASK_ANTIDIAG;
    a.S = g.S;
    const size_t lds = static_cast<size_t>(a.P) * (sizeof(uint64_t) + sizeof(uint16_t)) + s.NKB;
    if (lds > kAssignMaxLds) return hipErrorNotSupported;
    hipLaunchKernelGGL(k_cert_assign, dim3(static_cast<unsigned>(std::min(c.cap, 1024))),
                       dim3(kAssignThreads), lds, st, a, c);
    return hipGetLastError();
}

hipError_t launch_mask_assign(const Shape& s, const psa_mask_params& mp, const float* block_mass,
                              const float* block_sim, int8_t* level_map, hipStream_t st) {
    AssignArgs a = assign_args(s, mp);
    a.M = block_mass;
    a.sim = mp.cos_sim_min > 0.f ? block_sim : nullptr;
    a.map = level_map;
    return launch_assign(s, a, st);
}

}  // namespace psa
