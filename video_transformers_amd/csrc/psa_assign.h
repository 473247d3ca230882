// Threshold assignment of one (batch, head, query block) row by one workgroup of
// kAssignThreads threads (summary article, "Results": threshold-based levels with a cosine
// constraint on pooling). Shared by the mask's assignment kernel and by the attention kernel
// that scores block means in its prologue, so both produce the same map bit for bit.
//
// Per row, over the candidate blocks (all; causal: those overlapping tokens <= the query
// block's last token): sort by mass descending (ties: lower kb first); exclusive running sum c
// in float64 in that order; level = min{l : c < t_l}, otherwise skip. Then: causal
// non-candidates -> skip; forced L0 (diagonal blocks if asked; blocks overlapping the forced
// span in either direction) -> 0; a pooled level on a block whose similarity < cos_min -> 0.
#pragma once

#include <stdint.h>

#include "psa_device.h"
#include "psa_internal.h"

namespace psa {

constexpr int kAssignThreads = 256;

struct AssignArgs {
    const float* M;     // given masses [rows][NKB] (psa_mask_assign), or null
    const float* L;     // log2 masses [B*H][NKB][rows_per_head] (psa_mask), or null
    float* M_out;       // masses computed from L, written here (may be null in the fused path)
    const float* sim;
    const double* sim64;  // the similarities in float64 (psa_mask), used instead of sim if set
    int8_t* map;
    // Certification (psa_mask): rows whose float32 decisions lie within cert_abs of a threshold
    // or cert_rel of a tie across a level change are listed here for float64 rescoring.
    // cert[0] counts flagged rows, cert[1] those beyond cert_cap (left as float32 decides).
    int* cert;          // null: no certification (given masses are exact by definition)
    int* cert_rows;     // [cert_cap]
    int cert_cap;
    double cert_abs, cert_rel;   // the margins (cert_margins: per scoring mode)
    int H, Hkv, N, Nv, BQ, BK, NQB, NKB, causal;
    int P;  // sort length: power of two >= NKB
    int RQ, rows_per_head, sampling, S;   // scoring rows per query block (L path)
    double t[4];
    float cos_min;
    int force_diag, force_lo, force_hi;
};

// Certification margins of a float32 assignment, per scoring mode. A running sum c carries at
// most the row's summed absolute error of its float32 block masses, and two masses can trade
// places only when their gap is below the sum of their relative errors. Measured against
// float64 at full size (32k-token layers, 17k for d = 64): summed absolute error per row at most
// 6.5e-7 (sampling) and 8.7e-7 (antidiagonal, whose logits sum S*d = 1024 products); relative
// error per mass at most 1.6e-6 and 6.6e-6. The margins take about five times the first
// (cert_abs) and two and a half times twice the second (cert_rel): a decision further than
// cert_abs from every threshold, with no tie closer than cert_rel (relative) across a level
// change, is the float64 decision. Block-mean masses come from float64 dots and take the
// sampling margins.
struct CertMargins {
    double abs, rel;
};
inline CertMargins cert_margins(int mode) {
    return mode == PSA_MASK_ANTIDIAG ? CertMargins{5e-6, 3.3e-5} : CertMargins{4e-6, 8e-6};
}

// The arguments every assignment shares for one problem and mask parameters (the per-call
// sources and destinations, M / L / M_out / sim / map and the log-mass geometry, are set by
// the caller).
inline AssignArgs assign_args_of(const Shape& s, const psa_mask_params& mp) {
    AssignArgs a{};
    a.H = s.H;
    a.Hkv = s.Hkv;
    a.N = s.N;
    a.Nv = s.Nv;
    a.BQ = s.BQ;
    a.BK = s.BK;
    a.NQB = s.NQB;
    a.NKB = s.NKB;
    a.causal = s.causal;
    int P = 1;
    while (P < s.NKB) P <<= 1;
    a.P = P;
    for (int i = 0; i < 4; ++i) a.t[i] = static_cast<double>(mp.thresholds[i]);
    a.cos_min = mp.cos_sim_min;
    a.force_diag = mp.force_diag_l0 != 0;
    a.force_lo = mp.force_l0_begin;
    a.force_hi = mp.force_l0_end;
    const CertMargins cm = cert_margins(mp.mode);
    a.cert_abs = cm.abs;
    a.cert_rel = cm.rel;
    return a;
}

// float <-> uint32 order-preserving maps (for a 64-bit sort key of mass and kb)
__device__ __forceinline__ uint32_t float_order(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_from_order(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// double <-> uint64 order-preserving maps (float64 assignment: key = ~order(mass), kb apart)
__device__ __forceinline__ uint64_t double_order(double d) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(d));
    return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double double_from_order(uint64_t o) {
    return __longlong_as_double(static_cast<long long>((o & 0x8000000000000000ull) ? (o & 0x7fffffffffffffffull) : ~o));
}

__device__ __forceinline__ int8_t level_of(const AssignArgs& a, double c) {
    return c < a.t[0] ? 0 : c < a.t[1] ? 1 : c < a.t[2] ? 2 : c < a.t[3] ? 3 : -1;
}

// The overrides of one row, after the threshold levels are in lvl: causal non-candidates ->
// skip; forced L0; a pooled level on a block whose similarity < cos_min -> L0 (the float64
// similarity when given, compared with cos_min as a float). Ends with a barrier.
__device__ inline void assign_overrides(const AssignArgs& a, int qb, int b, int hk, int8_t* lvl,
                                        int tid) {
    const int qlo = qb * a.BQ, qhi = qlo + a.BQ;
    const bool any_valid = qlo < a.Nv;
    const int last = a.causal ? min((qhi - 1) / a.BK, a.NKB - 1) : a.NKB - 1;
    for (int kb = tid; kb < a.NKB; kb += kAssignThreads) {
        int8_t L = any_valid ? lvl[kb] : static_cast<int8_t>(-1);
        if (any_valid && kb <= last) {
            const int klo = kb * a.BK, khi = klo + a.BK;
            bool forced = a.force_diag && klo < qhi && qlo < khi;
            if (a.force_lo < a.force_hi &&
                ((qlo < a.force_hi && a.force_lo < qhi) || (klo < a.force_hi && a.force_lo < khi)))
                forced = true;
            const int64_t si = (static_cast<int64_t>(b) * a.Hkv + hk) * a.NKB + kb;
            if (forced)
                L = 0;
            else if (L > 0 && a.sim64 != nullptr && a.sim64[si] < static_cast<double>(a.cos_min))
                L = 0;
            else if (L > 0 && a.sim64 == nullptr && a.sim != nullptr && a.sim[si] < a.cos_min)
                L = 0;
        } else if (kb > last) {
            L = -1;
        }
        lvl[kb] = L;
    }
    __syncthreads();
}

// Masses from log2-masses staged in LDS (Ls[kb * RQ + i] for the query block's RQ scoring rows):
// scoring row i has logsumexp lse_i = log2 sum_kb exp2(L[kb][i]); mass_kb = mean over the valid
// rows of exp2(L[kb][i] - lse_i). Rows with no visible key have L = -inf everywhere. Writes the
// masses to Ms (LDS) and, if M_out is not null, to M_out[kb]. Ends with a barrier.
__device__ inline void assign_masses(const AssignArgs& a, int qb, const float* Ls, float* Ms,
                                     float* M_out, int tid) {
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int RQ = a.RQ;   // power of two <= 32
    const int i = tid & (RQ - 1);
    const int kstep = kAssignThreads / RQ;
    __shared__ float lse[32];   // per scoring row of the query block
    float m = -INFINITY, sum = 0.f;   // online logsumexp of this thread's values
    for (int kb = tid / RQ; kb < a.NKB; kb += kstep) {
        const float v = Ls[kb * RQ + i];
        const float mn = fmaxf(m, v);
        if (mn != -INFINITY) sum = sum * fast_exp2(m - mn) + fast_exp2(v - mn);
        m = mn;
    }
    // merge across the lanes of the same row (lane xor RQ, 2 RQ, ... 32), then the waves
    for (int o = RQ; o < 64; o <<= 1) {
        const float mo = __shfl_xor(m, o, 64);
        const float so = __shfl_xor(sum, o, 64);
        const float mn = fmaxf(m, mo);
        sum = mn == -INFINITY ? 0.f : sum * fast_exp2(m - mn) + so * fast_exp2(mo - mn);
        m = mn;
    }
    __shared__ float wm[kAssignThreads / 64][32], ws[kAssignThreads / 64][32];
    if (lane < RQ) {
        wm[wave][lane] = m;
        ws[wave][lane] = sum;
    }
    __syncthreads();
    if (tid < RQ) {
        float mm = -INFINITY, ss = 0.f;
        for (int w = 0; w < kAssignThreads / 64; ++w) {
            const float mo = wm[w][tid], so = ws[w][tid];
            const float mn = fmaxf(mm, mo);
            ss = mn == -INFINITY ? 0.f : ss * fast_exp2(mm - mn) + so * fast_exp2(mo - mn);
            mm = mn;
        }
        lse[tid] = (mm == -INFINITY || ss <= 0.f) ? -INFINITY : mm + __builtin_amdgcn_logf(ss);
    }
    __syncthreads();
    int den;
    if (a.sampling)
        den = min(max(a.Nv - qb * a.BQ, 0), a.BQ) > 0 ? RQ : 0;
    else
        den = min(max(a.Nv / a.S - qb * RQ, 0), RQ);
    const float invd = den > 0 ? 1.f / static_cast<float>(den) : 0.f;
    for (int kb = tid; kb < a.NKB; kb += kAssignThreads) {
        float acc = 0.f;
        for (int r = 0; r < RQ; ++r) {
            const float lr = lse[r];
            if (lr != -INFINITY) acc += fast_exp2(Ls[kb * RQ + r] - lr);
        }
        const float mass = acc * invd;
        Ms[kb] = mass;
        if (M_out != nullptr) M_out[kb] = mass;
    }
    __syncthreads();
}

// Levels of one row from its masses Ms (LDS, NKB) into lvl (LDS, NKB int8), overrides applied;
// keys is LDS scratch of a.P uint64. With cflag (an LDS int the caller cleared) set, a decision
// within the certification margins sets *cflag = 1. Ends with a barrier.
__device__ inline void assign_levels(const AssignArgs& a, int qb, int b, int hk, const float* Ms,
                                     uint64_t* keys, int8_t* lvl, int tid, int* cflag = nullptr) {
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qlo = qb * a.BQ, qhi = qlo + a.BQ;
    const bool any_valid = qlo < a.Nv;
    const int last = a.causal ? min((qhi - 1) / a.BK, a.NKB - 1) : a.NKB - 1;
    const int ncand = last + 1;
    for (int i = tid; i < a.P; i += kAssignThreads) {
        uint64_t key = ~0ull;
        if (i < ncand) key = (static_cast<uint64_t>(~float_order(Ms[i])) << 32) | static_cast<uint32_t>(i);
        keys[i] = key;
    }
    for (int i = tid; i < a.NKB; i += kAssignThreads) lvl[i] = -1;
    __syncthreads();
    // bitonic sort, ascending keys = mass descending, kb ascending, of the first Pr keys: the
    // candidates padded to a power of two (causal rows have fewer); the keys past them are
    // all ~0 and already in place at the end
    int Pr = 1;
    while (Pr < ncand) Pr <<= 1;
    for (int size = 2; size <= Pr; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < Pr / 2; i += kAssignThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = ((lo & size) == 0);
                const uint64_t x = keys[lo], y = keys[hi];
                if ((x > y) == up) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    // Exclusive running sum of the sorted masses in float64 (a block scan; the summation
    // order differs from a left-to-right loop only in float64 rounding, ~1e-16 relative),
    // then each sorted entry's level from its exclusive sum. The mass comes back out of the
    // sort key.
    {
        const int per = a.P / kAssignThreads > 0 ? a.P / kAssignThreads : 1;   // entries per thread
        const int i0 = tid * per;
        double loc = 0.0;
        for (int u = 0; u < per; ++u) {
            const int i = i0 + u;
            if (i < ncand) loc += static_cast<double>(float_from_order(~static_cast<uint32_t>(keys[i] >> 32)));
        }
        // inclusive scan of the per-thread totals: within the wave, then across the waves
        double inc = loc;
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        __shared__ double wsum[kAssignThreads / 64];
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        double base = 0.0;
        for (int w = 0; w < wave; ++w) base += wsum[w];
        double c = base + inc - loc;   // exclusive sum before entry i0
        if (any_valid) {
            bool flag = false;
            // the entry before i0 (for a near-tie across a level change at the thread boundary)
            double mprev = 0.0;
            int8_t lprev = 0;
            if (cflag != nullptr && i0 > 0 && i0 < ncand) {
                mprev = static_cast<double>(float_from_order(~static_cast<uint32_t>(keys[i0 - 1] >> 32)));
                lprev = level_of(a, c - mprev);
            }
            for (int u = 0; u < per; ++u) {
                const int i = i0 + u;
                if (i >= ncand) break;
                const uint64_t key = keys[i];
                const int kb = static_cast<int>(key & 0xffffffffu);
                const int8_t L = level_of(a, c);
                lvl[kb] = L;
                const double m = static_cast<double>(float_from_order(~static_cast<uint32_t>(key >> 32)));
                if (cflag != nullptr) {
#pragma unroll
                    for (int l = 0; l < 4; ++l)
                        if (fabs(c - a.t[l]) < a.cert_abs) flag = true;
                    if (i > 0 && L != lprev && mprev - m <= a.cert_rel * mprev) flag = true;
                    mprev = m;
                    lprev = L;
                }
                c += m;
            }
            if (flag) *cflag = 1;
        }
    }
    __syncthreads();
    assign_overrides(a, qb, b, hk, lvl, tid);
}

// The float64 assignment of one row: keys[i] = ~double_order(mass of block idx[i]) for the
// candidates i < ncand (the caller fills them; `keys` holds a.P entries, `idx` a.P uint16),
// sorted by (mass descending, kb ascending), exclusive running sum in float64 (a block scan),
// level = min{l : c < t_l}, then the overrides. Ends with a barrier.
__device__ inline void assign_levels_f64(const AssignArgs& a, int qb, int b, int hk, uint64_t* keys,
                                         uint16_t* idx, int8_t* lvl, int tid) {
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool any_valid = qb * a.BQ < a.Nv;
    const int last = a.causal ? min((qb * a.BQ + a.BQ - 1) / a.BK, a.NKB - 1) : a.NKB - 1;
    const int ncand = last + 1;
    int Pr = 1;
    while (Pr < ncand) Pr <<= 1;
    for (int i = ncand + tid; i < Pr; i += kAssignThreads) {
        keys[i] = ~0ull;
        idx[i] = 0xffffu;
    }
    for (int i = tid; i < a.NKB; i += kAssignThreads) lvl[i] = -1;
    __syncthreads();
    for (int size = 2; size <= Pr; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < Pr / 2; i += kAssignThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = ((lo & size) == 0);
                const uint64_t x = keys[lo], y = keys[hi];
                const uint16_t xi = idx[lo], yi = idx[hi];
                const bool gt = x > y || (x == y && xi > yi);
                if (gt == up) {
                    keys[lo] = y;
                    keys[hi] = x;
                    idx[lo] = yi;
                    idx[hi] = xi;
                }
            }
            __syncthreads();
        }
    }
    {
        const int per = Pr / kAssignThreads > 0 ? Pr / kAssignThreads : 1;
        const int i0 = tid * per;
        double loc = 0.0;
        for (int u = 0; u < per; ++u) {
            const int i = i0 + u;
            if (i < ncand) loc += double_from_order(~keys[i]);
        }
        double inc = loc;
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        __shared__ double wsum64[kAssignThreads / 64];
        if (lane == 63) wsum64[wave] = inc;
        __syncthreads();
        double base = 0.0;
        for (int w = 0; w < wave; ++w) base += wsum64[w];
        double c = base + inc - loc;
        if (any_valid) {
            for (int u = 0; u < per; ++u) {
                const int i = i0 + u;
                if (i >= ncand) break;
                lvl[idx[i]] = level_of(a, c);
                c += double_from_order(~keys[i]);
            }
        }
    }
    __syncthreads();
    assign_overrides(a, qb, b, hk, lvl, tid);
}

// ---- float64 pieces of the certification, shared by psa_mask and the fused prologue ----

// q_bar of query block qb in float64 (threads e < D each sum their column over the valid rows
// in row order, then divide); 0 when the block has no valid row. No barrier.
__device__ inline void cert_qbar_f64(const bf16_bits* qh, int64_t qs2, int qb, int BQ, int Nv, int D,
                                     double* qbar, int tid) {
    const int rv = min(max(Nv - qb * BQ, 0), BQ);
    if (tid < D) {
        double s = 0.0;
        for (int i = 0; i < rv; ++i)
            s += static_cast<double>(bf16_to_f32(qh[static_cast<int64_t>(qb * BQ + i) * qs2 + tid]));
        qbar[tid] = rv > 0 ? s / rv : 0.0;
    }
}

// Block-mean log-mass of KV block kb in float64: scale * q_bar . (sum_t k_t) / n + ln n over
// the block's n valid keys, from the block's float64 key sums ksum[e] = sum_t k_t[e] (one row
// of D, written by the block-means kernel; the dot in d order); -inf for a non-candidate, a
// block with no valid key or a query block with no valid row.
__device__ inline double cert_meankey_logmass(const double* ksum, const double* qbar, int D, int kb,
                                              int Nv, bool usable, double scale) {
    const int nv = min(max(Nv - kb * 64, 0), 64);
    if (!usable || nv == 0) return -INFINITY;
    const double* kr = ksum + static_cast<int64_t>(kb) * D;
    double dot = 0.0;
    for (int e = 0; e < D; ++e) dot = fma(qbar[e], kr[e], dot);
    return scale * dot / nv + log(static_cast<double>(nv));
}

// Per scoring row i < RQ (a power of two <= 32) of one query block, the float64 logsumexp over
// the KV blocks of L[i * NKB + kb] (natural-log block masses) into lse[i] (LDS, 32 entries).
// wm, ws: LDS scratch [kAssignThreads / 64][32]. Ends with a barrier.
__device__ inline void cert_lse(const double* L, int RQ, int NKB, double* lse, double (*wm)[32],
                                double (*ws)[32], int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    const int i = tid & (RQ - 1);
    double m = -INFINITY, sum = 0.0;
    for (int kb = tid / RQ; kb < NKB; kb += kAssignThreads / RQ) {
        const double v = L[static_cast<int64_t>(i) * NKB + kb];
        const double mn = fmax(m, v);
        if (mn != -INFINITY) sum = sum * exp(m - mn) + exp(v - mn);
        m = mn;
    }
    for (int o = RQ; o < 64; o <<= 1) {
        const double mo = __shfl_xor(m, o, 64);
        const double so = __shfl_xor(sum, o, 64);
        const double mn = fmax(m, mo);
        sum = mn == -INFINITY ? 0.0 : sum * exp(m - mn) + so * exp(mo - mn);
        m = mn;
    }
    if (lane < RQ) {
        wm[wave][lane] = m;
        ws[wave][lane] = sum;
    }
    __syncthreads();
    if (tid < RQ) {
        double mm = -INFINITY, ss = 0.0;
        for (int w = 0; w < kAssignThreads / 64; ++w) {
            const double mo = wm[w][tid], so = ws[w][tid];
            const double mn = fmax(mm, mo);
            ss = mn == -INFINITY ? 0.0 : ss * exp(mm - mn) + so * exp(mo - mn);
            mm = mn;
        }
        lse[tid] = (mm == -INFINITY || ss <= 0.0) ? -INFINITY : mm + log(ss);
    }
    __syncthreads();
}

// The float64 mass of block kb: the mean over the `den` valid scoring rows of exp(L - lse).
__device__ inline double cert_mass(const double* L, const double* lse, int RQ, int NKB, int kb,
                                   int den) {
    double acc = 0.0;
    for (int j = 0; j < RQ; ++j)
        if (lse[j] != -INFINITY) acc += exp(L[static_cast<int64_t>(j) * NKB + kb] - lse[j]);
    return den > 0 ? acc / den : 0.0;
}

// Valid scoring rows of query block qb: sampling (and block means, one row) count all S rows
// of a block with a valid query; antidiagonal counts the valid compressed rows.
__device__ inline int cert_den(const AssignArgs& a, int qb) {
    if (a.sampling) return min(max(a.Nv - qb * a.BQ, 0), a.BQ) > 0 ? a.RQ : 0;
    return min(max(a.Nv / a.S - qb * a.RQ, 0), a.RQ);
}

}  // namespace psa
