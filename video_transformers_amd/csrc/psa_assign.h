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
    int8_t* map;
    int H, Hkv, N, Nv, BQ, BK, NQB, NKB, causal;
    int P;  // sort length: power of two >= NKB
    int RQ, rows_per_head, sampling, S;   // scoring rows per query block (L path)
    double t[4];
    float cos_min;
    int force_diag, force_lo, force_hi;
};

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
// keys is LDS scratch of a.P uint64. Ends with a barrier.
__device__ inline void assign_levels(const AssignArgs& a, int qb, int b, int hk, const float* Ms,
                                     uint64_t* keys, int8_t* lvl, int tid) {
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
            for (int u = 0; u < per; ++u) {
                const int i = i0 + u;
                if (i >= ncand) break;
                const uint64_t key = keys[i];
                const int kb = static_cast<int>(key & 0xffffffffu);
                int8_t L = -1;
                if (c < a.t[0]) L = 0;
                else if (c < a.t[1]) L = 1;
                else if (c < a.t[2]) L = 2;
                else if (c < a.t[3]) L = 3;
                lvl[kb] = L;
                c += static_cast<double>(float_from_order(~static_cast<uint32_t>(key >> 32)));
            }
        }
    }
    __syncthreads();
    for (int kb = tid; kb < a.NKB; kb += kAssignThreads) {
        int8_t L = any_valid ? lvl[kb] : static_cast<int8_t>(-1);
        if (any_valid && kb <= last) {
            const int klo = kb * a.BK, khi = klo + a.BK;
            bool forced = a.force_diag && klo < qhi && qlo < khi;
            if (a.force_lo < a.force_hi &&
                ((qlo < a.force_hi && a.force_lo < qhi) || (klo < a.force_hi && a.force_lo < khi)))
                forced = true;
            if (forced)
                L = 0;
            else if (a.sim != nullptr && L > 0 &&
                     a.sim[(static_cast<int64_t>(b) * a.Hkv + hk) * a.NKB + kb] < a.cos_min)
                L = 0;
        }
        lvl[kb] = L;
    }
    __syncthreads();
}

}  // namespace psa
