// Block index of a level map: a CSR over (row, level) keys listing, for every
// (batch, head, query block) row and level l, the KV blocks at level l in ascending order.
// This is how the attention kernel learns which blocks to fetch at which level and never
// touches a skipped block (PSA summary article at rg.mbintangr.com, "Method": the least
// important blocks are skipped entirely).
//
// Three launches, all integer and deterministic:
//   k_index_count  one wave per row: per-level counts via ballots (bad entries -> skip + flag)
//   k_index_scan   one workgroup: exclusive scan of the R*4 counts into row_ptr
//   k_index_fill   one wave per row: ballot compaction of each level's kb into col_idx
#include "psa_device.h"
#include "psa_internal.h"

namespace psa {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ void __launch_bounds__(256) k_clear_i32(int32_t* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

__global__ void __launch_bounds__(256)
    k_index_count(const int8_t* __restrict__ map, int64_t rows, int nkb,
                  int32_t* __restrict__ row_ptr, int32_t* __restrict__ dev_err) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int8_t* m = map + row * nkb;
    int cnt[4] = {0, 0, 0, 0};
    bool bad = false;
    for (int kb0 = 0; kb0 < nkb; kb0 += 64) {
        const int kb = kb0 + lane;
        const int v = kb < nkb ? static_cast<int>(m[kb]) : -1;
        bad |= (v < -1 || v > 3);
#pragma unroll
        for (int l = 0; l < 4; ++l) cnt[l] += __popcll(__ballot(v == l));
    }
    if (__ballot(bad) != 0ull && lane == 0) *dev_err = PSA_ERR_BAD_LEVEL_MAP;  // same value from every writer
    if (lane < 4) {
        int c = lane == 0 ? cnt[0] : lane == 1 ? cnt[1] : lane == 2 ? cnt[2] : cnt[3];
        row_ptr[row * 4 + lane + 1] = c;
    }
}

// Exclusive scan of counts held in row_ptr[1..n] into row_ptr[0..n] (row_ptr[0] = 0).
// One workgroup of 1024 threads; each thread owns a contiguous chunk.
__global__ void __launch_bounds__(1024) k_index_scan(int32_t* __restrict__ row_ptr, int64_t n) {
    __shared__ int64_t part[1024];
    const int t = threadIdx.x;
    const int64_t chunk = (n + 1023) / 1024;
    const int64_t lo = t * chunk;
    const int64_t hi = lo + chunk < n ? lo + chunk : n;
    int64_t s = 0;
    for (int64_t i = lo; i < hi; ++i) s += row_ptr[i + 1];
    part[t] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 partial sums.
    for (int off = 1; off < 1024; off <<= 1) {
        int64_t add = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int64_t run = part[t] - s;  // exclusive prefix of this chunk
    for (int64_t i = lo; i < hi; ++i) {
        const int64_t c = row_ptr[i + 1];
        run += c;
        row_ptr[i + 1] = static_cast<int32_t>(run);
    }
    if (t == 0) row_ptr[0] = 0;
}

__global__ void __launch_bounds__(256)
    k_index_fill(const int8_t* __restrict__ map, int64_t rows, int nkb,
                 const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int8_t* m = map + row * nkb;
    int pos[4];
#pragma unroll
    for (int l = 0; l < 4; ++l) pos[l] = row_ptr[row * 4 + l];
    const uint64_t below = lanemask_lt();
    for (int kb0 = 0; kb0 < nkb; kb0 += 64) {
        const int kb = kb0 + lane;
        const int v = kb < nkb ? static_cast<int>(m[kb]) : -1;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const uint64_t bal = __ballot(v == l);
            if (v == l) col_idx[pos[l] + __popcll(bal & below)] = kb;
            pos[l] += __popcll(bal);
        }
    }
}

}  // namespace

hipError_t launch_clear_i32(int32_t* p, int n, hipStream_t st) {
    hipLaunchKernelGGL(k_clear_i32, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_build_index(const Shape& s, const int8_t* level_map, const IndexBufs& ib,
                              hipStream_t st) {
    const int64_t rows = static_cast<int64_t>(s.B) * s.H * s.NQB;
    hipError_t e = launch_clear_i32(ib.dev_err, 1, st);
    if (e != hipSuccess) return e;
    const unsigned blocks = static_cast<unsigned>((rows + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(k_index_count, dim3(blocks), dim3(256), 0, st, level_map, rows, s.NKB,
                       ib.row_ptr, ib.dev_err);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_index_scan, dim3(1), dim3(1024), 0, st, ib.row_ptr, rows * 4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_index_fill, dim3(blocks), dim3(256), 0, st, level_map, rows, s.NKB,
                       ib.row_ptr, ib.col_idx);
    return hipGetLastError();
}

}  // namespace psa
