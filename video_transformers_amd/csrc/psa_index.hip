// Block index of a level map: a CSR over (row, level) keys listing, for every
// (batch, head, query block) row and level l, the KV blocks at level l in ascending order.
// This is how the attention kernel learns which blocks to fetch at which level and never
// touches a skipped block (PSA summary article at rg.mbintangr.com, "Method": the least
// important blocks are skipped entirely).
//
// Four launches, all integer and deterministic:
//   k_index_count       one wave per row: per-level counts via ballots (bad entries -> skip + flag)
//   k_index_tile_sums   one workgroup per tile of 4096 counts: the tile's total
//   k_index_scan_tiles  one workgroup per tile: the totals of the tiles before it, then the
//                       tile's inclusive scan into row_ptr (in place)
//   k_index_fill        one wave per row: ballot compaction of each level's kb into col_idx
// The tile totals are parked at the start of col_idx, which the fill overwrites afterwards
// (its capacity, rows * NKB, is at least the number of tiles).
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

// Scan of the counts held in row_ptr[1..n] into their inclusive prefix sums (row_ptr[0] = 0),
// in tiles of kScanTile counts, kScanPer consecutive counts per thread.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 4;
constexpr int kScanTile = kScanThreads * kScanPer;

// Inclusive scan of one value per thread over the workgroup; `total` receives the sum.
__device__ int64_t block_inclusive_scan(int64_t v, int64_t& total) {
    __shared__ int64_t wsum[kScanThreads / 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
        const int64_t x = wsum[w];
        if (w < wave) before += x;
        all += x;
    }
    __syncthreads();   // wsum is reused by the next call
    total = all;
    return before + v;
}

__global__ void __launch_bounds__(kScanThreads)
    k_index_tile_sums(const int32_t* __restrict__ row_ptr, int64_t n, int32_t* __restrict__ sums) {
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kScanTile + threadIdx.x * kScanPer;
    int64_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j)
        if (i0 + j < n) s += row_ptr[i0 + j + 1];
    int64_t total;
    block_inclusive_scan(s, total);
    if (threadIdx.x == 0) sums[blockIdx.x] = static_cast<int32_t>(total);
}

__global__ void __launch_bounds__(kScanThreads)
    k_index_scan_tiles(int32_t* __restrict__ row_ptr, int64_t n, const int32_t* __restrict__ sums) {
    // the totals of the tiles before this one
    int64_t b = 0;
    for (int k = threadIdx.x; k < static_cast<int>(blockIdx.x); k += kScanThreads) b += sums[k];
    int64_t base;
    block_inclusive_scan(b, base);
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kScanTile + threadIdx.x * kScanPer;
    int32_t c[kScanPer];
    int64_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
        c[j] = i0 + j < n ? row_ptr[i0 + j + 1] : 0;
        s += c[j];
    }
    int64_t total;
    int64_t run = base + block_inclusive_scan(s, total) - s;   // exclusive prefix of this thread
#pragma unroll
    for (int j = 0; j < kScanPer; ++j)
        if (i0 + j < n) {
            run += c[j];
            row_ptr[i0 + j + 1] = static_cast<int32_t>(run);
        }
    if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
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
    const int64_t n = rows * 4;
    const unsigned tiles = static_cast<unsigned>((n + kScanTile - 1) / kScanTile);
    hipLaunchKernelGGL(k_index_tile_sums, dim3(tiles), dim3(kScanThreads), 0, st, ib.row_ptr, n, ib.col_idx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_index_scan_tiles, dim3(tiles), dim3(kScanThreads), 0, st, ib.row_ptr, n, ib.col_idx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_index_fill, dim3(blocks), dim3(256), 0, st, level_map, rows, s.NKB,
                       ib.row_ptr, ib.col_idx);
    return hipGetLastError();
}

}  // namespace psa
