// Block index of a level map: a CSR over (row, level) keys listing, for every
// (batch, head, query block) row and level l, the KV blocks at level l in ascending order.
// This is how the attention kernel learns which blocks to fetch at which level and never
// touches a skipped block (PSA summary article at rg.mbintangr.com, "Method": the least
// important blocks are skipped entirely).
//
// Five launches, all integer and deterministic:
//   k_index_count       one wave per row: per-level counts via ballots (bad entries -> skip + flag)
//   k_index_tile_sums   one workgroup per tile of 4096 counts: the tile's total
//   k_index_scan_tiles  one workgroup per tile: the totals of the tiles before it, then the
//                       tile's inclusive scan into row_ptr (in place)
//   k_index_fill        one wave per row: ballot compaction of each level's kb into col_idx
//   k_index_order       one workgroup per XCD range: the attention's dispatch order of the rows
//                       (after the offsets in row_ptr)
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

// Diagnostics: every word of the workgroup's 32 KB of LDS set to `pattern`. Launched with
// enough workgroups to cover every CU's LDS several times over, so the next kernels on the
// stream start on CUs whose LDS holds the pattern (LDS is not cleared between kernels).
constexpr int kFillLdsWords = 32 * 1024 / 4;

__global__ void __launch_bounds__(256) k_fill_lds(uint32_t pattern, int32_t* sink) {
    __shared__ uint32_t lds[kFillLdsWords];
    for (int i = threadIdx.x; i < kFillLdsWords; i += 256) lds[i] = pattern;
    __syncthreads();
    // one read keeps the stores (never true for a pattern the host passes with sink null)
    if (sink != nullptr && threadIdx.x == 0 && lds[blockIdx.x % kFillLdsWords] == ~pattern) sink[0] = 1;
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

// Dispatch order of the attention workgroups. Workgroup i runs on XCD i % 8, and the attention
// kernels give XCD x the slots of one contiguous range [x * nper, (x + 1) * nper), nper =
// ceil(rows / 8). The rows are grouped by KV head (rows / unit, unit = NQB * heads_q /
// heads_kv: the query heads that read one KV head), groups in ascending order, and inside a
// group listed by their number of 64-row tiles (sum over levels l of ceil(n_l / 2^l)), largest
// first: rows of similar tile counts have similar maps and fetch mostly the same blocks, and
// the workgroups started last are short ones (longest-processing-time-first list scheduling).
// The list is laid over the XCDs in chunks: f consecutive XCD ranges form a chunk, and
// inside a chunk list position j goes to XCD (chunk's first + j mod f), its local slot j / f,
// so the f XCDs work through the same rows, and the same KV head, at the same time (while
// each range has slots left; the list's tail then fills the remaining slots in order). f is
// the smallest of 1, 2, 4, 8 for which the K and V rows of all levels of the 8 / f KV heads
// in flight fit in half the 256 MB last-level cache (f = 1 when there is one (batch, KV
// head) only):
//  * f = 1 (contiguous ranges): each XCD takes whole KV heads (a group cut by a range
//    boundary is sorted in two parts) and neighbouring query blocks of a head share its L2;
//  * f = 2, 4: as f = 1 inside each range, the chunk's ranges interleaved;
//  * f = 8: whole groups sorted, the whole list interleaved over the eight XCDs.
// Each group: a stable counting sort over kOrderBuckets buckets spanning the group's tile
// counts (exact for spans up to kOrderBuckets, bucketed beyond); deterministic.
constexpr int kOrderThreads = 256;
constexpr int kOrderBuckets = 32;

// slot of list position i with f XCD ranges per chunk (see above); f = 1 is the identity
__device__ __forceinline__ int64_t chunk_slot(int64_t i, int64_t rows, int64_t nper, int f) {
    auto len = [&](int64_t x) {   // slots of XCD range x
        const int64_t n = rows - x * nper;
        return n < 0 ? int64_t{0} : (n < nper ? n : nper);
    };
    const int64_t x0 = (i / (f * nper)) * f;   // the chunk's first range
    int64_t j = i - x0 * nper;                 // position inside the chunk
    int64_t m = nper;                          // slots every range of the chunk has
    for (int k = 0; k < f; ++k) m = len(x0 + k) < m ? len(x0 + k) : m;
    if (j < f * m) return (x0 + j % f) * nper + j / f;
    j -= f * m;
    for (int k = 0; k < f; ++k) {   // the tail: the ranges' remaining slots, in order
        const int64_t rem = len(x0 + k) - m;
        if (j < rem) return (x0 + k) * nper + m + j;
        j -= rem;
    }
    return -1;   // not reached: the chunk has as many slots as positions
}

__device__ __forceinline__ int row_tiles(const int32_t* rp, int64_t r) {
    const int32_t* p = rp + r * 4;
    int t = 0;
#pragma unroll
    for (int l = 0; l < 4; ++l) t += (p[l + 1] - p[l] + (1 << l) - 1) >> l;
    return t;
}

// exclusive scan of one value per thread over kOrderThreads threads
__device__ int order_exclusive_scan(int v, int* wsum) {
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
#pragma unroll
    for (int w = 0; w < kOrderThreads / 64; ++w)
        if (w < wave) before += wsum[w];
    __syncthreads();
    return before + x - v;
}

__global__ void __launch_bounds__(kOrderThreads)
    k_index_order(const int32_t* __restrict__ row_ptr, int64_t rows, int64_t nper, int64_t unit,
                  int f, int32_t* __restrict__ order) {
    __shared__ int hist[kOrderBuckets * kOrderThreads];   // [bucket][thread]
    __shared__ int wred[2][kOrderThreads / 64];
    __shared__ int wsum[kOrderThreads / 64];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    // f < 8: the KV-head groups (or parts) of range blockIdx.x, one after another; f = 8: the
    // whole groups blockIdx.x, blockIdx.x + 8, ... (uniform loops)
    const bool whole = f == 8;
    const int64_t lo = whole ? static_cast<int64_t>(blockIdx.x) * unit : static_cast<int64_t>(blockIdx.x) * nper;
    const int64_t hi = whole ? rows : (lo + nper < rows ? lo + nper : rows);
    for (int64_t g_lo = lo; g_lo < hi;) {
        const int64_t g_end = (g_lo / unit + 1) * unit;
        const int64_t g_hi = g_end < hi ? g_end : hi;
        // thread t takes the consecutive rows [s0, s1) of the group
        const int64_t seg = (g_hi - g_lo + kOrderThreads - 1) / kOrderThreads;
        const int64_t s0 = g_lo + t * seg < g_hi ? g_lo + t * seg : g_hi;
        const int64_t s1 = s0 + seg < g_hi ? s0 + seg : g_hi;
        // the span of the tile counts
        int cmin = 0x7fffffff, cmax = 0;
        for (int64_t r = s0; r < s1; ++r) {
            const int c = row_tiles(row_ptr, r);
            cmin = min(cmin, c);
            cmax = max(cmax, c);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            cmin = min(cmin, __shfl_xor(cmin, o, 64));
            cmax = max(cmax, __shfl_xor(cmax, o, 64));
        }
        if (lane == 0) {
            wred[0][wave] = cmin;
            wred[1][wave] = cmax;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kOrderThreads / 64; ++w) {
            cmin = min(cmin, wred[0][w]);
            cmax = max(cmax, wred[1][w]);
        }
        const int span = cmax - cmin + 1;
        auto bucket = [&](int c) { return static_cast<int>((static_cast<int64_t>(cmax - c) * kOrderBuckets) / span); };
        // per (bucket, thread) counts, then their exclusive scan in bucket-major order: the
        // first position of each thread's rows of each bucket (stable: bucket, thread, row)
#pragma unroll
        for (int b = 0; b < kOrderBuckets; ++b) hist[b * kOrderThreads + t] = 0;
        for (int64_t r = s0; r < s1; ++r) ++hist[bucket(row_tiles(row_ptr, r)) * kOrderThreads + t];
        __syncthreads();
        constexpr int PER = kOrderBuckets;   // entries per thread
        int loc = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) loc += hist[t * PER + j];
        int run = order_exclusive_scan(loc, wsum);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = hist[t * PER + j];
            hist[t * PER + j] = run;
            run += c;
        }
        __syncthreads();
        for (int64_t r = s0; r < s1; ++r) {
            int* slot = &hist[bucket(row_tiles(row_ptr, r)) * kOrderThreads + t];
            const int64_t i = g_lo + *slot;   // list position
            order[f == 1 ? i : chunk_slot(i, rows, nper, f)] = static_cast<int32_t>(r);
            ++*slot;
        }
        __syncthreads();   // hist and wred are reused by the next group
        g_lo = whole ? g_hi + 7 * unit : g_hi;
    }
}

}  // namespace

hipError_t launch_clear_i32(int32_t* p, int n, hipStream_t st) {
    hipLaunchKernelGGL(k_clear_i32, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_fill_lds(uint32_t pattern, hipStream_t st) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // 160 KB of LDS per CU = 5 workgroups of 32 KB; four times that many
    hipLaunchKernelGGL(k_fill_lds, dim3(static_cast<unsigned>(cus) * 20), dim3(256), 0, st, pattern,
                       static_cast<int32_t*>(nullptr));
    return hipGetLastError();
}

// XCD ranges per chunk of the dispatch order: the smallest f of 1, 2, 4, 8 for which the K
// and V rows of all levels (N + 7N/8 rows each) of the 8 / f KV heads in flight fit in half the
// 256 MB last-level cache; 1 with a single (batch, KV head).
int order_share(const Shape& s) {
    if (static_cast<int64_t>(s.B) * s.Hkv <= 1) return 1;
    const int64_t elem = s.dtype == PSA_F32 ? 4 : 2;
    const int64_t per_head = (static_cast<int64_t>(s.N) + s.pooled_rows) * s.D * elem * 2;
    int f = 1;
    while (f < 8 && (8 / f) * per_head > (int64_t{128} << 20)) f *= 2;
    return f;
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
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t unit = static_cast<int64_t>(s.NQB) * (s.H / s.Hkv);   // rows per KV head
    hipLaunchKernelGGL(k_index_order, dim3(8), dim3(kOrderThreads), 0, st, ib.row_ptr, rows, (rows + 7) / 8,
                       unit, order_share(s), ib.row_ptr + rows * 4 + 1);
    return hipGetLastError();
}

}  // namespace psa
