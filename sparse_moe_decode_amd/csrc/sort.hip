// Prefill grouping: stable counting sort of the T*K (row, slot) pairs by
// expert id (pairs keep their t*K+k order inside each expert group).
//   k_sort_hist     per-chunk expert histograms (LDS counters).
//   k_sort_scan     one workgroup: per expert, the pairs of earlier chunks
//                   (running sums over the chunks, loads batched 8 chunks at
//                   a time), then counts and offsets (a scan over experts);
//                   for the prefill GEMMs also the row tiles (expert, first
//                   sorted row, rows of each tile).
//   k_sort_scatter  per chunk: per-wave histograms give the pairs of earlier
//                   waves, a broadcast loop the earlier lanes of the same
//                   wave; perm[offset + earlier chunks + earlier waves +
//                   earlier lanes] = pair.
// Integer-only and deterministic (LDS atomics only count); the result is
// unique. Optionally also the inverse permutation inv[pair] = sorted position.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "internal.h"
#include "workspace.hpp"

namespace moe {

constexpr int kSortWaves = kSortChunk / kWave;    // one pair per thread (kSortChunk: workspace.hpp)

__global__ void __launch_bounds__(kSortChunk) k_sort_hist(const int32_t *ids, int n, int E, int *table)
{
    __shared__ int hist[kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x)
        hist[e] = 0;
    __syncthreads();
    const int i = blockIdx.x * kSortChunk + tid;
    if (i < n) {
        const int e = ids[i];
        if (e >= 0 && e < E)
            atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x)
        table[static_cast<size_t>(blockIdx.x) * E + e] = hist[e];
}

// table[c][e] becomes the pairs of expert e in chunks before c; counts and
// offsets (exclusive scan over experts, Hillis-Steele in LDS).
__global__ void __launch_bounds__(kSortChunk) k_sort_scan(int C, int E, int *table, int32_t *counts,
                                                         int32_t *offsets, int bm, int max_tiles, int4 *tiles)
{
    __shared__ int sc[kMaxE], soff[kMaxE], scnt[kMaxE];
    const int tid = threadIdx.x;
    int total = 0;
    if (tid < E) {
        for (int c0 = 0; c0 < C; c0 += 8) {
            int v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                v[k] = c0 + k < C ? table[static_cast<size_t>(c0 + k) * E + tid] : 0;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (c0 + k < C) {
                    table[static_cast<size_t>(c0 + k) * E + tid] = total;
                    total += v[k];
                }
        }
        sc[tid] = total;
    }
    __syncthreads();
    for (int off = 1; off < E; off <<= 1) {
        const int v = (tid < E && tid >= off) ? sc[tid - off] : 0;
        __syncthreads();
        if (tid < E)
            sc[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        counts[tid] = total;
        offsets[tid] = sc[tid] - total;
        soff[tid] = sc[tid] - total;
        scnt[tid] = total;
        if (tid == E - 1)
            offsets[E] = sc[tid];
    }
    if (bm <= 0)
        return;
    // row tiles of bm rows per expert, in expert order: tiles[tix] =
    // (expert, first sorted row, rows) for tix < the number of tiles, and
    // (-1, 0, 0) up to max_tiles, so that a GEMM workgroup finds its tile
    // with one load
    const int v = tid < E ? (total + bm - 1) / bm : 0;
    __syncthreads();
    if (tid < E)
        sc[tid] = v;
    __syncthreads();
    for (int off = 1; off < E; off <<= 1) {
        const int a = (tid < E && tid >= off) ? sc[tid - off] : 0;
        __syncthreads();
        if (tid < E)
            sc[tid] += a;
        __syncthreads();
    }
    // expert of tile tix: the first e whose inclusive tile sum exceeds tix
    const int ntiles = sc[E - 1];
    for (int tix = tid; tix < max_tiles; tix += blockDim.x) {
        int4 t = make_int4(-1, 0, 0, 0);
        if (tix < ntiles) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sc[mid] > tix)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            const int first = sc[lo] - (scnt[lo] + bm - 1) / bm;   // the expert's first tile
            const int r0 = soff[lo] + (tix - first) * bm;
            t = make_int4(lo, r0, min(bm, soff[lo] + scnt[lo] - r0), 0);
        }
        tiles[tix] = t;
    }
}

__global__ void __launch_bounds__(kSortChunk) k_sort_scatter(const int32_t *ids, int n, int E, const int *table,
                                                            const int32_t *offsets, int32_t *perm, int32_t *inv)
{
    __shared__ int wh[kSortWaves][kMaxE];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    for (int w = 0; w < kSortWaves; ++w)
        for (int e = tid; e < E; e += blockDim.x)
            wh[w][e] = 0;
    __syncthreads();
    const int i = blockIdx.x * kSortChunk + tid;
    const int e = i < n ? ids[i] : -1;
    const bool valid = e >= 0 && e < E;
    if (valid)
        atomicAdd(&wh[wave][e], 1);
    __syncthreads();
    // per expert: first position of each wave's pairs
    for (int x = tid; x < E; x += blockDim.x) {
        int run = offsets[x] + table[static_cast<size_t>(blockIdx.x) * E + x];
        for (int w = 0; w < kSortWaves; ++w) {
            const int h = wh[w][x];
            wh[w][x] = run;
            run += h;
        }
    }
    __syncthreads();
    // earlier lanes of this wave with the same expert
    int r = 0;
    for (int j = 0; j < kWave; ++j) {
        const int ej = __builtin_amdgcn_readlane(e, j);
        r += (ej == e) & (j < lane);
    }
    if (valid) {
        const int pos = wh[wave][e] + r;
        perm[pos] = i;
        if (inv)
            inv[i] = pos;
    } else if (inv && i < n) {
        inv[i] = -1;
    }
}

int launch_sort_by_expert(const int32_t *ids, int T, int K, int E, int32_t *counts, int32_t *offsets,
                          int32_t *perm, void *ws, hipStream_t s, int32_t *inv, int bm, int max_tiles, int4 *tiles)
{
    const int n = T * K;
    const int chunks = (n + kSortChunk - 1) / kSortChunk;
    uint8_t *p = static_cast<uint8_t *>(ws);
    int *table = reinterpret_cast<int *>(p + align256(sizeof(Control)));
    hipLaunchKernelGGL(k_sort_hist, dim3(chunks), dim3(kSortChunk), 0, s, ids, n, E, table);
    hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(kSortChunk), 0, s, chunks, E, table, counts, offsets, bm, max_tiles,
                       tiles);
    hipLaunchKernelGGL(k_sort_scatter, dim3(chunks), dim3(kSortChunk), 0, s, ids, n, E, table, offsets, perm, inv);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
