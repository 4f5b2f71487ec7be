// Prefill grouping: stable counting sort of the T*K (row, slot) pairs by
// expert id (pairs keep their t*K+k order inside each expert group).
//   k_sort_hist     per-chunk expert histograms; the last-arriving workgroup
//                   scans them into counts, offsets and per-(chunk, expert)
//                   base positions.
//   k_sort_scatter  each pair's rank among earlier pairs of its chunk with the
//                   same expert gives its slot: perm[base + rank] = pair.
// Integer-only and deterministic; the result is unique. Optionally also the
// inverse permutation inv[pair] = sorted position.
#include <hip/hip_runtime.h>

#include "device_common.cuh"
#include "internal.h"

namespace moe {

constexpr int kSortChunk = 1024;   // pairs per workgroup

size_t sort_ws_bytes_tke(int64_t n, int E)
{
    const int64_t chunks = (n + kSortChunk - 1) / kSortChunk;
    return align256(sizeof(Control)) + align256(sizeof(int) * static_cast<size_t>(chunks) * E);
}

__global__ void __launch_bounds__(1024) k_sort_hist(const int32_t *ids, int n, int E, int *table, int32_t *counts,
                                                   int32_t *offsets, unsigned int *ticket)
{
    __shared__ int hist[kMaxE];
    __shared__ int scan[kMaxE];
    __shared__ int is_last;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x)
        hist[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * kSortChunk;
    for (int i = tid; i < kSortChunk && base + i < n; i += blockDim.x) {
        const int e = ids[base + i];
        if (e >= 0 && e < E)
            atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x)
        table[static_cast<size_t>(blockIdx.x) * E + e] = hist[e];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        is_last = atomicAdd(ticket, 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();
    const int C = gridDim.x;
    // per expert: running base over chunks (relative to the expert's group)
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int c = 0; c < C; ++c) {
            const int v = table[static_cast<size_t>(c) * E + e];
            table[static_cast<size_t>(c) * E + e] = run;
            run += v;
        }
        scan[e] = run;
        counts[e] = run;
    }
    __syncthreads();
    // exclusive scan of counts over experts (Hillis-Steele on an inclusive copy)
    for (int off = 1; off < E; off <<= 1) {
        int v = 0;
        if (tid < E && tid >= off)
            v = scan[tid - off];
        __syncthreads();
        if (tid < E)
            scan[tid] += v;
        __syncthreads();
    }
    for (int e = tid; e < E; e += blockDim.x) {
        const int excl = scan[e] - counts[e];
        offsets[e] = excl;
        for (int c = 0; c < C; ++c)
            table[static_cast<size_t>(c) * E + e] += excl;
    }
    if (tid == 0) {
        offsets[E] = scan[E - 1];
        *ticket = 0u;
    }
}

__global__ void __launch_bounds__(1024) k_sort_scatter(const int32_t *ids, int n, int E, const int *table,
                                                      int32_t *perm, int32_t *inv)
{
    __shared__ int le[kSortChunk];
    const int tid = threadIdx.x;
    const int base = blockIdx.x * kSortChunk;
    const int len = min(kSortChunk, n - base);
    for (int i = tid; i < len; i += blockDim.x)
        le[i] = ids[base + i];
    __syncthreads();
    for (int i = tid; i < len; i += blockDim.x) {
        const int e = le[i];
        if (e < 0 || e >= E)
            continue;
        int rank = 0;
        for (int j = 0; j < i; ++j)
            rank += (le[j] == e);
        const int pos = table[static_cast<size_t>(blockIdx.x) * E + e] + rank;
        perm[pos] = base + i;
        if (inv)
            inv[base + i] = pos;
    }
}

int launch_sort_by_expert(const int32_t *ids, int T, int K, int E, int32_t *counts, int32_t *offsets,
                          int32_t *perm, void *ws, hipStream_t s, int32_t *inv)
{
    const int n = T * K;
    const int chunks = (n + kSortChunk - 1) / kSortChunk;
    uint8_t *p = static_cast<uint8_t *>(ws);
    unsigned int *ticket = reinterpret_cast<unsigned int *>(p);
    int *table = reinterpret_cast<int *>(p + align256(sizeof(Control)));
    hipLaunchKernelGGL(k_sort_hist, dim3(chunks), dim3(1024), 0, s, ids, n, E, table, counts, offsets, ticket);
    if (hipGetLastError() != hipSuccess)
        return MOE_EHIP;
    hipLaunchKernelGGL(k_sort_scatter, dim3(chunks), dim3(1024), 0, s, ids, n, E, table, perm, inv);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
