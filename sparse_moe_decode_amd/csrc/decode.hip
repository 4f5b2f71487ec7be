// Decode (1 row) and few-row (2..4 rows) path of the sparse MoE layer on gfx950.
//
// Three launches per call on the caller's stream; kernel boundaries are the
// only synchronization between workgroups (no fences, counters or spin waits):
//   k_logits   router logits in fp64 (products of bf16/fp32 weights with fp32
//              activations are exact in double) plus the shared-gate logit,
//              one row per workgroup (a quarter of it per wave).
//   k_gateup   the shared expert's gate/up channels, and - in every other
//              workgroup - the exact top-K per row, softmax weights, sigmoid
//              gate and slot table (the union of the rows' experts; slot 0 is
//              the shared expert weighted by the gate: router, top-k and
//              shared gate as one step, the shared expert as an extra slot,
//              Research notes page, section 1, "Metal"), repeated per
//              workgroup from the logits, followed by one intermediate
//              channel per wave of one selected expert: gate and up rows
//              streamed with 16-byte non-temporal loads, SwiGLU, scaled by the
//              route weight.
//   k_down     one output row per wave: D_s[j] . h'_s summed over all slots,
//              so the weighted combine happens inside the dot product and
//              each y element is written once.
// Each distinct selected expert is read once per call, however many rows
// selected it (the few-row verify idea of the same page, section 1).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstddef>
#include <climits>
#include <mutex>
#include <type_traits>
#include <vector>

#include "device_common.hpp"
#include "internal.h"
#include "routing.hpp"

namespace moe {

// ================================================================ routing

// Union of the rows' selections: slot 0 is the shared expert (weight g),
// slots 1.. are the distinct routed experts in order of first appearance
// (row-major over [R][K]); the weight of a slot for row q is that row's route
// weight of the expert (0 if the row did not select it). Run by one wave.
// With `tab` (E ints of LDS, contents arbitrary) the rows' selections must
// hold distinct experts within each row, as computed routing does: each
// expert's first selection is then an LDS minimum over the selections, its
// slot the count of first selections before it, and each selection sets its
// own row's weight and mask bit (a few steps per lane). Without `tab` (caller
// routing, where a row may repeat an expert and its weights add up) every
// selection is compared with every other in a loop over the selections.
template <int R>
__device__ __forceinline__ void build_slots(RouteLds &rl, int K, int lane, int *tab = nullptr)
{
    if (R == 1) {
        // selections with an id below 0 (given ids outside [0, E)) get no slot
        const int e = lane < K ? rl.sel_e[0][lane] : -1;
        const unsigned long long lt = (1ull << lane) - 1ull;
        const unsigned long long valid = __ballot(e >= 0);
        const int slot = 1 + __popcll(valid & lt), ns = 1 + __popcll(valid);
        if (e >= 0) {
            rl.slots.expert[slot] = e;
            rl.slots.w[slot][0] = rl.sel_w[0][lane];
        }
        if (lane < ns) {
            rl.slots.rmask[lane] = 1u;
            rl.slots.pstart[lane] = lane;
        }
        if (lane == 0) {
            rl.slots.nslots = ns;
            rl.slots.pstart[ns] = ns;
            rl.slots.expert[0] = -1;
            rl.slots.w[0][0] = rl.g[0];
        }
        return;
    }
    // lane l < R*K holds selection l (row l / K)
    const int RK = R * K;
    const bool in = lane < RK;
    const int lq = in ? lane / K : 0, lk = in ? lane - lq * K : 0;
    const int e = in ? rl.sel_e[lq][lk] : -1;
    const float wl = in ? rl.sel_w[lq][lk] : 0.0f;
    const bool live = e >= 0;   // an id below 0 (given ids outside [0, E)) gets no slot
    const unsigned long long lt = (1ull << lane) - 1ull;
    bool first;
    int slot, ns;
    uint32_t rm = 0;
    if (tab) {
        if (live)
            tab[e] = kWave;
        __builtin_amdgcn_wave_barrier();
        if (live)
            atomicMin(&tab[e], lane);
        __builtin_amdgcn_wave_barrier();
        const int f = live ? tab[e] : kWave;
        first = live && f == lane;
        const unsigned long long mask = __ballot(first);
        ns = 1 + __popcll(mask);
        slot = live ? 1 + __popcll(mask & ((1ull << f) - 1ull)) : 0;
        for (int i = lane; i < (ns - 1) * R; i += kWave)
            rl.slots.w[1 + i / R][i % R] = 0.0f;
        for (int i = lane; i < ns - 1; i += kWave)
            rl.slots.rmask[1 + i] = 0u;
        __builtin_amdgcn_wave_barrier();
        if (live) {
            rl.slots.w[slot][lq] = wl;
            atomicOr(&rl.slots.rmask[slot], 1u << lq);
        }
        if (first)
            rl.slots.expert[slot] = e;
        __builtin_amdgcn_wave_barrier();
        if (first)
            rm = rl.slots.rmask[slot];
    } else {
        // the other selections are broadcast with readlane in uniform loops
        first = live;
        float wq[R];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            wq[q] = 0.0f;
            for (int k = 0; k < K; ++k) {
                const int j = q * K + k;
                const int ej = __builtin_amdgcn_readlane(e, j);
                const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
                const bool m = ej == e;
                first = first && !(m && j < lane);
                wq[q] += m ? wj : 0.0f;
                rm |= m ? 1u << q : 0u;
            }
        }
        const unsigned long long mask = __ballot(first);
        slot = 1 + __popcll(mask & lt);
        ns = 1 + __popcll(mask);
        if (first) {
            rl.slots.expert[slot] = e;
#pragma unroll
            for (int q = 0; q < R; ++q)
                rl.slots.w[slot][q] = wq[q];
            rl.slots.rmask[slot] = rm;
        }
    }
    // pair numbering: slot 0 (all rows) first, then the slots in order; the
    // prefix of the per-slot pair counts (< 8) from ballots of their bits
    const int cnt = first ? __popc(rm) : 0;
    int excl = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
        const unsigned long long mb = __ballot((cnt >> bit) & 1);
        excl += __popcll(mb & lt) << bit;
        total += __popcll(mb) << bit;
    }
    if (first)
        rl.slots.pstart[slot] = R + excl;
    if (lane == 0) {
        rl.slots.nslots = ns;
        rl.slots.expert[0] = -1;
        rl.slots.rmask[0] = (1u << R) - 1u;
        rl.slots.pstart[0] = 0;
#pragma unroll
        for (int q = 0; q < R; ++q)
            rl.slots.w[0][q] = rl.g[q];
    }
    if (lane == 0)
        rl.slots.pstart[ns] = R + total;
}

// Pair (row i of hbuf) of row q in `slot`, or -1 if the row does not use it.
__device__ __forceinline__ int pair_of(const SlotTable &t, int slot, int q)
{
    const uint32_t m = t.rmask[slot];
    return ((m >> q) & 1u) ? t.pstart[slot] + __popc(m & ((1u << q) - 1u)) : -1;
}

struct RouteArgs {
    const double *logits;      // [R][E]
    const double *zlogit;      // [R]
    int E, K, renorm;
    const int32_t *ids_in;     // [R][K] or null: routing given by the caller
    const float *wts_in, *gate_in;
    int32_t *ids_out;          // optional outputs
    float *wts_out, *gate_out;
    SlotTable *slots;          // published for the expert kernels (or null)
    const float *wbias;        // the router bias when it enters the selection only (weights without it), or null
};

constexpr int kRouteThreads = 256;   // threads of every workgroup that routes

static_assert(kRouteThreads == 4 * kWave, "one-row routing compacts four waves' candidates");

// One row routed by the whole workgroup: thread i holds experts i + 256 j
// (j < PT). The maxima of the fp32 keys over groups of 8 lanes (32 groups)
// give the threshold (kth_of_32: at or below the K-th largest logit), each
// wave compacts its own candidates, and wave 0 ranks them (rank_packed) while
// wave 1 evaluates the gate and writes the fixed part of the slot table. More
// than 64 candidates (massive ties) fall back to wave_route on the staged
// logits; keys shared near the boundary to exact fp64 ranking.
template <int PT>
__device__ __forceinline__ void route_block1(const RouteArgs &a, double *lg, RouteLds &rl)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int E = a.E, K = a.K;
    double v[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int e = tid + j * kRouteThreads;
        v[j] = e < E ? a.logits[e] : 0.0;
    }
    const double z = a.zlogit[0];
    uint32_t key[PT], mk = 0;   // 0 is below every key of a non-NaN value
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int e = tid + j * kRouteThreads;
        if (e < E)
            lg[e] = v[j];   // staged for the fallbacks and the softmax over all E
        key[j] = e < E ? f32_key(static_cast<float>(v[j])) : 0u;
        mk = key[j] > mk ? key[j] : mk;
    }
    // maximum over 8 lanes: quad permutations [1,0,3,2] and [2,3,0,1], then
    // the mirror within each half row
    uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mk), 0xB1, 0xF, 0xF, false));
    mk = o > mk ? o : mk;
    o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mk), 0x4E, 0xF, 0xF, false));
    mk = o > mk ? o : mk;
    o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mk), 0x141, 0xF, 0xF, false));
    mk = o > mk ? o : mk;
    if ((lane & 7) == 0)
        rl.pmax[0][wave * 8 + (lane >> 3)] = mk;
    __syncthreads();
    const uint32_t t = kth_of_32(rl.pmax[0], K, lane);
    // compaction within the wave: exclusive prefix of the per-lane counts
    bool c[PT];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        c[j] = (key[j] >= t) & (key[j] != 0);
        cnt += c[j];
    }
    const unsigned long long lt = (1ull << lane) - 1ull;
    int pos = 0, Cw = 0;
#pragma unroll
    for (int b = 0; (1 << b) <= PT; ++b) {
        const unsigned long long mb = __ballot((cnt >> b) & 1);
        pos += __popcll(mb & lt) << b;
        Cw += __popcll(mb) << b;
    }
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        if (c[j] && pos < kWave) {
            const int e = tid + j * kRouteThreads;
            rl.seg_p[wave][pos] = (static_cast<uint64_t>(key[j]) << 32) | static_cast<uint32_t>(~e);
        }
        pos += c[j];
    }
    if (lane == 0)
        rl.seg_n[wave] = Cw;
    __syncthreads();
    const int4 n = *reinterpret_cast<const int4 *>(rl.seg_n);
    const int C = n.x + n.y + n.z + n.w;
    if (wave == 0) {
        if (C <= kWave) {
            // lane l takes candidate l of the concatenated segments
            const int o1 = n.x, o2 = o1 + n.y, o3 = o2 + n.z;
            const int sw = (lane >= o1) + (lane >= o2) + (lane >= o3);
            const int si = lane - (sw == 0 ? 0 : sw == 1 ? o1 : sw == 2 ? o2 : o3);
            uint64_t p = 0;
            double val = 0.0;
            if (lane < C) {
                p = rl.seg_p[sw][si];
                val = lg[~static_cast<uint32_t>(p)];
                rl.cand_p[0][lane] = p;
            }
            if (!rank_packed(C, K, a.renorm, E, lg, z, false, 0, rl, lane, [&](uint64_t) { return val; },
                             &rl.slots, a.wbias)) {
                if (lane < C) {
                    rl.cand[0][lane] = static_cast<int>(~static_cast<uint32_t>(p));
                    rl.cand_v[0][lane] = val;
                }
                rank_exact(C, K, 0, rl, lane);
                wave_weights(lg, E, K, a.renorm, z, 0, rl, lane, false, a.wbias);
                if (lane < K) {
                    rl.slots.expert[lane + 1] = rl.sel_e[0][lane];
                    rl.slots.w[lane + 1][0] = rl.sel_w[0][lane];
                }
            }
        } else {
            wave_route(lg, E, K, a.renorm, z, 0, rl, lane, a.wbias);
            build_slots<1>(rl, K, lane);
        }
    } else if (wave == 1 && C <= kWave) {
        // the gate and the slots' fixed part (slot 0 = shared expert)
        if (lane == 0) {
            const float g = 1.0f / (1.0f + expf(static_cast<float>(-z)));
            rl.g[0] = g;
            rl.slots.w[0][0] = g;
            rl.slots.expert[0] = -1;
            rl.slots.nslots = K + 1;
            rl.slots.pstart[K + 1] = K + 1;
        }
        if (lane <= K) {
            rl.slots.rmask[lane] = 1u;
            rl.slots.pstart[lane] = lane;
        }
    }
    __syncthreads();
}

// Routing of the call's R rows inside one workgroup of kRouteThreads: one
// row by the whole workgroup (route_block1), or wave q selects row q from the
// logits (staged in `lg`, R rows of (E+1)&~1 doubles) and wave 0 then builds
// the slot table; or the caller's selection is taken as given (ids outside
// [0, E) get no slot: nothing of them is read or added). Ends with a
// workgroup barrier, after which `lg` may be reused.
template <int R>
__device__ __forceinline__ void route_block(const RouteArgs &a, double *lg, RouteLds &rl)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    if (a.ids_in) {
        if (tid < R * a.K) {
            const int q = tid / a.K, k = tid - q * a.K;
            const int e = a.ids_in[tid];
            const bool ok = e >= 0 && e < a.E;
            rl.sel_e[q][k] = ok ? e : -1;
            rl.sel_w[q][k] = ok ? a.wts_in[tid] : 0.0f;
        }
        if (tid < R)
            rl.g[tid] = a.gate_in[tid];
    } else if (R == 1) {
        if (a.E <= kRouteThreads)
            route_block1<1>(a, lg, rl);
        else if (a.E <= 2 * kRouteThreads)
            route_block1<2>(a, lg, rl);
        else
            route_block1<kMaxE / kRouteThreads>(a, lg, rl);
        return;   // ends with a workgroup barrier
    } else {
        // every load is issued before the first LDS store
        constexpr int PT = kMaxE / kRouteThreads;
        const int lgs = (a.E + 1) & ~1;
        double v[R][PT];
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int u = 0; u < PT; ++u) {
                const int i = tid + u * kRouteThreads;
                v[q][u] = i < a.E ? a.logits[q * a.E + i] : 0.0;
            }
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int u = 0; u < PT; ++u) {
                const int i = tid + u * kRouteThreads;
                if (i < a.E)
                    lg[q * lgs + i] = v[q][u];
            }
        __syncthreads();
        if (wave < R) {
            wave_route(lg + wave * lgs, a.E, a.K, a.renorm, a.zlogit[wave], wave, rl, lane, a.wbias);
        }
    }
    __syncthreads();
    // the staged logits are no longer read: their space holds the per-expert
    // table of build_slots (computed routing only)
    if (wave == 0)
        build_slots<R>(rl, a.K, lane, a.ids_in ? nullptr : reinterpret_cast<int *>(lg));
    __syncthreads();
}

// The routing of route_block to global memory: the selection, weights and
// gate (when computed here and asked for) and the slot table (if a.slots).
template <int R>
__device__ __forceinline__ void publish_route(const RouteArgs &a, const RouteLds &rl)
{
    const int tid = threadIdx.x;
    if (!a.ids_in) {
        if (tid < R * a.K) {
            const int q = tid / a.K, k = tid - q * a.K;
            if (a.ids_out)
                a.ids_out[tid] = rl.sel_e[q][k];
            if (a.wts_out)
                a.wts_out[tid] = rl.sel_w[q][k];
        }
        if (tid < R && a.gate_out)
            a.gate_out[tid] = rl.g[tid];
    }
    if (a.slots) {
        const int ns = rl.slots.nslots;
        if (tid == 0)
            a.slots->nslots = ns;
        for (int i = tid; i < ns; i += blockDim.x) {
            a.slots->expert[i] = rl.slots.expert[i];
            a.slots->rmask[i] = rl.slots.rmask[i];
            a.slots->pstart[i] = rl.slots.pstart[i];
#pragma unroll
            for (int q = 0; q < R; ++q)
                a.slots->w[i][q] = rl.slots.w[i][q];
        }
        if (tid == 0)
            a.slots->pstart[ns] = rl.slots.pstart[ns];
    }
}

// Routing on its own (the route-only entry point): one workgroup.
template <int R>
__global__ void __launch_bounds__(kRouteThreads) k_route(RouteArgs a)
{
    extern __shared__ __align__(16) unsigned char lds_raw[];
    __shared__ RouteLds rl;
    route_block<R>(a, reinterpret_cast<double *>(lds_raw), rl);
    publish_route<R>(a, rl);
}

// ============================================================ gate / up

struct GateUpArgs {
    const float *x;            // [R][H]
    const float *norm_w;       // RMS norm gamma [H], or null
    float norm_eps;
    int H, I, Is, Imax;
    const uint8_t *eg, *eu;    // routed gate/up stacks
    size_t estride;            // bytes per routed [I][H] matrix
    const uint8_t *sg, *su;    // shared gate/up
    const SlotTable *slots;
    float *hbuf;               // [S][R][Imax]
    int ch_per_wg;             // channels per workgroup (one per wave)
    int wg_per_slot;           // workgroups per routed slot
};

constexpr int kGuWaves = 4;
static_assert(kGuWaves * kWave == kRouteThreads, "gate/up workgroups route");
// Waves per SIMD the one-row gate/up kernel is compiled for (a register
// budget of 512/6 per lane): six 4-wave workgroups per CU keep a decode
// call's 1,400-odd workgroups resident at once, so none waits for a free slot
// and then repeats the routing late.
constexpr int kGuMinWaves = 6;
// Few-row calls: four waves per SIMD (128 registers), enough for the two
// sets of rows in flight of 2-bit rows; bf16 / fp32 rows (four 16-byte
// chunks per row and lane) get three (168 registers: at four they spilled,
// and R = 2 / 3 calls of the bf16 layer took 45 / 71 us instead of 41 / 58).
constexpr int kGuMinWavesRows = 4;
constexpr int kGuMinWavesRowsWide = 3;
// Chunks per lane in flight per row: four 16-byte chunks (a 2048-wide bf16
// row per wave), or one 2-bit block (a 2048-wide row per wave; wider rows
// stream in steps).
template <typename W>
struct GuChunks {
    static constexpr int value = 4;
};
template <int B>
struct GuChunks<QB<B>> {
    static constexpr int value = 1;
};

// Raw row chunks of one channel (gate and up), GuChunks<W> per lane.
template <typename W>
struct RowChunks {
    uint4 g[GuChunks<W>::value], u[GuChunks<W>::value];
};
template <int B>
struct RowChunks<QB<B>> {   // 3- and 4-bit blocks: the block's code dwords and its scale/min word
    uint32_t gc[B], uc[B];
    uint32_t gs, us;
};
template <>
struct RowChunks<Q2> {
    uint2 gc[GuChunks<Q2>::value], uc[GuChunks<Q2>::value];
    uint32_t gs[GuChunks<Q2>::value], us[GuChunks<Q2>::value];
};

template <typename W>
__device__ __forceinline__ void load_rows(W, const MatRef &G, const MatRef &U, int ch, int base, int lane, int nch,
                                          RowChunks<W> &r)
{
    constexpr int esz = W::kChunk == 4 ? 4 : 2;   // f32 / bf16 element bytes
#pragma unroll
    for (int u = 0; u < GuChunks<W>::value; ++u) {
        const int k = base + u * kWave + lane;
        if (k < nch) {
            r.g[u] = ld_nt16(G.base + (static_cast<size_t>(ch) * G.cols + k * W::kChunk) * esz);
            r.u[u] = ld_nt16(U.base + (static_cast<size_t>(ch) * U.cols + k * W::kChunk) * esz);
        }
    }
}
__device__ __forceinline__ void load_rows(Q2, const MatRef &G, const MatRef &U, int ch, int base, int lane, int nch,
                                          RowChunks<Q2> &r)
{
    const int nb = G.cols >> 5;
#pragma unroll
    for (int u = 0; u < GuChunks<Q2>::value; ++u) {
        const int b = base + u * kWave + lane;
        if (b < nch) {
            r.gc[u] = ld_nt8(G.base + static_cast<size_t>(ch) * (G.cols >> 2) + b * 8);
            r.uc[u] = ld_nt8(U.base + static_cast<size_t>(ch) * (U.cols >> 2) + b * 8);
            r.gs[u] = ld_nt4(G.base + static_cast<size_t>(G.rows) * (G.cols >> 2) +
                                                          (static_cast<size_t>(ch) * nb + b) * 4);
            r.us[u] = ld_nt4(U.base + static_cast<size_t>(U.rows) * (U.cols >> 2) +
                                                          (static_cast<size_t>(ch) * nb + b) * 4);
        }
    }
}

// The 4b code bytes of a 3- or 4-bit block (4-byte aligned) as dwords.
template <int B>
__device__ __forceinline__ void load_block_codes(const uint8_t *p, uint32_t (&cw)[B])
{
    if constexpr (B == 4) {
        const uint4 v = ld_nt16(p);
        cw[0] = v.x;
        cw[1] = v.y;
        cw[2] = v.z;
        cw[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < B; ++i)
            cw[i] = ld_nt4(p + 4 * i);
    }
}
template <int B>
__device__ __forceinline__ void load_rows(QB<B>, const MatRef &G, const MatRef &U, int ch, int base, int lane, int nch,
                                          RowChunks<QB<B>> &r)
{
    const int nb = G.cols >> 5;
    const int b = base + lane;
    if (b < nch) {
        const size_t blk = static_cast<size_t>(ch) * nb + b;
        load_block_codes<B>(G.base + blk * 4 * B, r.gc);
        load_block_codes<B>(U.base + blk * 4 * B, r.uc);
        r.gs = ld_nt4(G.base + static_cast<size_t>(G.rows) * nb * 4 * B + blk * 4);
        r.us = ld_nt4(U.base + static_cast<size_t>(U.rows) * nb * 4 * B + blk * 4);
    }
}

template <int R>
__device__ __forceinline__ void dot_chunk(F32, const uint4 &w, int k, const float *xs, int H, float (&acc)[R])
{
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 xv = *reinterpret_cast<const float4 *>(xs + q * H + k * 4);
        acc[q] = fmaf(__uint_as_float(w.x), xv.x, acc[q]);
        acc[q] = fmaf(__uint_as_float(w.y), xv.y, acc[q]);
        acc[q] = fmaf(__uint_as_float(w.z), xv.z, acc[q]);
        acc[q] = fmaf(__uint_as_float(w.w), xv.w, acc[q]);
    }
}
template <int R>
__device__ __forceinline__ void dot_chunk(BF16, const uint4 &w, int k, const float *xs, int H, float (&acc)[R])
{
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 x0 = *reinterpret_cast<const float4 *>(xs + q * H + k * 8);
        const float4 x1 = *reinterpret_cast<const float4 *>(xs + q * H + k * 8 + 4);
        float a = acc[q];
        a = fmaf(bf16_lo(w.x), x0.x, a);
        a = fmaf(bf16_hi(w.x), x0.y, a);
        a = fmaf(bf16_lo(w.y), x0.z, a);
        a = fmaf(bf16_hi(w.y), x0.w, a);
        a = fmaf(bf16_lo(w.z), x1.x, a);
        a = fmaf(bf16_hi(w.z), x1.y, a);
        a = fmaf(bf16_lo(w.w), x1.z, a);
        a = fmaf(bf16_hi(w.w), x1.w, a);
        acc[q] = a;
    }
}
// 2-bit blocks read x one block per lane, 128 bytes apart, which would put
// eight lanes of every ds_read_b128 quarter on the same banks. x is staged
// with the 16-byte chunks of block b permuted by c -> c ^ (b & 7) (see
// stage_x), so step s of a lane reads physical chunk s (an immediate offset)
// and the lanes of a quarter spread over the banks; the block's code bytes
// are permuted the same way once per block.
__device__ __forceinline__ int x_chunk_slot(int b, int c) { return c ^ (b & 7); }

// Code word of a 32-weight block with its 4-weight bytes reordered so that
// byte s holds the codes of logical chunk s ^ m (m = b & 7).
__device__ __forceinline__ uint2 codes_for_slots(const uint2 &cw, int m)
{
    const uint32_t w0 = (m & 4) ? cw.y : cw.x, w1 = (m & 4) ? cw.x : cw.y;
    const uint32_t sel = 0x03020100u ^ (static_cast<uint32_t>(m & 3) * 0x01010101u);
    return make_uint2(__builtin_amdgcn_perm(0u, w0, sel), __builtin_amdgcn_perm(0u, w1, sel));
}

// The gate and up blocks at the same position share their x values: each
// float4 of x is used for both as soon as it is read. Codes are converted
// four at a time: (d >> 2k) & 0x03030303 holds code k of the four slots of
// dword d, one per byte, and each byte becomes a float with one byte
// conversion (1.5 instructions per code instead of an extract and a
// conversion each).
template <int R>
__device__ __forceinline__ void dot_block2(const uint2 &gc0, uint32_t gsm, const uint2 &uc0, uint32_t usm, int b,
                                           const float *xs, int H, const float *xsum, float (&a)[R], float (&c)[R])
{
    const float gsc = f16_to_f32(gsm & 0xffffu), gmn = f16_to_f32(gsm >> 16);
    const float usc = f16_to_f32(usm & 0xffffu), umn = f16_to_f32(usm >> 16);
    const uint2 gc = codes_for_slots(gc0, b & 7), uc = codes_for_slots(uc0, b & 7);
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 *x = reinterpret_cast<const float4 *>(xs + q * H + b * 32);
        float ga = 0.0f, ua = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t dg = half ? gc.y : gc.x, du = half ? uc.y : uc.x;
            const float4 x0 = x[4 * half], x1 = x[4 * half + 1], x2 = x[4 * half + 2], x3 = x[4 * half + 3];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // byte j of mg / mu: code k of slot 4 * half + j; opaque, so that
                // the byte conversions are not folded back into 2-bit extracts
                uint32_t mg = (dg >> (2 * k)) & 0x03030303u, mu = (du >> (2 * k)) & 0x03030303u;
                asm("" : "+v"(mg), "+v"(mu));
                const float e0 = k == 0 ? x0.x : k == 1 ? x0.y : k == 2 ? x0.z : x0.w;
                const float e1 = k == 0 ? x1.x : k == 1 ? x1.y : k == 2 ? x1.z : x1.w;
                const float e2 = k == 0 ? x2.x : k == 1 ? x2.y : k == 2 ? x2.z : x2.w;
                const float e3 = k == 0 ? x3.x : k == 1 ? x3.y : k == 2 ? x3.z : x3.w;
                ga = fmaf(static_cast<float>(mg & 0xffu), e0, ga);
                ga = fmaf(static_cast<float>((mg >> 8) & 0xffu), e1, ga);
                ga = fmaf(static_cast<float>((mg >> 16) & 0xffu), e2, ga);
                ga = fmaf(static_cast<float>(mg >> 24), e3, ga);
                ua = fmaf(static_cast<float>(mu & 0xffu), e0, ua);
                ua = fmaf(static_cast<float>((mu >> 8) & 0xffu), e1, ua);
                ua = fmaf(static_cast<float>((mu >> 16) & 0xffu), e2, ua);
                ua = fmaf(static_cast<float>(mu >> 24), e3, ua);
            }
        }
        const float sx = xsum[q * (H >> 5) + b];
        a[q] = fmaf(gsc, ga, fmaf(gmn, sx, a[q]));
        c[q] = fmaf(usc, ua, fmaf(umn, sx, c[q]));
    }
}

// 3- and 4-bit blocks: the codes stay in place (extracted at fixed bit
// positions) and x chunk c of the block is read from its staged slot
// x_chunk_slot(b, c).
template <int B, int R>
__device__ __forceinline__ void dot_block_b(const uint32_t (&gc)[B], uint32_t gsm, const uint32_t (&uc)[B],
                                            uint32_t usm, int b, const float *xs, int H, const float *xsum,
                                            float (&a)[R], float (&c)[R])
{
    float ga[R], ua[R];
#pragma unroll
    for (int q = 0; q < R; ++q)
        ga[q] = ua[q] = 0.0f;
    // the slot offset of the block, opaque so that the eight slot addresses
    // are formed here (one xor each) rather than hoisted out of the item
    // loop, where they would be held in registers for the whole kernel
    int m = b & 7;
    asm volatile("" : "+v"(m));
    // chunk by chunk: its 4 gate and 4 up codes once, then every row
#pragma unroll
    for (int cl = 0; cl < 8; ++cl) {
        float g[4], u[4];
        if constexpr (B == 4) {
            // dword cl / 2 holds chunks cl & ~1 and cl | 1; masking nibble k of
            // every byte gives codes (k, k + 2) of both chunks, one per byte,
            // converted with one byte conversion each (done for the even chunk)
            const int t = cl >> 1, hb = 2 * (cl & 1);
            uint32_t g0 = gc[t] & 0x0f0f0f0fu, g1 = (gc[t] >> 4) & 0x0f0f0f0fu;
            uint32_t u0 = uc[t] & 0x0f0f0f0fu, u1 = (uc[t] >> 4) & 0x0f0f0f0fu;
            asm("" : "+v"(g0), "+v"(g1), "+v"(u0), "+v"(u1));
            g[0] = static_cast<float>((g0 >> (8 * hb)) & 0xffu);
            g[1] = static_cast<float>((g1 >> (8 * hb)) & 0xffu);
            g[2] = static_cast<float>((g0 >> (8 * hb + 8)) & 0xffu);
            g[3] = static_cast<float>((g1 >> (8 * hb + 8)) & 0xffu);
            u[0] = static_cast<float>((u0 >> (8 * hb)) & 0xffu);
            u[1] = static_cast<float>((u1 >> (8 * hb)) & 0xffu);
            u[2] = static_cast<float>((u0 >> (8 * hb + 8)) & 0xffu);
            u[3] = static_cast<float>((u1 >> (8 * hb + 8)) & 0xffu);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                g[k] = static_cast<float>(block_code<B>(gc, 4 * cl + k));
                u[k] = static_cast<float>(block_code<B>(uc, 4 * cl + k));
            }
        }
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const float4 xv = reinterpret_cast<const float4 *>(xs + q * H + b * 32)[cl ^ m];   // x_chunk_slot(b, cl)
            ga[q] = fmaf(g[0], xv.x, fmaf(g[1], xv.y, fmaf(g[2], xv.z, fmaf(g[3], xv.w, ga[q]))));
            ua[q] = fmaf(u[0], xv.x, fmaf(u[1], xv.y, fmaf(u[2], xv.z, fmaf(u[3], xv.w, ua[q]))));
        }
    }
    const float gsc = f16_to_f32(gsm & 0xffffu), gmn = f16_to_f32(gsm >> 16);
    const float usc = f16_to_f32(usm & 0xffffu), umn = f16_to_f32(usm >> 16);
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float sx = xsum[q * (H >> 5) + b];
        a[q] = fmaf(gsc, ga[q], fmaf(gmn, sx, a[q]));
        c[q] = fmaf(usc, ua[q], fmaf(umn, sx, c[q]));
    }
}

template <int R, typename W>
__device__ __forceinline__ void dot_rows(W, const RowChunks<W> &r, int base, int lane, int nch, const float *xs,
                                         int H, const float *, float (&a)[R], float (&c)[R])
{
#pragma unroll
    for (int u = 0; u < GuChunks<W>::value; ++u) {
        const int k = base + u * kWave + lane;
        if (k < nch) {
            dot_chunk<R>(W{}, r.g[u], k, xs, H, a);
            dot_chunk<R>(W{}, r.u[u], k, xs, H, c);
        }
    }
}
template <int R>
__device__ __forceinline__ void dot_rows(Q2, const RowChunks<Q2> &r, int base, int lane, int nch, const float *xs,
                                         int H, const float *xsum, float (&a)[R], float (&c)[R])
{
#pragma unroll
    for (int u = 0; u < GuChunks<Q2>::value; ++u) {
        const int b = base + u * kWave + lane;
        if (b < nch)
            dot_block2<R>(r.gc[u], r.gs[u], r.uc[u], r.us[u], b, xs, H, xsum, a, c);
    }
}
template <int R, int B>
__device__ __forceinline__ void dot_rows(QB<B>, const RowChunks<QB<B>> &r, int base, int lane, int nch,
                                         const float *xs, int H, const float *xsum, float (&a)[R], float (&c)[R])
{
    const int b = base + lane;
    if (b < nch)
        dot_block_b<B, R>(r.gc, r.gs, r.uc, r.us, b, xs, H, xsum, a, c);
}

// x of all rows into LDS (with the layer's RMS norm applied when gamma is
// given), plus per-32 block sums when W is a block format.
template <int R, typename W>
__device__ __forceinline__ void stage_x(const float *x, int H, float *xs, float *xsum, const float *gamma, float eps)
{
    // block formats: chunk c of block b of a row at slot x_chunk_slot(b, c)
    const int n4 = H >> 2;
    for (int i = threadIdx.x; i < R * n4; i += blockDim.x) {
        int d = i;
        if (W::kChunk == 32) {
            const int q = i / n4, r = i - q * n4;
            d = q * n4 + (r & ~7) + x_chunk_slot(r >> 3, r & 7);
        }
        reinterpret_cast<float4 *>(xs)[d] = reinterpret_cast<const float4 *>(x)[i];
    }
    if (gamma) {
        if (W::kChunk == 32)
            rms_norm_rows<R>(xs, H, gamma, eps, SlotsQ2{});
        else
            rms_norm_rows<R>(xs, H, gamma, eps, SlotsInOrder{});
    } else {
        __syncthreads();
    }
    if (W::kChunk == 32) {
        for (int i = threadIdx.x; i < R * (H >> 5); i += blockDim.x) {
            float s = 0.0f;
            for (int j = 0; j < 32; ++j)
                s += xs[i * 32 + j];
            xsum[i] = s;
        }
        __syncthreads();
    }
}

// h'(pair of row q)[ch] = w_q * silu(a_q) * c_q for one channel, from lane
// partials; rows with pair < 0 are not written.
template <int R>
__device__ __forceinline__ void finish_channel(const GateUpArgs &p, const int (&pair)[R], int ch, float (&a)[R],
                                               float (&c)[R], const float (&wq)[R], int lane)
{
#pragma unroll
    for (int q = 0; q < R; ++q) {
        a[q] = wave_sum(a[q]);
        c[q] = wave_sum(c[q]);
    }
    if (lane < R) {
        float hv = 0.0f;
        int pr = -1;
#pragma unroll
        for (int q = 0; q < R; ++q)
            if (q == lane) {
                hv = silu_mul(a[q], c[q]) * wq[q];
                pr = pair[q];
            }
        if (pr >= 0)
            p.hbuf[static_cast<size_t>(pr) * p.Imax + ch] = hv;
    }
}

// One routed channel for the rows that use its slot: the rows' dot products
// one at a time from the loaded gate/up rows, h' written to the row's pair.
template <int R, typename W>
__device__ __forceinline__ void routed_channel(const GateUpArgs &p, const RowChunks<W> &r, const SlotTable &t,
                                               int slot, int ch, const float *xs, const float *xsum, int lane)
{
    const int nck = p.H / W::kChunk;
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int pr = R == 1 ? slot : pair_of(t, slot, q);   // one row: every slot is the row's, pair = slot
        if (pr >= 0) {
            float a[1] = {0.0f}, c[1] = {0.0f};
            dot_rows<1>(W{}, r, 0, lane, nck, xs + q * p.H, p.H, xsum + q * (p.H >> 5), a, c);
            const float hv = silu_mul(wave_sum(a[0]), wave_sum(c[0])) * t.w[slot][q];
            if (lane == 0)
                p.hbuf[static_cast<size_t>(pr) * p.Imax + ch] = hv;
        }
    }
}

// One channel of rows wider than one chunk set (H > 256 * chunk): the gate
// and up rows stream in steps; x is already staged.
template <int R, typename W>
__device__ __forceinline__ void gateup_wide(const GateUpArgs &p, const MatRef &G, const MatRef &U, const int (&pair)[R],
                                            int ch, const float (&wq)[R], const float *xs, const float *xsum)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int nck = p.H / W::kChunk;
    float a[R], c[R];
#pragma unroll
    for (int q = 0; q < R; ++q)
        a[q] = c[q] = 0.0f;
    for (int base = 0; base < nck; base += kWave * GuChunks<W>::value) {
        RowChunks<W> part;
        load_rows(W{}, G, U, ch, base, lane, nck, part);
        dot_rows<R>(W{}, part, base, lane, nck, xs, p.H, xsum, a, c);
    }
    finish_channel<R>(p, pair, ch, a, c, wq, lane);
}

// Channel ch (< n, or nothing) of the shared expert by this wave, all rows
// with weight 1. x is staged here (every wave takes part in the barrier).
// When a row fits one chunk set (H <= 256 * chunk), the gate and up rows
// are requested before x is staged, so the weight stream overlaps the staging.
template <int R, typename W>
__device__ __forceinline__ void gateup_one(const GateUpArgs &p, const MatRef &G, const MatRef &U, int ch, int n,
                                           const float (&wq)[R], float *xs, float *xsum)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int nck = p.H / W::kChunk;
    int pair[R];   // the shared expert's pairs are rows 0..R-1
#pragma unroll
    for (int q = 0; q < R; ++q)
        pair[q] = q;
    if (nck <= kWave * GuChunks<W>::value) {
        float a[R], c[R];
#pragma unroll
        for (int q = 0; q < R; ++q)
            a[q] = c[q] = 0.0f;
        RowChunks<W> r;
        if (ch < n)
            load_rows(W{}, G, U, ch, 0, lane, nck, r);
        stage_x<R, W>(p.x, p.H, xs, xsum, p.norm_w, p.norm_eps);
        if (ch < n) {
            dot_rows<R>(W{}, r, 0, lane, nck, xs, p.H, xsum, a, c);
            finish_channel<R>(p, pair, ch, a, c, wq, lane);
        }
        return;
    }
    stage_x<R, W>(p.x, p.H, xs, xsum, p.norm_w, p.norm_eps);
    if (ch < n)
        gateup_wide<R, W>(p, G, U, pair, ch, wq, xs, xsum);
}

// Gate/up of one call. Workgroups [0, n_sh) take channels of the shared
// expert (unweighted; the gate multiplies them in the down pass) and start
// streaming at once. Every later workgroup b first repeats the call's routing
// from the logits (route_block: about a microsecond of one wave per row, hidden
// behind the shared expert's stream), then takes channels of slot
// 1 + b / wg_per_slot; workgroup b == 0 publishes the routing for the down pass
// and the caller.
template <int R, typename ET, typename ST>
__global__ void __launch_bounds__(kGuWaves * kWave,
                                  R == 1 ? kGuMinWaves : (ET::kChunk == 32 ? kGuMinWavesRows : kGuMinWavesRowsWide))
    k_gateup(GateUpArgs p, RouteArgs ra, int n_sh)
{
    extern __shared__ __align__(16) unsigned char lds_raw[];
    float *xs = reinterpret_cast<float *>(lds_raw);   // [R][H]
    float *xsum = xs + R * p.H;                       // [R][H/32]
    __shared__ RouteLds rl;
    const int wave = threadIdx.x / kWave;
    if (static_cast<int>(blockIdx.x) < n_sh) {
        const MatRef G{p.sg, p.Is, p.H}, U{p.su, p.Is, p.H};
        float one[R];
#pragma unroll
        for (int q = 0; q < R; ++q)
            one[q] = 1.0f;
        gateup_one<R, ST>(p, G, U, blockIdx.x * p.ch_per_wg + wave, p.Is, one, xs, xsum);
        return;
    }
    const int b = blockIdx.x - n_sh;
    route_block<R>(ra, reinterpret_cast<double *>(lds_raw), rl);
    if (b == 0)
        publish_route<R>(ra, rl);
    // work items: ch_per_wg channels of one routed slot; item i is slot
    // 1 + i / wg_per_slot; the routed workgroups stride over the items
    const int nitems = (rl.slots.nslots - 1) * p.wg_per_slot;
    if (b >= nitems)
        return;
    const int stride = gridDim.x - n_sh;
    const int lane = threadIdx.x & (kWave - 1);
    auto item_mats = [&](int it, int &slot, int &ch, MatRef &G, MatRef &U) {
        slot = 1 + it / p.wg_per_slot;
        ch = (it % p.wg_per_slot) * p.ch_per_wg + wave;
        const int e = rl.slots.expert[slot];
        G = MatRef{p.eg + e * p.estride, p.I, p.H};
        U = MatRef{p.eu + e * p.estride, p.I, p.H};
    };
    const int nck = p.H / ET::kChunk;
    if (nck > kWave * GuChunks<ET>::value) {
        // wide rows: each item streams its rows in steps
        stage_x<R, ET>(p.x, p.H, xs, xsum, p.norm_w, p.norm_eps);
        for (int it = b; it < nitems; it += stride) {
            int slot, ch;
            MatRef G, U;
            item_mats(it, slot, ch, G, U);
            float w[R];
            int pair[R];
#pragma unroll
            for (int q = 0; q < R; ++q) {
                w[q] = rl.slots.w[slot][q];
                pair[q] = pair_of(rl.slots, slot, q);
            }
            if (ch < p.I)
                gateup_wide<R, ET>(p, G, U, pair, ch, w, xs, xsum);
        }
        return;
    }
    if constexpr (R == 1) {
        // decode: normally one item per routed workgroup
        auto one_item = [&](int it, bool first) {
            int slot, ch;
            MatRef G, U;
            item_mats(it, slot, ch, G, U);
            RowChunks<ET> r;
            if (ch < p.I)
                load_rows(ET{}, G, U, ch, 0, lane, nck, r);
            if (first)
                stage_x<R, ET>(p.x, p.H, xs, xsum, p.norm_w, p.norm_eps);
            if (ch < p.I)
                routed_channel<R, ET>(p, r, rl.slots, slot, ch, xs, xsum, lane);
        };
        one_item(b, true);
        for (int it = b + stride; it < nitems; it += stride)
            one_item(it, false);
    } else {
        // few-row: the next item's rows are requested before the current
        // one is reduced
        int it = b, slot, ch;
        MatRef G, U;
        item_mats(it, slot, ch, G, U);
        RowChunks<ET> cur, nxt;
        if (ch < p.I)
            load_rows(ET{}, G, U, ch, 0, lane, nck, cur);
        stage_x<R, ET>(p.x, p.H, xs, xsum, p.norm_w, p.norm_eps);
        while (true) {
            const int nx = it + stride;
            int nslot = 0, nch = 0;
            if (nx < nitems) {
                MatRef G2, U2;
                item_mats(nx, nslot, nch, G2, U2);
                if (nch < p.I)
                    load_rows(ET{}, G2, U2, nch, 0, lane, nck, nxt);
            }
            if (ch < p.I)
                routed_channel<R, ET>(p, cur, rl.slots, slot, ch, xs, xsum, lane);
            if (nx >= nitems)
                break;
            cur = nxt;
            it = nx;
            slot = nslot;
            ch = nch;
        }
    }
}

// ================================================================= dense

struct LogitArgs {
    const float *x;          // [R][H]
    const float *norm_w;     // RMS norm gamma [H], or null
    float norm_eps;
    int H, E;
    const uint8_t *router_w; // [E][H]
    const float *bias;       // [E] or null
    const uint8_t *gate_w;   // [H]
    double *logits;          // [R][E]
    double *zlogit;          // [R]
};

constexpr int kLgThreads = 256;   // one router row per workgroup, four waves (the four quarters)
constexpr int kLgPrefetch = 4;    // 16-byte chunks per thread requested first

// x values (R rows) of the elements of one 16-byte router chunk c, read from
// global memory (cached: every workgroup reads the same x); with a norm, the
// normalized u = fp32((x r) gamma) of rms_norm_rows.
template <int R, int EPC>
__device__ __forceinline__ void chunk_x(const float *x, int H, int c, const float *gamma, const double (&r)[R],
                                        float (&xv)[R][EPC])
{
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
        for (int i = 0; i < EPC; i += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(x + static_cast<size_t>(q) * H + c * EPC + i);
            xv[q][i] = v.x;
            xv[q][i + 1] = v.y;
            xv[q][i + 2] = v.z;
            xv[q][i + 3] = v.w;
        }
    if (gamma) {
#pragma unroll
        for (int i = 0; i < EPC; i += 4) {
            const float4 g = *reinterpret_cast<const float4 *>(gamma + c * EPC + i);
            const float gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
            for (int q = 0; q < R; ++q)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    xv[q][i + k] = static_cast<float>(static_cast<double>(xv[q][i + k]) * r[q] * static_cast<double>(gv[k]));
        }
    }
}

// One chunk's products (weights in element order) added to acc[q].
template <int R>
__device__ __forceinline__ void chunk_fma(F32, const uint4 &u, const float (&xv)[R][4], double (&acc)[R])
{
    const float w[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[q] = fma(static_cast<double>(w[i]), static_cast<double>(xv[q][i]), acc[q]);
}
template <int R>
__device__ __forceinline__ void chunk_fma(BF16, const uint4 &u, const float (&xv)[R][8], double (&acc)[R])
{
    const float w[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                        bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[q] = fma(static_cast<double>(w[i]), static_cast<double>(xv[q][i]), acc[q]);
}

// Router logits of a call: one router row per workgroup (row E is the
// shared-gate vector), in the quartered order of router_chunk (wave w takes
// quarter w: chunks c with (c >> 6) & 3 == w). Each thread reads its own
// weight chunks and the x values they multiply straight from memory, so the
// row's one HBM round trip is not preceded by staging x in LDS; with a norm,
// the rows' sums of squares are formed first exactly as in rms_norm_rows
// (float4 i = tid, tid + 256, ..., then wave_sum, then the waves in order),
// so r matches the other kernels' bit for bit.
template <int R, typename RT>
__global__ void __launch_bounds__(kLgThreads) k_logits(LogitArgs a)
{
    constexpr int EPC = RT::kChunk;   // elements per 16-byte chunk
    __shared__ double part[R][kLgThreads / kWave];
    __shared__ double rr[R];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int e = blockIdx.x;
    const size_t rb = static_cast<size_t>(a.H) * (EPC == 4 ? 4 : 2);
    const uint8_t *row = e < a.E ? a.router_w + e * rb : a.gate_w;
    const int nch = static_cast<int>(rb / 16);
    // thread tid takes chunks c = tid + 256 k: quarter (c >> 6) & 3 = wave
    uint4 w[kLgPrefetch];
#pragma unroll
    for (int u = 0; u < kLgPrefetch; ++u) {
        const int c = tid + u * kLgThreads;
        if (c < nch)
            w[u] = ld_nt16(row + c * 16);
    }
    double r[R];
    if (a.norm_w) {
        const int n4 = a.H >> 2;
        const float4 *x4 = reinterpret_cast<const float4 *>(a.x);
#pragma unroll
        for (int q = 0; q < R; ++q) {
            double ss = 0.0;
            for (int i = tid; i < n4; i += kLgThreads) {
                const float4 v = x4[q * n4 + i];
                ss += static_cast<double>(v.x) * v.x + static_cast<double>(v.y) * v.y +
                      static_cast<double>(v.z) * v.z + static_cast<double>(v.w) * v.w;
            }
            ss = wave_sum(ss);
            if (lane == 0)
                part[q][wave] = ss;
        }
        __syncthreads();
        if (tid < R) {
            double t = 0.0;
            for (int v = 0; v < kLgThreads / kWave; ++v)
                t += part[tid][v];
            rr[tid] = 1.0 / sqrt(t / a.H + static_cast<double>(a.norm_eps));
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < R; ++q)
            r[q] = rr[q];
    } else {
#pragma unroll
        for (int q = 0; q < R; ++q)
            r[q] = 1.0;
    }
    double acc[R];
#pragma unroll
    for (int q = 0; q < R; ++q)
        acc[q] = 0.0;
#pragma unroll
    for (int u = 0; u < kLgPrefetch; ++u) {
        const int c = tid + u * kLgThreads;
        if (c < nch) {
            float xv[R][EPC];
            chunk_x<R, EPC>(a.x, a.H, c, a.norm_w, r, xv);
            chunk_fma<R>(RT{}, w[u], xv, acc);
        }
    }
    for (int c = tid + kLgPrefetch * kLgThreads; c < nch; c += kLgThreads) {
        const uint4 u = ld_nt16(row + c * 16);
        float xv[R][EPC];
        chunk_x<R, EPC>(a.x, a.H, c, a.norm_w, r, xv);
        chunk_fma<R>(RT{}, u, xv, acc);
    }
    __syncthreads();   // part[] is reused
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const double p = wave_sum(acc[q]);
        if (lane == 0)
            part[q][wave] = p;
    }
    __syncthreads();
    if (tid < R) {
        const double v = combine_quarters(part[tid][0], part[tid][1], part[tid][2], part[tid][3]);
        if (e < a.E)
            a.logits[tid * a.E + e] = v + (a.bias ? static_cast<double>(a.bias[e]) : 0.0);
        else
            a.zlogit[tid] = v;
    }
}

// ================================================================= down

struct DownArgs {
    float *y;                  // [R][H]
    const float *xres;         // [R][H] the layer input added to y (residual), or null
    int H, I, Is, Imax;
    const uint8_t *ed;         // routed down stack
    size_t estride;            // bytes per routed [H][I] matrix
    const uint8_t *sd;         // shared down
    size_t sbytes;             // bytes of the shared [H][Is] matrix
    const SlotTable *slots;
    const float *hbuf;         // [pairs][Imax]
    int max_pairs;             // R * (K + 1): bound on the (slot, row) pairs
};

constexpr int kDnWaves = 8;    // one output row per wave
// LDS for the staged h' rows of the down pass; beyond it h' is read from L2
constexpr size_t kDnStageLds = 144 * 1024;

// The first pieces of a down row are read through buffer descriptors over
// one matrix: a piece that is not needed gets an offset past the end, which
// returns zeros without a memory access. Every lane then issues the same
// loads, so the compiler can count them and wait for just the earlier ones.
constexpr int kAuxNT = 2;                   // non-temporal
constexpr uint32_t kPastEnd = 0xFFFFFFF0u;  // an offset beyond every matrix
constexpr int kRsrcWord3 = 0x00020000;      // raw 32-bit dwords, range-checked
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mat_rsrc(const uint8_t *base, size_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// Down rows are read in pieces of 8 elements (bf16: 16 bytes; 2-bit: 2 bytes
// of codes plus the block's scale/min) or 4 elements (fp32: 16 bytes). Lane
// c of a row takes piece c (then c+64, ...). fma1 adds piece . h[piece] of
// one h' row.
template <typename W>
struct DnPiece;
template <>
struct DnPiece<BF16> {
    static constexpr int kElems = 8;
    uint4 v;
    __device__ __forceinline__ void load(const MatRef &M, int j, int c)
    {
        v = ld_nt16(M.base + (static_cast<size_t>(j) * M.cols + c * 8) * 2);
    }
    __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t r, const MatRef &M, int j, int c, bool ok)
    {
        const uint32_t off = ok ? static_cast<uint32_t>((j * M.cols + c * 8) * 2) : kPastEnd;
        v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNT));
    }
    __device__ __forceinline__ void fma1(const float *h, int c, float &acc) const
    {
        const float4 h0 = *reinterpret_cast<const float4 *>(h + c * 8);
        const float4 h1 = *reinterpret_cast<const float4 *>(h + c * 8 + 4);
        float s = acc;
        s = fmaf(bf16_lo(v.x), h0.x, s);
        s = fmaf(bf16_hi(v.x), h0.y, s);
        s = fmaf(bf16_lo(v.y), h0.z, s);
        s = fmaf(bf16_hi(v.y), h0.w, s);
        s = fmaf(bf16_lo(v.z), h1.x, s);
        s = fmaf(bf16_hi(v.z), h1.y, s);
        s = fmaf(bf16_lo(v.w), h1.z, s);
        s = fmaf(bf16_hi(v.w), h1.w, s);
        acc = s;
    }
};
template <>
struct DnPiece<F32> {
    static constexpr int kElems = 4;
    float4 v;
    __device__ __forceinline__ void load(const MatRef &M, int j, int c)
    {
        const uint4 u = ld_nt16(M.base + (static_cast<size_t>(j) * M.cols + c * 4) * 4);
        v = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    }
    __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t r, const MatRef &M, int j, int c, bool ok)
    {
        const uint32_t off = ok ? static_cast<uint32_t>((j * M.cols + c * 4) * 4) : kPastEnd;
        const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNT));
        v = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    }
    __device__ __forceinline__ void fma1(const float *h, int c, float &acc) const
    {
        const float4 hv = *reinterpret_cast<const float4 *>(h + c * 4);
        acc = fmaf(v.x, hv.x, fmaf(v.y, hv.y, fmaf(v.z, hv.z, fmaf(v.w, hv.w, acc))));
    }
};
template <>
struct DnPiece<Q2> {
    static constexpr int kElems = 8;
    uint32_t codes;   // 16 bits used
    uint32_t sm;
    __device__ __forceinline__ void load(const MatRef &M, int j, int c)
    {
        const int nb = M.cols >> 5;
        const int b = c >> 2;
        codes = ld_nt2(M.base + static_cast<size_t>(j) * (M.cols >> 2) + c * 2);
        sm = ld_nt4(M.base + static_cast<size_t>(M.rows) * (M.cols >> 2) + (static_cast<size_t>(j) * nb + b) * 4);
    }
    __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t r, const MatRef &M, int j, int c, bool ok)
    {
        const int nb = M.cols >> 5;
        const uint32_t oc = ok ? static_cast<uint32_t>(j * (M.cols >> 2) + c * 2) : kPastEnd;
        const uint32_t os = ok ? static_cast<uint32_t>(M.rows * (M.cols >> 2) + (j * nb + (c >> 2)) * 4) : kPastEnd;
        codes = __builtin_amdgcn_raw_buffer_load_b16(r, oc, 0, kAuxNT);
        sm = __builtin_amdgcn_raw_buffer_load_b32(r, os, 0, kAuxNT);
    }
    // The piece as floats: codes (each with one byte conversion), scale, min.
    struct Dec {
        float c[8];
        float s, m;
    };
    __device__ __forceinline__ Dec dec() const
    {
        // byte 0 / 1 of wk: code k / k + 4; opaque so that the byte
        // conversions are not folded back into 2-bit extracts
        uint32_t w0 = codes & 0x0303u, w1 = (codes >> 2) & 0x0303u, w2 = (codes >> 4) & 0x0303u,
                 w3 = (codes >> 6) & 0x0303u;
        asm("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
        Dec d;
        d.c[0] = static_cast<float>(w0 & 0xffu);
        d.c[1] = static_cast<float>(w1 & 0xffu);
        d.c[2] = static_cast<float>(w2 & 0xffu);
        d.c[3] = static_cast<float>(w3 & 0xffu);
        d.c[4] = static_cast<float>((w0 >> 8) & 0xffu);
        d.c[5] = static_cast<float>((w1 >> 8) & 0xffu);
        d.c[6] = static_cast<float>((w2 >> 8) & 0xffu);
        d.c[7] = static_cast<float>((w3 >> 8) & 0xffu);
        d.s = f16_to_f32(sm & 0xffffu);
        d.m = f16_to_f32(sm >> 16);
        return d;
    }
    // sum of the 8 h values of piece c
    static __device__ __forceinline__ float hsum(const float *h, int c)
    {
        const float4 h0 = *reinterpret_cast<const float4 *>(h + c * 8);
        const float4 h1 = *reinterpret_cast<const float4 *>(h + c * 8 + 4);
        return ((h0.x + h0.y) + (h0.z + h0.w)) + ((h1.x + h1.y) + (h1.z + h1.w));
    }
    // sum_i (code_i * s + m) h_i = s * sum_i code_i h_i + m * sum_i h_i, with
    // hs = sum_i h_i given
    static __device__ __forceinline__ void fma_d(const Dec &d, const float *h, int c, float hs, float &acc)
    {
        const float4 h0 = *reinterpret_cast<const float4 *>(h + c * 8);
        const float4 h1 = *reinterpret_cast<const float4 *>(h + c * 8 + 4);
        float cx = 0.0f;
        cx = fmaf(d.c[0], h0.x, cx);
        cx = fmaf(d.c[1], h0.y, cx);
        cx = fmaf(d.c[2], h0.z, cx);
        cx = fmaf(d.c[3], h0.w, cx);
        cx = fmaf(d.c[4], h1.x, cx);
        cx = fmaf(d.c[5], h1.y, cx);
        cx = fmaf(d.c[6], h1.z, cx);
        cx = fmaf(d.c[7], h1.w, cx);
        acc = fmaf(d.s, cx, fmaf(d.m, hs, acc));
    }
    __device__ __forceinline__ void fma1(const float *h, int c, float &acc) const
    {
        fma_d(dec(), h, c, hsum(h, c), acc);
    }
};

// 3- and 4-bit pieces: 8 codes of B bits (B bytes at byte 8*B*c/8 of the
// row's codes: one aligned dword for B = 4; for B = 3 the two aligned dwords
// around the 3 bytes, joined by a funnel shift), plus the block's scale/min.
template <int B>
struct DnPiece<QB<B>> {
    static constexpr int kElems = 8;
    using Dec = DnPiece<Q2>::Dec;
    uint32_t codes;   // code k at bits B*k
    uint32_t sm;
    static __device__ __forceinline__ size_t row_bytes(const MatRef &M) { return static_cast<size_t>(M.cols) * B / 8; }
    __device__ __forceinline__ void load(const MatRef &M, int j, int c)
    {
        const int nb = M.cols >> 5;
        const uint8_t *row = M.base + static_cast<size_t>(j) * row_bytes(M);
        if constexpr (B == 4) {
            codes = ld_nt4(row + c * 4);
        } else {
            const int o = c * B;
            const uint32_t lo = ld_nt4(row + (o & ~3)), hi = ld_nt4(row + (o & ~3) + 4);
            codes = __builtin_amdgcn_alignbit(hi, lo, 8 * (o & 3));
        }
        sm = ld_nt4(M.base + static_cast<size_t>(M.rows) * row_bytes(M) + (static_cast<size_t>(j) * nb + (c >> 2)) * 4);
    }
    __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t r, const MatRef &M, int j, int c, bool ok)
    {
        const int nb = M.cols >> 5;
        const uint32_t rb = static_cast<uint32_t>(row_bytes(M));
        const uint32_t os = ok ? static_cast<uint32_t>(M.rows * rb + (j * nb + (c >> 2)) * 4) : kPastEnd;
        if constexpr (B == 4) {
            codes = __builtin_amdgcn_raw_buffer_load_b32(r, ok ? j * rb + c * 4 : kPastEnd, 0, kAuxNT);
        } else {
            const int o = c * B;
            const uint32_t oc = ok ? static_cast<uint32_t>(j * rb + (o & ~3)) : kPastEnd;
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(r, oc, 0, kAuxNT);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(r, ok ? oc + 4 : kPastEnd, 0, kAuxNT);
            codes = __builtin_amdgcn_alignbit(hi, lo, 8 * (o & 3));
        }
        sm = __builtin_amdgcn_raw_buffer_load_b32(r, os, 0, kAuxNT);
    }
    __device__ __forceinline__ Dec dec() const
    {
        Dec d;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            d.c[k] = static_cast<float>((codes >> (B * k)) & ((1u << B) - 1u));
        d.s = f16_to_f32(sm & 0xffffu);
        d.m = f16_to_f32(sm >> 16);
        return d;
    }
    __device__ __forceinline__ void fma1(const float *h, int c, float &acc) const
    {
        DnPiece<Q2>::fma_d(dec(), h, c, DnPiece<Q2>::hsum(h, c), acc);
    }
};

template <typename W>
struct DnBatch {
    static constexpr int value = 12;   // 16-byte pieces in flight per lane
};
template <int B>
struct DnBatch<QB<B>> {
    static constexpr int value = B == 3 ? 24 : 32;   // 2-4 bytes of codes (3 bits: two dwords) + 4 per piece
};

// Down projection and combine, one output row j per wave:
//   y[q][j] = sum over routed slots s used by row q of D_s[j] . h'(s, q)
//             + gate_q * D_shared[j] . h'(0, q)
// (h' carries the route weight). Only the (slot, row) pairs that carry
// weight exist, so a few-row call costs one row's arithmetic per slot.
// Request order: the first part of h' (STAGED: h' goes to LDS; otherwise it
// is read from L2), then the shared piece and the first batch of routed
// pieces. Loads complete in order, so h' is in LDS while the weight stream
// is still arriving, and each piece's products start as soon as it lands.
template <int R, typename ET, typename ST, bool STAGED>
__global__ void __launch_bounds__(kDnWaves * kWave) k_down(DownArgs p)
{
    extern __shared__ __align__(16) unsigned char lds_raw[];
    constexpr int B = DnBatch<ET>::value;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int j = blockIdx.x * kDnWaves + wave;
    const bool live = j < p.H;
    const int nslots = p.slots->nslots;
    const int npr = p.I / DnPiece<ET>::kElems, nps = p.Is / DnPiece<ST>::kElems;
    const MatRef SD{p.sd, p.H, p.Is};

    // h' and the slot-table entries for the LDS copies are requested first.
    // Every load of this prologue is unconditional (indices are clamped;
    // the weight pieces go through range-checked buffer loads), so the waits
    // before the LDS writes below cover only these early loads, not the
    // weight stream behind them; clamped duplicates rewrite equal values.
    constexpr int kT = kDnWaves * kWave;
    const int n4 = STAGED ? p.max_pairs * p.Imax / 4 : 1;
    const float4 *hsrc = reinterpret_cast<const float4 *>(p.hbuf);
    // float4 of h' per thread requested at once: all of it for top-10
    // routing and 512 channels (R (K + 1) pairs of 128 float4), so that the
    // staging is one round trip; larger shapes stage the rest in a loop
    constexpr int NH = R == 1 ? 4 : (R * 11 + 3) / 4;
    int hix[NH];
    float4 hv[NH];   // indexed only by unrolled constants: registers
    if (STAGED) {
#pragma unroll
        for (int k = 0; k < NH; ++k) {
            hix[k] = min(tid + k * kT, n4 - 1);
            hv[k] = hsrc[hix[k]];
        }
    }
    const int ti = min(tid, kMaxRows * kMaxK), tq = min(tid, R - 1);
    const int t_expert = p.slots->expert[ti];
    const uint32_t t_rmask = R > 1 ? p.slots->rmask[ti] : 0u;
    const int t_pstart = R > 1 ? p.slots->pstart[ti] : 0;
    const float t_gate = p.slots->w[0][tq];
    __builtin_amdgcn_sched_barrier(0);
    DnPiece<ST> ps;
    DnPiece<ET> pc[B];
    ps.load_b(mat_rsrc(p.sd, p.sbytes), SD, j, lane, live && lane < nps);
    {
        // the first batch's expert ids in one go (16-byte reads of the table)
        constexpr int NV = (B + 4) / 4;
        int4 ev[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k)
            ev[k] = reinterpret_cast<const int4 *>(p.slots->expert)[k];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int4 &v = ev[(1 + u) >> 2];
            const int r = (1 + u) & 3;
            const bool used = 1 + u < nslots;
            const int e = used ? (r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w) : 0;
            const MatRef M{p.ed + e * p.estride, p.H, p.I};
            pc[u].load_b(mat_rsrc(M.base, p.estride), M, j, lane, live && used && lane < npr);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the slot table's pair layout and gates into LDS, beside the h' staging
    __shared__ uint32_t rmask[kMaxRows * kMaxK + 1];
    __shared__ int pstart[kMaxRows * kMaxK + 1];
    __shared__ float gate[kMaxRows];
    __shared__ int expert[kMaxRows * kMaxK + 1];
    expert[ti] = t_expert;
    if (R > 1) {
        rmask[ti] = t_rmask;
        pstart[ti] = t_pstart;
    }
    gate[tq] = t_gate;
    const float *hl = p.hbuf;
    // One-row calls with block-format pieces also use the sum of each 8-value piece
    // of h': formed here once per workgroup from the two float4 halves held
    // by lanes 2i, 2i+1 (measured slower with several rows)
    constexpr bool HS = STAGED && R == 1 && is_block_format<ET>::value;
    float *hsl = reinterpret_cast<float *>(lds_raw) + (HS ? p.max_pairs * p.Imax : 0);
    if (STAGED) {
        float4 *dst = reinterpret_cast<float4 *>(lds_raw);
        auto put = [&](int i, int ic, float4 v) {
            dst[ic] = v;
            if constexpr (HS) {
                const float part = (v.x + v.y) + (v.z + v.w);
                const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0xB1, 0xF, 0xF, false));
                if ((i & 1) == 0 && i < n4)
                    hsl[i >> 1] = part + other;
            }
        };
#pragma unroll
        for (int k = 0; k < NH; ++k)
            put(tid + k * kT, hix[k], hv[k]);
        for (int i = tid + NH * kT; i < n4; i += kT)
            put(i, i, hsrc[i]);
        hl = reinterpret_cast<const float *>(lds_raw);
    }
    __syncthreads();
    if (!live)
        return;

    float acc[R], sh[R];
#pragma unroll
    for (int q = 0; q < R; ++q)
        acc[q] = sh[q] = 0.0f;
    // shared expert: pairs 0..R-1
    for (int base = 0; base < nps; base += kWave) {
        const int c = base + lane;
        if (base > 0 && c < nps)
            ps.load(SD, j, c);
        if (c < nps) {
#pragma unroll
            for (int q = 0; q < R; ++q)
                ps.fma1(hl + q * p.Imax, c, sh[q]);
        }
    }
    // routed slots in batches of B
    for (int s0 = 1; s0 < nslots; s0 += B) {
        for (int base = 0; base < npr; base += kWave) {
            const int c = base + lane;
            if (s0 > 1 || base > 0) {
#pragma unroll
                for (int u = 0; u < B; ++u)
                    if (s0 + u < nslots && c < npr)
                        pc[u].load(MatRef{p.ed + expert[s0 + u] * p.estride, p.H, p.I}, j, c);
            }
#pragma unroll
            for (int u = 0; u < B; ++u) {
                if (s0 + u < nslots && c < npr) {
                    if constexpr (HS) {
                        // pair = slot; the piece's h' sum from LDS
                        const float *h = hl + static_cast<size_t>(s0 + u) * p.Imax;
                        DnPiece<Q2>::fma_d(pc[u].dec(), h, c, hsl[(s0 + u) * (p.Imax >> 3) + c], acc[0]);
                    } else if constexpr (R == 1) {
                        pc[u].fma1(hl + static_cast<size_t>(s0 + u) * p.Imax, c, acc[0]);   // pair = slot
                    } else {
                        const uint32_t m = rmask[s0 + u];
                        int pp = pstart[s0 + u];
#pragma unroll
                        for (int q = 0; q < R; ++q)
                            if ((m >> q) & 1u)
                                pc[u].fma1(hl + static_cast<size_t>(pp++) * p.Imax, c, acc[q]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float v = wave_sum(acc[q]) + gate[q] * wave_sum(sh[q]);
        if (lane == 0)
            p.y[q * p.H + j] = p.xres ? p.xres[q * p.H + j] + v : v;
    }
}

// ================================================================ launch

static inline int imax_of(const moe_layer_desc *d) { return d->inter > d->shared_inter ? d->inter : d->shared_inter; }

static_assert(sizeof(RouteLds) <= kDecodeStaticLds, "routing state exceeds its LDS bound");
static_assert(offsetof(SlotTable, expert) % 16 == 0 && sizeof(SlotTable) % 16 == 0,
              "the down pass reads expert ids 16 bytes at a time");


struct RoutingIO {
    const int32_t *ids_in;
    const float *wts_in, *gate_in;
    int32_t *ids_out;
    float *wts_out, *gate_out;
};

template <typename ET>
static GateUpArgs gateup_args(const moe_layer_desc *d, const float *x, const DecodeWs &w)
{
    GateUpArgs g;
    g.x = x;
    g.norm_w = d->norm_w;
    g.norm_eps = d->norm_eps;
    g.H = d->hidden;
    g.I = d->inter;
    g.Is = d->shared_inter;
    g.Imax = imax_of(d);
    g.eg = static_cast<const uint8_t *>(d->exp_gate);
    g.eu = static_cast<const uint8_t *>(d->exp_up);
    g.estride = mat_bytes<ET>(g.I, g.H);
    g.sg = static_cast<const uint8_t *>(d->sh_gate);
    g.su = static_cast<const uint8_t *>(d->sh_up);
    g.slots = w.slots;
    g.hbuf = w.hbuf;
    g.ch_per_wg = kGuWaves;
    g.wg_per_slot = (g.I + g.ch_per_wg - 1) / g.ch_per_wg;
    return g;
}

// Workgroups of kernel `fn` (block threads, dynamic LDS bytes) that the
// current device holds at once: occupancy per CU times the CU count, cached
// per (kernel, LDS size, device). 0 if the runtime cannot tell.
static int resident_blocks(const void *fn, int block, size_t lds)
{
    struct Entry {
        const void *fn;
        size_t lds;
        int dev, n;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : cache)
            if (e.fn == fn && e.lds == lds && e.dev == dev)
                return e.n;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int n = per_cu * cus;
    std::lock_guard<std::mutex> lock(mu);
    cache.push_back(Entry{fn, lds, dev, n});
    return n;
}

// k_logits: the router logits and the shared-gate logit of R rows.
template <typename RT>
static int launch_logits_t(const moe_layer_desc *d, const float *x, int R, const DecodeWs &w, hipStream_t s)
{
    LogitArgs a;
    a.x = x;
    a.norm_w = d->norm_w;
    a.norm_eps = d->norm_eps;
    a.H = d->hidden;
    a.E = d->n_experts;
    a.router_w = static_cast<const uint8_t *>(d->router_w);
    a.bias = d->router_bias;
    a.gate_w = static_cast<const uint8_t *>(d->shared_gate_w);
    a.logits = w.logits;
    a.zlogit = w.zlogit;
    const dim3 grid(a.E + 1), block(kLgThreads);
    switch (R) {
    case 1: hipLaunchKernelGGL((k_logits<1, RT>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_logits<2, RT>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_logits<3, RT>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_logits<4, RT>), grid, block, 0, s, a); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

static int launch_logits(const moe_layer_desc *d, const float *x, int R, const DecodeWs &w, hipStream_t s)
{
    return d->router_t == MOE_F32 ? launch_logits_t<F32>(d, x, R, w, s) : launch_logits_t<BF16>(d, x, R, w, s);
}

static RouteArgs route_args(const moe_layer_desc *d, const RoutingIO &io, const DecodeWs &w, bool slots)
{
    RouteArgs a;
    a.logits = w.logits;
    a.zlogit = w.zlogit;
    a.E = d->n_experts;
    a.K = d->top_k;
    a.renorm = d->renormalize;
    a.ids_in = io.ids_in;
    a.wts_in = io.wts_in;
    a.gate_in = io.gate_in;
    a.ids_out = io.ids_out;
    a.wts_out = io.wts_out;
    a.gate_out = io.gate_out;
    a.slots = slots ? w.slots : nullptr;
    a.wbias = d->bias_mode == MOE_BIAS_SELECT_ONLY ? d->router_bias : nullptr;
    return a;
}

static int launch_route(const moe_layer_desc *d, int R, const RoutingIO &io, const DecodeWs &w, hipStream_t s)
{
    const RouteArgs a = route_args(d, io, w, false);
    const size_t lds = sizeof(double) * R * ((a.E + 1) & ~1);
    switch (R) {
    case 1: hipLaunchKernelGGL((k_route<1>), dim3(1), dim3(kRouteThreads), lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_route<2>), dim3(1), dim3(kRouteThreads), lds, s, a); break;
    case 3: hipLaunchKernelGGL((k_route<3>), dim3(1), dim3(kRouteThreads), lds, s, a); break;
    default: hipLaunchKernelGGL((k_route<4>), dim3(1), dim3(kRouteThreads), lds, s, a); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <typename ET, typename ST>
static int launch_experts_t(const moe_layer_desc *d, const float *x, int R, float *y, const RoutingIO &io,
                            const DecodeWs &w, hipStream_t s)
{
    const int H = d->hidden, I = d->inter, Is = d->shared_inter, K = d->top_k;
    const int Imax = imax_of(d);
    if (!io.ids_in) {
        const int rc = launch_logits(d, x, R, w, s);
        if (rc != MOE_OK)
            return rc;
    }
    {
        const GateUpArgs g = gateup_args<ET>(d, x, w);
        const RouteArgs ra = route_args(d, io, w, true);
        const int n_sh = (Is + g.ch_per_wg - 1) / g.ch_per_wg;
        const size_t lds = gateup_lds_bytes(R, H, d->n_experts);
        const void *fn = R == 1   ? reinterpret_cast<const void *>(&k_gateup<1, ET, ST>)
                         : R == 2 ? reinterpret_cast<const void *>(&k_gateup<2, ET, ST>)
                         : R == 3 ? reinterpret_cast<const void *>(&k_gateup<3, ET, ST>)
                                  : reinterpret_cast<const void *>(&k_gateup<4, ET, ST>);
        // routed workgroups: one per work item up to what stays resident
        // beside the shared ones (each routes once, then strides over items)
        int n_rt = R * K * g.wg_per_slot;
        const int resident = resident_blocks(fn, kGuWaves * kWave, lds) - n_sh;
        if (resident > 0 && n_rt > resident)
            n_rt = resident;
        const dim3 grid(n_sh + n_rt), block(kGuWaves * kWave);
        switch (R) {
        case 1: hipLaunchKernelGGL((k_gateup<1, ET, ST>), grid, block, lds, s, g, ra, n_sh); break;
        case 2: hipLaunchKernelGGL((k_gateup<2, ET, ST>), grid, block, lds, s, g, ra, n_sh); break;
        case 3: hipLaunchKernelGGL((k_gateup<3, ET, ST>), grid, block, lds, s, g, ra, n_sh); break;
        default: hipLaunchKernelGGL((k_gateup<4, ET, ST>), grid, block, lds, s, g, ra, n_sh); break;
        }
        if (hipGetLastError() != hipSuccess)
            return MOE_EHIP;
    }
    DownArgs dn;
    dn.y = y;
    dn.xres = d->residual ? x : nullptr;
    dn.H = H;
    dn.I = I;
    dn.Is = Is;
    dn.Imax = Imax;
    dn.ed = static_cast<const uint8_t *>(d->exp_down);
    dn.estride = mat_bytes<ET>(H, I);
    dn.sd = static_cast<const uint8_t *>(d->sh_down);
    dn.sbytes = mat_bytes<ST>(H, Is);
    dn.slots = w.slots;
    dn.hbuf = w.hbuf;
    dn.max_pairs = max_pairs(R, K);
    const dim3 dgrid((H + kDnWaves - 1) / kDnWaves), dblock(kDnWaves * kWave);
    // staged h' (and, for one row with block-format experts, one sum per 8-value piece)
    const size_t stage =
        static_cast<size_t>(dn.max_pairs) * Imax * sizeof(float) * (R == 1 && is_block_format<ET>::value ? 9 : 8) / 8;
    if (stage <= kDnStageLds) {
        switch (R) {
        case 1: hipLaunchKernelGGL((k_down<1, ET, ST, true>), dgrid, dblock, stage, s, dn); break;
        case 2: hipLaunchKernelGGL((k_down<2, ET, ST, true>), dgrid, dblock, stage, s, dn); break;
        case 3: hipLaunchKernelGGL((k_down<3, ET, ST, true>), dgrid, dblock, stage, s, dn); break;
        default: hipLaunchKernelGGL((k_down<4, ET, ST, true>), dgrid, dblock, stage, s, dn); break;
        }
    } else {
        switch (R) {
        case 1: hipLaunchKernelGGL((k_down<1, ET, ST, false>), dgrid, dblock, 0, s, dn); break;
        case 2: hipLaunchKernelGGL((k_down<2, ET, ST, false>), dgrid, dblock, 0, s, dn); break;
        case 3: hipLaunchKernelGGL((k_down<3, ET, ST, false>), dgrid, dblock, 0, s, dn); break;
        default: hipLaunchKernelGGL((k_down<4, ET, ST, false>), dgrid, dblock, 0, s, dn); break;
        }
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}


int launch_decode_forward(const moe_layer_desc *d, const float *x, int R, float *y, const int32_t *ids_in,
                          const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out,
                          float *gate_out, void *ws, hipStream_t s)
{
    const DecodeWs w = decode_ws_carve(ws, R, d->n_experts, d->top_k, imax_of(d));
    const RoutingIO io{ids_in, wts_in, gate_in, ids_out, wts_out, gate_out};
    const int et = d->expert_t, st = d->shared_t;
    if (st == MOE_F32) {
        switch (et) {
        case MOE_F32: return launch_experts_t<F32, F32>(d, x, R, y, io, w, s);
        case MOE_BF16: return launch_experts_t<BF16, F32>(d, x, R, y, io, w, s);
        case MOE_Q2B32: return launch_experts_t<Q2, F32>(d, x, R, y, io, w, s);
        case MOE_Q3B32: return launch_experts_t<Q3, F32>(d, x, R, y, io, w, s);
        default: return launch_experts_t<Q4, F32>(d, x, R, y, io, w, s);
        }
    }
    switch (et) {
    case MOE_F32: return launch_experts_t<F32, BF16>(d, x, R, y, io, w, s);
    case MOE_BF16: return launch_experts_t<BF16, BF16>(d, x, R, y, io, w, s);
    case MOE_Q2B32: return launch_experts_t<Q2, BF16>(d, x, R, y, io, w, s);
    case MOE_Q3B32: return launch_experts_t<Q3, BF16>(d, x, R, y, io, w, s);
    default: return launch_experts_t<Q4, BF16>(d, x, R, y, io, w, s);
    }
}

// Routing only: the logits, then the routing workgroup (no slot table).
int launch_decode_route(const moe_layer_desc *d, const float *x, int R, int32_t *ids, float *wts, float *gate,
                        void *ws, hipStream_t s)
{
    const DecodeWs w = decode_ws_carve(ws, R, d->n_experts, d->top_k, imax_of(d));
    const int rc = launch_logits(d, x, R, w, s);
    if (rc != MOE_OK)
        return rc;
    const RoutingIO io{nullptr, nullptr, nullptr, ids, wts, gate};
    return launch_route(d, R, io, w, s);
}

}  // namespace moe
