// Workspace layouts and the launch-shape choices they depend on: pure host
// arithmetic, shared by the kernel launchers (which carve the caller's
// workspace) and the C-ABI layer (which sizes it). No kernels here, so the
// sizing code also builds on its own for host-side checks.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "device_common.hpp"
#include "moe.h"

namespace moe {

// prefill grouped GEMMs: B rows (weight rows) per workgroup
constexpr int kGN = 256;
// K slices of the prefill router GEMM, summed by the selection kernel
constexpr int kMaxRouterSplits = 8;
// pairs per workgroup of the counting sort by expert
constexpr int kSortChunk = 1024;


// Reduction slices of a dense (shared-expert) GEMM with `blocks` output
// workgroups and Kd-deep rows: up to about 512 workgroups in all, at least
// one 32-deep step per slice.
inline int dense_splits(int blocks, int Kd)
{
    int ks = 1;
    while (blocks * ks * 2 <= 512 && ks * 2 <= Kd / 32 && ks < 64)
        ks *= 2;
    return ks;
}
inline int shared_gu_splits(const moe_layer_desc *d, int T)
{
    return dense_splits(((d->shared_inter + kGN / 2 - 1) / (kGN / 2)) * ((T + 63) / 64), d->hidden);
}
inline int shared_dn_splits(const moe_layer_desc *d, int T)
{
    // the down GEMM gains from slices only while it has few workgroups
    // (measured: at 256 workgroups two slices plus their sum were slower)
    const int blocks = ((d->hidden + kGN - 1) / kGN) * ((T + 63) / 64);
    return blocks < 128 ? dense_splits(blocks, d->shared_inter) : 1;
}
// The selection kernel sums the router GEMM's slices itself, so slices beyond
// those that give each of the 256 compute units a workgroup only add partial
// sums for it to read (measured at 2048 rows: 4 slices 6 us faster than 8; at
// 64 and 256 rows, where 8 slices are needed to fill the chip, 4-7 us slower).
inline int router_splits(const moe_layer_desc *d, int T)
{
    constexpr int kCUs = 256;
    const int blocks = ((d->n_experts + kGN - 1) / kGN) * ((T + 63) / 64);
    int ks = dense_splits(blocks, d->hidden);
    while (ks > 1 && blocks * (ks / 2) >= kCUs)
        ks /= 2;
    return ks < kMaxRouterSplits ? ks : kMaxRouterSplits;
}
inline size_t shared_kpart_bytes(const moe_layer_desc *d, int T)
{
    const int a = shared_gu_splits(d, T), b = shared_dn_splits(d, T);
    const size_t gu = a > 1 ? sizeof(float) * a * static_cast<size_t>(T) * 2 * d->shared_inter : 0;
    const size_t dn = b > 1 ? sizeof(float) * b * static_cast<size_t>(T) * d->hidden : 0;
    return gu > dn ? gu : dn;
}
inline size_t router_kpart_bytes(const moe_layer_desc *d, int T)
{
    const int c = router_splits(d, T);
    return c > 1 ? sizeof(float) * c * static_cast<size_t>(T) * d->n_experts : 0;
}

struct PrefillWs {
    uint8_t *sort_ws;
    size_t sort_bytes;
    uint4 *xh, *xl;
    float *lap;                      // approximate router logits [T][E]
    float *wn;                       // norms of the router rows [E]
    float *kpart;                    // split-K partial sums of the router GEMM
    float *kpart_sh;                 // split-K partial sums of the shared expert's GEMMs
    int32_t *ids;
    float *wts, *gate;
    int32_t *counts, *offsets, *perm, *inv;
    int4 *tiles;                     // row tiles (expert, first sorted row, rows)
    uint16_t *hh, *hl, *shh, *shl;   // h of the routed pairs [T*K][I] and of the shared expert [T][Is], bf16 hi/lo
    float *xsum, *hsum;              // 32-element block sums of x [T][H/32] and of h [T*K][I/32]
    float *rout, *sout;
    float *u;                        // the normalized input [T][H] (layers with a norm)
};

inline PrefillWs prefill_carve(void *ws, const moe_layer_desc *d, int T, bool carve)
{
    const int H = d->hidden, E = d->n_experts, K = d->top_k, I = d->inter, Is = d->shared_inter;
    const int64_t P = static_cast<int64_t>(T) * K;
    uint8_t *base = static_cast<uint8_t *>(ws);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        uint8_t *p = carve ? base + off : nullptr;
        off += align256(bytes);
        return p;
    };
    PrefillWs w;
    w.sort_bytes = sort_ws_bytes_tke(P, E);
    w.sort_ws = take(w.sort_bytes);
    w.xh = reinterpret_cast<uint4 *>(take(sizeof(uint16_t) * T * H));
    w.xl = reinterpret_cast<uint4 *>(take(sizeof(uint16_t) * T * H));
    w.lap = reinterpret_cast<float *>(take(sizeof(float) * T * E));
    w.wn = reinterpret_cast<float *>(take(sizeof(float) * E));
    w.ids = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * P));
    w.wts = reinterpret_cast<float *>(take(sizeof(float) * P));
    w.gate = reinterpret_cast<float *>(take(sizeof(float) * T));
    w.counts = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * E));
    w.offsets = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (E + 1)));
    w.perm = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * P));
    w.inv = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * P));
    w.tiles = reinterpret_cast<int4 *>(take(sizeof(int4) * ((P + 31) / 32 + E)));   // tiles at the smallest bm
    w.hh = reinterpret_cast<uint16_t *>(take(sizeof(uint16_t) * P * I));
    w.hl = reinterpret_cast<uint16_t *>(take(sizeof(uint16_t) * P * I));
    w.shh = reinterpret_cast<uint16_t *>(take(sizeof(uint16_t) * T * Is));
    w.shl = reinterpret_cast<uint16_t *>(take(sizeof(uint16_t) * T * Is));
    w.xsum = reinterpret_cast<float *>(take(sizeof(float) * T * (H / 32)));
    w.hsum = reinterpret_cast<float *>(take(sizeof(float) * P * (I / 32)));
    w.rout = reinterpret_cast<float *>(take(sizeof(float) * P * H));
    w.sout = reinterpret_cast<float *>(take(sizeof(float) * T * H));
    w.kpart = reinterpret_cast<float *>(take(router_kpart_bytes(d, T)));
    w.kpart_sh = reinterpret_cast<float *>(take(shared_kpart_bytes(d, T)));
    w.u = reinterpret_cast<float *>(take(d->norm_w ? sizeof(float) * T * H : 0));
    w.sort_bytes = off;   // total, when not carving
    return w;
}


}  // namespace moe
