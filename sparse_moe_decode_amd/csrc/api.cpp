// C ABI of the MoE layer library: host-side argument validation, workspace
// sizing and path dispatch. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "device_common.hpp"
#include "internal.h"
#include "moe.h"

namespace {

enum Path { kDecode = 0, kFewRow = 1, kPrefill = 2 };

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate_desc(const moe_layer_desc *d)
{
    if (!d)
        return MOE_EINVAL;
    if (d->reserved != 0)
        return MOE_EINVAL;
    if (d->bias_mode != MOE_BIAS_SELECT_AND_WEIGH && d->bias_mode != MOE_BIAS_SELECT_ONLY)
        return MOE_EINVAL;
    if (d->residual != 0 && d->residual != 1)
        return MOE_EINVAL;
    if (d->norm_w && !(d->norm_eps >= 0.0f && d->norm_eps <= 3.0e38f))
        return MOE_EINVAL;
    if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->inter <= 0 || d->shared_inter <= 0)
        return MOE_EINVAL;
    if (d->hidden % 32 || d->inter % 32 || d->shared_inter % 32)
        return MOE_EINVAL;
    if (d->top_k > d->n_experts || d->top_k > moe::kMaxK)
        return MOE_EINVAL;
    if (d->renormalize != 0 && d->renormalize != 1)
        return MOE_EINVAL;
    if ((d->router_t != MOE_F32 && d->router_t != MOE_BF16) ||
        (d->shared_t != MOE_F32 && d->shared_t != MOE_BF16) ||
        (d->expert_t < MOE_F32 || d->expert_t > MOE_Q4B32))
        return MOE_EINVAL;
    if (d->n_experts > moe::kMaxE || d->hidden > 8192 || d->inter > 4096 || d->shared_inter > 4096)
        return MOE_EUNSUPPORTED;
    const void *req[] = {d->router_w, d->shared_gate_w, d->exp_gate, d->exp_up, d->exp_down,
                         d->sh_gate,  d->sh_up,         d->sh_down};
    for (const void *p : req) {
        if (!p)
            return MOE_EINVAL;
        if (!aligned16(p))
            return MOE_EALIGN;
    }
    if (d->router_bias && (reinterpret_cast<uintptr_t>(d->router_bias) & 3u))
        return MOE_EALIGN;
    if (d->norm_w && !aligned16(d->norm_w))
        return MOE_EALIGN;
    return MOE_OK;
}

// Rows per decode / few-row launch: the gate/up kernel stages x of all rows
// (plus 2-bit block sums) and their router logits in LDS; keep that, with the
// kernel's static routing state, within 60 KiB.
int max_rows(const moe_layer_desc *d)
{
    for (int r = moe::kMaxRows; r > 1; --r)
        if (moe::gateup_lds_bytes(r, d->hidden, d->n_experts) + moe::kDecodeStaticLds <= 60u * 1024u)
            return r;
    return 1;
}

// Calls of up to this many rows run as few-row launches (see group_at) when
// the layer allows groups of kMaxRows; larger calls take the grouped prefill
// path. Measured on the 2-bit layer (us per call, few-row / prefill): 8 rows
// 104 / 147, 12 rows 151 / 157, 13 rows 166 / 159, 16 rows 204 / 181.
constexpr int kFewRowMaxT = 12;

Path choose_path(const moe_layer_desc *d, int T)
{
    const char *f = std::getenv("MOE_FORCE_PATH");
    if (f && *f) {
        if (!std::strcmp(f, "decode"))
            return kDecode;
        if (!std::strcmp(f, "fewrow"))
            return kFewRow;
        if (!std::strcmp(f, "prefill"))
            return kPrefill;
    }
    if (T == 1)
        return kDecode;
    if (T <= moe::kMaxRows)
        return kFewRow;
    if (T <= kFewRowMaxT && max_rows(d) == moe::kMaxRows)
        return kFewRow;
    return kPrefill;
}

// Largest launch group of the decode / few-row kernels (workspace size).
int group_rows(const moe_layer_desc *d, Path p, int T)
{
    if (p == kDecode)
        return 1;
    const int r = max_rows(d);
    return T < r ? T : r;
}

// Rows of the launch group that starts at row t. A call that fits one
// launch is one group; a longer few-row call runs in groups of three rows,
// the cheapest per row where measured (2-bit layer: 14.0, 12.5 and 13.3 us
// per row at 2, 3 and 4 rows per launch), a remainder of one row joining the
// last group as four.
int group_at(const moe_layer_desc *d, Path p, int T, int t)
{
    if (p == kDecode)
        return 1;
    const int r = max_rows(d), rem = T - t;
    if (T <= r)
        return rem;
    if (r >= 4 && rem == 4)
        return 4;
    const int g = r < 3 ? r : 3;
    return rem < g ? rem : g;
}

// Rows per prefill chunk. The prefill kernels address their workspace
// buffers with 32-bit offsets (buffer descriptors and int indices), so one
// chunk's workspace stays below 1.5 GiB; a longer call runs as consecutive
// chunks on the same workspace. MOE_PREFILL_CHUNK (rows) lowers the chunk
// (to test the chunk loop on small calls).
int prefill_chunk_rows(const moe_layer_desc *d)
{
    constexpr size_t kMaxChunkWs = static_cast<size_t>(3) << 29;
    int lo = 1, hi = 1 << 22;   // largest T in [lo, hi) whose workspace fits
    while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        if (moe::prefill_ws_bytes(d, mid) <= kMaxChunkWs)
            lo = mid;
        else
            hi = mid;
    }
    const char *f = std::getenv("MOE_PREFILL_CHUNK");
    if (f && *f) {
        const long v = std::strtol(f, nullptr, 10);
        if (v >= 1 && v < lo)
            lo = static_cast<int>(v);
    }
    return lo;
}

size_t ws_bytes_for(const moe_layer_desc *d, int T)
{
    if (T <= 0)
        return 256;
    const Path p = choose_path(d, T);
    if (p == kPrefill) {
        const int c = prefill_chunk_rows(d);
        if (T <= c)
            return moe::prefill_ws_bytes(d, T);
        const size_t full = moe::prefill_ws_bytes(d, c), rest = T % c ? moe::prefill_ws_bytes(d, T % c) : 0;
        return full > rest ? full : rest;
    }
    return static_cast<size_t>(moe::decode_ws_size(d, group_rows(d, p, T)));
}

}  // namespace

extern "C" {

uint32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_strerror(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported size or format";
    case MOE_EWORKSPACE: return "workspace or destination buffer too small";
    case MOE_EALIGN: return "pointer not 16-byte aligned";
    case MOE_EHIP: return "HIP launch or runtime error";
    case MOE_ENONFINITE: return "non-finite input or value out of fp16 range";
    default: return "unknown status";
    }
}

size_t moe_workspace_bytes(const moe_layer_desc *d, int32_t T)
{
    if (validate_desc(d) != MOE_OK || T < 0)
        return 0;
    return ws_bytes_for(d, T);
}

int moe_route(const moe_layer_desc *d, const float *x, int32_t T, int32_t *ids, float *wts, float *gate, void *ws,
              size_t ws_bytes, void *stream)
{
    int rc = validate_desc(d);
    if (rc != MOE_OK)
        return rc;
    if (T < 0)
        return MOE_EINVAL;
    if (T == 0)
        return MOE_OK;
    if (!x || !ids || !wts || !gate || !ws)
        return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(ws) || (reinterpret_cast<uintptr_t>(ids) & 3u) ||
        (reinterpret_cast<uintptr_t>(wts) & 3u) || (reinterpret_cast<uintptr_t>(gate) & 3u))
        return MOE_EALIGN;
    if (ws_bytes < ws_bytes_for(d, T))
        return MOE_EWORKSPACE;
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Path path = choose_path(d, T);
    const int H = d->hidden, K = d->top_k;
    if (path == kPrefill) {
        const int c = prefill_chunk_rows(d);
        for (int t = 0; t < T; t += c) {
            const int r = T - t < c ? T - t : c;
            const size_t ok = static_cast<size_t>(t) * K;
            rc = moe::launch_prefill_route(d, x + static_cast<size_t>(t) * H, r, ids + ok, wts + ok, gate + t, ws, s);
            if (rc != MOE_OK)
                return rc;
        }
        return MOE_OK;
    }
    for (int t = 0, r = 0; t < T; t += r) {
        r = group_at(d, path, T, t);
        rc = moe::launch_decode_route(d, x + static_cast<size_t>(t) * H, r, ids + static_cast<size_t>(t) * K,
                                      wts + static_cast<size_t>(t) * K, gate + t, ws, s);
        if (rc != MOE_OK)
            return rc;
    }
    return MOE_OK;
}

int moe_forward(const moe_layer_desc *d, const float *x, int32_t T, float *y, const int32_t *ids_in,
                const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out, float *gate_out,
                void *ws, size_t ws_bytes, void *stream)
{
    int rc = validate_desc(d);
    if (rc != MOE_OK)
        return rc;
    if (T < 0)
        return MOE_EINVAL;
    if (T == 0)
        return MOE_OK;
    if (!x || !y || !ws)
        return MOE_EINVAL;
    if (ids_in && (!wts_in || !gate_in))
        return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(ws))
        return MOE_EALIGN;
    const void *small[] = {ids_in, wts_in, gate_in, ids_out, wts_out, gate_out};
    for (const void *p : small)
        if (p && (reinterpret_cast<uintptr_t>(p) & 3u))
            return MOE_EALIGN;
    if (ws_bytes < ws_bytes_for(d, T))
        return MOE_EWORKSPACE;
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Path path = choose_path(d, T);
    const int H = d->hidden, K = d->top_k;
    const int chunk = path == kPrefill ? prefill_chunk_rows(d) : 0;
    for (int t = 0, r = 0; t < T; t += r) {
        r = path == kPrefill ? (T - t < chunk ? T - t : chunk) : group_at(d, path, T, t);
        const size_t ok = static_cast<size_t>(t) * K;
        rc = (path == kPrefill ? moe::launch_prefill_forward : moe::launch_decode_forward)(d, x + static_cast<size_t>(t) * H, r, y + static_cast<size_t>(t) * H,
                                        ids_in ? ids_in + ok : nullptr, ids_in ? wts_in + ok : nullptr,
                                        ids_in ? gate_in + t : nullptr, ids_out ? ids_out + ok : nullptr,
                                        wts_out ? wts_out + ok : nullptr, gate_out ? gate_out + t : nullptr, ws, s);
        if (rc != MOE_OK)
            return rc;
    }
    return MOE_OK;
}

size_t moe_sort_workspace_bytes(int32_t T, int32_t K, int32_t E)
{
    if (T < 0 || K <= 0 || E <= 0 || E > moe::kMaxE)
        return 0;
    return moe::sort_ws_bytes_tke(static_cast<int64_t>(T) * K, E);
}

int moe_sort_by_expert(const int32_t *ids, int32_t T, int32_t K, int32_t E, int32_t *counts, int32_t *offsets,
                       int32_t *perm, void *ws, size_t ws_bytes, void *stream)
{
    if (T < 0 || K <= 0 || E <= 0)
        return MOE_EINVAL;
    if (E > moe::kMaxE || static_cast<int64_t>(T) * K > 0x7fffffff)
        return MOE_EUNSUPPORTED;
    if (!ids || !counts || !offsets || !perm || !ws)
        return MOE_EINVAL;
    const void *ps[] = {ids, counts, offsets, perm};
    for (const void *p : ps)
        if (reinterpret_cast<uintptr_t>(p) & 3u)
            return MOE_EALIGN;
    if (!aligned16(ws))
        return MOE_EALIGN;
    if (ws_bytes < moe_sort_workspace_bytes(T, K, E))
        return MOE_EWORKSPACE;
    if (T == 0)
        return MOE_OK;
    (void)hipGetLastError();
    return moe::launch_sort_by_expert(ids, T, K, E, counts, offsets, perm, ws, static_cast<hipStream_t>(stream),
                                      nullptr);
}

int moe_qb_unpack(int32_t bits, const void *packed, int64_t rows, int64_t cols, float *dst, void *stream)
{
    if (bits < 2 || bits > 4 || !packed || !dst || rows <= 0 || cols <= 0 || cols % 32 != 0)
        return MOE_EINVAL;
    if (!aligned16(packed) || !aligned16(dst))
        return MOE_EALIGN;
    (void)hipGetLastError();
    return moe::launch_qb_unpack(bits, packed, rows, cols, dst, static_cast<hipStream_t>(stream));
}

int moe_q2_unpack(const void *packed, int64_t rows, int64_t cols, float *dst, void *stream)
{
    return moe_qb_unpack(2, packed, rows, cols, dst, stream);
}

}  // extern "C"
