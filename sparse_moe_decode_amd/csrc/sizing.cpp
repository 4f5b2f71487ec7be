// Workspace and LDS sizing of the launchers (host only, no kernels).
#include "internal.h"
#include "workspace.hpp"

namespace moe {

size_t gateup_lds_bytes(int R, int H, int E)
{
    const size_t a = sizeof(float) * (R * H + R * (H >> 5)), b = sizeof(double) * R * ((E + 1) & ~1);
    return a > b ? a : b;
}

int decode_ws_size(const moe_layer_desc *d, int R)
{
    const int imax = d->inter > d->shared_inter ? d->inter : d->shared_inter;
    return static_cast<int>(decode_ws_bytes(R, d->n_experts, d->top_k, imax));
}

size_t sort_ws_bytes_tke(int64_t n, int E)
{
    const int64_t chunks = (n + kSortChunk - 1) / kSortChunk;
    return align256(sizeof(Control)) + align256(sizeof(int) * static_cast<size_t>(chunks) * E);
}

size_t prefill_ws_bytes(const moe_layer_desc *d, int T)
{
    return prefill_carve(nullptr, d, T, false).sort_bytes;
}

}  // namespace moe
