// moe_forward_noalloc: moe_forward on a scratch buffer the library owns, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array per GPU (each device that loads
// the library holds its own copy until the process ends). Host code never
// uses the array's name as an address: on the first call on a device, with
// that device current, its address is taken with hipGetSymbolAddress and kept
// per device; that pointer is what the kernels receive, exactly as they
// receive a caller's workspace in moe_forward. The kernels need no
// initialization of it (no state survives between calls), so nothing is
// cleared here. Every call on one GPU shares that GPU's array: calls that
// overlap in time on one GPU (two streams, two host threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

namespace {

__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of this GPU's scratch array, or null if it cannot be had.
void *scratch_of_current_device()
{
    static std::mutex mu;
    static void *ptr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        ptr[dev] = p;
    }
    return ptr[dev];
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_layer_desc *d, const float *x, int32_t T, float *y,
                                   const int32_t *ids_in, const float *wts_in, const float *gate_in,
                                   int32_t *ids_out, float *wts_out, float *gate_out, void *stream)
{
    if (T < 0)
        return MOE_EINVAL;
    if (T == 0)
        return MOE_OK;
    const size_t need = moe_workspace_bytes(d, T);
    if (need == 0)   // an invalid descriptor: moe_forward returns its status before using a workspace
        return moe_forward(d, x, T, y, ids_in, wts_in, gate_in, ids_out, wts_out, gate_out, nullptr, 0, stream);
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_EWORKSPACE;
    void *ws = scratch_of_current_device();
    if (!ws)
        return MOE_EHIP;
    return moe_forward(d, x, T, y, ids_in, wts_in, gate_in, ids_out, wts_out, gate_out, ws,
                       MOE_NOALLOC_SCRATCH_BYTES, stream);
}
