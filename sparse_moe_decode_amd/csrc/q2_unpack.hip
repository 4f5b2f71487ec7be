// Device unpack of one 2-bit packed matrix to fp32 (bit-exact test hook).
// One thread per 32-weight block: w = code * scale + min, where the product
// is exact (an fp16 significand times a value <= 3 fits binary32) and the
// add rounds once, so the result equals the format definition bit for bit.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "internal.h"

namespace moe {

__global__ void __launch_bounds__(256) k_q2_unpack(const uint8_t *packed, int64_t rows, int64_t cols, float *dst)
{
    const int64_t nb = cols >> 5;
    const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (blk >= rows * nb)
        return;
    const int64_t r = blk / nb, b = blk % nb;
    const uint2 cw = *reinterpret_cast<const uint2 *>(packed + r * (cols >> 2) + b * 8);
    const uint32_t sm = *reinterpret_cast<const uint32_t *>(packed + rows * (cols >> 2) + blk * 4);
    const float s = f16_to_f32(sm & 0xffffu);
    const float m = f16_to_f32(sm >> 16);
    float *out = dst + r * cols + b * 32;
#pragma unroll
    for (int j4 = 0; j4 < 8; ++j4) {
        const uint32_t d = (j4 < 4 ? cw.x : cw.y) >> (8 * (j4 & 3));
        float4 v;
        v.x = __fmaf_rn(static_cast<float>(d & 3u), s, m);
        v.y = __fmaf_rn(static_cast<float>((d >> 2) & 3u), s, m);
        v.z = __fmaf_rn(static_cast<float>((d >> 4) & 3u), s, m);
        v.w = __fmaf_rn(static_cast<float>((d >> 6) & 3u), s, m);
        *reinterpret_cast<float4 *>(out + j4 * 4) = v;
    }
}

int launch_q2_unpack(const void *packed, int64_t rows, int64_t cols, float *dst, hipStream_t s)
{
    const int64_t blocks = rows * (cols / 32);
    const int64_t grid = (blocks + 255) / 256;
    if (grid > 0x7fffffff)
        return MOE_EUNSUPPORTED;
    hipLaunchKernelGGL(k_q2_unpack, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                       static_cast<const uint8_t *>(packed), rows, cols, dst);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
