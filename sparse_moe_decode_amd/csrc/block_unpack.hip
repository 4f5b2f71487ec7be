// Device unpack of one b-bit packed matrix to fp32 (bit-exact test hook).
// One thread per 32-weight block: w = code * scale + min, where the product
// is exact (an fp16 significand times a code below 16 fits binary32) and the
// add rounds once, so the result equals the format definition bit for bit.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "internal.h"

namespace moe {

template <int B>
__global__ void __launch_bounds__(256) k_qb_unpack(const uint8_t *packed, int64_t rows, int64_t cols, float *dst)
{
    const int64_t nb = cols >> 5;
    const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (blk >= rows * nb)
        return;
    // codes of block blk: 4B bytes at blk * 4B (4-byte aligned)
    uint32_t cw[B];
    const uint32_t *src = reinterpret_cast<const uint32_t *>(packed + blk * 4 * B);
#pragma unroll
    for (int i = 0; i < B; ++i)
        cw[i] = src[i];
    const uint32_t sm = *reinterpret_cast<const uint32_t *>(packed + rows * nb * 4 * B + blk * 4);
    const float s = f16_to_f32(sm & 0xffffu);
    const float m = f16_to_f32(sm >> 16);
    float *out = dst + blk * 32;
#pragma unroll
    for (int j4 = 0; j4 < 8; ++j4) {
        float4 v;
        v.x = __fmaf_rn(static_cast<float>(block_code<B>(cw, 4 * j4)), s, m);
        v.y = __fmaf_rn(static_cast<float>(block_code<B>(cw, 4 * j4 + 1)), s, m);
        v.z = __fmaf_rn(static_cast<float>(block_code<B>(cw, 4 * j4 + 2)), s, m);
        v.w = __fmaf_rn(static_cast<float>(block_code<B>(cw, 4 * j4 + 3)), s, m);
        *reinterpret_cast<float4 *>(out + j4 * 4) = v;
    }
}

int launch_qb_unpack(int bits, const void *packed, int64_t rows, int64_t cols, float *dst, hipStream_t s)
{
    const int64_t blocks = rows * (cols / 32);
    const int64_t grid = (blocks + 255) / 256;
    if (grid > 0x7fffffff)
        return MOE_EUNSUPPORTED;
    const uint8_t *p = static_cast<const uint8_t *>(packed);
    const dim3 g(static_cast<unsigned>(grid)), b(256);
    if (bits == 2)
        hipLaunchKernelGGL(k_qb_unpack<2>, g, b, 0, s, p, rows, cols, dst);
    else if (bits == 3)
        hipLaunchKernelGGL(k_qb_unpack<3>, g, b, 0, s, p, rows, cols, dst);
    else if (bits == 4)
        hipLaunchKernelGGL(k_qb_unpack<4>, g, b, 0, s, p, rows, cols, dst);
    else
        return MOE_EINVAL;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
