// Host-side packer for the b-bit block weight formats (MOE_Q2B32,
// MOE_Q3B32, MOE_Q4B32; b = 2, 3, 4).
//
// Format: 32 weights per block along a row, b-bit unsigned codes, fp16 scale
// and fp16 minimum, w = code * scale + min. The pages' kernels work on
// 32-weight chunks of the expert rows (Red Lite "Research notes, October
// 2026", section 4, narrow-row mul_mv entry); the block, code width and
// formula are the layer's stated 2-bit format, and the 3- and 4-bit widths
// are the higher-precision expert files of the same model ("DwarfStar Red
// Lite" guide, the IQ3_XXS file). Quantizer rule and physical layout are
// documented in include/moe.h.
//
// Built with -ffp-contract=off: every float operation below is one IEEE
// binary32 operation with round-to-nearest-even.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "moe.h"

namespace {

// fp32 -> fp16 bits, round to nearest even, by integer manipulation of the
// binary32 encoding.
uint16_t f32_to_f16_bits(float f)
{
    uint32_t x;
    std::memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7fffffffu;
    if (ax > 0x7f800000u)
        return static_cast<uint16_t>(sign | 0x7e00u);           // NaN
    if (ax >= 0x477ff000u)                                        // >= 65520 rounds to inf
        return static_cast<uint16_t>(sign | 0x7c00u);
    if (ax < 0x38800000u) {                                       // below 2^-14: subnormal result
        if (ax <= 0x33000000u)                                    // <= 2^-25 rounds to 0 (tie -> even)
            return static_cast<uint16_t>(sign);
        const uint32_t e = ax >> 23;                              // 102..112
        const uint32_t m = (ax & 0x7fffffu) | 0x800000u;
        const uint32_t shift = 126u - e;                          // value / 2^-24 = m >> shift
        uint32_t q = m >> shift;
        const uint32_t rem = m & ((1u << shift) - 1u);
        const uint32_t half = 1u << (shift - 1u);
        if (rem > half || (rem == half && (q & 1u)))
            ++q;
        return static_cast<uint16_t>(sign | q);
    }
    uint32_t r = ax - 0x38000000u;                                // rebias 127 -> 15
    r = (r + 0x0fffu + ((r >> 13) & 1u)) >> 13;                   // 23 -> 10 mantissa bits, RNE
    return static_cast<uint16_t>(sign | r);
}

float f16_bits_to_f32(uint16_t h)
{
    const uint32_t sign = static_cast<uint32_t>(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t m = h & 0x3ffu;
    uint32_t x;
    if (e == 0) {
        if (m == 0) {
            x = sign;
        } else {
            int s = 0;
            while (!(m & 0x400u)) {
                m <<= 1;
                ++s;
            }
            x = sign | (static_cast<uint32_t>(113 - s) << 23) | ((m & 0x3ffu) << 13);
        }
    } else if (e == 31) {
        x = sign | 0x7f800000u | (m << 13);
    } else {
        x = sign | ((e + 112u) << 23) | (m << 13);
    }
    float f;
    std::memcpy(&f, &x, 4);
    return f;
}

bool bits_ok(int32_t bits) { return bits >= 2 && bits <= 4; }

}  // namespace

extern "C" size_t moe_qb_packed_bytes(int32_t bits, int64_t rows, int64_t cols)
{
    if (!bits_ok(bits) || rows <= 0 || cols <= 0 || cols % 32 != 0)
        return 0;
    // b bits of code plus 32 bits of scale/min per 32 weights: (b + 1) / 8 bytes per weight
    const uint64_t raw = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols) / 8u * static_cast<uint64_t>(bits + 1);
    return static_cast<size_t>((raw + 255u) / 256u * 256u);
}

extern "C" int moe_qb_pack(int32_t bits, const float *src, int64_t rows, int64_t cols, void *dst, size_t dst_bytes)
{
    if (!bits_ok(bits) || !src || !dst || rows <= 0 || cols <= 0 || cols % 32 != 0)
        return MOE_EINVAL;
    const size_t need = moe_qb_packed_bytes(bits, rows, cols);
    if (dst_bytes < need)
        return MOE_EWORKSPACE;
    const int top = (1 << bits) - 1;
    const float levels = static_cast<float>(top);
    const int64_t nb = cols / 32, cbytes = 4 * bits;   // code bytes per block
    uint8_t *out = static_cast<uint8_t *>(dst);
    uint8_t *codes = out;
    uint8_t *sm = out + rows * nb * cbytes;
    const size_t used = static_cast<size_t>(rows * nb * (cbytes + 4));
    std::memset(out + used, 0, need - used);

    for (int64_t r = 0; r < rows; ++r) {
        const float *row = src + r * cols;
        for (int64_t b = 0; b < nb; ++b) {
            const float *w = row + b * 32;
            float lo = w[0], hi = w[0];
            for (int j = 0; j < 32; ++j) {
                if (!std::isfinite(w[j]))
                    return MOE_ENONFINITE;
                lo = w[j] < lo ? w[j] : lo;
                hi = w[j] > hi ? w[j] : hi;
            }
            const uint16_t min_h = f32_to_f16_bits(lo);
            const float minf = f16_bits_to_f32(min_h);
            const float span = hi - minf;
            const float step = span / levels;
            const uint16_t scale_h = f32_to_f16_bits(step);
            const float scalef = f16_bits_to_f32(scale_h);
            if (!std::isfinite(minf) || !std::isfinite(scalef))
                return MOE_ENONFINITE;
            // the block's codes as one little-endian integer of 32*b bits,
            // weight j at bits b*j .. b*j+b-1
            uint64_t acc[2] = {0, 0};
            if (scalef != 0.0f) {
                for (int j = 0; j < 32; ++j) {
                    const float t = (w[j] - minf) / scalef;
                    const float n = std::nearbyint(t);
                    const uint64_t c = n <= 0.0f ? 0u : (n >= levels ? static_cast<uint64_t>(top)
                                                                      : static_cast<uint64_t>(n));
                    const int bit = bits * j;
                    acc[bit >> 6] |= c << (bit & 63);
                    if ((bit & 63) + bits > 64)
                        acc[(bit >> 6) + 1] |= c >> (64 - (bit & 63));
                }
            }
            uint8_t *cb = codes + (r * nb + b) * cbytes;
            for (int i = 0; i < cbytes; ++i)
                cb[i] = static_cast<uint8_t>(acc[i >> 3] >> (8 * (i & 7)));
            uint8_t *p = sm + (r * nb + b) * 4;
            p[0] = static_cast<uint8_t>(scale_h & 0xff);
            p[1] = static_cast<uint8_t>(scale_h >> 8);
            p[2] = static_cast<uint8_t>(min_h & 0xff);
            p[3] = static_cast<uint8_t>(min_h >> 8);
        }
    }
    return MOE_OK;
}

extern "C" size_t moe_q2_packed_bytes(int64_t rows, int64_t cols) { return moe_qb_packed_bytes(2, rows, cols); }

extern "C" int moe_q2_pack(const float *src, int64_t rows, int64_t cols, void *dst, size_t dst_bytes)
{
    return moe_qb_pack(2, src, rows, cols, dst, dst_bytes);
}
