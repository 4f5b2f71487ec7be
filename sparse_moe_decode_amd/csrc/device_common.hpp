// Device helpers shared by the gfx950 kernels: weight-format access, wave64
// reductions and the workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxK = 16;
constexpr int kMaxE = 1024;
constexpr int kMaxRows = 4;   // rows per few-row call

// ------------------------------------------------------------ formats
//
// Every matrix is read in 16-byte "chunks" (f32: 4 values, bf16: 8 values)
// or, for the b-bit block formats, in 32-weight blocks (4b bytes of codes
// plus one dword holding the fp16 scale and min).

struct F32 {
    static constexpr int kChunk = 4;   // elements per chunk
};
struct BF16 {
    static constexpr int kChunk = 8;
};
template <int B>
struct QB {
    static constexpr int kChunk = 32;
    static constexpr int kBits = B;
};
using Q2 = QB<2>;
using Q3 = QB<3>;
using Q4 = QB<4>;

template <typename W>
struct is_block_format {
    static constexpr bool value = false;
};
template <int B>
struct is_block_format<QB<B>> {
    static constexpr bool value = true;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp16 bits -> fp32 (exact; fp16 subnormals are kept by the conversion)
__device__ __forceinline__ float f16_to_f32(uint32_t bits16)
{
    _Float16 h;
    uint16_t b = static_cast<uint16_t>(bits16);
    __builtin_memcpy(&h, &b, 2);
    return static_cast<float>(h);
}

// A dense matrix of type F32/BF16: row-major, `cols` elements per row.
// A b-bit matrix: codes plane then scale/min plane (see moe_qb_pack).
struct MatRef {
    const uint8_t *base;   // matrix start
    int rows, cols;
};

// Byte size of one stacked b-bit matrix: (b + 1) / 8 bytes per weight,
// rounded up to 256.
__host__ __device__ inline size_t qb_packed_bytes(int bits, int64_t rows, int64_t cols)
{
    const uint64_t raw = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols) / 8u * static_cast<uint64_t>(bits + 1);
    return static_cast<size_t>((raw + 255u) / 256u * 256u);
}

template <typename W>
struct MatBytes;
template <>
struct MatBytes<F32> {
    __host__ __device__ static size_t of(int64_t rows, int64_t cols) { return rows * cols * 4; }
};
template <>
struct MatBytes<BF16> {
    __host__ __device__ static size_t of(int64_t rows, int64_t cols) { return rows * cols * 2; }
};
template <int B>
struct MatBytes<QB<B>> {
    __host__ __device__ static size_t of(int64_t rows, int64_t cols) { return qb_packed_bytes(B, rows, cols); }
};
template <typename W>
__host__ __device__ inline size_t mat_bytes(int64_t rows, int64_t cols) { return MatBytes<W>::of(rows, cols); }

// Code j (0..31) of a b-bit block held as dwords cw[] (the block's 4b bytes
// read little-endian): bits b*j .. b*j+b-1; a code that straddles two
// dwords is joined with one funnel shift. j is a compile-time constant after
// unrolling, so each code costs one or two instructions.
template <int B, int N>
__device__ __forceinline__ uint32_t block_code(const uint32_t (&cw)[N], int j)
{
    const int bit = B * j, w = bit >> 5, sh = bit & 31;
    const uint32_t v = sh + B <= 32 ? cw[w] >> sh : __builtin_amdgcn_alignbit(cw[w + 1], cw[w], sh);
    return v & ((1u << B) - 1u);
}

// ----------------------------------------------------------- reductions

template <typename T>
__device__ __forceinline__ T lane_group_sum(T v, int width)
{
    for (int off = width >> 1; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// Loads of weight data, which each call reads once: non-temporal, so the
// stream does not displace the small hot data (activations, routing state)
// from the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt16(const void *p)
{
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void *p)
{
    const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint32_t ld_nt4(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ uint32_t ld_nt2(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}

// Sum over the 64 lanes of a wave, returned in every lane: DPP adds within
// each row of 16 lanes (quad permutations [1,0,3,2] and [2,3,0,1], then row
// rotations by 4 and 8), then the four row sums read from lanes 0/16/32/48.
__device__ __forceinline__ float dpp_row_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
    v = dpp_row_sum(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ double wave_sum(double v)
{
#define MOE_DPP_ADD_F64(ctrl)                                                                                    \
    {                                                                                                            \
        const long long b = __double_as_longlong(v);                                                             \
        const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b & 0xffffffff), ctrl, 0xF, 0xF, false);  \
        const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), ctrl, 0xF, 0xF, false);         \
        v += __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));              \
    }
    MOE_DPP_ADD_F64(0xB1)
    MOE_DPP_ADD_F64(0x4E)
    MOE_DPP_ADD_F64(0x124)
    MOE_DPP_ADD_F64(0x128)
#undef MOE_DPP_ADD_F64
    double r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const long long b = __double_as_longlong(v);
        const int lo = __builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffff), 16 * i);
        const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 16 * i);
        r[i] = __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
}

// Pre-MoE RMS norm of R rows of H fp32 values staged in LDS (row q at
// xs + q * H), in place: u_h = fp32(x_h * r * gamma_h) with
// r = 1 / sqrt(sum_h x_h^2 / H + eps); the sum of squares is in double (each
// square is exact there; only the order of the additions differs from a
// sequential sum), r and the products too, u rounded once. The float4 at
// slot i of a row holds the values of float4 logical(i) (the 2-bit chunk
// order of x). Every thread of the workgroup (at most 16 waves) calls it; it
// begins and ends with a workgroup barrier.
template <int R, typename Map>
__device__ __forceinline__ void rms_norm_rows(float *xs, int H, const float *gamma, float eps, Map logical)
{
    __shared__ double part[R][16];
    __shared__ double rr[R];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, nw = blockDim.x / kWave;
    const int n4 = H >> 2;
    float4 *x4 = reinterpret_cast<float4 *>(xs);
    __syncthreads();
    for (int q = 0; q < R; ++q) {
        double ss = 0.0;
        for (int i = tid; i < n4; i += blockDim.x) {
            const float4 v = x4[q * n4 + i];
            ss += static_cast<double>(v.x) * v.x + static_cast<double>(v.y) * v.y + static_cast<double>(v.z) * v.z +
                  static_cast<double>(v.w) * v.w;
        }
        ss = wave_sum(ss);
        if (lane == 0)
            part[q][wave] = ss;
    }
    __syncthreads();
    if (tid < R) {
        double t = 0.0;
        for (int w = 0; w < nw; ++w)
            t += part[tid][w];
        rr[tid] = 1.0 / sqrt(t / H + static_cast<double>(eps));
    }
    __syncthreads();
    const float4 *g4 = reinterpret_cast<const float4 *>(gamma);
    for (int i = tid; i < n4; i += blockDim.x) {
        const float4 g = g4[logical(i)];
        for (int q = 0; q < R; ++q) {
            const double r = rr[q];
            float4 v = x4[q * n4 + i];
            v.x = static_cast<float>(static_cast<double>(v.x) * r * static_cast<double>(g.x));
            v.y = static_cast<float>(static_cast<double>(v.y) * r * static_cast<double>(g.y));
            v.z = static_cast<float>(static_cast<double>(v.z) * r * static_cast<double>(g.z));
            v.w = static_cast<float>(static_cast<double>(v.w) * r * static_cast<double>(g.w));
            x4[q * n4 + i] = v;
        }
    }
    __syncthreads();
}

// The float4 slot maps of rms_norm_rows: rows in order, or the 2-bit chunk
// order (chunk c of 32-value block b at c ^ (b & 7), an involution).
struct SlotsInOrder {
    __device__ int operator()(int i) const { return i; }
};
struct SlotsQ2 {
    __device__ int operator()(int i) const { return (i & ~7) | ((i & 7) ^ ((i >> 3) & 7)); }
};

__device__ __forceinline__ float silu_mul(float a, float c)
{
    return a / (1.0f + __expf(-a)) * c;
}

__device__ __forceinline__ int next_pow2(int v)
{
    int p = 1;
    while (p < v)
        p <<= 1;
    return p;
}

// ------------------------------------------------------------ workspace
//
// Layout of the decode / few-row workspace (all offsets 256-byte aligned):
//   control     : counters and flags (256 B)
//   logits      : [R][E] double
//   zlogit      : [R] double
//   slot table  : nslots, slot_expert[S], slot_w[S][R] (S = R*K + 1)
//   hbuf        : [S][R][Imax] fp32   (weighted SwiGLU activations, one row
//                 per (slot, row) pair; at most R*(K+1) rows are used)
// Reserved header at the start of every workspace (no kernel keeps state
// in it; the workspaces need no initialization).
struct Control {
    unsigned int reserved[64];
};

// Slots of a decode / few-row call: slot 0 is the shared expert, slots
// 1.. the distinct routed experts. The (slot, row) pairs of the rows that use
// a slot are numbered slot-major: pair pstart[s] + (rank of row q among the
// rows of rmask[s]); the gate/up pass writes h' of pair i to row i of hbuf.
struct SlotTable {
    int nslots;
    int pad[3];
    int expert[kMaxRows * kMaxK + 1];          // slot 0 = shared expert (-1)
    float w[kMaxRows * kMaxK + 1][kMaxRows];   // per-row weight (0: row does not use the slot)
    uint32_t rmask[kMaxRows * kMaxK + 1];      // rows that use the slot
    int pstart[kMaxRows * kMaxK + 2];          // first pair of each slot; [nslots] = pair count
};

// Bound on the pairs of a call of R rows: each row uses K routed slots and
// the shared one.
__host__ __device__ inline int max_pairs(int R, int K) { return R * (K + 1); }

struct DecodeWs {
    Control *ctl;
    double *logits;
    double *zlogit;
    SlotTable *slots;
    float *hbuf;
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

__host__ __device__ inline size_t decode_ws_bytes(int R, int E, int K, int Imax)
{
    const int S = R * K + 1;
    return align256(sizeof(Control)) + align256(sizeof(double) * R * E) + align256(sizeof(double) * R) +
           align256(sizeof(SlotTable)) + align256(sizeof(float) * S * R * Imax);
}

__host__ __device__ inline DecodeWs decode_ws_carve(void *ws, int R, int E, int K, int Imax)
{
    (void)K;
    (void)Imax;
    uint8_t *p = static_cast<uint8_t *>(ws);
    DecodeWs w;
    w.ctl = reinterpret_cast<Control *>(p);
    p += align256(sizeof(Control));
    w.logits = reinterpret_cast<double *>(p);
    p += align256(sizeof(double) * R * E);
    w.zlogit = reinterpret_cast<double *>(p);
    p += align256(sizeof(double) * R);
    w.slots = reinterpret_cast<SlotTable *>(p);
    p += align256(sizeof(SlotTable));
    w.hbuf = reinterpret_cast<float *>(p);
    return w;
}

}  // namespace moe
