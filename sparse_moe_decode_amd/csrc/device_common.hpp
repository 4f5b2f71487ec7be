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
// or, for the 2-bit format, in 32-weight blocks (8 bytes of codes plus one
// dword holding the fp16 scale and min).

struct F32 {
    static constexpr int kChunk = 4;   // elements per chunk
};
struct BF16 {
    static constexpr int kChunk = 8;
};
struct Q2 {
    static constexpr int kChunk = 32;
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
// A Q2 matrix: codes plane then scale/min plane (see moe_q2_pack).
struct MatRef {
    const uint8_t *base;   // matrix start
    int rows, cols;
};

// Byte size of one stacked matrix of each format.
__host__ __device__ inline size_t q2_packed_bytes(int64_t rows, int64_t cols)
{
    const uint64_t raw = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols) / 8u * 3u;
    return static_cast<size_t>((raw + 255u) / 256u * 256u);
}

template <typename W>
__host__ __device__ inline size_t mat_bytes(int64_t rows, int64_t cols);
template <>
__host__ __device__ inline size_t mat_bytes<F32>(int64_t rows, int64_t cols) { return rows * cols * 4; }
template <>
__host__ __device__ inline size_t mat_bytes<BF16>(int64_t rows, int64_t cols) { return rows * cols * 2; }
template <>
__host__ __device__ inline size_t mat_bytes<Q2>(int64_t rows, int64_t cols) { return q2_packed_bytes(rows, cols); }

// ----------------------------------------------------------- chunk dots
//
// dot of chunk `c` of row `r` with a vector v (fp32, in LDS), accumulated
// into acc[R] for R vectors laid out with stride `vs`. For Q2 `vsum` holds
// the per-block sums of each vector (stride vss), used for the min term:
//   sum_j (code_j*s + m) v_j = s * sum_j code_j v_j + m * sum_j v_j.

template <int R>
__device__ __forceinline__ void chunk_dot(F32, const MatRef &M, int r, int c, const float *v, int vs,
                                          const float *, int, float (&acc)[R])
{
    const float4 w = *reinterpret_cast<const float4 *>(M.base + (static_cast<size_t>(r) * M.cols + c * 4) * 4);
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 xv = *reinterpret_cast<const float4 *>(v + q * vs + c * 4);
        acc[q] = fmaf(w.x, xv.x, acc[q]);
        acc[q] = fmaf(w.y, xv.y, acc[q]);
        acc[q] = fmaf(w.z, xv.z, acc[q]);
        acc[q] = fmaf(w.w, xv.w, acc[q]);
    }
}

template <int R>
__device__ __forceinline__ void chunk_dot(BF16, const MatRef &M, int r, int c, const float *v, int vs,
                                          const float *, int, float (&acc)[R])
{
    const uint4 w = *reinterpret_cast<const uint4 *>(M.base + (static_cast<size_t>(r) * M.cols + c * 8) * 2);
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 x0 = *reinterpret_cast<const float4 *>(v + q * vs + c * 8);
        const float4 x1 = *reinterpret_cast<const float4 *>(v + q * vs + c * 8 + 4);
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

// codes of one 32-weight block: two dwords, weight j at bits 2*(j%16) of dword j/16
template <int R>
__device__ __forceinline__ void chunk_dot(Q2, const MatRef &M, int r, int b, const float *v, int vs,
                                          const float *vsum, int vss, float (&acc)[R])
{
    const int nb = M.cols >> 5;
    const uint2 cw = *reinterpret_cast<const uint2 *>(M.base + static_cast<size_t>(r) * (M.cols >> 2) + b * 8);
    const uint32_t sm = *reinterpret_cast<const uint32_t *>(
        M.base + static_cast<size_t>(M.rows) * (M.cols >> 2) + (static_cast<size_t>(r) * nb + b) * 4);
    const float s = f16_to_f32(sm & 0xffffu);
    const float m = f16_to_f32(sm >> 16);
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float *x = v + q * vs + b * 32;
        float cx = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t d = half ? cw.y : cw.x;
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const float4 xv = *reinterpret_cast<const float4 *>(x + half * 16 + j4 * 4);
                const uint32_t byte = d >> (8 * j4);
                cx = fmaf(static_cast<float>(byte & 3u), xv.x, cx);
                cx = fmaf(static_cast<float>((byte >> 2) & 3u), xv.y, cx);
                cx = fmaf(static_cast<float>((byte >> 4) & 3u), xv.z, cx);
                cx = fmaf(static_cast<float>((byte >> 6) & 3u), xv.w, cx);
            }
        }
        acc[q] = fmaf(s, cx, fmaf(m, vsum[q * vss + b], acc[q]));
    }
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
