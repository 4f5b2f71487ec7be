// Prefill path (many rows per call): rows grouped by expert, grouped bf16 MFMA
// GEMMs on gfx950 (the batched-prefill chunk of the Red Lite "guide" page,
// section "Chat defaults", processes 2048 prompt tokens per pass).
//
//   k_split_x         x (fp32) -> x_hi + x_lo (bf16 pair; x - hi - lo is
//                     below 2^-17 |x|)
//   k_logits64        router logits [T][E] and shared-gate logits [T] in
//                     fp64: exact products, a fixed summation order
//   k_select_rows     exact top-K per row (one wave per row), softmax weights,
//                     sigmoid gate
//   sort (sort.hip)   stable counting sort of the T*K (row, slot) pairs by
//                     expert, with the inverse permutation
//   k_tiles           per-expert 64-row tile offsets
//   k_gemm_gateup     per (expert, 64-row tile, 64-channel block): gathered
//                     x rows times the gate and up rows of the expert, SwiGLU,
//                     times the route weight -> h (fp32, sorted row order)
//   k_gemm_down       per (expert, 64-row tile, 128-column block): h times the
//                     expert's down rows -> one output row per (row, slot)
//   k_combine         y[t] = sum_k out[(t, k)] + g_t * shared(t)
// The shared expert uses the same GEMM kernels over all rows.
//
// MFMA precision: weights enter as an exact bf16 (bf16 weights) or as a
// bf16 hi+lo pair of their fp32 value (2-bit weights are first decoded
// exactly, w = code*scale + min); activations enter as hi+lo pairs. The
// products hi*hi + hi*lo + lo*hi are accumulated in fp32 by
// v_mfma_f32_16x16x32_bf16, giving ~2^-16 relative error per term.
#include <hip/hip_runtime.h>

#include "device_common.cuh"
#include "internal.h"
#include "routing.cuh"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ uint32_t bf16_rne_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 8 fp32 values -> bf16 hi (packed, 4 dwords) and lo = bf16(v - hi).
__device__ __forceinline__ void split8(const float (&v)[8], uint4 &hi, uint4 &lo)
{
    uint32_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        h[j] = bf16_rne_bits(v[j]);
        l[j] = bf16_rne_bits(v[j] - __uint_as_float(h[j] << 16));
    }
    hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}

// ============================================================== split x

__global__ void __launch_bounds__(256) k_split_x(const float *x, int64_t n8, uint4 *xh, uint4 *xl)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n8)
        return;
    const float4 a = reinterpret_cast<const float4 *>(x)[2 * i];
    const float4 b = reinterpret_cast<const float4 *>(x)[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint4 hi, lo;
    split8(v, hi, lo);
    xh[i] = hi;
    xl[i] = lo;
}

// =========================================================== fp64 logits

constexpr int kLgTile = 64;

// One 64x64 tile of logits (rows t, experts e; expert index E is the
// shared-gate vector). 16x16 threads, 4x4 outputs each, k in steps of 32.
template <typename RT>
__global__ void __launch_bounds__(256) k_logits64(const float *x, int T, int H, int E, const uint8_t *router_w,
                                                  const uint8_t *gate_w, const float *bias, double *logits,
                                                  double *z)
{
    __shared__ float xs[kLgTile][33];
    __shared__ float wsm[kLgTile][33];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int e0 = blockIdx.x * kLgTile, t0 = blockIdx.y * kLgTile;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = 0.0;
    const int lr = tid >> 2, lp = tid & 3;   // loader: row, 8-element part
    for (int k0 = 0; k0 < H; k0 += 32) {
        {
            const int t = t0 + lr;
            float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (t < T) {
                const float4 a = *reinterpret_cast<const float4 *>(x + static_cast<size_t>(t) * H + k0 + lp * 8);
                const float4 b = *reinterpret_cast<const float4 *>(x + static_cast<size_t>(t) * H + k0 + lp * 8 + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                xs[lr][lp * 8 + j] = v[j];
        }
        {
            const int e = e0 + lr;
            float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (e <= E) {
                if (RT::kChunk == 4) {
                    const float *row = reinterpret_cast<const float *>(e < E ? router_w + static_cast<size_t>(e) * H * 4
                                                                             : gate_w);
                    const float4 a = *reinterpret_cast<const float4 *>(row + k0 + lp * 8);
                    const float4 b = *reinterpret_cast<const float4 *>(row + k0 + lp * 8 + 4);
                    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
                } else {
                    const uint16_t *row = reinterpret_cast<const uint16_t *>(
                        e < E ? router_w + static_cast<size_t>(e) * H * 2 : gate_w);
                    const uint4 u = *reinterpret_cast<const uint4 *>(row + k0 + lp * 8);
                    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
                    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                wsm[lr][lp * 8 + j] = v[j];
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < 32; ++k) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = static_cast<double>(xs[ty * 4 + i][k]);
                b[i] = static_cast<double>(wsm[tx * 4 + i][k]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= T)
            continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E)
                logits[static_cast<size_t>(t) * E + e] = acc[i][j] + (bias ? static_cast<double>(bias[e]) : 0.0);
            else if (e == E)
                z[t] = acc[i][j];
        }
    }
}

// ============================================================ selection

// One wave per row: exact top-K, weights, gate (routing.cuh).
__global__ void __launch_bounds__(256) k_select_rows(const double *logits, const double *z, int T, int E, int K,
                                                     int renorm, int32_t *ids, float *wts, float *gate,
                                                     int32_t *ids_out, float *wts_out, float *gate_out)
{
    __shared__ RouteLds rl;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int t = blockIdx.x * (blockDim.x / kWave) + wave;
    if (t >= T)
        return;
    const double *lg = logits + static_cast<size_t>(t) * E;
    wave_route(lg, E, K, renorm, z[t], wave, rl, lane);
    __builtin_amdgcn_wave_barrier();
    if (lane < K) {
        const int e = rl.sel_e[wave][lane];
        const float w = rl.sel_w[wave][lane];
        ids[t * K + lane] = e;
        wts[t * K + lane] = w;
        if (ids_out)
            ids_out[t * K + lane] = e;
        if (wts_out)
            wts_out[t * K + lane] = w;
    }
    if (lane == 0) {
        gate[t] = rl.g[wave];
        if (gate_out)
            gate_out[t] = rl.g[wave];
    }
}

// Caller-supplied routing: ids outside [0, E) become expert 0 with weight 0.
__global__ void __launch_bounds__(256) k_take_routing(const int32_t *ids_in, const float *wts_in, const float *gate_in,
                                                      int n, int T, int E, int32_t *ids, float *wts, float *gate)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const int e = ids_in[i];
        const bool ok = e >= 0 && e < E;
        ids[i] = ok ? e : 0;
        wts[i] = ok ? wts_in[i] : 0.0f;
    }
    if (i < T)
        gate[i] = gate_in[i];
}

// Per-expert tile offsets: tile_off[e] = sum_{e' < e} ceil(count[e'] / 64).
__global__ void __launch_bounds__(1024) k_tiles(const int32_t *counts, int E, int32_t *tile_off)
{
    __shared__ int s[kMaxE];
    const int t = threadIdx.x;
    const int v = t < E ? (counts[t] + 63) / 64 : 0;
    if (t < E)
        s[t] = v;
    __syncthreads();
    for (int off = 1; off < E; off <<= 1) {
        int a = 0;
        if (t < E && t >= off)
            a = s[t - off];
        __syncthreads();
        if (t < E)
            s[t] += a;
        __syncthreads();
    }
    if (t < E)
        tile_off[t] = s[t] - v;
    if (t == 0)
        tile_off[E] = s[E - 1];
}

// ================================================================= GEMMs

constexpr int kBM = 64;          // rows per tile
constexpr int kLDK = 40;         // LDS row stride in bf16 (32 + 8 padding)

// 8 consecutive weights (k0 .. k0+7) of row n of a [rows][cols] matrix as
// bf16 hi/lo. Rows past the end give zeros.
__device__ __forceinline__ void b_piece(Q2, const uint8_t *base, int rows, int cols, int n, int k0, uint4 &hi,
                                        uint4 &lo)
{
    if (n >= rows) {
        hi = lo = make_uint4(0, 0, 0, 0);
        return;
    }
    const int nb = cols >> 5, b = k0 >> 5, part = (k0 & 31) >> 3;
    const uint32_t codes =
        *reinterpret_cast<const uint16_t *>(base + static_cast<size_t>(n) * (cols >> 2) + b * 8 + part * 2);
    const uint32_t sm = *reinterpret_cast<const uint32_t *>(base + static_cast<size_t>(rows) * (cols >> 2) +
                                                            (static_cast<size_t>(n) * nb + b) * 4);
    const float s = f16_to_f32(sm & 0xffffu), m = f16_to_f32(sm >> 16);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = __fmaf_rn(static_cast<float>((codes >> (2 * j)) & 3u), s, m);
    split8(v, hi, lo);
}
__device__ __forceinline__ void b_piece(BF16, const uint8_t *base, int rows, int cols, int n, int k0, uint4 &hi,
                                        uint4 &lo)
{
    lo = make_uint4(0, 0, 0, 0);
    hi = n < rows ? *reinterpret_cast<const uint4 *>(base + (static_cast<size_t>(n) * cols + k0) * 2) : lo;
}
__device__ __forceinline__ void b_piece(F32, const uint8_t *base, int rows, int cols, int n, int k0, uint4 &hi,
                                        uint4 &lo)
{
    if (n >= rows) {
        hi = lo = make_uint4(0, 0, 0, 0);
        return;
    }
    const float *p = reinterpret_cast<const float *>(base) + static_cast<size_t>(n) * cols + k0;
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split8(v, hi, lo);
}

struct GemmArgs {
    // rows: routed (sorted pair rows of expert groups) or shared (all T rows)
    int routed;
    int T, K, E;
    const int32_t *tile_off;   // [E+1] (routed)
    const int32_t *offsets;    // [E+1] (routed)
    const int32_t *perm;       // [T*K] sorted row -> pair index (routed)
    const float *wts;          // [T*K] route weights by pair index (routed)
    // A operand
    const uint4 *xh, *xl;      // gate/up: x as bf16 hi/lo [T][H]
    const float *a32;          // down: h rows (fp32) [rows][Kd]
    // B operand: matrices [N][Kd]; routed expert e at base + e * stride
    const uint8_t *b0, *b1;    // gate/up: gate, up; down: down (b1 unused)
    size_t bstride;
    int N, Kd;
    float *out;                // gate/up: h [rows][N]; down: [rows][N]
};

// Rows of this workgroup: (first row index, row count), the row -> source
// row map (token for gate/up A rows, sorted row for h) and route weights.
struct TileRows {
    int e, r0, nrows;
};

__device__ inline bool tile_rows(const GemmArgs &p, TileRows &tr)
{
    __shared__ int sh[3];
    const int tix = blockIdx.y;
    if (threadIdx.x == 0) {
        if (p.routed) {
            int lo = 0, hi = p.E;   // largest e with tile_off[e] <= tix
            if (tix >= p.tile_off[p.E]) {
                sh[0] = -1;
            } else {
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (p.tile_off[mid] <= tix)
                        lo = mid;
                    else
                        hi = mid;
                }
                const int mt = tix - p.tile_off[lo];
                const int r0 = p.offsets[lo] + mt * kBM;
                sh[0] = lo;
                sh[1] = r0;
                sh[2] = min(kBM, p.offsets[lo + 1] - r0);
            }
        } else {
            const int r0 = tix * kBM;
            sh[0] = r0 < p.T ? 0 : -1;
            sh[1] = r0;
            sh[2] = min(kBM, p.T - r0);
        }
    }
    __syncthreads();
    tr.e = sh[0];
    tr.r0 = sh[1];
    tr.nrows = sh[2];
    return tr.e >= 0 && tr.nrows > 0;
}

// acc[rt][ct] += A(rows wr*32 + rt*16 ..) x B(cols bcol[ct] ..) over one
// 32-deep step, with hi/lo passes (B lo skipped for exact bf16 weights).
template <bool BLO>
__device__ __forceinline__ void mfma_step(const uint16_t *Ah, const uint16_t *Al, const uint16_t *Bh,
                                          const uint16_t *Bl, int arow0, const int (&bcol)[4], int lane,
                                          f32x4 (&acc)[2][4])
{
    const int li = lane & 15, kq = lane >> 4;
    bf16x8 ah[2], al[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = arow0 + rt * 16 + li;
        ah[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Ah + r * kLDK + kq * 8));
        al[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Al + r * kLDK + kq * 8));
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int c = bcol[ct] + li;
        const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Bh + c * kLDK + kq * 8));
        bf16x8 bl;
        if (BLO)
            bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Bl + c * kLDK + kq * 8));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[rt], bh, acc[rt][ct], 0, 0, 0);
            if (BLO)
                acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[rt], bl, acc[rt][ct], 0, 0, 0);
            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[rt], bh, acc[rt][ct], 0, 0, 0);
        }
    }
}

template <typename W>
struct HasLo {
    static constexpr bool value = true;
};
template <>
struct HasLo<BF16> {
    static constexpr bool value = false;
};

// Gate/up: tile of 64 rows x 64 channels (both gate and up), 4 waves in 2x2,
// each wave 32 rows x 32 channels of gate and of up. h = silu(g) * u * w.
template <typename W>
__global__ void __launch_bounds__(256) k_gemm_gateup(GemmArgs p)
{
    __shared__ __align__(16) uint16_t Ah[kBM * kLDK], Al[kBM * kLDK];
    __shared__ __align__(16) uint16_t Bh[128 * kLDK], Bl[128 * kLDK];
    __shared__ int tok[kBM];
    __shared__ float rw[kBM];
    TileRows tr;
    if (!tile_rows(p, tr))
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 64;
    if (tid < kBM) {
        int t = -1;
        float w = 0.0f;
        if (tid < tr.nrows) {
            if (p.routed) {
                const int pi = p.perm[tr.r0 + tid];
                t = pi / p.K;
                w = p.wts[pi];
            } else {
                t = tr.r0 + tid;
                w = 1.0f;
            }
        }
        tok[tid] = t;
        rw[tid] = w;
    }
    __syncthreads();
    const uint8_t *G = p.b0 + (p.routed ? tr.e * p.bstride : 0);
    const uint8_t *U = p.b1 + (p.routed ? tr.e * p.bstride : 0);
    const int wr = wave >> 1, wc = wave & 1;
    const int bcol[4] = {wc * 32, wc * 32 + 16, 64 + wc * 32, 64 + wc * 32 + 16};
    f32x4 acc[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int lr = tid >> 2, lp = tid & 3;
    const int Hd = p.Kd;
    for (int k0 = 0; k0 < Hd; k0 += 32) {
        // A: 64 gathered x rows, 32 columns, hi and lo
        {
            const int t = tok[lr];
            uint4 h = make_uint4(0, 0, 0, 0), l = h;
            if (t >= 0) {
                const size_t idx = (static_cast<size_t>(t) * Hd + k0 + lp * 8) / 8;
                h = p.xh[idx];
                l = p.xl[idx];
            }
            *reinterpret_cast<uint4 *>(Ah + lr * kLDK + lp * 8) = h;
            *reinterpret_cast<uint4 *>(Al + lr * kLDK + lp * 8) = l;
        }
        // B: 64 gate rows then 64 up rows, 32 columns
        {
            uint4 h, l;
            b_piece(W{}, G, p.N, Hd, n0 + lr, k0 + lp * 8, h, l);
            *reinterpret_cast<uint4 *>(Bh + lr * kLDK + lp * 8) = h;
            *reinterpret_cast<uint4 *>(Bl + lr * kLDK + lp * 8) = l;
            b_piece(W{}, U, p.N, Hd, n0 + lr, k0 + lp * 8, h, l);
            *reinterpret_cast<uint4 *>(Bh + (64 + lr) * kLDK + lp * 8) = h;
            *reinterpret_cast<uint4 *>(Bl + (64 + lr) * kLDK + lp * 8) = l;
        }
        __syncthreads();
        mfma_step<HasLo<W>::value>(Ah, Al, Bh, Bl, wr * 32, bcol, lane, acc);
        __syncthreads();
    }
    // epilogue: lane holds rows 4*(lane/16)+i of each 16x16 tile, column lane%16
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int ch = n0 + wc * 32 + ct * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wr * 32 + rt * 16 + 4 * (lane >> 4) + i;
                if (r < tr.nrows && ch < p.N) {
                    const float h = silu_mul(acc[rt][ct][i], acc[rt][ct + 2][i]) * rw[r];
                    p.out[static_cast<size_t>(tr.r0 + r) * p.N + ch] = h;
                }
            }
        }
    }
}

// Down: tile of 64 rows x 128 output columns; 4 waves in 2x2, each wave 32
// rows x 64 columns. A = h rows (fp32, split to hi/lo as they are staged).
template <typename W>
__global__ void __launch_bounds__(256) k_gemm_down(GemmArgs p)
{
    __shared__ __align__(16) uint16_t Ah[kBM * kLDK], Al[kBM * kLDK];
    __shared__ __align__(16) uint16_t Bh[128 * kLDK], Bl[128 * kLDK];
    TileRows tr;
    if (!tile_rows(p, tr))
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 128;
    const uint8_t *D = p.b0 + (p.routed ? tr.e * p.bstride : 0);
    const int wr = wave >> 1, wc = wave & 1;
    const int bcol[4] = {wc * 64, wc * 64 + 16, wc * 64 + 32, wc * 64 + 48};
    f32x4 acc[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int lr = tid >> 2, lp = tid & 3;
    const int Kd = p.Kd;
    for (int k0 = 0; k0 < Kd; k0 += 32) {
        {
            uint4 h = make_uint4(0, 0, 0, 0), l = h;
            if (lr < tr.nrows) {
                const float *src = p.a32 + static_cast<size_t>(tr.r0 + lr) * Kd + k0 + lp * 8;
                const float4 a = *reinterpret_cast<const float4 *>(src);
                const float4 b = *reinterpret_cast<const float4 *>(src + 4);
                const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                split8(v, h, l);
            }
            *reinterpret_cast<uint4 *>(Ah + lr * kLDK + lp * 8) = h;
            *reinterpret_cast<uint4 *>(Al + lr * kLDK + lp * 8) = l;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint4 h, l;
            b_piece(W{}, D, p.N, Kd, n0 + half * 64 + lr, k0 + lp * 8, h, l);
            *reinterpret_cast<uint4 *>(Bh + (half * 64 + lr) * kLDK + lp * 8) = h;
            *reinterpret_cast<uint4 *>(Bl + (half * 64 + lr) * kLDK + lp * 8) = l;
        }
        __syncthreads();
        mfma_step<HasLo<W>::value>(Ah, Al, Bh, Bl, wr * 32, bcol, lane, acc);
        __syncthreads();
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int col = n0 + bcol[ct] + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wr * 32 + rt * 16 + 4 * (lane >> 4) + i;
                if (r < tr.nrows && col < p.N)
                    p.out[static_cast<size_t>(tr.r0 + r) * p.N + col] = acc[rt][ct][i];
            }
        }
    }
}

// y[t] = sum_k out[inv[t*K + k]] + g_t * shared[t]   (float4 per thread)
__global__ void __launch_bounds__(256) k_combine(const float *routed_out, const float *shared_out,
                                                 const int32_t *inv, const float *gate, int T, int K, int H, float *y)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int h4 = H / 4;
    if (i >= static_cast<int64_t>(T) * h4)
        return;
    const int t = static_cast<int>(i / h4), c = static_cast<int>(i % h4);
    float4 s = reinterpret_cast<const float4 *>(shared_out + static_cast<size_t>(t) * H)[c];
    const float g = gate[t];
    float4 acc = make_float4(g * s.x, g * s.y, g * s.z, g * s.w);
    for (int k = 0; k < K; ++k) {
        const int r = inv[t * K + k];
        const float4 v = reinterpret_cast<const float4 *>(routed_out + static_cast<size_t>(r) * H)[c];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    reinterpret_cast<float4 *>(y + static_cast<size_t>(t) * H)[c] = acc;
}

// ============================================================ workspace

struct PrefillWs {
    uint8_t *sort_ws;
    size_t sort_bytes;
    uint4 *xh, *xl;
    double *logits, *z;
    int32_t *ids;
    float *wts, *gate;
    int32_t *counts, *offsets, *perm, *inv, *tile_off;
    float *hbuf, *hsh, *rout, *sout;
};

static PrefillWs prefill_carve(void *ws, const moe_layer_desc *d, int T, bool carve)
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
    w.logits = reinterpret_cast<double *>(take(sizeof(double) * T * E));
    w.z = reinterpret_cast<double *>(take(sizeof(double) * T));
    w.ids = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * P));
    w.wts = reinterpret_cast<float *>(take(sizeof(float) * P));
    w.gate = reinterpret_cast<float *>(take(sizeof(float) * T));
    w.counts = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * E));
    w.offsets = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (E + 1)));
    w.perm = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * P));
    w.inv = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * P));
    w.tile_off = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (E + 1)));
    w.hbuf = reinterpret_cast<float *>(take(sizeof(float) * P * I));
    w.hsh = reinterpret_cast<float *>(take(sizeof(float) * T * Is));
    w.rout = reinterpret_cast<float *>(take(sizeof(float) * P * H));
    w.sout = reinterpret_cast<float *>(take(sizeof(float) * T * H));
    w.sort_bytes = off;   // total, when not carving
    return w;
}

size_t prefill_ws_bytes(const moe_layer_desc *d, int T)
{
    return prefill_carve(nullptr, d, T, false).sort_bytes;
}

template <typename ET, typename ST>
static int run_gemms(const moe_layer_desc *d, int T, const PrefillWs &w, hipStream_t s)
{
    const int H = d->hidden, E = d->n_experts, K = d->top_k, I = d->inter, Is = d->shared_inter;
    const int64_t P = static_cast<int64_t>(T) * K;
    const int max_tiles = static_cast<int>((P + kBM - 1) / kBM + E);
    GemmArgs g{};
    g.T = T;
    g.K = K;
    g.E = E;
    g.tile_off = w.tile_off;
    g.offsets = w.offsets;
    g.perm = w.perm;
    g.wts = w.wts;
    g.xh = w.xh;
    g.xl = w.xl;
    // routed gate/up
    g.routed = 1;
    g.b0 = static_cast<const uint8_t *>(d->exp_gate);
    g.b1 = static_cast<const uint8_t *>(d->exp_up);
    g.bstride = mat_bytes<ET>(I, H);
    g.N = I;
    g.Kd = H;
    g.out = w.hbuf;
    hipLaunchKernelGGL((k_gemm_gateup<ET>), dim3((I + 63) / 64, max_tiles), dim3(256), 0, s, g);
    // shared gate/up
    GemmArgs sg = g;
    sg.routed = 0;
    sg.b0 = static_cast<const uint8_t *>(d->sh_gate);
    sg.b1 = static_cast<const uint8_t *>(d->sh_up);
    sg.bstride = 0;
    sg.N = Is;
    sg.out = w.hsh;
    hipLaunchKernelGGL((k_gemm_gateup<ST>), dim3((Is + 63) / 64, (T + kBM - 1) / kBM), dim3(256), 0, s, sg);
    // routed down
    GemmArgs dg = g;
    dg.b0 = static_cast<const uint8_t *>(d->exp_down);
    dg.b1 = nullptr;
    dg.bstride = mat_bytes<ET>(H, I);
    dg.N = H;
    dg.Kd = I;
    dg.a32 = w.hbuf;
    dg.out = w.rout;
    hipLaunchKernelGGL((k_gemm_down<ET>), dim3((H + 127) / 128, max_tiles), dim3(256), 0, s, dg);
    // shared down
    GemmArgs sd = dg;
    sd.routed = 0;
    sd.b0 = static_cast<const uint8_t *>(d->sh_down);
    sd.bstride = 0;
    sd.Kd = Is;
    sd.a32 = w.hsh;
    sd.out = w.sout;
    hipLaunchKernelGGL((k_gemm_down<ST>), dim3((H + 127) / 128, (T + kBM - 1) / kBM), dim3(256), 0, s, sd);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Router logits and the exact per-row routing (ids / weights / gate in the
// workspace, and in the caller's outputs when given).
static int prefill_route(const moe_layer_desc *d, const float *x, int T, const PrefillWs &w, int32_t *ids_out,
                         float *wts_out, float *gate_out, hipStream_t s)
{
    const int H = d->hidden, E = d->n_experts, K = d->top_k;
    const dim3 lg((E + 1 + kLgTile - 1) / kLgTile, (T + kLgTile - 1) / kLgTile);
    if (d->router_t == MOE_F32)
        hipLaunchKernelGGL((k_logits64<F32>), lg, dim3(256), 0, s, x, T, H, E,
                           static_cast<const uint8_t *>(d->router_w), static_cast<const uint8_t *>(d->shared_gate_w),
                           d->router_bias, w.logits, w.z);
    else
        hipLaunchKernelGGL((k_logits64<BF16>), lg, dim3(256), 0, s, x, T, H, E,
                           static_cast<const uint8_t *>(d->router_w), static_cast<const uint8_t *>(d->shared_gate_w),
                           d->router_bias, w.logits, w.z);
    hipLaunchKernelGGL(k_select_rows, dim3((T + 3) / 4), dim3(256), 0, s, w.logits, w.z, T, E, K, d->renormalize,
                       w.ids, w.wts, w.gate, ids_out, wts_out, gate_out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_prefill_route(const moe_layer_desc *d, const float *x, int T, int32_t *ids, float *wts, float *gate,
                         void *ws, hipStream_t s)
{
    const PrefillWs w = prefill_carve(ws, d, T, true);
    return prefill_route(d, x, T, w, ids, wts, gate, s);
}

int launch_prefill_forward(const moe_layer_desc *d, const float *x, int T, float *y, const int32_t *ids_in,
                           const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out,
                           float *gate_out, void *ws, hipStream_t s)
{
    const int H = d->hidden, E = d->n_experts, K = d->top_k;
    const int64_t P = static_cast<int64_t>(T) * K;
    const PrefillWs w = prefill_carve(ws, d, T, true);
    const int64_t n8 = static_cast<int64_t>(T) * H / 8;
    hipLaunchKernelGGL(k_split_x, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, s, x, n8, w.xh, w.xl);
    int rc;
    if (ids_in) {
        hipLaunchKernelGGL(k_take_routing, dim3(static_cast<unsigned>((P + 255) / 256)), dim3(256), 0, s, ids_in,
                           wts_in, gate_in, static_cast<int>(P), T, E, w.ids, w.wts, w.gate);
        rc = hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
    } else {
        rc = prefill_route(d, x, T, w, ids_out, wts_out, gate_out, s);
    }
    if (rc != MOE_OK)
        return rc;
    rc = launch_sort_by_expert(w.ids, T, K, E, w.counts, w.offsets, w.perm, w.sort_ws, s, w.inv);
    if (rc != MOE_OK)
        return rc;
    hipLaunchKernelGGL(k_tiles, dim3(1), dim3(1024), 0, s, w.counts, E, w.tile_off);
    const int et = d->expert_t, st = d->shared_t;
    if (st == MOE_F32) {
        rc = et == MOE_F32 ? run_gemms<F32, F32>(d, T, w, s)
                           : (et == MOE_BF16 ? run_gemms<BF16, F32>(d, T, w, s) : run_gemms<Q2, F32>(d, T, w, s));
    } else {
        rc = et == MOE_F32 ? run_gemms<F32, BF16>(d, T, w, s)
                           : (et == MOE_BF16 ? run_gemms<BF16, BF16>(d, T, w, s) : run_gemms<Q2, BF16>(d, T, w, s));
    }
    if (rc != MOE_OK)
        return rc;
    const int64_t n4 = static_cast<int64_t>(T) * H / 4;
    hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s, w.rout, w.sout,
                       w.inv, w.gate, T, K, H, y);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
