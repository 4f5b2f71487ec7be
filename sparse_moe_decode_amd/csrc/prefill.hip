// Prefill path (many rows per call): rows grouped by expert, grouped bf16 MFMA
// GEMMs on gfx950 (the batched-prefill chunk of the Red Lite "guide" page,
// section "Chat defaults", processes 2048 prompt tokens per pass).
//
//   k_split_x         x (fp32) -> x_hi + x_lo (bf16 pair; x - hi - lo is
//                     below 2^-17 |x|), and the router row norms
//   k_ggemm (router)  approximate router logits [T][E] (bf16 MFMA, bounded
//                     error)
//   k_select_approx   per row: the experts the bound cannot rule out, their
//                     logits exactly in fp64, exact top-K, softmax weights,
//                     sigmoid gate
//   sort (sort.hip)   stable counting sort of the T*K (row, slot) pairs by
//                     expert, with the inverse permutation and the per-expert
//                     row tiles (32 or 64 rows) with each tile's expert
//   k_ggemm (dual)    per (expert row tile, 128-channel block): gathered x
//                     rows times the gate and up rows of the expert, SwiGLU,
//                     times the route weight -> h (bf16 hi/lo, sorted rows)
//   k_ggemm           per (expert row tile, 256-column block): h times the
//                     expert's down rows -> one output row per (row, slot)
//   k_rmsnorm         (layers with a pre-MoE norm) u = RMS norm of x, the
//                     input of everything above
//   k_combine         y[t] = sum_k out[(t, k)] + g_t * shared(t) (+ x[t] with
//                     the residual)
// The shared expert uses the same GEMM kernels over all rows. Everything runs
// on the caller's stream, in order.
//
// MFMA precision: activations enter as bf16 hi+lo pairs; 2-bit weights as
// the exact bf16 values 1 + c/4 of their codes with 4 x the block scale
// applied to each 32-deep partial sum, and (minimum - 4 scale) times the
// block sums of the activations as one more MFMA for every 4 blocks; bf16
// weights exactly; fp32 weights as hi+lo pairs.
// v_mfma_f32_16x16x32_bf16 accumulates in fp32; the dropped lo*lo terms are
// below 2^-16 of each product.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "device_common.hpp"
#include "internal.h"
#include "routing.hpp"
#include "workspace.hpp"

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

template <typename RT>
__device__ void router_norm(const uint8_t *router_w, int E, int H, float *wn, int e, int lane);

// Blocks [0, nbx): x split; blocks from nbx on (when wn is given): norms of
// the router rows, one wave per row (router_norm).
template <typename RT>
__global__ void __launch_bounds__(256) k_split_x(const float *x, int64_t n8, uint4 *xh, uint4 *xl, float *xsum,
                                                 int nbn, const uint8_t *router_w, int E, int H, float *wn)
{
    // the norm blocks come first, so that their longer dependent loads
    // overlap the element-wise blocks instead of trailing them
    if (static_cast<int>(blockIdx.x) < nbn) {
        router_norm<RT>(router_w, E, H, wn, blockIdx.x * 4 + threadIdx.x / kWave, threadIdx.x & (kWave - 1));
        return;
    }
    const int64_t i = static_cast<int64_t>(blockIdx.x - nbn) * blockDim.x + threadIdx.x;
    if (i >= n8)   // n8 is a multiple of 4: a lane quad is all in or all out
        return;
    const float4 a = reinterpret_cast<const float4 *>(x)[2 * i];
    const float4 b = reinterpret_cast<const float4 *>(x)[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint4 hi, lo;
    split8(v, hi, lo);
    xh[i] = hi;
    xl[i] = lo;
    // sums of the 32-element blocks (4 lanes of a quad), for 2-bit weights
    float s = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));
    if ((i & 3) == 0)
        xsum[i >> 2] = s;
}

// ============================================================ selection

// Routing of many rows from approximate logits. L' = x W^T comes from the
// dense bf16 GEMM below (x as hi + lo bf16, each product exact, fp32 sums);
// for every row t and expert e
//   |L'_te - sum_k x_tk w_ek| <= c_H ||x_t|| ||w_e||,
//   c_H = 1.01 (3 * 2^-16 + (3H + 64) * 2^-23),
// which covers the dropped low parts (of x, and of fp32 weights), any order
// of at most 3H + 64 fp32 additions with an error of up to one ulp each, and
// sum |x w| <= ||x|| ||w|| (Cauchy-Schwarz). With lower and upper bounds
// lo_e <= logit_e <= hi_e, the K-th largest lower bound is at or below the
// K-th largest logit, so an expert of the exact top K has hi_e at or above
// any value at or below it: those are the candidates. Their logits are then
// computed exactly in fp64 in the order of the decode path (router_chunk,
// wave_sum, + bias) and ranked exactly. More than 64 candidates, or weights
// over all E logits, take every logit exactly.

// ||w_e||, rounded up, of router row e by one wave.
template <typename RT>
__device__ void router_norm(const uint8_t *router_w, int E, int H, float *wn, int e, int lane)
{
    if (e >= E)
        return;
    const size_t rb = static_cast<size_t>(H) * (RT::kChunk == 4 ? 4 : 2);
    const uint8_t *row = router_w + e * rb;
    const int nch = static_cast<int>(rb / 16);
    double ss = 0.0;
    for (int c = lane; c < nch; c += kWave) {
        const uint4 u = *reinterpret_cast<const uint4 *>(row + static_cast<size_t>(c) * 16);
        if (RT::kChunk == 4) {
            const float w[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ss = fma(static_cast<double>(w[i]), static_cast<double>(w[i]), ss);
        } else {
            const float w[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                                bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ss = fma(static_cast<double>(w[i]), static_cast<double>(w[i]), ss);
        }
    }
    ss = wave_sum(ss);
    if (lane == 0)
        wn[e] = static_cast<float>(sqrt(ss) * (1.0 + 1e-6));
}

// Exact fp64 dot product of a router row (or the gate vector) with the x row
// in LDS, by the whole wave, in the quartered order of the decode path
// (router_chunk per quarter, wave_sum, combine_quarters).
template <typename RT>
__device__ __forceinline__ double exact_dot(const uint8_t *row, int nch, const float *xs, int H, int lane)
{
    double acc[4][1] = {{0.0}, {0.0}, {0.0}, {0.0}};
    for (int c0 = lane; c0 < nch; c0 += 4 * kWave) {
        uint4 u4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * kWave;
            u4[u] = *reinterpret_cast<const uint4 *>(row + static_cast<size_t>(c < nch ? c : 0) * 16);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * kWave;   // quarter u
            if (c < nch)
                router_chunk<1>(RT{}, u4[u], c, xs, H, acc[u]);
        }
    }
    return combine_quarters(wave_sum(acc[0][0]), wave_sum(acc[1][0]), wave_sum(acc[2][0]), wave_sum(acc[3][0]));
}

// Exact logits of experts cand[j] (cand null: expert j), j = j0, j0 + step,
// ... < n, by one wave, two at a time so that the second row's loads overlap
// the first one's sums; lane 0 stores them in out[j].
template <typename RT>
__device__ __forceinline__ void exact_logits(const int *cand, int j0, int step, int n, const uint8_t *router_w,
                                             size_t rb, int nch, const float *bias, const float *xs, int H, int lane,
                                             double *out)
{
    for (int j = j0; j < n; j += 2 * step) {
        const int ja = j, jb = j + step < n ? j + step : j;
        const int ea = cand ? cand[ja] : ja, eb = cand ? cand[jb] : jb;
        double a0[4][1] = {{0.0}, {0.0}, {0.0}, {0.0}}, a1[4][1] = {{0.0}, {0.0}, {0.0}, {0.0}};
        // four chunks per lane of both rows (one per quarter) requested at once
        for (int c0 = lane; c0 < nch; c0 += 4 * kWave) {
            uint4 ua[4], ub[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * kWave;
                const size_t o = static_cast<size_t>(c < nch ? c : 0) * 16;
                ua[u] = *reinterpret_cast<const uint4 *>(router_w + ea * rb + o);
                ub[u] = *reinterpret_cast<const uint4 *>(router_w + eb * rb + o);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * kWave;
                if (c < nch) {
                    router_chunk<1>(RT{}, ua[u], c, xs, H, a0[u]);
                    router_chunk<1>(RT{}, ub[u], c, xs, H, a1[u]);
                }
            }
        }
        const double va = combine_quarters(wave_sum(a0[0][0]), wave_sum(a0[1][0]), wave_sum(a0[2][0]),
                                           wave_sum(a0[3][0])) + (bias ? static_cast<double>(bias[ea]) : 0.0);
        const double vb = combine_quarters(wave_sum(a1[0][0]), wave_sum(a1[1][0]), wave_sum(a1[2][0]),
                                           wave_sum(a1[3][0])) + (bias ? static_cast<double>(bias[eb]) : 0.0);
        if (lane == 0) {
            out[ja] = va;
            out[jb] = vb;
        }
    }
}

constexpr int kSelWaves = 4;          // waves per row in k_select_approx

// One row per workgroup of kSelWaves waves: the x row in LDS; wave 0 sums
// the approximate logits of the GEMM's ks slices (lap [ks][T][E]), forms the
// bounds and the candidates; all waves compute exact logits (of the
// candidates, or of all E experts); one wave the gate logit; wave 0 ranks
// and writes the routing.
template <typename RT, int PL>
__global__ void __launch_bounds__(kSelWaves * kWave) k_select_approx(
    const float *x, const float *lap, int ks, const float *wn, const uint8_t *router_w, const uint8_t *gate_w,
    const float *bias, const float *wbias, int T, int H, int E, int K, int renorm, double cH, int32_t *ids,
    float *wts, float *gate, int32_t *ids_out, float *wts_out, float *gate_out)
{
    extern __shared__ __align__(16) float xs[];   // [H] x row, then [E] exact logits (all-E path)
    __shared__ RouteLds rl;
    __shared__ double xss[kSelWaves];
    __shared__ double zsh;
    __shared__ int csh;   // candidates, or -1: every logit exactly
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, t = blockIdx.x;
    const size_t rb = static_cast<size_t>(H) * (RT::kChunk == 4 ? 4 : 2);
    const int nch = static_cast<int>(rb / 16);
    double *lg = reinterpret_cast<double *>(xs + ((H + 3) & ~3));
    // wave 0 requests what its bounds need before the x row: the GEMM's K
    // slices (at most kMaxRouterSplits), the norms and the bias, all with
    // clamped indices so that the loads are unconditional and are waited for
    // together
    float lv[PL][kMaxRouterSplits], wv[PL], bv[PL];
    if (wave == 0) {
        const float *bp = bias ? bias : wn;
#pragma unroll
        for (int m = 0; m < PL; ++m) {
            const int e = lane + m * kWave, ec = e < E ? e : 0;
#pragma unroll
            for (int z = 0; z < kMaxRouterSplits; ++z)
                lv[m][z] = lap[(static_cast<size_t>(z < ks ? z : 0) * T + t) * E + ec];
            wv[m] = wn[ec];
            bv[m] = bp[ec];
        }
    }
    // x row to LDS; ||x|| in fp64 (rounded up)
    double ss = 0.0;
    const float4 *xr = reinterpret_cast<const float4 *>(x + static_cast<size_t>(t) * H);
    for (int i = tid; i < H / 4; i += blockDim.x) {
        const float4 v = xr[i];
        reinterpret_cast<float4 *>(xs)[i] = v;
        ss = fma(static_cast<double>(v.x), static_cast<double>(v.x), ss);
        ss = fma(static_cast<double>(v.y), static_cast<double>(v.y), ss);
        ss = fma(static_cast<double>(v.z), static_cast<double>(v.z), ss);
        ss = fma(static_cast<double>(v.w), static_cast<double>(v.w), ss);
    }
    ss = wave_sum(ss);
    if (lane == 0)
        xss[wave] = ss;
    __syncthreads();
    if (wave == 0) {
        double sx = 0.0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w)
            sx += xss[w];
        const double xb = cH * sqrt(sx) * (1.0 + 1e-6);
        // the slices added in slice order (within the bound)
        float lsum[PL];
#pragma unroll
        for (int m = 0; m < PL; ++m) {
            lsum[m] = lv[m][0];
#pragma unroll
            for (int z = 1; z < kMaxRouterSplits; ++z)
                lsum[m] += z < ks ? lv[m][z] : 0.0f;
        }
        // bounds as fp32 keys, lower bounds rounded down and upper bounds up
        uint32_t klo[PL], khi[PL];
        uint32_t mk = 0;
#pragma unroll
        for (int m = 0; m < PL; ++m) {
            const int e = lane + m * kWave;
            klo[m] = khi[m] = 0u;
            if (e < E) {
                const double lp = lsum[m];
                const double b = bias ? static_cast<double>(bv[m]) : 0.0;
                const double v = lp + b;
                const double B = (xb * wv[m] + 1e-15 * (fabs(lp) + fabs(b)) + 1e-30) * (1.0 + 1e-9);
                const double lo = v - B, hi = v + B;
                klo[m] = f32_key(static_cast<float>(lo - fabs(lo) * 1e-6 - 1e-30));
                khi[m] = f32_key(static_cast<float>(hi + fabs(hi) * 1e-6 + 1e-30));
            }
            mk = klo[m] > mk ? klo[m] : mk;
        }
        // threshold at or below the K-th largest lower bound: the K-th
        // largest of the 32 lane-pair maxima
        const uint32_t other =
            static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mk), 0xB1, 0xF, 0xF, false));
        const uint32_t pm = other > mk ? other : mk;
        if ((lane & 1) == 0)
            rl.pmax[0][lane >> 1] = pm;
        __builtin_amdgcn_wave_barrier();
        const uint32_t th = kth_of_32(rl.pmax[0], K, lane);
        // candidates: upper bound at or above the threshold
        int cnt = 0;
#pragma unroll
        for (int m = 0; m < PL; ++m)
            cnt += (khi[m] >= th) & (khi[m] != 0);
        const unsigned long long lt = (1ull << lane) - 1ull;
        int pos = 0, C = 0;
#pragma unroll
        for (int b = 0; (1 << b) <= PL; ++b) {
            const unsigned long long mb = __ballot((cnt >> b) & 1);
            pos += __popcll(mb & lt) << b;
            C += __popcll(mb) << b;
        }
#pragma unroll
        for (int m = 0; m < PL; ++m) {
            const bool c = (khi[m] >= th) & (khi[m] != 0);
            if (c && pos < kWave)
                rl.cand[0][pos] = lane + m * kWave;
            pos += c;
        }
        if (lane == 0)
            csh = (C <= kWave && renorm) ? C : -1;
    }
    __syncthreads();
    const int C = csh;
    if (C >= 0) {
        exact_logits<RT>(rl.cand[0], wave, kSelWaves, C, router_w, rb, nch, bias, xs, H, lane, rl.cand_v[0]);
        if (wave == (C + kSelWaves - 1) % kSelWaves) {   // the wave with the fewest candidates
            const double z = exact_dot<RT>(gate_w, nch, xs, H, lane);
            if (lane == 0)
                zsh = z;
        }
    } else {
        exact_logits<RT>(nullptr, wave, kSelWaves, E, router_w, rb, nch, bias, xs, H, lane, lg);
        if (wave == (E + kSelWaves - 1) % kSelWaves) {
            const double z = exact_dot<RT>(gate_w, nch, xs, H, lane);
            if (lane == 0)
                zsh = z;
        }
    }
    __syncthreads();
    if (wave != 0)
        return;
    if (C >= 0) {
        rank_exact(C, K, 0, rl, lane);
        wave_weights(nullptr, E, K, renorm, zsh, 0, rl, lane, true, wbias);
    } else {
        wave_route(lg, E, K, renorm, zsh, 0, rl, lane, wbias);
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < K) {
        const int e = rl.sel_e[0][lane];
        const float w = rl.sel_w[0][lane];
        ids[t * K + lane] = e;
        wts[t * K + lane] = w;
        if (ids_out)
            ids_out[t * K + lane] = e;
        if (wts_out)
            wts_out[t * K + lane] = w;
    }
    if (lane == 0) {
        gate[t] = rl.g[0];
        if (gate_out)
            gate_out[t] = rl.g[0];
    }
}

// Caller-supplied routing: ids outside [0, E) become -1, which the sort
// skips (no GEMM row) and the combine adds nothing for.
__global__ void __launch_bounds__(256) k_take_routing(const int32_t *ids_in, const float *wts_in, const float *gate_in,
                                                      int n, int T, int E, int32_t *ids, float *wts, float *gate)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const int e = ids_in[i];
        const bool ok = e >= 0 && e < E;
        ids[i] = ok ? e : -1;
        wts[i] = ok ? wts_in[i] : 0.0f;
    }
    if (i < T)
        gate[i] = gate_in[i];
}

// ================================================================= GEMMs
//
// Grouped GEMM  C[r][n] = sum_k A[r][k] B[n][k]  over the rows r of one row
// tile (rows of one expert group, or of the chunk for the shared expert) and
// the B rows n of one column block, K = Kd, on v_mfma_f32_16x16x32_bf16.
//   A: bf16 hi/lo pairs of fp32 values (x - hi - lo below 2^-17 |x|); rows
//      gathered by token (gate/up) or taken in sorted order (down).
//   B: 2-bit blocks, bf16 (exact) or fp32 (as hi/lo pairs).
// 2-bit weights enter as the bf16 values v = 1 + c/4 of their codes (exact):
// each 32-deep step is one block, t = A_hi.v + A_lo.v, then
// acc += 4s * t with the block's scale s (per B row), and the remaining terms
// (m - 4s) * asum (m: the block's minimum, asum: the block sum of the A row)
// as one more MFMA per tile for every 4 blocks: m and -4s as exact bf16
// hi + lo, asum as hi + lo, the six products of 4 blocks in one 32-deep step.
// bf16 weights: two passes (A_hi.w + A_lo.w); fp32 weights: three
// (A_hi.w_hi + A_hi.w_lo + A_lo.w_hi).
// Workgroup: 4 waves, BM rows x kGN B rows. Gate/up (DUAL) puts the gate and
// up rows of the same channels in the same wave (the LDS B rows alternate
// gate / up chunks) and ends with SwiGLU times the route weight, written as
// bf16 hi/lo (the A operand of the down pass) with its 32-channel block sums.

constexpr int kLD = 40;          // LDS row stride in bf16 (32 + 8 padding)

template <int BM>
struct GemmShape {
    static constexpr int WR = 1;                  // waves along rows
    static constexpr int WC = 4 / WR;             // waves along B rows
    static constexpr int TR = BM / WR;            // rows per wave
    static constexpr int TC = kGN / WC;           // B rows per wave
    static constexpr int RT = TR / 16, CT = TC / 16;
};

struct GemmArgs {
    int routed, T, K, E;
    const int4 *tiles;         // [tiles] expert, first sorted row, rows of each row tile (routed)
    const int32_t *offsets;    // [E+1] (routed)
    const int32_t *perm;       // [T*K] sorted row -> pair index (routed)
    const float *wts;          // [T*K] route weights by pair index (routed)
    const uint16_t *ah, *al;   // A rows, bf16 hi/lo [rows][Kd]
    int a_bytes;               // bytes of each of ah, al
    int a_lo_off;              // bytes from ah to al (al follows ah)
    const float *asum;         // block-format B: block sums of the A rows [rows][Kd/32]
    int asum_bytes;            // bytes of asum
    int a_gather;              // A row of a tile row: token of the pair (1) or the row itself (0)
    const uint8_t *b0, *b1;    // B: gate, up (dual) or one matrix; routed expert e at base + e * bstride
    size_t bstride;
    int N, Kd;
    uint16_t *hh, *hl;         // dual: h hi/lo [rows][N]
    float *hsum;               // dual, optional: block sums of h [rows][N/32]
    float *out;                // single: [rows][N]
    float *kpart;              // split K (dense, non-routed; gridDim.z slices): fp32 partial sums,
                               // dual [z][rows][2][N] (gate, up), single [z][rows][N]
};

// 8 fp32 -> bf16 hi and lo = bf16(v - hi), packed as the MFMA operand.
__device__ __forceinline__ void split_frag(const float (&v)[8], bf16x8 &hi, bf16x8 &lo)
{
    uint4 h, l;
    split8(v, h, l);
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// The tile of this workgroup (blockIdx.y): expert, first sorted row, rows;
// the A source row and route weight of each tile row. Every thread calls it.
template <int BM>
__device__ __forceinline__ bool gemm_tile(const GemmArgs &p, int *tile, int *tok, float *rw)
{
    if (threadIdx.x == 0) {
        const int tix = blockIdx.y;
        int e = -1, r0 = 0, nr = 0;
        if (p.routed) {
            const int4 t = p.tiles[tix];   // e = -1 past the last tile
            e = t.x;
            r0 = t.y;
            nr = t.z;
        } else if (tix * BM < p.T) {
            e = 0;
            r0 = tix * BM;
            nr = min(BM, p.T - r0);
        }
        tile[0] = e;
        tile[1] = r0;
        tile[2] = nr;
    }
    __syncthreads();
    const int e = tile[0], r0 = tile[1], nrows = tile[2];
    if (e < 0 || nrows <= 0)
        return false;
    if (threadIdx.x < BM) {
        const int t = threadIdx.x;
        int src = -1;
        float w = 0.0f;
        if (t < nrows) {
            if (p.routed) {
                const int pi = p.perm[r0 + t];
                src = p.a_gather ? pi / p.K : r0 + t;
                w = p.wts[pi];
            } else {
                src = r0 + t;
                w = 1.0f;
            }
        }
        tok[t] = src;
        rw[t] = w;
    }
    __syncthreads();
    return true;
}

// B row (channel or output column) and matrix of LDS B row t. DUAL: chunks
// of kGN / (2 WC) rows alternate gate / up.
template <bool DUAL, int BM>
__device__ __forceinline__ int gemm_brow(const GemmArgs &p, int e, int n0, int t, const uint8_t *&mat)
{
    const size_t eoff = p.routed ? static_cast<size_t>(e) * p.bstride : 0;
    if (DUAL) {
        constexpr int chunk = kGN / (2 * GemmShape<BM>::WC);
        const int blk = t / chunk;
        mat = ((blk & 1) ? p.b1 : p.b0) + eoff;
        return n0 + (blk >> 1) * chunk + t % chunk;
    }
    mat = p.b0 + eoff;
    return n0 + t;
}

// lane holds rows 4*(lane/16)+i of each 16x16 tile, column lane%16
template <bool DUAL, int BM>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &p,
                                              f32x4 (&acc)[GemmShape<BM>::RT][GemmShape<BM>::CT], int n0, int r0,
                                              int nrows, const float *rw, int wr, int wc, int lane)
{
    using S = GemmShape<BM>;
    const int li = lane & 15, kq = lane >> 4;
    if (DUAL) {
        constexpr int chunk = kGN / (2 * S::WC);
        const int nb32 = p.N >> 5;
#pragma unroll
        for (int rt = 0; rt < S::RT; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wr * S::TR + rt * 16 + 4 * kq + i;
                float bs = 0.0f;
#pragma unroll
                for (int ct = 0; ct < S::CT / 2; ++ct) {
                    const int ch = n0 + wc * chunk + ct * 16 + li;
                    const float h = silu_mul(acc[rt][ct][i], acc[rt][ct + S::CT / 2][i]) * (r < nrows ? rw[r] : 0.0f);
                    if (r < nrows && ch < p.N) {
                        const uint32_t hb = bf16_rne_bits(h);
                        const uint32_t lb = bf16_rne_bits(h - __uint_as_float(hb << 16));
                        const size_t o = static_cast<size_t>(r0 + r) * p.N + ch;
                        p.hh[o] = static_cast<uint16_t>(hb);
                        p.hl[o] = static_cast<uint16_t>(lb);
                    }
                    // 32-channel block sums: two tiles of 16 channels, summed over the 16 lanes
                    bs += h;
                    if (ct & 1) {
                        const float tot = dpp_row_sum(bs);
                        const int blk = (n0 + wc * chunk + (ct - 1) * 16) >> 5;
                        if (p.hsum && li == 0 && r < nrows && blk < nb32)
                            p.hsum[static_cast<size_t>(r0 + r) * nb32 + blk] = tot;
                        bs = 0.0f;
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int rt = 0; rt < S::RT; ++rt) {
#pragma unroll
            for (int ct = 0; ct < S::CT; ++ct) {
                const int col = n0 + wc * S::TC + ct * 16 + li;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wr * S::TR + rt * 16 + 4 * kq + i;
                    if (r < nrows && col < p.N)
                        p.out[static_cast<size_t>(r0 + r) * p.N + col] = acc[rt][ct][i];
                }
            }
        }
    }
}

// Next step's B rows in registers. All variants: init() once per workgroup,
// load(step) for the 32-deep step, store() of that step to the LDS B tile.
template <typename W>
struct BStage;
// bf16 weights: four lanes per B row, 16 bytes each, so one wave-wide load
// covers 16 rows x 64 contiguous bytes; thread t holds LDS rows t/4 + 64q
// (q = 0..3), part t%4. Plain loads: the dense weights are reread by every
// row tile, so they stay in L2.
template <>
struct BStage<BF16> {
    const uint8_t *row[4];   // this thread's 16-byte column of its B rows (row 0 for rows past the end)
    uint32_t ok;             // bit q: row q exists
    uint4 v[4];
    template <bool DUAL, int BM>
    __device__ __forceinline__ void init(const GemmArgs &p, int e, int n0, int tid)
    {
        ok = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint8_t *m;
            const int bn = gemm_brow<DUAL, BM>(p, e, n0, (tid >> 2) + 64 * q, m);
            ok |= (bn < p.N ? 1u : 0u) << q;
            row[q] = m + (static_cast<size_t>(bn < p.N ? bn : 0) * p.Kd + (tid & 3) * 8) * 2;
        }
    }
    __device__ __forceinline__ void load(int blk)
    {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 w = *reinterpret_cast<const uint4 *>(row[q] + blk * 64);
            v[q] = ((ok >> q) & 1u) ? w : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(uint16_t *Bh, uint16_t *, int tid) const
    {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint4 *>(Bh + ((tid >> 2) + 64 * q) * kLD + (tid & 3) * 8) = v[q];
    }
};
// fp32 weights (split to bf16 hi/lo when stored): one B row per thread.
template <>
struct BStage<F32> {
    const uint8_t *M;
    int n, rows, cols;
    uint4 v[8];
    template <bool DUAL, int BM>
    __device__ __forceinline__ void init(const GemmArgs &p, int e, int n0, int tid)
    {
        n = gemm_brow<DUAL, BM>(p, e, n0, tid, M);
        rows = p.N;
        cols = p.Kd;
    }
    __device__ __forceinline__ void load(int blk)
    {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = n < rows ? ld_nt16(M + (static_cast<size_t>(n) * cols + blk * 32 + q * 4) * 4) : make_uint4(0, 0, 0, 0);
    }
    __device__ __forceinline__ void store(uint16_t *Bh, uint16_t *Bl, int row) const
    {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float f[8] = {__uint_as_float(v[2 * q].x), __uint_as_float(v[2 * q].y), __uint_as_float(v[2 * q].z),
                                __uint_as_float(v[2 * q].w), __uint_as_float(v[2 * q + 1].x),
                                __uint_as_float(v[2 * q + 1].y), __uint_as_float(v[2 * q + 1].z),
                                __uint_as_float(v[2 * q + 1].w)};
            uint4 h, l;
            split8(f, h, l);
            *reinterpret_cast<uint4 *>(Bh + row * kLD + q * 8) = h;
            *reinterpret_cast<uint4 *>(Bl + row * kLD + q * 8) = l;
        }
    }
};

// bf16 / fp32 weights: one 32-deep step in LDS, the next one's global loads
// in registers while the current one is multiplied.
template <typename W, bool DUAL, int BM>
__global__ void __launch_bounds__(256) k_ggemm(GemmArgs p)
{
    using S = GemmShape<BM>;
    constexpr bool kBLo = W::kChunk == 4;
    __shared__ __align__(16) uint16_t Lah[BM * kLD], Lal[BM * kLD], Lbh[kGN * kLD];
    __shared__ __align__(16) uint16_t Lbl[kBLo ? kGN * kLD : 8];
    __shared__ int Ltok[BM];
    __shared__ float Lrw[BM];
    __shared__ int Ltile[3];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kq = lane >> 4;
    const int wr = wave / S::WC, wc = wave % S::WC;
    if (!gemm_tile<BM>(p, Ltile, Ltok, Lrw))
        return;
    const int e = Ltile[0], r0 = Ltile[1], nrows = Ltile[2];
    const int n0 = blockIdx.x * (DUAL ? kGN / 2 : kGN);
    const bool a_loader = tid < BM * 4;
    const int arow = (tid >> 2) % BM, apart = tid & 3;
    const int asrc = Ltok[arow];

    f32x4 acc[S::RT][S::CT];
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < S::CT; ++ct)
            acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    // reduction slice (split K over gridDim.z)
    const int nsteps_all = p.Kd / 32, ks = gridDim.z;
    const int s_begin = static_cast<int>(blockIdx.z) * nsteps_all / ks;
    const int nsteps = (static_cast<int>(blockIdx.z) + 1) * nsteps_all / ks - s_begin;
    uint4 rah = make_uint4(0, 0, 0, 0), ral = rah;
    BStage<W> rb;
    rb.template init<DUAL, BM>(p, e, n0, tid);
    // unconditional loads (rows without a source read row 0, then zero)
    const bool a_live = a_loader && asrc >= 0;
    const size_t a_base = (static_cast<size_t>(a_live ? asrc : 0) * p.Kd + apart * 8) / 8;
    auto load_step = [&](int s) {
        s += s_begin;
        const uint4 h = reinterpret_cast<const uint4 *>(p.ah)[a_base + s * 4];
        const uint4 l = reinterpret_cast<const uint4 *>(p.al)[a_base + s * 4];
        rah = a_live ? h : make_uint4(0, 0, 0, 0);
        ral = a_live ? l : make_uint4(0, 0, 0, 0);
        rb.load(s);
    };
    load_step(0);
    for (int s = 0; s < nsteps; ++s) {
        if (a_loader) {
            *reinterpret_cast<uint4 *>(Lah + arow * kLD + apart * 8) = rah;
            *reinterpret_cast<uint4 *>(Lal + arow * kLD + apart * 8) = ral;
        }
        rb.store(Lbh, Lbl, tid);
        __syncthreads();
        if (s + 1 < nsteps)
            load_step(s + 1);
        bf16x8 fah[S::RT], fal[S::RT];
#pragma unroll
        for (int rt = 0; rt < S::RT; ++rt) {
            const int r = wr * S::TR + rt * 16 + li;
            fah[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Lah + r * kLD + kq * 8));
            fal[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Lal + r * kLD + kq * 8));
        }
#pragma unroll
        for (int ct = 0; ct < S::CT; ++ct) {
            const int c = wc * S::TC + ct * 16 + li;
            const bf16x8 fb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Lbh + c * kLD + kq * 8));
            bf16x8 fbl;
            if (kBLo)
                fbl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Lbl + c * kLD + kq * 8));
#pragma unroll
            for (int rt = 0; rt < S::RT; ++rt) {
                acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fah[rt], fb, acc[rt][ct], 0, 0, 0);
                acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fal[rt], fb, acc[rt][ct], 0, 0, 0);
                if (kBLo)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fah[rt], fbl, acc[rt][ct], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    if (ks > 1) {
        // partial sums of this slice; k_dual_sum / k_single_sum finish them
        const size_t zr = static_cast<size_t>(blockIdx.z) * p.T;
#pragma unroll
        for (int rt = 0; rt < S::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < S::CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wr * S::TR + rt * 16 + 4 * kq + i;
                    if (r >= nrows)
                        continue;
                    const size_t row = zr + r0 + r;
                    if (DUAL) {
                        constexpr int chunk = kGN / (2 * S::WC);
                        const int half = ct / (S::CT / 2), cc = ct % (S::CT / 2);
                        const int ch = n0 + wc * chunk + cc * 16 + li;
                        if (ch < p.N)
                            p.kpart[(row * 2 + half) * p.N + ch] = acc[rt][ct][i];
                    } else {
                        const int col = n0 + wc * S::TC + ct * 16 + li;
                        if (col < p.N)
                            p.kpart[row * p.N + col] = acc[rt][ct][i];
                    }
                }
        return;
    }
    gemm_epilogue<DUAL, BM>(p, acc, n0, r0, nrows, Lrw, wr, wc, lane);
}

// Split-K finish of the dense dual GEMM (non-routed rows, weight 1): the
// slices' gate and up sums in slice order (loads issued eight slices at a
// time), then the SwiGLU and bf16 hi/lo split of gemm_epilogue.
__global__ void __launch_bounds__(256) k_dual_sum(const float *part, int ks, int T, int N, uint16_t *hh,
                                                  uint16_t *hl)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;   // row * N + ch
    if (i >= static_cast<int64_t>(T) * N)
        return;
    const int64_t t = i / N, ch = i - t * N;
    float g = 0.0f, u = 0.0f;
    for (int z0 = 0; z0 < ks; z0 += 8) {
        float vg[8], vu[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const size_t row = static_cast<size_t>(z0 + k) * T + t;
            const bool ok = z0 + k < ks;
            vg[k] = ok ? part[(row * 2 + 0) * N + ch] : 0.0f;
            vu[k] = ok ? part[(row * 2 + 1) * N + ch] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            g += vg[k];
            u += vu[k];
        }
    }
    const float h = silu_mul(g, u) * 1.0f;
    const uint32_t hb = bf16_rne_bits(h);
    hh[i] = static_cast<uint16_t>(hb);
    hl[i] = static_cast<uint16_t>(bf16_rne_bits(h - __uint_as_float(hb << 16)));
}

// Split-K finish of the dense single GEMM: the slices' sums in slice order.
__global__ void __launch_bounds__(256) k_single_sum(const float *part, int ks, int T, int N, float *out)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n = static_cast<int64_t>(T) * N;
    if (i >= n)
        return;
    float s = 0.0f;
    for (int z0 = 0; z0 < ks; z0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = z0 + k < ks ? part[static_cast<size_t>(z0 + k) * n + i] : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            s += v[k];
    }
    out[i] = s;
}

// Block-format main loop (b-bit codes, b = 2, 3, 4; the weight operand is
// called B below). B arrives in mega-steps of 4 blocks: 4 consecutive lanes
// read one B row's 4 blocks (4 * 4b bytes of codes and 16 of scale/min
// words), so each wave-wide load touches 16 rows of one matrix; the raw
// words are held in registers one mega-step ahead, then the codes go to LDS
// as they are, the scales as fp32, and the minima and scales as the operands
// of the minimum term, with the block sums of the tile's A rows. Each wave
// expands the codes of its own B operands to bf16 in registers (8 codes per
// lane per operand). A: each thread holds BM/32 16-byte pieces (row, part,
// hi or lo) of 4 consecutive blocks; a group of 4 blocks goes to LDS at once
// (one barrier per group) and each block's pieces are reloaded with the
// block 4 steps ahead as soon as they are stored. Loads go through buffer
// descriptors: rows past the end read as zero.
constexpr int kMS = 4;           // blocks per mega-step (a divisor of 64)
constexpr int kAG = 4;           // A blocks per LDS group (and register ring slots)
// Word 3 of a raw buffer descriptor on gfx9 targets (32-bit data format;
// offsets past num_records read as zero).
constexpr int kBufWord3 = 0x00020000;
constexpr int kRawS = kMS + 1;       // LDS row stride (floats) of scales
constexpr int kMinS = 12;            // LDS row stride (dwords) of the minimum-term fragments
static_assert(kMS == 4, "the minimum term packs 4 blocks x 6 products into one 32-deep MFMA");
// LDS row stride (dwords) of the raw codes of b-bit blocks
template <int BITS>
struct RawCodes {
    static constexpr int kStride = BITS * kMS + 1;
};

// 8 codes (16 bits, code i at bits 2i..2i+1) -> the bf16 values 1 + c/4
// (exact): each code becomes the top two mantissa bits of 1.0 (0x3F80), so
// one block's dot product with A is asum + (sum of a*c)/4 and the weight
// s*c + m equals (4s)*v + (m - 4s). y holds code 2j at bit 4j and code 2j+1
// at bit 4j+16; each bf16 pair is then one mask and one shift of y.
// one2 = 0x3F803F80 (a pair of bf16 1.0) in a register the compiler cannot
// see through, so that each (shifted y & mask) | one2 is one bit-field insert
// (one2 has no bits under the mask).
template <int BITS>
__device__ __forceinline__ bf16x8 codes_bf16(uint32_t c, uint32_t one2);
template <>
__device__ __forceinline__ bf16x8 codes_bf16<2>(uint32_t c16, uint32_t one2)
{
    constexpr uint32_t m = 0x00600060u;
    const uint32_t y = c16 | (c16 << 14);
    const uint32_t w0 = ((y << 5) & m) | (one2 & ~m);
    const uint32_t w1 = ((y << 1) & m) | (one2 & ~m);
    const uint32_t w2 = ((y >> 3) & m) | (one2 & ~m);
    const uint32_t w3 = ((y >> 7) & m) | (one2 & ~m);
    return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}
// 3- and 4-bit codes (code i at bits b*i of c): the bf16 values 1 + c/2^b,
// exact for b <= 7, with the code in the top b mantissa bits; the weight
// s*c + m equals (2^b s)*v + (m - 2^b s).
template <int BITS>
__device__ __forceinline__ bf16x8 codes_bf16(uint32_t c, uint32_t one2)
{
    constexpr uint32_t mask = (1u << BITS) - 1u;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (c >> (2 * j * BITS)) & mask, hi = (c >> ((2 * j + 1) * BITS)) & mask;
        w[j] = (lo << (7 - BITS)) | (hi << (23 - BITS)) | one2;
    }
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// The raw words of one (B row, block): BITS dwords of codes.
template <int BITS>
__device__ __forceinline__ void load_raw_codes(__amdgpu_buffer_rsrc_t r, int off, uint32_t (&cw)[BITS])
{
    if constexpr (BITS == 2) {
        const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        cw[0] = v.x;
        cw[1] = v.y;
    } else if constexpr (BITS == 3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
        cw[0] = v[0];
        cw[1] = v[1];
        cw[2] = v[2];
    } else {
        const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        cw[0] = v.x;
        cw[1] = v.y;
        cw[2] = v.z;
        cw[3] = v.w;
    }
}

// The 8 codes (8*BITS bits) of quarter kq of one block's raw words in LDS.
template <int BITS>
__device__ __forceinline__ uint32_t quarter_codes(const uint32_t *raw, int kq)
{
    if constexpr (BITS == 2)
        return (raw[kq >> 1] >> (16 * (kq & 1))) & 0xffffu;
    else if constexpr (BITS == 4)
        return raw[kq];
    else {
        const int bit = 24 * kq, w = bit >> 5;   // the 24 bits may straddle two dwords
        return __builtin_amdgcn_alignbit(raw[w + 1], raw[w], bit & 31) & 0xffffffu;
    }
}

// Workgroups per CU: three for 32-row tiles of 2-bit blocks (48 KiB of LDS
// each); two for the wider raw codes of 3- and 4-bit blocks and for 64-row
// tiles (their A staging and accumulators).
template <int BITS, bool DUAL, int BM>
__global__ void __launch_bounds__(256, BM == 32 && BITS == 2 ? 3 : 2) k_ggemm_qb(GemmArgs p)
{
    constexpr int kRawC = RawCodes<BITS>::kStride;
    constexpr float kLevels = static_cast<float>(1 << BITS);   // 2^b
    using S = GemmShape<BM>;
    constexpr int AP = BM / 32;            // A pieces per thread per block
    constexpr int BL = kGN * kMS / 256;    // (row, block) words per thread per mega-step
    constexpr int ASN = (BM * kMS + 255) / 256;   // (A row, block) sums per thread per mega-step (at most)
    constexpr int RPI = 64 / kMS;          // B rows per wave-wide load
    __shared__ __align__(16) uint16_t La[kAG][2][BM * kLD];
    __shared__ __align__(16) uint32_t Lrc[kGN * kRawC];
    __shared__ float Lsc[kGN * kRawS];
    // minimum-term operands of the mega-step, three MFMA fragments per B row
    // and per A row (see the staging below), and a zero fragment
    __shared__ __align__(16) uint32_t Lmb[kGN * kMinS];
    __shared__ __align__(16) uint32_t Lma[BM * kMinS];
    __shared__ __align__(16) uint32_t Lz[4];
    __shared__ int Ltok[BM];
    __shared__ float Lrw[BM];
    __shared__ int Ltile[3];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kq = lane >> 4;
    const int wr = wave / S::WC, wc = wave % S::WC;
    if (!gemm_tile<BM>(p, Ltile, Ltok, Lrw))
        return;
    const int e = Ltile[0], r0 = Ltile[1], nrows = Ltile[2];
    const int n0 = blockIdx.x * (DUAL ? kGN / 2 : kGN);
    const int NB = p.Kd / 32;
    const size_t plane = static_cast<size_t>(p.N) * (p.Kd / 32) * 4 * BITS;   // bytes of the codes plane

    // B raw words: wave w loads 64 consecutive B rows of one matrix (DUAL:
    // waves 0-1 gate, 2-3 up), RPI rows per instruction
    const int bl = tid % kMS;
    const size_t eoff = p.routed ? static_cast<size_t>(e) * p.bstride : 0;
    const int rowb = (p.Kd / 32) * 4 * BITS;   // bytes of codes per B row
    const int msel = DUAL ? __builtin_amdgcn_readfirstlane(tid >> 7) : 0;   // wave-uniform
    const uint8_t *mbase = (msel ? p.b1 : p.b0) + eoff;
    const __amdgpu_buffer_rsrc_t rcode =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(mbase), 0, static_cast<int>(plane), kBufWord3);
    const __amdgpu_buffer_rsrc_t rsmw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(mbase + plane), 0, p.N * NB * 4, kBufWord3);
    const int chl0 = (DUAL ? ((tid >> 6) & 1) : (tid >> 6)) * 64 + (tid & 63) / kMS;   // local channel of row j: + RPI j
    const int ch0 = n0 + chl0;
    // two register sets (even and odd mega-steps), both loaded at once, so
    // that each B row's words of 8 consecutive blocks (64 or 128 bytes of
    // codes) are requested together; 4-bit codes in 64-row tiles (no
    // registers to spare) and 3-bit codes (measured: the second set fetches
    // less but runs slower, 984 against 914 us per 2048-row chunk): one set,
    // reloaded after each mega-step
    constexpr int NSET = BITS == 2 || (BITS == 4 && BM == 32) ? 2 : 1;
    uint32_t rc[NSET][BL][BITS];
    uint32_t rs[NSET][BL];
    // block sums of A: value j of this thread is (row q / kMS, block q % kMS)
    // of the mega-step, q = tid + 256 j, loaded through a buffer descriptor
    // (padding rows read past its range: zeros)
    const __amdgpu_buffer_rsrc_t rsum =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.asum), 0, p.asum_bytes, kBufWord3);
    float ras[NSET][ASN];
    int asoff[ASN];
#pragma unroll
    for (int j = 0; j < ASN; ++j) {
        const int q = tid + 256 * j;
        const int src = q < BM * kMS ? Ltok[q / kMS] : -1;
        asoff[j] = src >= 0 ? (src * NB + q % kMS) * 4 : 0x7fff0000;
    }
    // the words of mega-step M into register set `set`
    auto load_b = [&](int M, auto set) {
        constexpr int R = decltype(set)::value;
        const int blk = M * kMS + bl;
        const int bb = blk < NB ? blk : 0;
#pragma unroll
        for (int j = 0; j < BL; ++j) {
            const int n = ch0 + RPI * j;
            load_raw_codes<BITS>(rcode, n * rowb + bb * 4 * BITS, rc[R][j]);
            rs[R][j] = __builtin_amdgcn_raw_buffer_load_b32(rsmw, (n * NB + bb) * 4, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < ASN; ++j) {
            const float v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsum, asoff[j] + M * kMS * 4, 0, 0));
            ras[R][j] = M * kMS + (tid + 256 * j) % kMS < NB ? v : 0.0f;
        }
    };
    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, NSET - 1>;
    // LDS B row of local channel c of matrix msel (DUAL: chunks alternate gate / up)
    auto lds_row = [&](int c) {
        if (!DUAL)
            return c;
        constexpr int chunk = kGN / (2 * S::WC);
        return (c / chunk) * 2 * chunk + msel * chunk + c % chunk;
    };

    // A pieces of this thread: piece q -> row q/8, part (q/2)%4, hi (even q)
    // or lo; one descriptor over hi and lo (lo starts a_lo_off bytes after hi),
    // padding rows read past its range (zeros)
    const __amdgpu_buffer_rsrc_t ra_rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.ah), 0, p.a_lo_off + p.a_bytes, kBufWord3);
    int arow[AP], apart[AP], ahl[AP], aoff[AP];
#pragma unroll
    for (int j = 0; j < AP; ++j) {
        const int q = tid + 256 * j;
        arow[j] = q >> 3;
        apart[j] = (q >> 1) & 3;
        ahl[j] = q & 1;
        const int src = Ltok[arow[j]];
        aoff[j] = src >= 0 ? (ahl[j] ? p.a_lo_off : 0) + (src * p.Kd + apart[j] * 8) * 2 : 0x7fff0000;
    }
    uint4 ra[kAG][AP];
    auto load_a = [&](int slot, int blk) {
        const int bb = blk < NB ? blk : 0;
#pragma unroll
        for (int j = 0; j < AP; ++j)
            ra[slot][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra_rs, aoff[j] + bb * 64, 0, 0));
    };

    f32x4 acc[S::RT][S::CT];
#pragma unroll
    for (int rt = 0; rt < S::RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < S::CT; ++ct)
            acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (tid < 4)
        Lz[tid] = 0u;   // ordered before its first read by the first group's barrier
    uint32_t one2 = 0x3F803F80u;   // see codes_bf16
    asm volatile("" : "+v"(one2));
    const int nms = (NB + kMS - 1) / kMS;
    load_b(0, Set0{});
    if (NSET == 2 && nms > 1)
        load_b(1, Set1{});
#pragma unroll
    for (int u = 0; u < kAG; ++u)
        load_a(u, u);
    // The main loop for NA 16-row MFMA tiles that hold rows of the tile (the
    // others hold padding only and are skipped), one instance per count, so
    // that no branch separates an MFMA from the instructions that read its
    // result.
    auto main_loop = [&](auto na) {
        constexpr int NA = decltype(na)::value;
        // mega-step M from register set R (R = M % NSET)
        auto mstep = [&](int M, auto set) {
            constexpr int R = decltype(set)::value;
            // raw codes and scales of this mega-step to LDS, then the words
            // of the next one (one set) or, after an odd one, of the next two
            {
                const bool in = M * kMS + bl < NB;
#pragma unroll
                for (int j = 0; j < BL; ++j) {
                    const int row = lds_row(chl0 + RPI * j);
#pragma unroll
                    for (int i = 0; i < BITS; ++i)
                        Lrc[row * kRawC + BITS * bl + i] = in ? rc[R][j][i] : 0u;
                    const float s = in ? f16_to_f32(rs[R][j] & 0xffffu) : 0.0f;
                    Lsc[row * kRawS + bl] = kLevels * s;
                    // m and -2^b s as exact bf16 hi + lo: hi keeps the top 8 of
                    // the 11 significant bits of the fp16 value, lo = v - hi (at
                    // most 3 bits, exact); the pairs (m_hi, m_lo), (m_hi, s_hi),
                    // (s_lo, s_hi) of block bl, each packed by one byte permute of
                    // the fp32 bit patterns' upper halves
                    const float mf = in ? f16_to_f32(rs[R][j] >> 16) : 0.0f, sf = -kLevels * s;
                    const uint32_t mh = __float_as_uint(mf) & 0xffff0000u, sh = __float_as_uint(sf) & 0xffff0000u;
                    const uint32_t ml = __float_as_uint(mf - __uint_as_float(mh));
                    const uint32_t sl = __float_as_uint(sf - __uint_as_float(sh));
                    Lmb[row * kMinS + bl] = __builtin_amdgcn_perm(ml, mh, 0x07060302u);
                    Lmb[row * kMinS + 4 + bl] = __builtin_amdgcn_perm(sh, mh, 0x07060302u);
                    Lmb[row * kMinS + 8 + bl] = __builtin_amdgcn_perm(sh, sl, 0x07060302u);
                }
                // the A rows' block sums as bf16 hi + lo (residual below 2^-17):
                // the matching pairs (a_hi, a_hi), (a_lo, a_hi), (a_hi, a_lo), so
                // that fragment f of both sides multiplies to
                // a_hi m_hi + a_hi m_lo | a_lo m_hi + a_hi s_hi | a_hi s_lo + a_lo s_hi
#pragma unroll
                for (int j = 0; j < ASN; ++j) {
                    const int q = tid + 256 * j;
                    if (q < BM * kMS) {
                        const float av = ras[R][j];
                        const uint32_t ah = bf16_rne_bits(av), al = bf16_rne_bits(av - __uint_as_float(ah << 16));
                        uint32_t *ma = &Lma[(q / kMS) * kMinS + q % kMS];
                        ma[0] = ah | (ah << 16);
                        ma[4] = al | (ah << 16);
                        ma[8] = ah | (al << 16);
                    }
                }
            }
            if constexpr (NSET == 1) {
                if (M + 1 < nms)
                    load_b(M + 1, Set0{});
            } else if constexpr (R == 1) {
                if (M + 1 < nms)
                    load_b(M + 1, Set0{});
                if (M + 2 < nms)
                    load_b(M + 2, Set1{});
            }
            // A in groups of kAG blocks (the register ring): the group goes to
            // LDS, its slots are refilled kAG blocks ahead, one barrier, then the
            // group's blocks are computed
#pragma unroll
            for (int g = 0; g < kMS; g += kAG) {
                if (M * kMS + g >= NB)
                    break;
#pragma unroll
                for (int u = 0; u < kAG; ++u) {
#pragma unroll
                    for (int j = 0; j < AP; ++j)
                        *reinterpret_cast<uint4 *>(&La[u][ahl[j]][arow[j] * kLD + apart[j] * 8]) = ra[u][j];
                    load_a(u, M * kMS + g + u + kAG);
                }
                __syncthreads();
#pragma unroll
                for (int u = 0; u < kAG; ++u) {
                    const int b = g + u;
                    if (M * kMS + b >= NB)
                        break;
                    bf16x8 fah[S::RT], fal[S::RT];
#pragma unroll
                    for (int rt = 0; rt < NA; ++rt) {
                        const int r = wr * S::TR + rt * 16 + li;
                        fah[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&La[u][0][r * kLD + kq * 8]));
                        fal[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&La[u][1][r * kLD + kq * 8]));
                    }
#pragma unroll
                    for (int ct = 0; ct < S::CT; ++ct) {
                        const int c = wc * S::TC + ct * 16 + li;
                        const bf16x8 fb = codes_bf16<BITS>(quarter_codes<BITS>(&Lrc[c * kRawC + BITS * b], kq), one2);
                        const float sc = Lsc[c * kRawS + b];
#pragma unroll
                        for (int rt = 0; rt < NA; ++rt) {
                            f32x4 t =
                                __builtin_amdgcn_mfma_f32_16x16x32_bf16(fah[rt], fb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fal[rt], fb, t, 0, 0, 0);
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[rt][ct][i] = fmaf(sc, t[i], acc[rt][ct][i]);
                        }
                    }
                }
                // the minimum terms of the mega-step's blocks: one MFMA per tile
                // (lanes kq = 0..2 hold fragments 0..2, lanes kq = 3 zeros)
                {
                    bf16x8 fma_[S::RT];
#pragma unroll
                    for (int rt = 0; rt < NA; ++rt) {
                        const int r = wr * S::TR + rt * 16 + li;
                        fma_[rt] = __builtin_bit_cast(
                            bf16x8, *reinterpret_cast<const uint4 *>(kq < 3 ? &Lma[r * kMinS + 4 * kq] : Lz));
                    }
#pragma unroll
                    for (int ct = 0; ct < S::CT; ++ct) {
                        const int c = wc * S::TC + ct * 16 + li;
                        const bf16x8 fmb = __builtin_bit_cast(
                            bf16x8, *reinterpret_cast<const uint4 *>(kq < 3 ? &Lmb[c * kMinS + 4 * kq] : Lz));
#pragma unroll
                        for (int rt = 0; rt < NA; ++rt)
                            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fma_[rt], fmb, acc[rt][ct], 0, 0, 0);
                    }
                }
                __syncthreads();
            }
        };
        if constexpr (NSET == 1) {
            for (int M = 0; M < nms; ++M)
                mstep(M, Set0{});
        } else {
            for (int M = 0; M < nms; M += 2) {
                mstep(M, Set0{});
                if (M + 1 < nms)
                    mstep(M + 1, Set1{});
            }
        }
    };
    static_assert(S::RT == 2 || S::RT == 4, "32- or 64-row tiles");
    const int nact = (nrows + 15) >> 4;   // wave-uniform, 1..RT
    if (nact >= S::RT)
        main_loop(std::integral_constant<int, S::RT>{});
    else if (nact == 1)
        main_loop(std::integral_constant<int, 1>{});
    else if constexpr (S::RT == 4) {
        if (nact == 2)
            main_loop(std::integral_constant<int, 2>{});
        else
            main_loop(std::integral_constant<int, 3>{});
    }

    gemm_epilogue<DUAL, BM>(p, acc, n0, r0, nrows, Lrw, wr, wc, lane);
}

// y[t] = sum_k out[inv[t*K + k]] + g_t * shared[t]   (float4 per thread);
// a pair the sort skipped (inv < 0) adds nothing
__global__ void __launch_bounds__(256) k_combine(const float *routed_out, const float *shared_out,
                                                 const int32_t *inv, const float *gate, int T, int K, int H,
                                                 const float *xres, float *y)
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
        if (r < 0)
            continue;
        const float4 v = reinterpret_cast<const float4 *>(routed_out + static_cast<size_t>(r) * H)[c];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if (xres) {
        const float4 xv = reinterpret_cast<const float4 *>(xres + static_cast<size_t>(t) * H)[c];
        acc.x = xv.x + acc.x;
        acc.y = xv.y + acc.y;
        acc.z = xv.z + acc.z;
        acc.w = xv.w + acc.w;
    }
    reinterpret_cast<float4 *>(y + static_cast<size_t>(t) * H)[c] = acc;
}

// The layer's pre-MoE RMS norm, one row per workgroup: u = fp32(x r gamma)
// (rms_norm_rows).
__global__ void __launch_bounds__(256) k_rmsnorm(const float *x, int H, const float *gamma, float eps, float *u)
{
    extern __shared__ __align__(16) float row[];
    const size_t off = static_cast<size_t>(blockIdx.x) * H;
    for (int i = threadIdx.x; i < H / 4; i += blockDim.x)
        reinterpret_cast<float4 *>(row)[i] = reinterpret_cast<const float4 *>(x + off)[i];
    rms_norm_rows<1>(row, H, gamma, eps, SlotsInOrder{});
    for (int i = threadIdx.x; i < H / 4; i += blockDim.x)
        reinterpret_cast<float4 *>(u + off)[i] = reinterpret_cast<const float4 *>(row)[i];
}

// ============================================================ workspace
// (the carve and the reduction-slice counts are in workspace.hpp)

// Rows per routed tile: 32 when the expert groups are small on average (three
// workgroups per CU, less padding), else 64 (each wave's B operands serve
// four 16-row MFMA tiles). The block-format kernels skip 16-row tiles that
// hold no rows. At 40 pairs per expert (2048 rows, top-10 of 512) 32-row
// tiles measured faster (407 against 415 us for the routed gate/up GEMM).
static int routed_bm(int64_t P, int E) { return P < 48 * static_cast<int64_t>(E) ? 32 : 64; }

template <typename W, bool DUAL>
static void launch_ggemm(const GemmArgs &g, int bm, int tiles, hipStream_t s, int ks = 1)
{
    const dim3 grid((g.N + (DUAL ? kGN / 2 : kGN) - 1) / (DUAL ? kGN / 2 : kGN), tiles, ks), block(256);
    if constexpr (is_block_format<W>::value) {
        if (bm == 32)
            hipLaunchKernelGGL((k_ggemm_qb<W::kBits, DUAL, 32>), grid, block, 0, s, g);
        else
            hipLaunchKernelGGL((k_ggemm_qb<W::kBits, DUAL, 64>), grid, block, 0, s, g);
    } else {
        if (bm == 32)
            hipLaunchKernelGGL((k_ggemm<W, DUAL, 32>), grid, block, 0, s, g);
        else
            hipLaunchKernelGGL((k_ggemm<W, DUAL, 64>), grid, block, 0, s, g);
    }
}

// Routed and shared GEMMs on stream s, in order.
template <typename ET, typename ST>
static int run_gemms(const moe_layer_desc *d, int T, const PrefillWs &w, int bm, hipStream_t s)
{
    const int H = d->hidden, E = d->n_experts, K = d->top_k, I = d->inter, Is = d->shared_inter;
    const int64_t P = static_cast<int64_t>(T) * K;
    const int max_tiles = static_cast<int>((P + bm - 1) / bm + E);
    const int sh_tiles = (T + 63) / 64;
    GemmArgs g{};
    g.T = T;
    g.K = K;
    g.E = E;
    g.tiles = w.tiles;
    g.offsets = w.offsets;
    g.perm = w.perm;
    g.wts = w.wts;
    // routed gate/up: A = x rows of the pairs' tokens
    g.routed = 1;
    g.ah = reinterpret_cast<const uint16_t *>(w.xh);
    g.a_bytes = static_cast<int>(sizeof(uint16_t) * T * H);
    g.a_lo_off = static_cast<int>(reinterpret_cast<const uint8_t *>(w.xl) - reinterpret_cast<const uint8_t *>(w.xh));
    g.al = reinterpret_cast<const uint16_t *>(w.xl);
    g.a_gather = 1;
    g.b0 = static_cast<const uint8_t *>(d->exp_gate);
    g.b1 = static_cast<const uint8_t *>(d->exp_up);
    g.bstride = mat_bytes<ET>(I, H);
    g.N = I;
    g.Kd = H;
    g.hh = w.hh;
    g.hl = w.hl;
    g.asum = w.xsum;
    g.asum_bytes = static_cast<int>(sizeof(float) * T * (H / 32));
    g.hsum = ET::kChunk == 32 ? w.hsum : nullptr;
    launch_ggemm<ET, true>(g, bm, max_tiles, s);
    // shared gate/up: A = all x rows
    GemmArgs sg = g;
    sg.routed = 0;
    sg.a_gather = 0;
    sg.b0 = static_cast<const uint8_t *>(d->sh_gate);
    sg.b1 = static_cast<const uint8_t *>(d->sh_up);
    sg.bstride = 0;
    sg.N = Is;
    sg.hh = w.shh;
    sg.hl = w.shl;
    sg.hsum = nullptr;
    sg.kpart = w.kpart_sh;
    const int gks = shared_gu_splits(d, T);
    launch_ggemm<ST, true>(sg, 64, sh_tiles, s, gks);
    if (gks > 1) {
        const int64_t n = static_cast<int64_t>(T) * Is;
        hipLaunchKernelGGL(k_dual_sum, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, w.kpart_sh, gks, T,
                           Is, w.shh, w.shl);
    }
    // routed down: A = h of the pairs (sorted order)
    GemmArgs dg = g;
    dg.ah = w.hh;
    dg.a_bytes = static_cast<int>(sizeof(uint16_t) * P * I);
    dg.a_lo_off = static_cast<int>(reinterpret_cast<const uint8_t *>(w.hl) - reinterpret_cast<const uint8_t *>(w.hh));
    dg.al = w.hl;
    dg.a_gather = 0;
    dg.asum = w.hsum;
    dg.asum_bytes = static_cast<int>(sizeof(float) * P * (I / 32));
    dg.b0 = static_cast<const uint8_t *>(d->exp_down);
    dg.b1 = nullptr;
    dg.bstride = mat_bytes<ET>(H, I);
    dg.N = H;
    dg.Kd = I;
    dg.out = w.rout;
    launch_ggemm<ET, false>(dg, bm, max_tiles, s);
    // shared down
    GemmArgs sd = dg;
    sd.routed = 0;
    sd.ah = w.shh;
    sd.a_bytes = static_cast<int>(sizeof(uint16_t) * T * Is);
    sd.a_lo_off = static_cast<int>(reinterpret_cast<const uint8_t *>(w.shl) - reinterpret_cast<const uint8_t *>(w.shh));
    sd.al = w.shl;
    sd.b0 = static_cast<const uint8_t *>(d->sh_down);
    sd.bstride = 0;
    sd.Kd = Is;
    sd.out = w.sout;
    sd.kpart = w.kpart_sh;
    const int dks = shared_dn_splits(d, T);
    launch_ggemm<ST, false>(sd, 64, sh_tiles, s, dks);
    if (dks > 1) {
        const int64_t n = static_cast<int64_t>(T) * H;
        hipLaunchKernelGGL(k_single_sum, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, w.kpart_sh, dks,
                           T, H, w.sout);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// The per-row routing (ids / weights / gate in the workspace, and in the
// caller's outputs when given): router norms, approximate logits from the
// dense GEMM of x (hi + lo, from k_split_x), then candidates and their exact
// logits (k_select_approx).
template <typename RT>
static void prefill_route_t(const moe_layer_desc *d, const float *x, int T, const PrefillWs &w, int32_t *ids_out,
                            float *wts_out, float *gate_out, hipStream_t s)
{
    const int H = d->hidden, E = d->n_experts, K = d->top_k;
    GemmArgs g{};
    g.T = T;
    g.K = K;
    g.E = E;
    g.routed = 0;
    g.a_gather = 0;
    g.ah = reinterpret_cast<const uint16_t *>(w.xh);
    g.al = reinterpret_cast<const uint16_t *>(w.xl);
    g.a_bytes = static_cast<int>(sizeof(uint16_t) * T * H);
    g.a_lo_off = static_cast<int>(reinterpret_cast<const uint8_t *>(w.xl) - reinterpret_cast<const uint8_t *>(w.xh));
    g.b0 = static_cast<const uint8_t *>(d->router_w);
    g.bstride = 0;
    g.N = E;
    g.Kd = H;
    g.out = w.lap;
    g.kpart = w.kpart;
    const int ks = router_splits(d, T);
    launch_ggemm<RT, false>(g, 64, (T + 63) / 64, s, ks);
    const float *lap = ks > 1 ? w.kpart : w.lap;
    const double cH = 1.01 * (3.0 * std::ldexp(1.0, -16) + (3.0 * H + 64.0) * std::ldexp(1.0, -23));
    const size_t lds = sizeof(float) * ((H + 3) & ~3) + sizeof(double) * E;
    const float *wb = d->bias_mode == MOE_BIAS_SELECT_ONLY ? d->router_bias : nullptr;
    if (E <= 8 * kWave)
        hipLaunchKernelGGL((k_select_approx<RT, 8>), dim3(T), dim3(kSelWaves * kWave), lds, s, x, lap, ks, w.wn,
                           static_cast<const uint8_t *>(d->router_w), static_cast<const uint8_t *>(d->shared_gate_w),
                           d->router_bias, wb, T, H, E, K, d->renormalize, cH, w.ids, w.wts, w.gate, ids_out, wts_out,
                           gate_out);
    else
        hipLaunchKernelGGL((k_select_approx<RT, kMaxE / kWave>), dim3(T), dim3(kSelWaves * kWave), lds, s, x, lap, ks, w.wn,
                           static_cast<const uint8_t *>(d->router_w), static_cast<const uint8_t *>(d->shared_gate_w),
                           d->router_bias, wb, T, H, E, K, d->renormalize, cH, w.ids, w.wts, w.gate, ids_out, wts_out,
                           gate_out);
}

static int prefill_route(const moe_layer_desc *d, const float *x, int T, const PrefillWs &w, int32_t *ids_out,
                         float *wts_out, float *gate_out, hipStream_t s)
{
    if (d->router_t == MOE_F32)
        prefill_route_t<F32>(d, x, T, w, ids_out, wts_out, gate_out, s);
    else
        prefill_route_t<BF16>(d, x, T, w, ids_out, wts_out, gate_out, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// x hi/lo and block sums; with `norms`, also the router row norms (for the
// routing) in leading blocks of the same launch.
static void split_x(const moe_layer_desc *d, const float *x, int T, const PrefillWs &w, bool norms, hipStream_t s)
{
    const int H = d->hidden, E = d->n_experts;
    const int64_t n8 = static_cast<int64_t>(T) * H / 8;
    const int nbx = static_cast<int>((n8 + 255) / 256), nbn = norms ? (E + 3) / 4 : 0;
    const dim3 grid(nbn + nbx);
    const uint8_t *rw = static_cast<const uint8_t *>(d->router_w);
    if (d->router_t == MOE_F32)
        hipLaunchKernelGGL((k_split_x<F32>), grid, dim3(256), 0, s, x, n8, w.xh, w.xl, w.xsum, nbn, rw, E, H, w.wn);
    else
        hipLaunchKernelGGL((k_split_x<BF16>), grid, dim3(256), 0, s, x, n8, w.xh, w.xl, w.xsum, nbn, rw, E, H, w.wn);
}

// The layer's input: x, or its RMS norm (k_rmsnorm into the workspace).
static const float *layer_input(const moe_layer_desc *d, const float *x, int T, const PrefillWs &w, hipStream_t s)
{
    if (!d->norm_w)
        return x;
    hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), sizeof(float) * d->hidden, s, x, d->hidden, d->norm_w,
                       d->norm_eps, w.u);
    return w.u;
}

int launch_prefill_route(const moe_layer_desc *d, const float *x, int T, int32_t *ids, float *wts, float *gate,
                         void *ws, hipStream_t s)
{
    const PrefillWs w = prefill_carve(ws, d, T, true);
    const float *u = layer_input(d, x, T, w, s);
    split_x(d, u, T, w, true, s);
    return prefill_route(d, u, T, w, ids, wts, gate, s);
}

// Everything between the x split and the combine: the routing (computed or
// given), the sort, the tiles and the GEMMs.
static int prefill_middle(const moe_layer_desc *d, const float *x, int T, const PrefillWs &w, const int32_t *ids_in,
                          const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out,
                          float *gate_out, hipStream_t s)
{
    const int E = d->n_experts, K = d->top_k;
    const int64_t P = static_cast<int64_t>(T) * K;
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
    const int bm = routed_bm(P, E);
    rc = launch_sort_by_expert(w.ids, T, K, E, w.counts, w.offsets, w.perm, w.sort_ws, s, w.inv, bm,
                               static_cast<int>((P + bm - 1) / bm + E), w.tiles);
    if (rc != MOE_OK)
        return rc;
    const int et = d->expert_t, st = d->shared_t;
    if (st == MOE_F32) {
        switch (et) {
        case MOE_F32: return run_gemms<F32, F32>(d, T, w, bm, s);
        case MOE_BF16: return run_gemms<BF16, F32>(d, T, w, bm, s);
        case MOE_Q2B32: return run_gemms<Q2, F32>(d, T, w, bm, s);
        case MOE_Q3B32: return run_gemms<Q3, F32>(d, T, w, bm, s);
        default: return run_gemms<Q4, F32>(d, T, w, bm, s);
        }
    }
    switch (et) {
    case MOE_F32: return run_gemms<F32, BF16>(d, T, w, bm, s);
    case MOE_BF16: return run_gemms<BF16, BF16>(d, T, w, bm, s);
    case MOE_Q2B32: return run_gemms<Q2, BF16>(d, T, w, bm, s);
    case MOE_Q3B32: return run_gemms<Q3, BF16>(d, T, w, bm, s);
    default: return run_gemms<Q4, BF16>(d, T, w, bm, s);
    }
}

int launch_prefill_forward(const moe_layer_desc *d, const float *x, int T, float *y, const int32_t *ids_in,
                           const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out,
                           float *gate_out, void *ws, hipStream_t s)
{
    const int H = d->hidden, K = d->top_k;
    const PrefillWs w = prefill_carve(ws, d, T, true);
    const float *u = layer_input(d, x, T, w, s);
    split_x(d, u, T, w, ids_in == nullptr, s);
    const int rc = prefill_middle(d, u, T, w, ids_in, wts_in, gate_in, ids_out, wts_out, gate_out, s);
    if (rc != MOE_OK)
        return rc;
    const int64_t n4 = static_cast<int64_t>(T) * H / 4;
    hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s, w.rout, w.sout,
                       w.inv, w.gate, T, K, H, d->residual ? x : nullptr, y);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
