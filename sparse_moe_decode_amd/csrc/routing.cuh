// Exact per-row routing shared by the decode and prefill paths: top-K of a
// row of fp64 router logits under the order "logit desc, then id asc", the
// softmax weights over the selection and the sigmoid shared-expert gate.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>

#include "device_common.cuh"

namespace moe {

// Routing state of up to kMaxRows rows, in LDS.
struct RouteLds {
    int sel_e[kMaxRows][kMaxK];
    double sel_l[kMaxRows][kMaxK];
    float sel_w[kMaxRows][kMaxK];
    double ex[kMaxRows][kMaxK];
    int cand[kMaxRows][kWave];
    double cand_v[kMaxRows][kWave];
    float g[kMaxRows];
    SlotTable slots;
};

// Order-preserving integer key of a float: a > b iff key(a) > key(b).
__device__ __forceinline__ uint32_t f32_key(float v)
{
    const uint32_t u = __float_as_uint(v + 0.0f);   // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-K of one row of E logits (double, in LDS) by one wave, under the order
// "logit desc, then id asc". Writes rl.sel_e[q][0..K) and rl.sel_l[q][0..K)
// in that order. Expert e = lane + 64*m is element m of lane `lane`.
//  1. Each lane's maximum; the K-th largest lane maximum M is at most the
//     K-th largest logit (the K lanes above it hold K distinct logits >= M).
//  2. Candidates: logits whose fp32 rounding is >= fp32(M). Rounding to fp32
//     is monotone, so every logit of the true top K is a candidate and every
//     non-candidate is below M, hence below the K-th largest.
//  3. The candidates are ranked exactly (fp64 compare, then id).
// The threshold is found by a bitwise binary search whose counts are
// wave-wide ballots; the candidates are compacted into LDS and ranked there.
__device__ inline void wave_select(const double *lg, int E, int K, int q, RouteLds &rl, int lane)
{
    constexpr int PL = kMaxE / kWave;
    const int npl = (E + kWave - 1) / kWave;
    // Every slot is written on every path (no divergent writes into the
    // array), so the keys stay plain registers.
    uint32_t key[PL];
    uint32_t mk = 0;   // 0 is below every real key
#pragma unroll
    for (int m = 0; m < PL; ++m) {
        const int e = lane + m * kWave;
        const bool in = e < E;
        const uint32_t k = f32_key(static_cast<float>(lg[in ? e : 0]));
        key[m] = in ? k : 0u;
        mk = key[m] > mk ? key[m] : mk;
    }
    uint32_t t = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = t | (1u << b);
        if (__popcll(__ballot(mk >= c)) >= K)
            t = c;
    }
    const unsigned long long lt = (1ull << lane) - 1ull;
    int C = 0;
#pragma unroll
    for (int m = 0; m < PL; ++m) {
        if (m < npl) {
            const bool cand = key[m] >= t && key[m] != 0;
            const unsigned long long mask = __ballot(cand);
            const int pos = C + __popcll(mask & lt);
            if (cand && pos < kWave) {
                const int e = lane + m * kWave;
                rl.cand[q][pos] = e;
                rl.cand_v[q][pos] = lg[e];
            }
            C += __popcll(mask);
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (C <= kWave) {
        // rank of each candidate among the candidates; the table is read
        // with same-address (broadcast) LDS loads
        const int e = lane < C ? rl.cand[q][lane] : 0;
        const double v = lane < C ? rl.cand_v[q][lane] : 0.0;
        int rank = 0;
#pragma unroll 4
        for (int j = 0; j < C; ++j) {
            const double vj = rl.cand_v[q][j];
            const int ej = rl.cand[q][j];
            rank += (vj > v) | ((vj == v) & (ej < e));
        }
        if (lane < C && rank < K) {
            rl.sel_e[q][rank] = e;
            rl.sel_l[q][rank] = v;
        }
        __builtin_amdgcn_wave_barrier();
        return;
    }
    // many candidates (massive exact ties): rank each against all logits
#pragma unroll
    for (int m = 0; m < PL; ++m) {
        const int e = lane + m * kWave;
        if (e >= E || key[m] < t)
            continue;
        const double v = lg[e];
        int rank = 0;
        for (int e2 = 0; e2 < E; ++e2) {
            const double o = lg[e2];
            rank += (o > v) | ((o == v) & (e2 < e));
        }
        if (rank < K) {
            rl.sel_e[q][rank] = e;
            rl.sel_l[q][rank] = v;
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// Route weights of row q by the wave that selected it, in selection order:
// w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0) over the selection
// (renormalized) or over all E logits; the gate sigmoid(z_q).
__device__ inline void wave_weights(const double *lg, int E, int K, int renorm, double z, int q, RouteLds &rl,
                                    int lane)
{
    __builtin_amdgcn_wave_barrier();
    const double l0 = rl.sel_l[q][0];
    double v = 0.0;
    if (lane < K) {
        v = exp(rl.sel_l[q][lane] - l0);
        rl.ex[q][lane] = v;
    }
    __builtin_amdgcn_wave_barrier();
    double denom = 0.0;
    if (renorm) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < K)
                denom += rl.ex[q][j];
    } else {
        double s = 0.0;
        for (int e = lane; e < E; e += kWave)
            s += exp(lg[e] - l0);
        denom = lane_group_sum(s, kWave);
    }
    if (lane < K)
        rl.sel_w[q][lane] = static_cast<float>(v / denom);
    if (lane == 0)
        rl.g[q] = static_cast<float>(1.0 / (1.0 + exp(-z)));
}

}  // namespace moe
