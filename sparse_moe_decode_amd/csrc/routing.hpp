// Exact per-row routing shared by the decode and prefill paths: top-K of a
// row of fp64 router logits under the order "logit desc, then id asc", the
// softmax weights over the selection and the sigmoid shared-expert gate.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>

#include "device_common.hpp"

namespace moe {

// Routing state of up to kMaxRows rows, in LDS.
struct RouteLds {
    int sel_e[kMaxRows][kMaxK];
    double sel_l[kMaxRows][kMaxK];
    float sel_w[kMaxRows][kMaxK];
    alignas(16) int cand[kMaxRows][kWave];
    alignas(16) double cand_v[kMaxRows][kWave];
    alignas(16) uint64_t cand_p[kMaxRows][kWave];
    alignas(16) uint32_t pmax[kMaxRows][kWave / 2];
    // one row routed by a whole workgroup of 4 waves: each wave's candidates
    // (packed as in cand_p) and their counts
    alignas(16) uint64_t seg_p[4][kWave];
    alignas(16) int seg_n[4];
    float g[kMaxRows];
    SlotTable slots;
};

// Router dot products in fp64 (exact products of an fp32 activation and a
// bf16/fp32 weight): one 16-byte chunk c of a router row (4 fp32 or 8 bf16
// weights) against x (fp32, R rows of H in `xs`), accumulated in element order.
//
// The order of an exact logit, the same on every path so that all paths
// produce the same bits: chunk c of a row belongs to quarter (c >> 6) & 3
// and lane c & 63; each lane sums its chunks of a quarter in increasing c
// (router_chunk), each quarter is summed over the wave (wave_sum), and the
// logit is (P0 + P1) + (P2 + P3), then + bias. Four waves compute the four
// quarters side by side (the decode logits kernel); one wave computes them
// with four accumulators (the prefill selection).
template <int R>
__device__ __forceinline__ void router_chunk(F32, const uint4 &u, int c, const float *xs, int H, double (&acc)[R])
{
    const float w[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 xv = *reinterpret_cast<const float4 *>(xs + q * H + c * 4);
        acc[q] = fma(static_cast<double>(w[0]), static_cast<double>(xv.x), acc[q]);
        acc[q] = fma(static_cast<double>(w[1]), static_cast<double>(xv.y), acc[q]);
        acc[q] = fma(static_cast<double>(w[2]), static_cast<double>(xv.z), acc[q]);
        acc[q] = fma(static_cast<double>(w[3]), static_cast<double>(xv.w), acc[q]);
    }
}

template <int R>
__device__ __forceinline__ void router_chunk(BF16, const uint4 &u, int c, const float *xs, int H, double (&acc)[R])
{
    const float wf[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                         bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 x0 = *reinterpret_cast<const float4 *>(xs + q * H + c * 8);
        const float4 x1 = *reinterpret_cast<const float4 *>(xs + q * H + c * 8 + 4);
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[q] = fma(static_cast<double>(wf[i]), static_cast<double>(xv[i]), acc[q]);
    }
}

__device__ __forceinline__ double combine_quarters(double p0, double p1, double p2, double p3)
{
    return (p0 + p1) + (p2 + p3);
}

// v[l] + v[l ^ 32] on every lane, with one VALU swap of the wave's halves
// (v_permlane32_swap: each returned register holds one half of each).
__device__ __forceinline__ int add_halves(int v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] + r[1];
}

// Order-preserving integer key of a float: a > b iff key(a) > key(b).
__device__ __forceinline__ uint32_t f32_key(float v)
{
    const uint32_t u = __float_as_uint(v + 0.0f);   // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact rank of candidate `lane` among the C <= 64 candidates of row q
// (rl.cand / rl.cand_v, padded with NaN to a multiple of 8), fp64 compare then
// id; lanes with rank < K write the selection.
__device__ __forceinline__ void rank_exact(int C, int K, int q, RouteLds &rl, int lane)
{
    const int C8 = (C + 7) & ~7;
    if (lane >= C && lane < C8)
        rl.cand_v[q][lane] = __builtin_nan("");
    __builtin_amdgcn_wave_barrier();
    const int e = lane < C ? rl.cand[q][lane] : 0;
    const double v = lane < C ? rl.cand_v[q][lane] : 0.0;
    int rank = 0;
    for (int j = 0; j < C; j += 8) {
        double2 pv[4];
        int4 pe[2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            pv[u] = *reinterpret_cast<const double2 *>(&rl.cand_v[q][j + 2 * u]);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            pe[u] = *reinterpret_cast<const int4 *>(&rl.cand[q][j + 4 * u]);
        const double vj[8] = {pv[0].x, pv[0].y, pv[1].x, pv[1].y, pv[2].x, pv[2].y, pv[3].x, pv[3].y};
        const int ej[8] = {pe[0].x, pe[0].y, pe[0].z, pe[0].w, pe[1].x, pe[1].y, pe[1].z, pe[1].w};
#pragma unroll
        for (int u = 0; u < 8; ++u)
            rank += (vj[u] > v) | ((vj[u] == v) & (ej[u] < e));
    }
    if (lane < C && rank < K) {
        rl.sel_e[q][rank] = e;
        rl.sel_l[q][rank] = v;
    }
    __builtin_amdgcn_wave_barrier();
}

// Weight logit of expert e from its selection logit l: l itself, or l - b_e
// when the router bias enters the selection only (wb = the bias, else null).
__device__ __forceinline__ double weight_logit(double l, int e, const float *wb)
{
    return wb ? l - static_cast<double>(wb[e]) : l;
}

// Route weights of row q by the wave that selected it, in selection order:
// w_k = exp(v_k - v_0) / sum_j exp(v_j - v_0) over the selection
// (renormalized) or over all E, with v the weight logits (weight_logit); the
// gate sigmoid(z_q) = 1/(1+exp(-z_q)). The differences v_k - v_0 are taken
// in fp64 and rounded once; the exponentials, sums and quotients are fp32
// (the outputs are fp32). Lane k < K evaluates exp(v_k - v_0), lane K
// evaluates exp(-z), in one pass; sums are wave reductions in a fixed order.
__device__ __forceinline__ void wave_weights(const double *lg, int E, int K, int renorm, double z, int q, RouteLds &rl,
                                             int lane, bool gate = true, const float *wb = nullptr)
{
    __builtin_amdgcn_wave_barrier();
    const double l0 = weight_logit(rl.sel_l[q][0], rl.sel_e[q][0], wb);
    float arg = 0.0f;
    if (lane < K)
        arg = static_cast<float>(weight_logit(rl.sel_l[q][lane], rl.sel_e[q][lane], wb) - l0);
    else if (lane == K)
        arg = static_cast<float>(-z);
    const float v = expf(arg);
    float denom;
    if (renorm) {
        denom = wave_sum(lane < K ? v : 0.0f);
    } else {
        float s = 0.0f;
        for (int e = lane; e < E; e += kWave)
            s += expf(static_cast<float>(weight_logit(lg[e], e, wb) - l0));
        denom = wave_sum(s);
    }
    const float r = (lane < K ? v : 1.0f) / (lane < K ? denom : 1.0f + v);
    if (lane < K)
        rl.sel_w[q][lane] = r;
    if (gate && lane == K)
        rl.g[q] = r;
    __builtin_amdgcn_wave_barrier();
}

// The K-th largest of 32 keys gm[0..32) (LDS), or, if it is tied, a value
// with fewer than K keys above it and at least K at or above: lane l counts
// the keys above key l%32 in half l/32 of the array; the halves are added.
__device__ __forceinline__ uint32_t kth_of_32(const uint32_t *gm, int K, int lane)
{
    const uint32_t v = gm[lane & 31];
    const uint32_t *half = gm + 16 * (lane >> 5);
    uint4 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = *reinterpret_cast<const uint4 *>(half + 4 * j);
    int gt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        gt += (o[j].x > v) + (o[j].y > v) + (o[j].z > v) + (o[j].w > v);
    gt = add_halves(gt);
    // exactly K-1 above: the K-th largest; with ties at that value no lane
    // may see K-1, then: fewer than K above and at least K at or above
    unsigned long long hit = __ballot(lane < 32 && gt == K - 1);
    if (hit == 0) {
        int ge = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ge += (o[j].x >= v) + (o[j].y >= v) + (o[j].z >= v) + (o[j].w >= v);
        ge = add_halves(ge);
        hit = __ballot(lane < 32 && gt < K && ge >= K);
    }
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), __builtin_ctzll(hit)));
}

// Ranking of the C <= 64 candidates of row q compacted in rl.cand_p[q][0..C)
// as packed (fp32 key, ~id) words; value(p) gives the fp64 logit of the
// lane's candidate p. Distinct keys order their values exactly: unless one of
// the first K+1 shares its key with another candidate, the selection, its
// weights (as in wave_weights) and, if `gate`, the gate are written (and the
// routed slots 1..K of `st`, if given) and true is returned; else nothing is
// written and the candidates need exact fp64 ranking.
template <typename ValueOf>
__device__ __forceinline__ bool rank_packed(int C, int K, int renorm, int E, const double *lg, double z, bool gate,
                                            int q, RouteLds &rl, int lane, ValueOf value, SlotTable *st,
                                            const float *wb)
{
    // padding 0 is below every candidate and shares no key with one; up to
    // 16 candidates (the usual case) are read in one unrolled batch
    const int CP = C <= 16 ? 16 : (C + 3) & ~3;
    if (lane >= C && lane < CP)
        rl.cand_p[q][lane] = 0;
    __builtin_amdgcn_wave_barrier();
    const uint64_t p = rl.cand_p[q][lane];
    const uint32_t pk = static_cast<uint32_t>(p >> 32);
    int rank = 0, tie = 0;
    auto count4 = [&](const ulonglong2 &a, const ulonglong2 &b) {
        rank += (a.x > p) + (a.y > p) + (b.x > p) + (b.y > p);
        tie += (static_cast<uint32_t>(a.x >> 32) == pk) + (static_cast<uint32_t>(a.y >> 32) == pk) +
               (static_cast<uint32_t>(b.x >> 32) == pk) + (static_cast<uint32_t>(b.y >> 32) == pk);
    };
    if (C <= 16) {
        ulonglong2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = *reinterpret_cast<const ulonglong2 *>(&rl.cand_p[q][2 * u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            count4(v[2 * u], v[2 * u + 1]);
    } else {
        for (int j = 0; j < C; j += 4)
            count4(*reinterpret_cast<const ulonglong2 *>(&rl.cand_p[q][j]),
                   *reinterpret_cast<const ulonglong2 *>(&rl.cand_p[q][j + 2]));
    }
    const bool live = lane < C;
    if (__ballot(live && rank <= K && tie > 1) != 0)
        return false;
    const int e = static_cast<int>(~static_cast<uint32_t>(p));
    const double val = live ? value(p) : 0.0;
    const double wv = live ? weight_logit(val, e, wb) : 0.0;
    // v_0: the weight logit of the candidate ranked first
    const int r0 = __builtin_ctzll(__ballot(live && rank == 0));
    const long long vb = __double_as_longlong(wv);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(vb & 0xffffffff), r0);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(vb >> 32), r0);
    const double l0 = __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
    const bool sel = live && rank < K;
    const float ex = sel ? expf(static_cast<float>(wv - l0)) : 0.0f;
    float denom;
    if (renorm) {
        denom = wave_sum(ex);
    } else {
        float sum = 0.0f;
        for (int e2 = lane; e2 < E; e2 += kWave)
            sum += expf(static_cast<float>(weight_logit(lg[e2], e2, wb) - l0));
        denom = wave_sum(sum);
    }
    if (sel) {
        const float w = ex / denom;
        rl.sel_e[q][rank] = e;
        rl.sel_l[q][rank] = val;
        rl.sel_w[q][rank] = w;
        if (st) {
            st->expert[rank + 1] = e;
            st->w[rank + 1][0] = w;
        }
    }
    if (gate && lane == 0)
        rl.g[q] = 1.0f / (1.0f + expf(static_cast<float>(-z)));
    __builtin_amdgcn_wave_barrier();
    return true;
}

// Routing of one row of E logits (double, in LDS) by one wave: the top K
// under the order "logit desc, then id asc" into rl.sel_e[q][0..K) and
// rl.sel_l[q][0..K), the route weights into rl.sel_w[q] and the gate into
// rl.g[q] (weights as in wave_weights). Expert e = lane + 64*m is element m of
// lane `lane`; PL is the number of elements per lane (E <= 64*PL).
//  1. Keys: order-preserving integers of the fp32 roundings (rounding to
//     fp32 is monotone). M = the K-th largest of the 32 maxima of lane pairs;
//     the K pairs at or above it hold K distinct logits whose keys are >= M,
//     so the K-th largest logit has key >= M.
//  2. Candidates: logits with key >= M (every logit of the true top K is
//     one), compacted into LDS by a ballot prefix of the per-lane counts.
//  3. Ranking by (key desc, id asc) packed in 64 bits. Distinct keys order
//     their values exactly; if any of the first K+1 shares its key with
//     another candidate, the candidates are ranked in fp64 instead
//     (rank_exact). The weights are then computed by the ranked lanes
//     themselves. More than 64 candidates (massive ties) take a slower exact
//     path.
template <int PL>
__device__ __forceinline__ void wave_route_pl(const double *lg, int E, int K, int renorm, double z, int q,
                                              RouteLds &rl, int lane, const float *wb)
{
    uint32_t key[PL];
    uint32_t mk = 0;   // 0 is below every key of a non-NaN value
#pragma unroll
    for (int m = 0; m < PL; ++m) {
        const int e = lane + m * kWave;
        const bool in = e < E;
        const uint32_t k = f32_key(static_cast<float>(lg[in ? e : 0]));
        key[m] = in ? k : 0u;
        mk = key[m] > mk ? key[m] : mk;
    }
    // 1. maximum over the lane pair (2i, 2i+1): DPP quad permutation [1,0,3,2]
    const uint32_t other =
        static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mk), 0xB1, 0xF, 0xF, false));
    const uint32_t pm = other > mk ? other : mk;
    if ((lane & 1) == 0)
        rl.pmax[q][lane >> 1] = pm;
    __builtin_amdgcn_wave_barrier();
    const uint32_t t = kth_of_32(rl.pmax[q], K, lane);

    // 2. compaction: exclusive prefix of the per-lane counts from ballots of
    // their bits
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < PL; ++m)
        cnt += (key[m] >= t) & (key[m] != 0);
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
        const bool c = (key[m] >= t) & (key[m] != 0);
        if (c && pos < kWave) {
            const int e = lane + m * kWave;
            rl.cand[q][pos] = e;
            rl.cand_p[q][pos] = (static_cast<uint64_t>(key[m]) << 32) | static_cast<uint32_t>(~e);
        }
        pos += c;
    }
    if (C <= kWave) {
        // 3. rank by packed key
        if (rank_packed(C, K, renorm, E, lg, z, true, q, rl, lane,
                        [&](uint64_t p) { return lg[~static_cast<uint32_t>(p)]; }, nullptr, wb))
            return;
        // a key shared near the boundary: exact fp64 ranking
        if (lane < C)
            rl.cand_v[q][lane] = lg[rl.cand[q][lane]];
        rank_exact(C, K, q, rl, lane);
    } else {
        // many candidates (massive exact ties): rank each against all logits
#pragma unroll
        for (int m = 0; m < PL; ++m) {
            const int e = lane + m * kWave;
            if (e >= E || key[m] < t)
                continue;
            const double val = lg[e];
            int rank = 0;
            for (int e2 = 0; e2 < E; ++e2) {
                const double o2 = lg[e2];
                rank += (o2 > val) | ((o2 == val) & (e2 < e));
            }
            if (rank < K) {
                rl.sel_e[q][rank] = e;
                rl.sel_l[q][rank] = val;
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    wave_weights(lg, E, K, renorm, z, q, rl, lane, true, wb);
}

// Routing of row q by one wave (see wave_route_pl); wb: the router bias when
// it enters the selection only (the weights then use the unbiased logits).
__device__ __forceinline__ void wave_route(const double *lg, int E, int K, int renorm, double z, int q, RouteLds &rl,
                                           int lane, const float *wb)
{
    if (E <= 8 * kWave)
        wave_route_pl<8>(lg, E, K, renorm, z, q, rl, lane, wb);
    else
        wave_route_pl<kMaxE / kWave>(lg, E, K, renorm, z, q, rl, lane, wb);
}

}  // namespace moe
