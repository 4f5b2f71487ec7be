// Decode (1 row) and few-row (2..4 rows) path of the sparse MoE layer on gfx950.
//
// Three launches per call, all on the caller's stream:
//   k_route   router logits (fp64 accumulation) + shared-gate logit, then the
//             last-arriving workgroup runs the wave-level top-K, the softmax
//             weights, the sigmoid gate and builds the slot table (the union
//             of the rows' experts; slot 0 is the shared expert, weighted by
//             the gate - the "extra slot" design of the Research notes page,
//             section 1, "Metal").
//   k_gateup  one wave per (slot, intermediate channel): gate and up rows
//             read once with 16-byte loads, dotted with every row's x,
//             SwiGLU, scaled by the row's route weight -> hbuf.
//   k_down    each wave owns output rows j and sums D_s[j] . hbuf_s over all
//             slots: the weighted combine happens inside the dot, no partial
//             results leave the chip, every y element is written once.
// Each selected expert is read exactly once per call, whatever the number of
// rows that selected it (the few-row idea of the Research notes page,
// section 1, MTP "Verify" entry).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>

#include "device_common.cuh"
#include "internal.h"

namespace moe {

// ============================================================== route

struct RouteArgs {
    const float *x;          // [R][H]
    int H, E, K, renorm;
    const uint8_t *router_w; // [E][H]
    const float *bias;       // [E] or null
    const uint8_t *gate_w;   // [H]
    int32_t *ids_out;        // [R][K] or null
    float *wts_out;          // [R][K] or null
    float *gate_out;         // [R] or null
    DecodeWs ws;
    int rows_per_wave;
};

// fp64 dot of router row `row` with each staged x row. Products of a bf16 or
// fp32 weight with an fp32 activation are exact in double.
template <int R>
__device__ __forceinline__ void router_dot(F32, const uint8_t *row, int H, const float *xs, int lane,
                                           double (&acc)[R])
{
    const int nch = H >> 2;
    for (int c = lane; c < nch; c += kWave) {
        const float4 w = *reinterpret_cast<const float4 *>(row + c * 16);
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const float4 xv = *reinterpret_cast<const float4 *>(xs + q * H + c * 4);
            acc[q] = fma(static_cast<double>(w.x), static_cast<double>(xv.x), acc[q]);
            acc[q] = fma(static_cast<double>(w.y), static_cast<double>(xv.y), acc[q]);
            acc[q] = fma(static_cast<double>(w.z), static_cast<double>(xv.z), acc[q]);
            acc[q] = fma(static_cast<double>(w.w), static_cast<double>(xv.w), acc[q]);
        }
    }
}

template <int R>
__device__ __forceinline__ void router_dot(BF16, const uint8_t *row, int H, const float *xs, int lane,
                                           double (&acc)[R])
{
    const int nch = H >> 3;
    for (int c = lane; c < nch; c += kWave) {
        const uint4 w = *reinterpret_cast<const uint4 *>(row + c * 16);
        const float wf[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                             bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
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
}

// Selection for one row by one wave: K rounds of a wave-wide argmax over
// (logit desc, id asc). Returns the selected ids / logits in every lane.
__device__ inline void wave_topk(const double *logits, int E, int K, int lane, int (&sel_id)[kMaxK],
                                 double (&sel_l)[kMaxK], double &sum_all_exp_shift, bool need_all)
{
    constexpr int kPerLane = kMaxE / kWave;   // 16
    double lv[kPerLane];
#pragma unroll
    for (int m = 0; m < kPerLane; ++m) {
        const int e = lane + m * kWave;
        lv[m] = e < E ? logits[e] : -DBL_MAX;
    }
    uint32_t taken = 0;
    for (int k = 0; k < K; ++k) {
        double bv = -DBL_MAX;
        int bi = INT_MAX;
#pragma unroll
        for (int m = 0; m < kPerLane; ++m) {
            const int e = lane + m * kWave;
            if (e < E && !((taken >> m) & 1u) && (lv[m] > bv || (lv[m] == bv && e < bi))) {
                bv = lv[m];
                bi = e;
            }
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            const double ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        sel_id[k] = bi;
        sel_l[k] = bv;
        if ((bi & (kWave - 1)) == lane)
            taken |= 1u << (bi / kWave);
    }
    sum_all_exp_shift = 0.0;
    if (need_all) {
        double s = 0.0;
#pragma unroll
        for (int m = 0; m < kPerLane; ++m) {
            const int e = lane + m * kWave;
            if (e < E)
                s += exp(lv[m] - sel_l[0]);
        }
        for (int off = kWave / 2; off > 0; off >>= 1)
            s += __shfl_xor(s, off, kWave);
        sum_all_exp_shift = s;
    }
}

// Slot table from per-row selections held in LDS (sel_e/sel_w [R][K], g[R]).
template <int R>
__device__ inline void build_slots(SlotTable *st, const int *sel_e, const float *sel_w, const float *g, int K,
                                   int lane)
{
    const int RK = R * K;
    bool first = false;
    int e = -1;
    if (lane < RK) {
        e = sel_e[lane];
        first = true;
        for (int j = 0; j < lane; ++j)
            if (sel_e[j] == e)
                first = false;
    }
    const unsigned long long mask = __ballot(first);
    const int slot = 1 + __popcll(mask & ((1ull << lane) - 1ull));
    if (first) {
        st->expert[slot] = e;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            float w = 0.0f;
            for (int k = 0; k < K; ++k)
                if (sel_e[q * K + k] == e)
                    w = sel_w[q * K + k];
            st->w[slot][q] = w;
        }
    }
    if (lane == 0) {
        st->nslots = 1 + __popcll(mask);
        st->expert[0] = -1;
#pragma unroll
        for (int q = 0; q < R; ++q)
            st->w[0][q] = g[q];
    }
}

template <int R, typename RT>
__global__ void __launch_bounds__(256) k_route(RouteArgs a)
{
    extern __shared__ float xs[];   // [R][H]
    const int tid = threadIdx.x;
    for (int i = tid; i < R * a.H / 4; i += blockDim.x)
        reinterpret_cast<float4 *>(xs)[i] = reinterpret_cast<const float4 *>(a.x)[i];
    __syncthreads();

    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int gwave = blockIdx.x * (blockDim.x / kWave) + wave;
    const size_t rb = static_cast<size_t>(a.H) * (RT::kChunk == 4 ? 4 : 2);
    for (int i = 0; i < a.rows_per_wave; ++i) {
        const int e = gwave * a.rows_per_wave + i;
        if (e > a.E)
            break;
        const uint8_t *row = e < a.E ? a.router_w + e * rb : a.gate_w;
        double acc[R];
#pragma unroll
        for (int q = 0; q < R; ++q)
            acc[q] = 0.0;
        router_dot<R>(RT{}, row, a.H, xs, lane, acc);
#pragma unroll
        for (int q = 0; q < R; ++q)
            acc[q] = lane_group_sum(acc[q], kWave);
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < R; ++q) {
                if (e < a.E)
                    a.ws.logits[q * a.E + e] = acc[q] + (a.bias ? static_cast<double>(a.bias[e]) : 0.0);
                else
                    a.ws.zlogit[q] = acc[q];
            }
        }
    }

    // Last-arriving workgroup does the selection.
    __shared__ int is_last;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned int t = atomicAdd(&a.ws.ctl->route_done, 1u);
        is_last = (t == gridDim.x - 1);
    }
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();

    __shared__ int sel_e[kMaxRows * kMaxK];
    __shared__ float sel_w[kMaxRows * kMaxK];
    __shared__ float gq[kMaxRows];
    if (wave < R) {
        const int q = wave;
        int ids[kMaxK];
        double ls[kMaxK];
        double sum_all;
        const double *lg = a.ws.logits + q * a.E;
        wave_topk(lg, a.E, a.K, lane, ids, ls, sum_all, a.renorm == 0);
        double denom = 0.0;
        if (a.renorm) {
            for (int k = 0; k < a.K; ++k)
                denom += exp(ls[k] - ls[0]);
        } else {
            denom = sum_all;
        }
        const double z = __builtin_nontemporal_load(&a.ws.zlogit[q]);
        const float g = static_cast<float>(1.0 / (1.0 + exp(-z)));
        for (int k = 0; k < a.K; ++k) {
            if (lane == k) {
                const float w = static_cast<float>(exp(ls[k] - ls[0]) / denom);
                sel_e[q * a.K + k] = ids[k];
                sel_w[q * a.K + k] = w;
                if (a.ids_out)
                    a.ids_out[q * a.K + k] = ids[k];
                if (a.wts_out)
                    a.wts_out[q * a.K + k] = w;
            }
        }
        if (lane == 0) {
            gq[q] = g;
            if (a.gate_out)
                a.gate_out[q] = g;
        }
    }
    __syncthreads();
    if (wave == 0)
        build_slots<R>(a.ws.slots, sel_e, sel_w, gq, a.K, lane);
    if (tid == 0)
        a.ws.ctl->route_done = 0u;   // every other workgroup has finished with it
}

// Slot table from routing supplied by the caller.
// Ids outside [0, E) contribute nothing (they become expert 0 with weight 0).
template <int R>
__global__ void __launch_bounds__(64) k_slots_from_routing(const int32_t *ids, const float *wts, const float *gate,
                                                           int K, int E, SlotTable *st)
{
    __shared__ int sel_e[kMaxRows * kMaxK];
    __shared__ float sel_w[kMaxRows * kMaxK];
    __shared__ float gq[kMaxRows];
    const int lane = threadIdx.x;
    if (lane < R * K) {
        const int e = ids[lane];
        const bool ok = e >= 0 && e < E;
        sel_e[lane] = ok ? e : 0;
        sel_w[lane] = ok ? wts[lane] : 0.0f;
    }
    if (lane < R)
        gq[lane] = gate[lane];
    __syncthreads();
    build_slots<R>(st, sel_e, sel_w, gq, K, lane);
}

// ============================================================ gate/up

struct GateUpArgs {
    const float *x;   // [R][H]
    int H, I, Is, Imax;
    const uint8_t *eg, *eu;   // routed gate/up stacks
    size_t estride;           // bytes per routed [I][H] matrix
    const uint8_t *sg, *su;   // shared gate/up
    DecodeWs ws;
    int units;                // Is + R*K*I
    int ch_per_wave;
};

template <int R, typename W>
__device__ __forceinline__ void gateup_unit(const MatRef &G, const MatRef &U, int ch, const float *xs, int H,
                                            const float *xsum, int lane, float (&a)[R], float (&c)[R])
{
    const int nch = H / W::kChunk;
#pragma unroll
    for (int q = 0; q < R; ++q) {
        a[q] = 0.0f;
        c[q] = 0.0f;
    }
    for (int k = lane; k < nch; k += kWave) {
        chunk_dot<R>(W{}, G, ch, k, xs, H, xsum, H >> 5, a);
        chunk_dot<R>(W{}, U, ch, k, xs, H, xsum, H >> 5, c);
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
        a[q] = lane_group_sum(a[q], kWave);
        c[q] = lane_group_sum(c[q], kWave);
    }
}

template <int R, typename ET, typename ST>
__global__ void __launch_bounds__(256) k_gateup(GateUpArgs p)
{
    extern __shared__ float smem[];
    float *xs = smem;                   // [R][H]
    float *xsum = smem + R * p.H;       // [R][H/32] (block sums, 2-bit weights only)
    const int tid = threadIdx.x;
    for (int i = tid; i < R * p.H / 4; i += blockDim.x)
        reinterpret_cast<float4 *>(xs)[i] = reinterpret_cast<const float4 *>(p.x)[i];
    __syncthreads();
    if (ET::kChunk == 32) {
        for (int i = tid; i < R * (p.H >> 5); i += blockDim.x) {
            float s = 0.0f;
            for (int j = 0; j < 32; ++j)
                s += xs[i * 32 + j];
            xsum[i] = s;
        }
        __syncthreads();
    }
    const int lane = tid & (kWave - 1);
    const int gwave = blockIdx.x * (blockDim.x / kWave) + tid / kWave;
    const SlotTable *st = p.ws.slots;
    const int nslots = st->nslots;
    for (int i = 0; i < p.ch_per_wave; ++i) {
        const int u = gwave * p.ch_per_wave + i;
        if (u >= p.units)
            break;
        int slot, ch;
        if (u < p.Is) {
            slot = 0;
            ch = u;
        } else {
            slot = 1 + (u - p.Is) / p.I;
            ch = (u - p.Is) % p.I;
        }
        if (slot >= nslots)
            break;
        float a[R], c[R];
        if (slot == 0) {
            const MatRef G{p.sg, p.Is, p.H}, U{p.su, p.Is, p.H};
            gateup_unit<R, ST>(G, U, ch, xs, p.H, xsum, lane, a, c);
        } else {
            const int e = st->expert[slot];
            const MatRef G{p.eg + e * p.estride, p.I, p.H}, U{p.eu + e * p.estride, p.I, p.H};
            gateup_unit<R, ET>(G, U, ch, xs, p.H, xsum, lane, a, c);
        }
        if (lane < R) {
            float hv = 0.0f;
#pragma unroll
            for (int q = 0; q < R; ++q)
                if (q == lane)
                    hv = silu_mul(a[q], c[q]) * st->w[slot][q];
            p.ws.hbuf[(static_cast<size_t>(slot) * R + lane) * p.Imax + ch] = hv;
        }
    }
}

// ============================================================== down

struct DownArgs {
    float *y;   // [R][H]
    int H, I, Is, Imax;
    const uint8_t *ed;        // routed down stack
    size_t estride;           // bytes per routed [H][I] matrix
    const uint8_t *sd;        // shared down
    DecodeWs ws;
    int group;                // slots staged in LDS at a time
};

constexpr int kDownRowsPerWave = 4;

// Partial dots of rows j0 .. j0+3 of matrix M with the staged h of one slot.
template <int R, typename W>
__device__ __forceinline__ void down_slot(const MatRef &M, int j0, const float *h, const float *hs, int Imax,
                                          int lane, float (&acc)[kDownRowsPerWave][R])
{
    const int nch = M.cols / W::kChunk;
    const int lpr = nch >= kWave ? kWave : next_pow2(nch);
    const int rpi = kWave / lpr;
    const int lr = lane / lpr;
    const int lc = lane % lpr;
#pragma unroll
    for (int t = 0; t < kDownRowsPerWave; ++t) {
        if (t * rpi >= kDownRowsPerWave)
            break;
        const int j = j0 + t * rpi + lr;
        if (j >= M.rows || t * rpi + lr >= kDownRowsPerWave)
            continue;
        for (int c = lc; c < nch; c += lpr)
            chunk_dot<R>(W{}, M, j, c, h, Imax, hs, Imax >> 5, acc[t]);
    }
}

template <int R, typename W>
__device__ __forceinline__ void down_reduce_store(int n, int lane, float (&acc)[kDownRowsPerWave][R],
                                                  float *ybuf /* [rows][R] */, bool add)
{
    const int nch = n / W::kChunk;
    const int lpr = nch >= kWave ? kWave : next_pow2(nch);
    const int rpi = kWave / lpr;
    const int lr = lane / lpr;
    const int lc = lane % lpr;
#pragma unroll
    for (int t = 0; t < kDownRowsPerWave; ++t) {
        if (t * rpi >= kDownRowsPerWave)
            break;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const float v = lane_group_sum(acc[t][q], lpr);
            const int row = t * rpi + lr;
            if (lc == 0 && row < kDownRowsPerWave) {
                if (add)
                    ybuf[row * R + q] += v;
                else
                    ybuf[row * R + q] = v;
            }
        }
    }
}

template <int R, typename ET, typename ST>
__global__ void __launch_bounds__(256) k_down(DownArgs p)
{
    extern __shared__ float smem[];
    const int G = p.group;
    float *hl = smem;                              // [G][R][Imax]
    float *hs = smem + G * R * p.Imax;             // [G][R][Imax/32]
    __shared__ float ybuf[4][kDownRowsPerWave * R];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int j0 = (blockIdx.x * (blockDim.x / kWave) + wave) * kDownRowsPerWave;
    const SlotTable *st = p.ws.slots;
    const int nslots = st->nslots;

    float acc_r[kDownRowsPerWave][R], acc_s[kDownRowsPerWave][R];
#pragma unroll
    for (int t = 0; t < kDownRowsPerWave; ++t)
#pragma unroll
        for (int q = 0; q < R; ++q) {
            acc_r[t][q] = 0.0f;
            acc_s[t][q] = 0.0f;
        }

    for (int s0 = 0; s0 < nslots; s0 += G) {
        const int gs = min(G, nslots - s0);
        __syncthreads();
        const int n4 = gs * R * p.Imax / 4;
        for (int i = tid; i < n4; i += blockDim.x)
            reinterpret_cast<float4 *>(hl)[i] =
                reinterpret_cast<const float4 *>(p.ws.hbuf + static_cast<size_t>(s0) * R * p.Imax)[i];
        __syncthreads();
        if (ET::kChunk == 32) {
            const int nb = p.Imax >> 5;
            for (int i = tid; i < gs * R * nb; i += blockDim.x) {
                float s = 0.0f;
                for (int j = 0; j < 32; ++j)
                    s += hl[i * 32 + j];
                hs[i] = s;
            }
            __syncthreads();
        }
        if (j0 < p.H) {
            for (int g = 0; g < gs; ++g) {
                const int slot = s0 + g;
                const float *h = hl + g * R * p.Imax;
                const float *hsum = hs + g * R * (p.Imax >> 5);
                if (slot == 0) {
                    const MatRef M{p.sd, p.H, p.Is};
                    down_slot<R, ST>(M, j0, h, hsum, p.Imax, lane, acc_s);
                } else {
                    const int e = st->expert[slot];
                    const MatRef M{p.ed + e * p.estride, p.H, p.I};
                    down_slot<R, ET>(M, j0, h, hsum, p.Imax, lane, acc_r);
                }
            }
        }
    }
    const bool live = j0 < p.H;
    if (live)
        down_reduce_store<R, ET>(p.I, lane, acc_r, ybuf[wave], false);
    __syncthreads();
    if (live)
        down_reduce_store<R, ST>(p.Is, lane, acc_s, ybuf[wave], true);
    __syncthreads();
    if (live && lane < kDownRowsPerWave * R) {
        const int row = lane / R, q = lane % R;
        if (j0 + row < p.H)
            p.y[q * p.H + j0 + row] = ybuf[wave][row * R + q];
    }
}

// ============================================================ launch

template <typename RT>
static int launch_route_t(const moe_layer_desc *d, const float *x, int R, int32_t *ids, float *wts, float *gate,
                          const DecodeWs &ws, hipStream_t s)
{
    RouteArgs a;
    a.x = x;
    a.H = d->hidden;
    a.E = d->n_experts;
    a.K = d->top_k;
    a.renorm = d->renormalize;
    a.router_w = static_cast<const uint8_t *>(d->router_w);
    a.bias = d->router_bias;
    a.gate_w = static_cast<const uint8_t *>(d->shared_gate_w);
    a.ids_out = ids;
    a.wts_out = wts;
    a.gate_out = gate;
    a.ws = ws;
    a.rows_per_wave = 1;
    const int waves = (a.E + 1 + a.rows_per_wave - 1) / a.rows_per_wave;
    const dim3 grid((waves + 3) / 4), block(256);
    const size_t lds = sizeof(float) * R * a.H;
    switch (R) {
    case 1: hipLaunchKernelGGL((k_route<1, RT>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_route<2, RT>), grid, block, lds, s, a); break;
    case 3: hipLaunchKernelGGL((k_route<3, RT>), grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL((k_route<4, RT>), grid, block, lds, s, a); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <typename ET, typename ST>
static int launch_experts_t(const moe_layer_desc *d, const float *x, int R, float *y, const DecodeWs &ws,
                            hipStream_t s)
{
    const int H = d->hidden, I = d->inter, Is = d->shared_inter, K = d->top_k;
    const int Imax = I > Is ? I : Is;
    GateUpArgs g;
    g.x = x;
    g.H = H;
    g.I = I;
    g.Is = Is;
    g.Imax = Imax;
    g.eg = static_cast<const uint8_t *>(d->exp_gate);
    g.eu = static_cast<const uint8_t *>(d->exp_up);
    g.estride = mat_bytes<ET>(I, H);
    g.sg = static_cast<const uint8_t *>(d->sh_gate);
    g.su = static_cast<const uint8_t *>(d->sh_up);
    g.ws = ws;
    g.units = Is + R * K * I;
    g.ch_per_wave = 2;
    const int gw = (g.units + g.ch_per_wave - 1) / g.ch_per_wave;
    const dim3 ggrid((gw + 3) / 4), block(256);
    const size_t glds = sizeof(float) * R * H + (ET::kChunk == 32 ? sizeof(float) * R * (H / 32) : 0);
    switch (R) {
    case 1: hipLaunchKernelGGL((k_gateup<1, ET, ST>), ggrid, block, glds, s, g); break;
    case 2: hipLaunchKernelGGL((k_gateup<2, ET, ST>), ggrid, block, glds, s, g); break;
    case 3: hipLaunchKernelGGL((k_gateup<3, ET, ST>), ggrid, block, glds, s, g); break;
    default: hipLaunchKernelGGL((k_gateup<4, ET, ST>), ggrid, block, glds, s, g); break;
    }
    if (hipGetLastError() != hipSuccess)
        return MOE_EHIP;

    DownArgs dn;
    dn.y = y;
    dn.H = H;
    dn.I = I;
    dn.Is = Is;
    dn.Imax = Imax;
    dn.ed = static_cast<const uint8_t *>(d->exp_down);
    dn.estride = mat_bytes<ET>(H, I);
    dn.sd = static_cast<const uint8_t *>(d->sh_down);
    dn.ws = ws;
    // stage as many slots as fit in 48 KiB of LDS
    const size_t per_slot = sizeof(float) * R * Imax + sizeof(float) * R * (Imax / 32);
    int group = static_cast<int>((48u * 1024u) / per_slot);
    if (group < 1)
        group = 1;
    if (group > R * K + 1)
        group = R * K + 1;
    dn.group = group;
    const int rows_per_wg = 4 * kDownRowsPerWave;
    const dim3 dgrid((H + rows_per_wg - 1) / rows_per_wg);
    const size_t dlds = per_slot * group;
    switch (R) {
    case 1: hipLaunchKernelGGL((k_down<1, ET, ST>), dgrid, block, dlds, s, dn); break;
    case 2: hipLaunchKernelGGL((k_down<2, ET, ST>), dgrid, block, dlds, s, dn); break;
    case 3: hipLaunchKernelGGL((k_down<3, ET, ST>), dgrid, block, dlds, s, dn); break;
    default: hipLaunchKernelGGL((k_down<4, ET, ST>), dgrid, block, dlds, s, dn); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int decode_ws_size(const moe_layer_desc *d, int R)
{
    const int Imax = d->inter > d->shared_inter ? d->inter : d->shared_inter;
    return static_cast<int>(decode_ws_bytes(R, d->n_experts, d->top_k, Imax));
}

int launch_decode_route(const moe_layer_desc *d, const float *x, int R, int32_t *ids, float *wts, float *gate,
                        void *ws, hipStream_t s)
{
    const int Imax = d->inter > d->shared_inter ? d->inter : d->shared_inter;
    const DecodeWs w = decode_ws_carve(ws, R, d->n_experts, d->top_k, Imax);
    if (d->router_t == MOE_F32)
        return launch_route_t<F32>(d, x, R, ids, wts, gate, w, s);
    return launch_route_t<BF16>(d, x, R, ids, wts, gate, w, s);
}

int launch_decode_forward(const moe_layer_desc *d, const float *x, int R, float *y, const int32_t *ids_in,
                          const float *wts_in, const float *gate_in, int32_t *ids_out, float *wts_out,
                          float *gate_out, void *ws, hipStream_t s)
{
    const int Imax = d->inter > d->shared_inter ? d->inter : d->shared_inter;
    const DecodeWs w = decode_ws_carve(ws, R, d->n_experts, d->top_k, Imax);
    int rc;
    if (ids_in) {
        switch (R) {
        case 1: hipLaunchKernelGGL((k_slots_from_routing<1>), dim3(1), dim3(64), 0, s, ids_in, wts_in, gate_in, d->top_k, d->n_experts, w.slots); break;
        case 2: hipLaunchKernelGGL((k_slots_from_routing<2>), dim3(1), dim3(64), 0, s, ids_in, wts_in, gate_in, d->top_k, d->n_experts, w.slots); break;
        case 3: hipLaunchKernelGGL((k_slots_from_routing<3>), dim3(1), dim3(64), 0, s, ids_in, wts_in, gate_in, d->top_k, d->n_experts, w.slots); break;
        default: hipLaunchKernelGGL((k_slots_from_routing<4>), dim3(1), dim3(64), 0, s, ids_in, wts_in, gate_in, d->top_k, d->n_experts, w.slots); break;
        }
        rc = hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
    } else {
        rc = (d->router_t == MOE_F32) ? launch_route_t<F32>(d, x, R, ids_out, wts_out, gate_out, w, s)
                                      : launch_route_t<BF16>(d, x, R, ids_out, wts_out, gate_out, w, s);
    }
    if (rc != MOE_OK)
        return rc;
    const int et = d->expert_t, st = d->shared_t;
    if (st == MOE_F32) {
        if (et == MOE_F32) return launch_experts_t<F32, F32>(d, x, R, y, w, s);
        if (et == MOE_BF16) return launch_experts_t<BF16, F32>(d, x, R, y, w, s);
        return launch_experts_t<Q2, F32>(d, x, R, y, w, s);
    }
    if (et == MOE_F32) return launch_experts_t<F32, BF16>(d, x, R, y, w, s);
    if (et == MOE_BF16) return launch_experts_t<BF16, BF16>(d, x, R, y, w, s);
    return launch_experts_t<Q2, BF16>(d, x, R, y, w, s);
}

}  // namespace moe
