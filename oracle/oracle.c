/*
 * oracle.c - plain CPU oracle of one sparse Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library or its Python binding may
 * link, load or call this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code with the GPU path.
 *
 * What it computes (per token, everything accumulated in double):
 *   - the Qwen3-Next MoE layer shape from the Red Lite "Architecture" page,
 *     section "Qwen3-Next shape": routed experts, a top-k selection per token,
 *     one shared expert;
 *   - router, top-k and shared gate as the single routing step described in
 *     "Research notes, October 2026", section 1 (DwarfStar today, "Metal"):
 *     logits l_e = W_r[e] . x (+ b_e), selection of the K largest, softmax
 *     weights over the selection (renormalized), shared gate sigmoid(w_g . x);
 *   - SwiGLU experts: h = silu(G x) * (U x), d = D h; the combine
 *     y = sum_k w_k d_(ids[k]) + g * d_shared (the "weighted reduce" of the
 *     same page, section 4, "Techniques with evidence");
 *   - precision: a double-precision implementation of the same computation,
 *     as the "guide" page, section "Correctness", describes its kernel gate.
 *   - selection order: logit descending, then expert id ascending. The
 *     "Red Lite dev18" page, section "Scope boundary", reports an exact router
 *     tie that two implementations broke differently; this oracle fixes the
 *     rule (lower id first) so the result is unique.
 *   - a per-expert router bias b_e: either added to the logits for both the
 *     selection and the softmax weights (bias_mode 0), or used for the
 *     selection only, the weights coming from the unbiased logits
 *     (bias_mode 1: the opt-in cache-aware routing z + lambda * Delta *
 *     cached of "Research notes, October 2026", section 4, where the bias
 *     steers which experts are chosen);
 *   - optionally (multi-layer stacks) the layer's input x is first
 *     RMS-normalized and scaled, u = x / sqrt(mean(x^2) + eps) * gamma (the
 *     RMS_NORM+SCALE that precedes the MoE block, fused there per the MoE
 *     fusions row of the same page, section 4), u stored as fp32 like every
 *     activation of the layer, and the output carries the residual,
 *     y = x + MoE(u).
 *
 * Weight widening is exact: fp32 and bf16 values convert to double without
 * rounding; the 2-bit block format is decoded to fp32 first (its own
 * definition) and then widened.
 *
 * b-bit block formats, b = 2, 3, 4 (logical form used only inside this
 * oracle; the 3- and 4-bit variants are the higher-precision expert files of
 * the same model, "DwarfStar Red Lite" guide, IQ3_XXS, with the weight type a
 * function constant of the kernels, "Research notes, October 2026", section
 * 1, "Metal"):
 *   32 consecutive weights of a row (along the reduction dimension) form a
 *   block with 4b bytes of codes (weight j at bits b*j .. b*j+b-1 of the
 *   block's bytes read as one little-endian integer), an fp16 scale and an
 *   fp16 minimum; w = fp32(code * scale + min), code in 0 .. 2^b - 1. The
 *   quantizer below is written from that definition with IEEE binary32
 *   arithmetic, round-to-nearest-even.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_Q2 = 2, OR_Q3 = 3, OR_Q4 = 4 };

typedef struct {
    const uint8_t *codes;   /* [rows][cols*b/8] */
    const uint16_t *scale;  /* [rows][cols/32] fp16 bit patterns */
    const uint16_t *minv;   /* [rows][cols/32] fp16 bit patterns */
} oracle_q2_matrix;         /* a b-bit matrix; b from the layer's expert type */

typedef struct {
    int32_t hidden, n_experts, top_k, inter, shared_inter, renormalize;
    int32_t router_t, expert_t, shared_t;
    const void *router_w;        /* [E][H], router_t */
    const float *router_bias;    /* [E] or NULL */
    const void *gate_vec;        /* [H], router_t */
    const void *const *exp_gate; /* E entries: [I][H] (f32/bf16) or oracle_q2_matrix* (b-bit) */
    const void *const *exp_up;   /* E entries: [I][H] */
    const void *const *exp_down; /* E entries: [H][I] */
    const void *sh_gate;         /* [Is][H], shared_t */
    const void *sh_up;           /* [Is][H] */
    const void *sh_down;         /* [H][Is] */
    int32_t bias_mode;           /* 0: bias in selection and weights; 1: selection only */
    int32_t residual;            /* 1: y = x + MoE(u) */
    const float *norm_w;         /* [H] gamma, or NULL: u = x (no norm) */
    double norm_eps;
} oracle_desc;

/* ---------------------------------------------------------------- fp16 */

/* fp16 bit pattern -> float, from the IEEE 754 binary16 definition. */
float oracle_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* zero / subnormal */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp(1.0 + man / 1024.0, ex - 15);
    return (float)(sign ? -v : v);
}

/* float -> fp16 bit pattern, round to nearest, ties to even.
 * Works on the exact double value; every scaling below is by a power of two
 * and nearbyint() rounds ties to even in the default rounding mode. */
uint16_t oracle_float_to_half(float f)
{
    if (isnan(f))
        return 0x7e00;
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (a >= 65520.0)                                /* rounds past 65504 */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {                       /* subnormal range */
        double q = nearbyint(ldexp(a, 24));          /* units of 2^-24 */
        return sign | (uint16_t)q;                   /* q == 1024 is 2^-14 */
    }
    int e2;
    frexp(a, &e2);                                   /* a = fr * 2^e2, fr in [0.5,1) */
    int E = e2 - 1;                                  /* a in [2^E, 2^(E+1)) */
    double m = nearbyint((ldexp(a, -E) - 1.0) * 1024.0);
    if (m == 1024.0) {
        m = 0.0;
        E += 1;
    }
    if (E + 15 >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | (int)m);
}

/* ------------------------------------------------------ b-bit blocks */

/* Code j of a block (4b bytes, weight j at bits b*j..b*j+b-1). */
static int block_code(const uint8_t *cb, int bits, int j)
{
    int c = 0;
    for (int i = 0; i < bits; ++i) {
        const int bit = bits * j + i;
        c |= ((cb[bit / 8] >> (bit % 8)) & 1) << i;
    }
    return c;
}

static void set_block_code(uint8_t *cb, int bits, int j, int c)
{
    for (int i = 0; i < bits; ++i) {
        const int bit = bits * j + i;
        cb[bit / 8] |= (uint8_t)(((c >> i) & 1) << (bit % 8));
    }
}

/* Quantize one row-major fp32 matrix [rows][cols] (cols % 32 == 0) into the
 * logical b-bit block form (bits 2, 3 or 4). Returns 0, or -1 if a value is
 * not finite or a block's min or scale does not fit fp16. */
int oracle_qb_quantize(int bits, const float *src, int64_t rows, int64_t cols,
                       uint8_t *codes, uint16_t *scale, uint16_t *minv)
{
    if (cols % 32 != 0 || bits < 2 || bits > 4)
        return -1;
    const int top = (1 << bits) - 1;
    const float levels = (float)top;
    const int64_t nb = cols / 32, cbytes = 4 * bits;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *w = src + r * cols + b * 32;
            float lo = w[0], hi = w[0];
            for (int j = 0; j < 32; ++j) {
                if (!isfinite(w[j]))
                    return -1;
                if (w[j] < lo) lo = w[j];
                if (w[j] > hi) hi = w[j];
            }
            uint16_t mh = oracle_float_to_half(lo);
            float mf = oracle_half_to_float(mh);
            float range = hi - mf;                   /* binary32 subtract */
            float step = range / levels;             /* binary32 divide */
            uint16_t sh = oracle_float_to_half(step);
            float sf = oracle_half_to_float(sh);
            if (!isfinite(mf) || !isfinite(sf))
                return -1;
            uint8_t *cb = codes + r * (cols / 32) * cbytes + b * cbytes;
            memset(cb, 0, (size_t)cbytes);
            for (int j = 0; j < 32; ++j) {
                int c = 0;
                if (sf != 0.0f) {
                    float diff = w[j] - mf;
                    float q = diff / sf;
                    float n = nearbyintf(q);
                    c = n < 0.0f ? 0 : (n > levels ? top : (int)n);
                }
                set_block_code(cb, bits, j, c);
            }
            scale[r * nb + b] = sh;
            minv[r * nb + b] = mh;
        }
    }
    return 0;
}

/* Decode the logical block form back to fp32: w = code * scale + min. */
void oracle_qb_dequantize(int bits, const uint8_t *codes, const uint16_t *scale, const uint16_t *minv,
                          int64_t rows, int64_t cols, float *dst)
{
    const int64_t nb = cols / 32, cbytes = 4 * bits;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            float sf = oracle_half_to_float(scale[r * nb + b]);
            float mf = oracle_half_to_float(minv[r * nb + b]);
            const uint8_t *cb = codes + r * nb * cbytes + b * cbytes;
            for (int j = 0; j < 32; ++j) {
                int c = block_code(cb, bits, j);
                float prod = (float)c * sf;          /* exact: <= 15 significant bits */
                dst[r * cols + b * 32 + j] = prod + mf;  /* one rounding */
            }
        }
    }
}

/* The 2-bit instances. */
int oracle_q2_quantize(const float *src, int64_t rows, int64_t cols,
                       uint8_t *codes, uint16_t *scale, uint16_t *minv)
{
    return oracle_qb_quantize(2, src, rows, cols, codes, scale, minv);
}

void oracle_q2_dequantize(const uint8_t *codes, const uint16_t *scale, const uint16_t *minv,
                          int64_t rows, int64_t cols, float *dst)
{
    oracle_qb_dequantize(2, codes, scale, minv, rows, cols, dst);
}

/* ------------------------------------------------------------ widening */

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Row r (length cols) of a matrix of type t, widened exactly to double. */
static void row_to_double(const void *m, int32_t t, int64_t r, int64_t cols, double *out)
{
    if (t == OR_F32) {
        const float *p = (const float *)m + r * cols;
        for (int64_t c = 0; c < cols; ++c)
            out[c] = (double)p[c];
    } else if (t == OR_BF16) {
        const uint16_t *p = (const uint16_t *)m + r * cols;
        for (int64_t c = 0; c < cols; ++c)
            out[c] = bf16_to_double(p[c]);
    } else {
        const int bits = t == OR_Q2 ? 2 : (t == OR_Q3 ? 3 : 4);
        const oracle_q2_matrix *q = (const oracle_q2_matrix *)m;
        float tmp[32];
        for (int64_t b = 0; b < cols / 32; ++b) {
            oracle_qb_dequantize(bits, q->codes + r * (cols / 32) * 4 * bits + b * 4 * bits,
                                 q->scale + r * (cols / 32) + b,
                                 q->minv + r * (cols / 32) + b, 1, 32, tmp);
            for (int j = 0; j < 32; ++j)
                out[b * 32 + j] = (double)tmp[j];
        }
    }
}

static double dot(const double *a, const double *b, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += a[i] * b[i];
    return s;
}

/* ------------------------------------------------------------- routing */

typedef struct {
    double l;   /* selection logit (with the bias) */
    double w;   /* weight logit (with the bias in bias_mode 0, without it in bias_mode 1) */
    int32_t e;
} scored;

/* Order: larger logit first; equal logits, lower expert id first. */
static int by_logit_then_id(const void *pa, const void *pb)
{
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->l > b->l) return -1;
    if (a->l < b->l) return 1;
    return (a->e > b->e) - (a->e < b->e);
}

/* Route one token. logits[E] receives the selection logits l_e + b_e. */
static void route_one(const oracle_desc *d, const double *x, double *logits,
                      int32_t *ids, double *wts, double *gate, double *rowbuf, scored *sc)
{
    const int64_t H = d->hidden, E = d->n_experts, K = d->top_k;
    for (int64_t e = 0; e < E; ++e) {
        row_to_double(d->router_w, d->router_t, e, H, rowbuf);
        double l = dot(rowbuf, x, H);
        double b = d->router_bias ? (double)d->router_bias[e] : 0.0;
        logits[e] = l + b;
        sc[e].l = l + b;
        sc[e].w = d->bias_mode == 1 ? l : l + b;
        sc[e].e = (int32_t)e;
    }
    /* Brute force: a full sort of all experts by the selection order. */
    qsort(sc, (size_t)E, sizeof(scored), by_logit_then_id);
    for (int64_t k = 0; k < K; ++k)
        ids[k] = sc[k].e;
    /* Softmax of the weight logits over the selected experts (renormalized)
       or over all E, taken at the selected ones; m is the largest weight
       logit of the set summed over. */
    const int64_t n = d->renormalize ? K : E;
    double m = sc[0].w;
    for (int64_t i = 1; i < n; ++i)
        if (sc[i].w > m)
            m = sc[i].w;
    double denom = 0.0;
    for (int64_t i = 0; i < n; ++i)
        denom += exp(sc[i].w - m);
    for (int64_t k = 0; k < K; ++k)
        wts[k] = exp(sc[k].w - m) / denom;
    row_to_double(d->gate_vec, d->router_t, 0, H, rowbuf);
    double z = dot(rowbuf, x, H);
    *gate = 1.0 / (1.0 + exp(-z));
}

/*
 * RMS norm and scale of one row: u_h = fp32(x_h * r * gamma_h) with
 * r = 1 / sqrt(sum_h x_h^2 / H + eps), everything in double until u is
 * stored as fp32 (the layer's activation format).
 */
void oracle_rmsnorm(const float *x, int64_t H, const float *gamma, double eps, float *u)
{
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h)
        ss += (double)x[h] * (double)x[h];
    const double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int64_t h = 0; h < H; ++h)
        u[h] = (float)((double)x[h] * r * (double)gamma[h]);
}

/* The layer input of row t as double: x, or its RMS norm when the layer has one. */
static void input_row(const oracle_desc *d, const float *x, int64_t t, float *ubuf, double *xd)
{
    const int64_t H = d->hidden;
    const float *xr = x + t * H;
    if (d->norm_w) {
        oracle_rmsnorm(xr, H, d->norm_w, d->norm_eps, ubuf);
        xr = ubuf;
    }
    for (int64_t h = 0; h < H; ++h)
        xd[h] = (double)xr[h];
}

/* --------------------------------------------------------- expert FFN */

/* d_out[H] = D * (silu(G x) * (U x)) for one expert of intermediate size n. */
static void swiglu_ffn(const void *G, const void *U, const void *D, int32_t t,
                       int64_t H, int64_t n, const double *x, double *d_out,
                       double *rowbuf, double *h)
{
    for (int64_t i = 0; i < n; ++i) {
        row_to_double(G, t, i, H, rowbuf);
        double a = dot(rowbuf, x, H);
        row_to_double(U, t, i, H, rowbuf);
        double c = dot(rowbuf, x, H);
        double silu = a / (1.0 + exp(-a));
        h[i] = silu * c;
    }
    for (int64_t j = 0; j < H; ++j) {
        row_to_double(D, t, j, n, rowbuf);
        d_out[j] = dot(rowbuf, h, n);
    }
}

static int check_desc(const oracle_desc *d)
{
    if (!d || d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->top_k > d->n_experts ||
        d->inter <= 0 || d->shared_inter <= 0 || !d->router_w || !d->gate_vec)
        return -1;
    if (d->router_t != OR_F32 && d->router_t != OR_BF16)
        return -1;
    if (d->shared_t != OR_F32 && d->shared_t != OR_BF16)
        return -1;
    if (d->expert_t < OR_F32 || d->expert_t > OR_Q4)
        return -1;
    if (d->expert_t >= OR_Q2 && (d->hidden % 32 || d->inter % 32))
        return -1;
    if (d->bias_mode != 0 && d->bias_mode != 1)
        return -1;
    if (d->residual != 0 && d->residual != 1)
        return -1;
    if (d->norm_w && !(d->norm_eps >= 0.0))
        return -1;
    return 0;
}

/*
 * Route only: ids[T][K], wts[T][K], gate[T], logits[T][E] (logits may be NULL).
 */
int oracle_route(const oracle_desc *d, const float *x, int64_t T,
                 int32_t *ids, double *wts, double *gate, double *logits)
{
    if (check_desc(d))
        return -1;
    const int64_t H = d->hidden, E = d->n_experts, K = d->top_k;
    int rc = 0;
#pragma omp parallel
    {
        double *xd = malloc(sizeof(double) * H);
        double *rowbuf = malloc(sizeof(double) * H);
        double *lg = malloc(sizeof(double) * E);
        scored *sc = malloc(sizeof(scored) * E);
        float *ubuf = malloc(sizeof(float) * H);
        if (!xd || !rowbuf || !lg || !sc || !ubuf) {
#pragma omp atomic write
            rc = -2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                input_row(d, x, t, ubuf, xd);
                route_one(d, xd, lg, ids + t * K, wts + t * K, gate + t, rowbuf, sc);
                if (logits)
                    memcpy(logits + t * E, lg, sizeof(double) * E);
            }
        }
        free(xd);
        free(rowbuf);
        free(lg);
        free(sc);
        free(ubuf);
    }
    return rc;
}

/*
 * Whole layer for T tokens (each token independently; with a norm, on the
 * normalized input; with the residual, x is added to the output):
 *   ids[T][K] int32, wts[T][K] double, gate[T] double,
 *   y[T][H] float (the double result rounded once), y64[T][H] double or NULL.
 * Tokens are spread over OpenMP threads (set by the caller); every token is
 * computed by the same sequential code, so the result does not depend on the
 * thread count.
 */
int oracle_layer(const oracle_desc *d, const float *x, int64_t T,
                 int32_t *ids, double *wts, double *gate, float *y, double *y64)
{
    if (check_desc(d))
        return -1;
    const int64_t H = d->hidden, E = d->n_experts, K = d->top_k;
    const int64_t I = d->inter, Is = d->shared_inter;
    const int64_t nmax = (I > Is ? I : Is);
    const int64_t rowmax = (H > nmax ? H : nmax);
    int rc = 0;
#pragma omp parallel
    {
        double *xd = malloc(sizeof(double) * H);
        double *rowbuf = malloc(sizeof(double) * rowmax);
        double *lg = malloc(sizeof(double) * E);
        scored *sc = malloc(sizeof(scored) * E);
        double *h = malloc(sizeof(double) * (nmax > 0 ? nmax : 1));
        double *dv = malloc(sizeof(double) * H);
        double *acc = malloc(sizeof(double) * H);
        float *ubuf = malloc(sizeof(float) * H);
        if (!xd || !rowbuf || !lg || !sc || !h || !dv || !acc || !ubuf) {
#pragma omp atomic write
            rc = -2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                input_row(d, x, t, ubuf, xd);
                int32_t *tid = ids + t * K;
                double *tw = wts + t * K;
                route_one(d, xd, lg, tid, tw, gate + t, rowbuf, sc);
                for (int64_t j = 0; j < H; ++j)
                    acc[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    int32_t e = tid[k];
                    if (!d->exp_gate[e] || !d->exp_up[e] || !d->exp_down[e]) {
#pragma omp atomic write
                        rc = -3;                     /* selected expert not supplied */
                        continue;
                    }
                    swiglu_ffn(d->exp_gate[e], d->exp_up[e], d->exp_down[e], d->expert_t,
                               H, I, xd, dv, rowbuf, h);
                    for (int64_t j = 0; j < H; ++j)
                        acc[j] += tw[k] * dv[j];
                }
                swiglu_ffn(d->sh_gate, d->sh_up, d->sh_down, d->shared_t, H, Is, xd, dv, rowbuf, h);
                for (int64_t j = 0; j < H; ++j)
                    acc[j] += gate[t] * dv[j];
                if (d->residual)   /* the residual stream: the un-normalized input */
                    for (int64_t j = 0; j < H; ++j)
                        acc[j] += (double)x[t * H + j];
                for (int64_t j = 0; j < H; ++j) {
                    y[t * H + j] = (float)acc[j];
                    if (y64)
                        y64[t * H + j] = acc[j];
                }
            }
        }
        free(xd);
        free(rowbuf);
        free(lg);
        free(sc);
        free(h);
        free(dv);
        free(acc);
        free(ubuf);
    }
    return rc;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
