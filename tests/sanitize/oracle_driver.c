/* Exercises the oracle's C code under AddressSanitizer and
 * UndefinedBehaviorSanitizer (host-side check, no GPU): every buffer is a
 * heap block of exactly the size the call needs, so a read or write past it
 * is reported. Returns nonzero on a failed check. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const uint8_t *codes;
    const uint16_t *scale;
    const uint16_t *minv;
} qmat;

typedef struct {
    int32_t hidden, n_experts, top_k, inter, shared_inter, renormalize;
    int32_t router_t, expert_t, shared_t;
    const void *router_w;
    const float *router_bias;
    const void *gate_vec;
    const void *const *exp_gate;
    const void *const *exp_up;
    const void *const *exp_down;
    const void *sh_gate;
    const void *sh_up;
    const void *sh_down;
    int32_t bias_mode;
    int32_t residual;
    const float *norm_w;
    double norm_eps;
} odesc;

float oracle_half_to_float(uint16_t h);
uint16_t oracle_float_to_half(float f);
int oracle_qb_quantize(int bits, const float *src, int64_t rows, int64_t cols, uint8_t *codes, uint16_t *scale,
                       uint16_t *minv);
void oracle_qb_dequantize(int bits, const uint8_t *codes, const uint16_t *scale, const uint16_t *minv, int64_t rows,
                          int64_t cols, float *dst);
int oracle_route(const odesc *d, const float *x, int64_t T, int32_t *ids, double *wts, double *gate, double *logits);
int oracle_layer(const odesc *d, const float *x, int64_t T, int32_t *ids, double *wts, double *gate, float *y,
                 double *y64);
void oracle_rmsnorm(const float *x, int64_t H, const float *gamma, double eps, float *u);

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) /* splitmix64 -> [0, 1) */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-53;
}
static float nrand(double std) { return (float)((urand() + urand() + urand() - 1.5) * 2.0 * std); }

static float *fmat(int64_t n, double std)
{
    float *a = malloc(sizeof(float) * n);
    for (int64_t i = 0; i < n; ++i)
        a[i] = nrand(std);
    return a;
}
static uint16_t *bmat(int64_t n, double std) /* bf16 patterns, truncated draws */
{
    uint16_t *a = malloc(sizeof(uint16_t) * n);
    for (int64_t i = 0; i < n; ++i) {
        float f = nrand(std);
        uint32_t u;
        memcpy(&u, &f, 4);
        a[i] = (uint16_t)(u >> 16);
    }
    return a;
}

/* One b-bit matrix in exact-size heap blocks. */
static qmat *qmake(int bits, const float *w, int64_t rows, int64_t cols)
{
    qmat *q = malloc(sizeof(qmat));
    uint8_t *c = malloc((size_t)(rows * cols * bits / 8));
    uint16_t *s = malloc(sizeof(uint16_t) * rows * cols / 32);
    uint16_t *m = malloc(sizeof(uint16_t) * rows * cols / 32);
    CHECK(oracle_qb_quantize(bits, w, rows, cols, c, s, m) == 0);
    q->codes = c;
    q->scale = s;
    q->minv = m;
    return q;
}
static void qfree(qmat *q)
{
    free((void *)q->codes);
    free((void *)q->scale);
    free((void *)q->minv);
    free(q);
}

static void test_fp16(void)
{
    for (uint32_t h = 0; h < 0x10000; ++h) {
        const float f = oracle_half_to_float((uint16_t)h);
        if (!isnan(f))
            CHECK(oracle_float_to_half(f) == (uint16_t)h);
    }
    CHECK(oracle_float_to_half(1e10f) == 0x7c00);
    CHECK(oracle_float_to_half(-1e-30f) == 0x8000);
}

static void test_quantizer(void)
{
    const int64_t rows = 5, cols = 96;
    for (int bits = 2; bits <= 4; ++bits) {
        float *w = fmat(rows * cols, 0.02);
        w[7] = 0.99999f;                                   /* uneven blocks */
        for (int j = 32; j < 64; ++j)
            w[j] = 0.0123f;                                /* a constant block */
        qmat *q = qmake(bits, w, rows, cols);
        float *out = malloc(sizeof(float) * rows * cols);
        oracle_qb_dequantize(bits, q->codes, q->scale, q->minv, rows, cols, out);
        for (int64_t i = 0; i < rows * cols; ++i)
            CHECK(isfinite(out[i]) && fabsf(out[i] - w[i]) < 0.5f);
        free(out);
        qfree(q);
        w[3] = NAN;
        uint8_t *c = malloc((size_t)(rows * cols * bits / 8));
        uint16_t *s = malloc(sizeof(uint16_t) * rows * cols / 32), *m = malloc(sizeof(uint16_t) * rows * cols / 32);
        CHECK(oracle_qb_quantize(bits, w, rows, cols, c, s, m) == -1);
        CHECK(oracle_qb_quantize(bits, w, rows, 48, c, s, m) == -1);
        free(c);
        free(s);
        free(m);
        free(w);
    }
}

/* A tiny layer in every expert format, with and without norm / residual /
 * bias, through route and layer. */
static void test_layer(int expert_t, int norm, int residual, int bias_mode, int renorm)
{
    const int H = 64, E = 8, K = 3, I = 32, Is = 32, T = 5;
    float *rw = fmat((int64_t)E * H, 0.1), *gv = fmat(H, 0.1), *bias = fmat(E, 0.5);
    float *sg = fmat((int64_t)Is * H, 0.05), *su = fmat((int64_t)Is * H, 0.05), *sd = fmat((int64_t)H * Is, 0.05);
    float *gamma = norm ? fmat(H, 0.3) : NULL;
    const void **eg = malloc(sizeof(void *) * E), **eu = malloc(sizeof(void *) * E), **ed = malloc(sizeof(void *) * E);
    void *own[3 * 8];
    for (int e = 0; e < E; ++e) {
        float *g = fmat((int64_t)I * H, 0.05), *u = fmat((int64_t)I * H, 0.05), *dn = fmat((int64_t)H * I, 0.05);
        if (expert_t == 0) {
            eg[e] = own[3 * e] = g;
            eu[e] = own[3 * e + 1] = u;
            ed[e] = own[3 * e + 2] = dn;
            continue;
        }
        if (expert_t == 1) {
            eg[e] = own[3 * e] = bmat((int64_t)I * H, 0.05);
            eu[e] = own[3 * e + 1] = bmat((int64_t)I * H, 0.05);
            ed[e] = own[3 * e + 2] = bmat((int64_t)H * I, 0.05);
        } else {
            eg[e] = own[3 * e] = qmake(expert_t, g, I, H);
            eu[e] = own[3 * e + 1] = qmake(expert_t, u, I, H);
            ed[e] = own[3 * e + 2] = qmake(expert_t, dn, H, I);
        }
        free(g);
        free(u);
        free(dn);
    }
    odesc d = {H, E, K, I, Is, renorm, 0, expert_t, 0, rw, bias_mode >= 0 ? bias : NULL, gv, eg, eu, ed,
               sg, su, sd, bias_mode >= 0 ? bias_mode : 0, residual, gamma, 1e-6};
    float *x = fmat((int64_t)T * H, 1.0), *y = malloc(sizeof(float) * T * H);
    int32_t *ids = malloc(sizeof(int32_t) * T * K);
    double *wts = malloc(sizeof(double) * T * K), *gate = malloc(sizeof(double) * T);
    double *y64 = malloc(sizeof(double) * T * H), *lg = malloc(sizeof(double) * T * E);
    CHECK(oracle_route(&d, x, T, ids, wts, gate, lg) == 0);
    CHECK(oracle_layer(&d, x, T, ids, wts, gate, y, y64) == 0);
    for (int i = 0; i < T * K; ++i)
        CHECK(ids[i] >= 0 && ids[i] < E && wts[i] > 0.0 && wts[i] <= 1.0);
    for (int i = 0; i < T * H; ++i)
        CHECK(isfinite(y64[i]) && y[i] == (float)y64[i]);
    odesc bad = d;
    bad.top_k = E + 1;
    CHECK(oracle_layer(&bad, x, T, ids, wts, gate, y, y64) == -1);
    bad = d;
    bad.expert_t = 5;
    CHECK(oracle_route(&bad, x, T, ids, wts, gate, NULL) == -1);
    if (gamma) {
        float *u = malloc(sizeof(float) * H);
        oracle_rmsnorm(x, H, gamma, 1e-6, u);
        free(u);
    }
    for (int e = 0; e < E; ++e)
        for (int m = 0; m < 3; ++m) {
            if (expert_t >= 2)
                qfree(own[3 * e + m]);
            else
                free(own[3 * e + m]);
        }
    free(eg);
    free(eu);
    free(ed);
    free(rw);
    free(gv);
    free(bias);
    free(sg);
    free(su);
    free(sd);
    free(gamma);
    free(x);
    free(y);
    free(ids);
    free(wts);
    free(gate);
    free(y64);
    free(lg);
}

int main(void)
{
    test_fp16();
    test_quantizer();
    for (int et = 0; et <= 4; ++et)
        test_layer(et, et & 1, et >= 2, et == 3 ? 1 : (et == 4 ? 0 : -1), et != 2);
    test_layer(2, 1, 1, 1, 1);
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("oracle driver: all checks passed\n");
    return failures ? 1 : 0;
}
