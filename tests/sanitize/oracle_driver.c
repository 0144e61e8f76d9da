/*
 * Memory and undefined-behaviour exercise of the CPU oracle (test
 * infrastructure), built with AddressSanitizer and UBSan by
 * tests/test_sanitizers.py.  It runs every oracle entry on small seeded
 * inputs -- both formats, every tail, routing with ties and a splitting cap,
 * the routed half with and without seed, the sandwich tail -- and checks only
 * status codes: the results themselves are pinned elsewhere.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return st;
}
static double unif(void) { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
static uint16_t bf16(double v) { return or_bf16_round(v); }

/* One n x k matrix (E stacked) of format fmt, heap-allocated. */
static or_qmat make(int fmt, int n, int k, int E)
{
    or_qmat w;
    w.fmt = fmt;
    w.n = n;
    w.k = k;
    if (fmt == OR_FMT_INT8_ROW) {
        int8_t* q = malloc((size_t)E * n * k);
        float* s = malloc(sizeof(float) * (size_t)E * n);
        for (size_t i = 0; i < (size_t)E * n * k; ++i) q[i] = (int8_t)((int)(next() % 255) - 127);
        for (size_t i = 0; i < (size_t)E * n; ++i) s[i] = (float)((0.5 + unif()) / (127.0 * sqrt((double)k)));
        w.q = q;
        w.s = s;
        w.z = NULL;
    } else {
        uint8_t* q = malloc((size_t)E * n * k / 2);
        uint16_t* s = malloc(2 * (size_t)E * n * (k / 64));
        uint16_t* z = malloc(2 * (size_t)E * n * (k / 64));
        for (size_t i = 0; i < (size_t)E * n * k / 2; ++i) q[i] = (uint8_t)next();
        for (size_t i = 0; i < (size_t)E * n * (k / 64); ++i) {
            s[i] = bf16((0.5 + unif()) / (8.0 * sqrt((double)k)));
            z[i] = bf16(6.0 + 3.0 * unif());
        }
        w.q = q;
        w.s = s;
        w.z = z;
    }
    return w;
}

static void drop(or_qmat* w)
{
    free((void*)w->q);
    free((void*)w->s);
    free((void*)w->z);
}

static uint16_t* rows(int m, int n)
{
    uint16_t* r = malloc(2 * (size_t)m * n);
    for (size_t i = 0; i < (size_t)m * n; ++i) r[i] = bf16(2.0 * unif() - 1.0);
    return r;
}

#define CHECK(c)                                                     \
    do {                                                             \
        if (!(c)) {                                                  \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            return 1;                                                \
        }                                                            \
    } while (0)

int main(void)
{
    const int hidden = 128, inter = 192, m = 5;
    for (int fmt = OR_FMT_INT8_ROW; fmt <= OR_FMT_INT4_AFFINE_G64; ++fmt) {
        or_qmat g = make(fmt, inter, hidden, 1), u = make(fmt, inter, hidden, 1), d = make(fmt, hidden, inter, 1);
        uint16_t* x = rows(m, hidden);
        uint16_t* out = rows(m, hidden);
        uint16_t* nw = rows(1, hidden);
        float* dq = malloc(sizeof(float) * inter * hidden);
        or_dequant_matrix(&g, dq);
        double* xv = malloc(sizeof(double) * hidden);
        float* y = malloc(sizeof(float) * inter);
        for (int i = 0; i < hidden; ++i) xv[i] = or_bf16_value(x[i]);
        or_gemv(&g, xv, y);
        for (int act = OR_ACT_SILU; act <= OR_ACT_GELU_TANH; ++act) {
            CHECK(or_dense(&g, &u, &d, hidden, inter, m, act, OR_TAIL_RESIDUAL, x, out, NULL, 1e-6f) == OR_OK);
            CHECK(or_dense(&g, &u, &d, hidden, inter, m, act, OR_TAIL_RMSNORM, x, out, nw, 1e-6f) == OR_OK);
            for (int tail = OR_TAIL_NONE; tail <= OR_TAIL_SIGMOID_GATE; ++tail) {
                if (tail == OR_TAIL_RESIDUAL) continue;
                CHECK(or_shared_expert(&g, &u, &d, hidden, inter, m, act, tail, x, out, nw, 1e-6f) == OR_OK);
            }
        }
        CHECK(or_dense(&g, &u, &d, hidden + 64, inter, m, OR_ACT_SILU, OR_TAIL_RESIDUAL, x, out, NULL, 0.f) ==
              OR_ERR_INVALID);
        free(dq);
        free(xv);
        free(y);
        free(x);
        free(out);
        free(nw);
        drop(&g);
        drop(&u);
        drop(&d);
    }

    /* routing: random logits, ties, a NaN, a splitting cap; then the routed half */
    const int E = 9, k = 3, mr = 7;
    float* logits = malloc(sizeof(float) * mr * E);
    float* scale = malloc(sizeof(float) * E);
    for (int i = 0; i < mr * E; ++i) logits[i] = (float)(unif() * 4.0 - 2.0);
    logits[3] = logits[4];
    logits[E + 2] = NAN;
    for (int e = 0; e < E; ++e) scale[e] = (float)(0.5 + unif());
    int32_t* ids = malloc(sizeof(int32_t) * mr * k);
    float* w = malloc(sizeof(float) * mr * k);
    int32_t* plan = malloc(sizeof(int32_t) * OR_PLAN_INTS(mr, k));
    for (int cap = k; cap <= 12; cap += 3) {
        CHECK(or_moe_route(logits, scale, mr, E, k, cap, ids, w, plan) == OR_OK);
        CHECK(or_moe_route(logits, NULL, mr, E, k, cap, ids, w, plan) == OR_OK);
    }
    CHECK(or_moe_route(logits, NULL, mr, E, k, k - 1, ids, w, plan) == OR_ERR_CAPACITY);
    CHECK(or_moe_route(logits, NULL, mr, E, k, 33, ids, w, plan) == OR_ERR_UNSUPPORTED);
    or_qmat eg = make(OR_FMT_INT4_AFFINE_G64, inter, hidden, E), eu = make(OR_FMT_INT4_AFFINE_G64, inter, hidden, E);
    or_qmat ed = make(OR_FMT_INT4_AFFINE_G64, hidden, inter, E);
    uint16_t* x = rows(mr, hidden);
    uint16_t* seed = rows(mr, hidden);
    uint16_t* resid = rows(mr, hidden);
    CHECK(or_moe_routed(&eg, &eu, &ed, E, hidden, inter, mr, k, OR_ACT_SILU, x, ids, w, seed, resid) == OR_OK);
    ids[1] = -1;
    ids[4] = E;   /* out-of-range ids add nothing */
    CHECK(or_moe_routed(&eg, &eu, &ed, E, hidden, inter, mr, k, OR_ACT_GELU_TANH, x, ids, w, NULL, resid) == OR_OK);
    uint16_t* h1 = rows(mr, hidden);
    uint16_t* r = rows(mr, hidden);
    uint16_t* pw = rows(1, hidden);
    or_sandwich_tail(h1, r, pw, mr, hidden, 1e-6f, resid);
    float dd[3] = {1.f, 2.f, 3.f}, ww[3] = {0.5f, 0.25f, 0.25f};
    (void)or_seeded_sum(1.0f, ww, dd, 3);
    float* lg2 = malloc(sizeof(float) * mr * E);
    uint16_t* rw = rows(E, hidden);
    or_router_logits(x, rw, mr, hidden, E, lg2);
    free(lg2);
    free(rw);
    free(h1);
    free(r);
    free(pw);
    free(x);
    free(seed);
    free(resid);
    drop(&eg);
    drop(&eu);
    drop(&ed);
    free(logits);
    free(scale);
    free(ids);
    free(w);
    free(plan);
    printf("oracle sanitizer run: ok\n");
    return 0;
}
