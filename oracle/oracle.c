/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  The plain, slow, single-threaded CPU
 * definition of what libffnq computes, used to check the HIP path.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it; the product never does.  It shares no code, header, table or constant
 * generator with the HIP path.
 *
 * Source of the method (docs.rs pages of the `turbospark-runtime` crate):
 *   [llama/dense.rs]           module doc: m = rms_norm(x) (caller), h = down(act(gate@m, up@m)), x = x + h;
 *                              `encode_llama_layer_dense`: gate/up GEMVs, silu/gelu-mul, down GEMV, residual add
 *   [gemma4/shared_expert.rs]  `encode_shared_expert_branch(_batched)`: the same FFN with an in-place
 *                              RMSNorm tail (RMS_EPS = 1e-6, bf16 weight)
 *   [qwen/moe_batch.rs]        module doc and `encode_qwen_layer_moe_batched`: router top-k with
 *                              renormalised weights, union-bounded sub-batches, pair order, phase 1,
 *                              phase 2 seeded with the sigmoid-gated shared expert, raw residual add;
 *                              module doc, first bullet: the Gemma-style variant (routed sum from
 *                              zero, the normed shared branch joining in a sandwich tail)
 *
 * Precision: the pages fix none beyond 2-byte activation buffers, an fp32
 * router and an fp32 phase-2 accumulator.  The oracle therefore works in
 * double and rounds exactly where the library's contract stores a value:
 * weights are dequantised to fp32, dot products are accumulated in double
 * (increasing k) and rounded once to fp32, the fp32 intermediates g, u, act,
 * h, d, the gate logit and the route weights are rounded to fp32, and ABI
 * outputs are rounded once to bf16 (nearest, ties to even).  The phase-2
 * accumulator is an fp32 accumulator (seed first, then the ranks in order,
 * product and sum each rounded to fp32) because the pages make that order
 * part of the function.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no FMA contraction, IEEE double).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ---- bf16 ----------------------------------------------------------------- */

/* The real value of a bf16 bit pattern: the upper half of a binary32. */
double or_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a real (held exactly in a double) to the nearest bf16, ties to even.
 * bf16 has 8 significant bits, normal exponents -126..127 and subnormals
 * with spacing 2^-133.  The rounding is done on the double directly (one
 * rounding), by scaling to the bf16 grid spacing of v's binade. */
uint16_t or_bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                 /* a = f * 2^e2, f in [0.5, 1): leading bit 2^(e2-1) */
    int lead = e2 - 1;
    if (lead < -126) lead = -126;  /* subnormal range: fixed spacing */
    double spacing = ldexp(1.0, lead - 7);
    double r = rint(a / spacing) * spacing;   /* rint: round half to even */
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds past it is inf */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r;           /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* ---- O1: dequantisation ------------------------------------------------------
 * INT8 per-row: w = s[n] * q[n][k] ([gemma4/shared_expert.rs]: "INT8 gate/up").
 * INT4 affine, groups of 64 along k: w = s[n][g] * (code - z[n][g]) with the
 * code of input k in the low nibble of byte k/2 when k is even, the high
 * nibble when odd ([qwen/moe_batch.rs]: the Affine routed layout).  code - z
 * is exact in fp32; the product is rounded once to fp32. */
float or_dequant(const or_qmat* w, int row, int col)
{
    if (w->fmt == OR_FMT_INT8_ROW) {
        const int8_t* q = (const int8_t*)w->q;
        const float* s = (const float*)w->s;
        float qv = (float)q[(size_t)row * w->k + col];
        return s[row] * qv;
    }
    const uint8_t* q = (const uint8_t*)w->q;
    const uint16_t* s = (const uint16_t*)w->s;
    const uint16_t* z = (const uint16_t*)w->z;
    uint8_t byte = q[(size_t)row * (w->k / 2) + col / 2];
    int code = (col & 1) ? (byte >> 4) : (byte & 0x0F);
    size_t g = (size_t)row * (w->k / 64) + col / 64;
    float sc = (float)or_bf16_value(s[g]);
    float zp = (float)or_bf16_value(z[g]);
    float diff = (float)code - zp;
    return sc * diff;
}

void or_dequant_matrix(const or_qmat* w, float* out)
{
    for (int n = 0; n < w->n; ++n)
        for (int k = 0; k < w->k; ++k) out[(size_t)n * w->k + k] = or_dequant(w, n, k);
}

/* Matrix e of a stacked [E][...] expert tensor. */
or_qmat or_expert(const or_qmat* w, int e)
{
    or_qmat r = *w;
    size_t n = (size_t)w->n, k = (size_t)w->k;
    if (w->fmt == OR_FMT_INT8_ROW) {
        r.q = (const int8_t*)w->q + (size_t)e * n * k;
        r.s = (const float*)w->s + (size_t)e * n;
    } else {
        r.q = (const uint8_t*)w->q + (size_t)e * n * (k / 2);
        r.s = (const uint16_t*)w->s + (size_t)e * n * (k / 64);
        r.z = (const uint16_t*)w->z + (size_t)e * n * (k / 64);
    }
    return r;
}

/* ---- O2: y = W x ---------------------------------------------------------------
 * y[n] = sum_k w[n][k] * x[k], accumulated in double in increasing k and
 * rounded once to fp32 (the GEMV of `encode_gemv_any` / `encode_gemm_any`). */
void or_gemv(const or_qmat* w, const double* x, float* y)
{
    for (int n = 0; n < w->n; ++n) {
        double acc = 0.0;
        for (int k = 0; k < w->k; ++k) acc += (double)or_dequant(w, n, k) * x[k];
        y[n] = (float)acc;
    }
}

/* ---- O3: gated activation ---------------------------------------------------------
 * act = f(gate) * up, gate first ([llama/dense.rs]: `encode_silu_mul(ffn_gate,
 * ffn_up, ffn_act)`); SiLU or the tanh form of GELU, in double, rounded to fp32. */
double or_silu(double v) { return v / (1.0 + exp(-v)); }

double or_gelu_tanh(double v)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

float or_act(int act, float g, float u)
{
    double f = (act == OR_ACT_SILU) ? or_silu((double)g) : or_gelu_tanh((double)g);
    return (float)(f * (double)u);
}

/* One token through gate/up/act/down: h[hidden] (fp32). */
static void ffn_token(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int act,
                      const uint16_t* x_bf16, float* h)
{
    int hidden = gate->k, inter = gate->n;
    double* x = (double*)malloc(sizeof(double) * (size_t)hidden);
    float* g = (float*)malloc(sizeof(float) * (size_t)inter);
    float* u = (float*)malloc(sizeof(float) * (size_t)inter);
    double* a = (double*)malloc(sizeof(double) * (size_t)inter);
    for (int i = 0; i < hidden; ++i) x[i] = or_bf16_value(x_bf16[i]);
    or_gemv(gate, x, g);
    or_gemv(up, x, u);
    for (int i = 0; i < inter; ++i) a[i] = (double)or_act(act, g[i], u[i]);
    or_gemv(down, a, h);
    free(x); free(g); free(u); free(a);
}

/* ---- O4: tails ----------------------------------------------------------------------- */

/* Raw residual add, x <- x + h ([llama/dense.rs] `encode_residual_add`). */
uint16_t or_residual(uint16_t x, float h) { return or_bf16_round(or_bf16_value(x) + (double)h); }

/* RMSNorm with a bf16 weight: out = h / sqrt(mean(h^2) + eps) * w
 * ([gemma4/shared_expert.rs] `encode_rms_norm_bf16w(h1, post_ffn1, h1, hidden, RMS_EPS)`). */
void or_rmsnorm_row(const float* h, const uint16_t* w, int n, float eps, uint16_t* out)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += (double)h[i] * (double)h[i];
    double r = 1.0 / sqrt(ss / (double)n + (double)eps);
    for (int i = 0; i < n; ++i) out[i] = or_bf16_round((double)h[i] * r * or_bf16_value(w[i]));
}

/* Shared-expert gate logit: a one-row GEMV <w_gate, x> over hidden, fp32
 * ([qwen/moe_batch.rs]: `mlp.shared_expert_gate.weight` with rows = 1). */
float or_gate_logit(const uint16_t* wg, const uint16_t* x, int n)
{
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += or_bf16_value(wg[i]) * or_bf16_value(x[i]);
    return (float)acc;
}

/* Router logits ([qwen/moe_batch.rs] `encode_qwen_layer_moe_batched`: the M
 * router GEMVs run before the routed half, which reads their fp32 logits
 * back): logits[t][e] = <w_e, x_t> over hidden, each in double, rounded once
 * to fp32.  x bf16 [m][hidden], w bf16 [n_experts][hidden]. */
void or_router_logits(const uint16_t* x, const uint16_t* w, int m, int hidden, int n_experts, float* logits)
{
    for (int t = 0; t < m; ++t)
        for (int e = 0; e < n_experts; ++e) {
            double acc = 0.0;
            for (int i = 0; i < hidden; ++i)
                acc += or_bf16_value(w[(size_t)e * hidden + i]) * or_bf16_value(x[(size_t)t * hidden + i]);
            logits[(size_t)t * n_experts + e] = (float)acc;
        }
}

/* h * sigmoid(logit) ([qwen/moe_batch.rs] `encode_sigmoid_scalar_mul`). */
uint16_t or_sigmoid_gate(float h, float logit)
{
    double sg = 1.0 / (1.0 + exp(-(double)logit));
    return or_bf16_round((double)h * sg);
}

static int check_ffn(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int hidden, int inter)
{
    if (gate->n != inter || up->n != inter || gate->k != hidden || up->k != hidden) return OR_ERR_INVALID;
    if (down->n != hidden || down->k != inter) return OR_ERR_INVALID;
    return OR_OK;
}

/* Dense layer FFN half: tail RESIDUAL (out in/out) or RMSNORM (out written). */
int or_dense(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int hidden, int inter,
             int m, int act, int tail, const uint16_t* x, uint16_t* out, const uint16_t* norm_w, float eps)
{
    if (check_ffn(gate, up, down, hidden, inter)) return OR_ERR_INVALID;
    float* h = (float*)malloc(sizeof(float) * (size_t)hidden);
    for (int t = 0; t < m; ++t) {
        ffn_token(gate, up, down, act, x + (size_t)t * hidden, h);
        uint16_t* o = out + (size_t)t * hidden;
        if (tail == OR_TAIL_RESIDUAL) {
            for (int i = 0; i < hidden; ++i) o[i] = or_residual(o[i], h[i]);
        } else {
            or_rmsnorm_row(h, norm_w, hidden, eps, o);
        }
    }
    free(h);
    return OR_OK;
}

/* Shared expert: tail NONE, RMSNORM (aux = norm weight) or SIGMOID_GATE (aux = gate vector). */
int or_shared_expert(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int hidden, int inter,
                     int m, int act, int tail, const uint16_t* x, uint16_t* h_out, const uint16_t* aux,
                     float eps)
{
    if (check_ffn(gate, up, down, hidden, inter)) return OR_ERR_INVALID;
    float* h = (float*)malloc(sizeof(float) * (size_t)hidden);
    for (int t = 0; t < m; ++t) {
        const uint16_t* xt = x + (size_t)t * hidden;
        ffn_token(gate, up, down, act, xt, h);
        uint16_t* o = h_out + (size_t)t * hidden;
        if (tail == OR_TAIL_RMSNORM) {
            or_rmsnorm_row(h, aux, hidden, eps, o);
        } else if (tail == OR_TAIL_SIGMOID_GATE) {
            float l = or_gate_logit(aux, xt, hidden);
            for (int i = 0; i < hidden; ++i) o[i] = or_sigmoid_gate(h[i], l);
        } else {
            for (int i = 0; i < hidden; ++i) o[i] = or_bf16_round((double)h[i]);
        }
    }
    free(h);
    return OR_OK;
}

/* ---- O5: router top-k ------------------------------------------------------------------
 * The host top-k of [qwen/moe_batch.rs] (`router_topk_gemma4(logits_t, top_k,
 * per_expert_ones)` per token).  Rank by logit descending, ties to the lower
 * index, NaN as -inf.  Weights: softmax over the selected logits (the full
 * softmax renormalised over the top-k; the common denominator cancels), times
 * the per-expert scale. */
static double rank_value(float l) { return isnan(l) ? -INFINITY : (double)l; }

static int beats(const float* l, int a, int b) /* does expert a rank before expert b? */
{
    double va = rank_value(l[a]), vb = rank_value(l[b]);
    if (va != vb) return va > vb;
    return a < b;
}

void or_topk_token(const float* logits, const float* scale, int n_experts, int k, int32_t* ids, float* w)
{
    char* taken = (char*)calloc((size_t)n_experts, 1);
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int e = 0; e < n_experts; ++e)
            if (!taken[e] && (best < 0 || beats(logits, e, best))) best = e;
        taken[best] = 1;
        ids[r] = best;
    }
    free(taken);
    double l0 = rank_value(logits[ids[0]]);
    double* ex = (double*)malloc(sizeof(double) * (size_t)k);
    double sum = 0.0;
    for (int r = 0; r < k; ++r) {
        double lr = rank_value(logits[ids[r]]);
        ex[r] = (lr == l0) ? 1.0 : exp(lr - l0);
        sum += ex[r];
    }
    for (int r = 0; r < k; ++r) {
        double sc = scale ? (double)scale[ids[r]] : 1.0;
        w[r] = (float)(ex[r] / sum * sc);
    }
    free(ex);
}

/* ---- O7: the expert-union plan ----------------------------------------------------------
 * [qwen/moe_batch.rs]: sub-batches are bounded by their expert UNION, which
 * must not exceed cap = min(cache slots, 32); routes stay in pair order
 * (p = t*k + r).  Reading taken: each sub-batch is the longest run of tokens
 * from its start whose union fits; the union lists experts in first-appearance
 * pair order and an expert's slot is its position in it. */
int or_moe_plan(const int32_t* ids, int m, int k, int n_experts, int cap, int32_t* plan)
{
    size_t total = (size_t)OR_PLAN_INTS(m, k);
    for (size_t i = 0; i < total; ++i) plan[i] = -1;
    int32_t* sub_tok = plan + 1;
    int32_t* sub_uni = plan + (m + 2);
    int32_t* uexp = plan + (2 * m + 3);
    int32_t* pslot = plan + (2 * m + 3 + m * k);
    int32_t* spb = plan + (2 * m + 3 + 2 * m * k);
    int32_t* sp = plan + (2 * m + 4 + 3 * m * k);
    int* slot_of = (int*)malloc(sizeof(int) * (size_t)n_experts);
    int S = 0, U = 0, s = 0;
    while (s < m) {
        for (int e = 0; e < n_experts; ++e) slot_of[e] = -1;
        int base = U, usize = 0, t = s;
        while (t < m) {
            int fresh = 0;
            for (int r = 0; r < k; ++r) {
                int e = ids[t * k + r];
                int dup = 0;
                for (int r2 = 0; r2 < r; ++r2) dup |= (ids[t * k + r2] == e);
                if (slot_of[e] < 0 && !dup) ++fresh;
            }
            if (usize + fresh > cap) break;
            for (int r = 0; r < k; ++r) {
                int e = ids[t * k + r];
                if (slot_of[e] < 0) { slot_of[e] = usize; uexp[base + usize] = e; ++usize; }
            }
            ++t;
        }
        if (t == s) { free(slot_of); return OR_ERR_CAPACITY; }
        for (int p = s * k; p < t * k; ++p) pslot[p] = slot_of[ids[p]];
        sub_tok[S] = s;
        sub_uni[S] = base;
        ++S;
        U = base + usize;
        s = t;
    }
    sub_tok[S] = m;
    sub_uni[S] = U;
    plan[0] = S;
    int pos = 0;
    for (int b = 0; b < S; ++b) {
        int base = sub_uni[b], usize = sub_uni[b + 1] - sub_uni[b];
        for (int j = 0; j < usize; ++j) {
            spb[base + j] = pos;
            for (int p = sub_tok[b] * k; p < sub_tok[b + 1] * k; ++p)
                if (pslot[p] == j) sp[pos++] = p;
        }
    }
    spb[U] = pos;
    free(slot_of);
    return OR_OK;
}

int or_moe_route(const float* logits, const float* scale, int m, int n_experts, int k, int cap,
                 int32_t* ids, float* w, int32_t* plan)
{
    if (m < 0 || n_experts <= 0 || k < 1 || k > n_experts) return OR_ERR_INVALID;
    if (cap > 32) return OR_ERR_UNSUPPORTED;
    if (cap < k) return OR_ERR_CAPACITY;
    if (m == 0) return OR_OK;
    for (int t = 0; t < m; ++t)
        or_topk_token(logits + (size_t)t * n_experts, scale, n_experts, k, ids + (size_t)t * k,
                      w + (size_t)t * k);
    return or_moe_plan(ids, m, k, n_experts, cap, plan);
}

/* ---- O8: the seeded phase-2 accumulator ------------------------------------------------
 * [qwen/moe_batch.rs]: the accumulator starts at the gated shared-expert output
 * and then adds the ranks, w_r * d_r in rank order, in fp32. */
float or_seeded_sum(float seed, const float* w, const float* d, int k)
{
    float acc = seed;
    for (int r = 0; r < k; ++r) {
        float prod = w[r] * d[r];
        acc = acc + prod;
    }
    return acc;
}

/* ---- O6 + O8: the routed half ---------------------------------------------------------
 * Phase 1 per pair: act_p = f(gate_e x_t) * (up_e x_t); phase 2 per token:
 * acc = seed, += w_r * (down_e act_p) over r; tail: one raw residual add. */
int or_moe_routed(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int n_experts, int hidden,
                  int moe_inter, int m, int k, int act, const uint16_t* x, const int32_t* ids,
                  const float* w, const uint16_t* seed, uint16_t* resid)
{
    if (check_ffn(gate, up, down, hidden, moe_inter)) return OR_ERR_INVALID;
    float* d = (float*)malloc(sizeof(float) * (size_t)k * hidden);
    float* wt = (float*)malloc(sizeof(float) * (size_t)k);
    char* valid = (char*)malloc((size_t)k);
    for (int t = 0; t < m; ++t) {
        const uint16_t* xt = x + (size_t)t * hidden;
        for (int r = 0; r < k; ++r) {
            int e = ids[t * k + r];
            valid[r] = (e >= 0 && e < n_experts);
            wt[r] = w[t * k + r];
            if (!valid[r]) continue;
            or_qmat ge = or_expert(gate, e), ue = or_expert(up, e), de = or_expert(down, e);
            ffn_token(&ge, &ue, &de, act, xt, d + (size_t)r * hidden);
        }
        uint16_t* o = resid + (size_t)t * hidden;
        for (int i = 0; i < hidden; ++i) {
            float acc = seed ? (float)or_bf16_value(seed[(size_t)t * hidden + i]) : 0.0f;
            for (int r = 0; r < k; ++r) {
                if (!valid[r]) continue;
                float prod = wt[r] * d[(size_t)r * hidden + i];
                acc = acc + prod;
            }
            o[i] = or_residual(o[i], acc);
        }
    }
    free(d); free(wt); free(valid);
    return OR_OK;
}

/* ---- O9: the Gemma-style sandwich tail -----------------------------------------------------
 * [qwen/moe_batch.rs] module doc, first bullet: Gemma's routed sum starts from
 * zero (no seed) and its shared branch joins in the layer's sandwich tail after
 * its own norm ([gemma4/shared_expert.rs] `encode_shared_expert_branch`: the
 * down projection, then `post_feedforward_layernorm_1` in place, into the bf16
 * row h1).  The pages print no more of that tail.  Reading taken here: the
 * join is z = h1 + r, the bf16 shared row plus the bf16 routed row (the
 * unseeded routed sum rounded once), added exactly; one more RMSNorm with its
 * own bf16 weight w over z, written as a bf16 row (as every norm on the pages
 * writes one); then one raw residual add into the stream.  Per token t:
 *   n = bf16(z / sqrt(mean(z^2) + eps) * w),  resid <- bf16(resid + n). */
void or_sandwich_tail(const uint16_t* h1, const uint16_t* r, const uint16_t* w, int m, int n, float eps,
                      uint16_t* resid)
{
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    for (int t = 0; t < m; ++t) {
        const uint16_t* ht = h1 + (size_t)t * n;
        const uint16_t* rt = r + (size_t)t * n;
        uint16_t* o = resid + (size_t)t * n;
        double ss = 0.0;
        for (int i = 0; i < n; ++i) {
            z[i] = or_bf16_value(ht[i]) + or_bf16_value(rt[i]);
            ss += z[i] * z[i];
        }
        double inv = 1.0 / sqrt(ss / (double)n + (double)eps);
        for (int i = 0; i < n; ++i) {
            uint16_t nb = or_bf16_round(z[i] * inv * or_bf16_value(w[i]));
            o[i] = or_bf16_round(or_bf16_value(o[i]) + or_bf16_value(nb));
        }
    }
    free(z);
}
