/*
 * oracle.h -- TEST INFRASTRUCTURE ONLY: declarations of the CPU oracle in
 * oracle.c.  Constants are the oracle's own, defined to equal the library's
 * published values; nothing here is included by the HIP path.
 */
#ifndef OR_ORACLE_H
#define OR_ORACLE_H
#include <stdint.h>

#define OR_OK 0
#define OR_ERR_INVALID -1
#define OR_ERR_UNSUPPORTED -2
#define OR_ERR_CAPACITY -3

#define OR_FMT_INT8_ROW 1
#define OR_FMT_INT4_AFFINE_G64 2
#define OR_ACT_SILU 1
#define OR_ACT_GELU_TANH 2
#define OR_TAIL_NONE 0
#define OR_TAIL_RESIDUAL 1
#define OR_TAIL_RMSNORM 2
#define OR_TAIL_SIGMOID_GATE 3

#define OR_PLAN_INTS(m, k) (1 + 2 * ((m) + 1) + 4 * (m) * (k) + 1)

typedef struct or_qmat {
    int32_t fmt, n, k;
    const void* q;
    const void* s;
    const void* z;
} or_qmat;

double or_bf16_value(uint16_t b);
uint16_t or_bf16_round(double v);
float or_dequant(const or_qmat* w, int row, int col);
void or_dequant_matrix(const or_qmat* w, float* out);
or_qmat or_expert(const or_qmat* w, int e);
void or_gemv(const or_qmat* w, const double* x, float* y);
double or_silu(double v);
double or_gelu_tanh(double v);
float or_act(int act, float g, float u);
uint16_t or_residual(uint16_t x, float h);
void or_rmsnorm_row(const float* h, const uint16_t* w, int n, float eps, uint16_t* out);
float or_gate_logit(const uint16_t* wg, const uint16_t* x, int n);
uint16_t or_sigmoid_gate(float h, float logit);
void or_router_logits(const uint16_t* x, const uint16_t* w, int m, int hidden, int n_experts, float* logits);
int or_dense(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int hidden, int inter, int m,
             int act, int tail, const uint16_t* x, uint16_t* out, const uint16_t* norm_w, float eps);
int or_shared_expert(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int hidden, int inter,
                     int m, int act, int tail, const uint16_t* x, uint16_t* h_out, const uint16_t* aux,
                     float eps);
void or_topk_token(const float* logits, const float* scale, int n_experts, int k, int32_t* ids, float* w);
int or_moe_plan(const int32_t* ids, int m, int k, int n_experts, int cap, int32_t* plan);
int or_moe_route(const float* logits, const float* scale, int m, int n_experts, int k, int cap,
                 int32_t* ids, float* w, int32_t* plan);
float or_seeded_sum(float seed, const float* w, const float* d, int k);
int or_moe_routed(const or_qmat* gate, const or_qmat* up, const or_qmat* down, int n_experts, int hidden,
                  int moe_inter, int m, int k, int act, const uint16_t* x, const int32_t* ids,
                  const float* w, const uint16_t* seed, uint16_t* resid);
void or_sandwich_tail(const uint16_t* h1, const uint16_t* r, const uint16_t* w, int m, int n, float eps,
                      uint16_t* resid);
#endif
