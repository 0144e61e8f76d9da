// tail.h -- row-wise tails of libffnq that need a whole output row.
#pragma once
#include "device.h"

namespace ffnq {

// RMSNorm with a bf16 weight over rows of h (fp32):
//   out[t][i] = bf16(h[t][i] / sqrt(mean_i h^2 + eps) * w[i])
// ([gemma4/shared_expert.rs] encode_rms_norm_bf16w with RMS_EPS).  The sum
// of squares, the scale and the product are formed in double; the result is
// rounded to bf16 once.  One workgroup per row.
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ h, const uint16_t* __restrict__ w,
                                                      uint16_t* __restrict__ out, int n, float eps)
{
    __shared__ double part[256 / 64];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float* row = h + (size_t)t * n;
    double ss = 0.0;
    for (int i = tid; i < n; i += blockDim.x) ss += (double)row[i] * (double)row[i];
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += part[i];
    const double r = 1.0 / sqrt(tot / (double)n + (double)eps);
    for (int i = tid; i < n; i += blockDim.x)
        out[(size_t)t * n + i] = bf16_from_f64((double)row[i] * r * (double)bf16_f32(w[i]));
}

// The seeded phase-2 reduction and the raw residual add of the routed half
// ([qwen/moe_batch.rs]: moe_phase2_down_reduce_k8 starts its fp32
// accumulator at the gated shared expert, then adds the ranks in order; the
// tail is one residual add, no norm).  d = down_e(act_p) per pair p comes from
// the grouped down kernel.  Product and sum are each rounded to fp32
// (no fused multiply-add), in rank order.
__global__ void __launch_bounds__(256) moe_reduce_kernel(const float* __restrict__ pair_out,
                                                         const float* __restrict__ topk_w,
                                                         const int32_t* __restrict__ topk_ids, int n_experts,
                                                         const uint16_t* __restrict__ seed, uint16_t* __restrict__ resid,
                                                         int m, int k, int n)
{
    const size_t total = (size_t)m * n;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx / n), i = (int)(idx - (size_t)t * n);
        float acc = seed ? bf16_f32(seed[idx]) : 0.0f;
        for (int r = 0; r < k; ++r) {
            const int p = t * k + r;
            const int e = topk_ids[p];
            if (e < 0 || e >= n_experts) continue;
            const float prod = __fmul_rn(topk_w[p], pair_out[(size_t)p * n + i]);
            acc = __fadd_rn(acc, prod);
        }
        resid[idx] = bf16_from_f64((double)bf16_f32(resid[idx]) + (double)acc);
    }
}

}  // namespace ffnq
