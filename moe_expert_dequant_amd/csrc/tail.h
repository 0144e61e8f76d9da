// tail.h -- row-wise tails of libffnq that run after the down projection.
// The down kernel leaves fp32 partial sums part[r][row][i] over R K-ranges;
// these kernels add them in a fixed order (r = 0, 1, ...) before the tail.
#pragma once
#include "device.h"

namespace ffnq {

// part[0] + part[1] + ... + part[R-1] at idx, added in that order.  The loads
// go out in batches of 8 before the adds (a batch past R re-reads the last
// range, and its values are not added), so a batch costs one memory latency
// rather than one per range.
__device__ __forceinline__ float sum_parts(const float* part, int R, size_t stride, size_t idx)
{
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = part[(size_t)min(j, R - 1) * stride + idx];   // R >= 1
    float h = v[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) h = j < R ? h + v[j] : h;
    for (int r0 = 8; r0 < R; r0 += 8) {   // more than 8 ranges: further batches
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = part[(size_t)min(r0 + j, R - 1) * stride + idx];
#pragma unroll
        for (int j = 0; j < 8; ++j) h = r0 + j < R ? h + v[j] : h;
    }
    return h;
}

// sum_parts for 1 <= R <= NB: one batch, no loop, so that a caller's unrolled
// loop over elements can put several elements' loads in flight together.
template <int NB>
__device__ __forceinline__ float sum_parts_n(const float* part, int R, size_t stride, size_t idx)
{
    float v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = part[(size_t)min(j, R - 1) * stride + idx];
    float h = v[0];
#pragma unroll
    for (int j = 1; j < NB; ++j) h = j < R ? h + v[j] : h;
    return h;
}
__device__ __forceinline__ float sum_parts8(const float* part, int R, size_t stride, size_t idx)
{
    return sum_parts_n<8>(part, R, stride, idx);
}

// RMSNorm with a bf16 weight over rows of h:
//   out[t][i] = bf16(h[t][i] / sqrt(mean_i h^2 + eps) * w[i])
// ([gemma4/shared_expert.rs] encode_rms_norm_bf16w with RMS_EPS).  The sum
// of squares, the scale and the product are formed in double; the result is
// rounded to bf16 once.  One workgroup of kNormThreads per row, so that a row of
// up to 4 * kNormThreads values is summed from its K-range partials in one
// round of loads.  With `held` (rows of at most kRowLds values) the summed row
// and the weight are kept in dynamic LDS between the two passes, loaded
// together in the first; the host launches with n * 6 bytes of LDS then.
constexpr int kRowLds = 8192;
constexpr int kNormThreads = 1024;

// One row t of the RMSNorm, by a workgroup of kNormThreads; store(i, v)
// receives every rounded value.  hrow/wrow: the dynamic LDS row (used when
// n <= kRowLds); partial: kNormThreads / 64 doubles of LDS.
template <class Store>
__device__ __forceinline__ void rmsnorm_row(const float* __restrict__ part, int R, int m,
                                            const uint16_t* __restrict__ w, int n, float eps, int t, float* hrow,
                                            uint16_t* wrow, double* partial, Store store)
{
    const int tid = threadIdx.x;
    const size_t stride = (size_t)m * n;
    const bool held = n <= kRowLds;
    double ss = 0.0;
    // four elements per step, their loads together (indices clamped into the
    // row; only elements < n are kept), added to ss in element order
    auto first_pass = [&](auto sumf) {
        for (int i0 = tid; i0 < n; i0 += 4 * kNormThreads) {
            float h4[4];
            uint16_t w4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ic = min(i0 + kNormThreads * u, n - 1);
                h4[u] = sumf((size_t)t * n + ic);
                w4[u] = w[ic];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + kNormThreads * u;
                if (i < n) {
                    hrow[i] = h4[u];
                    wrow[i] = w4[u];
                    ss += (double)h4[u] * (double)h4[u];
                }
            }
        }
    };
    if (held && R <= 8) {
        first_pass([&](size_t ix) { return sum_parts_n<8>(part, R, stride, ix); });
    } else if (held && R <= 16) {
        first_pass([&](size_t ix) { return sum_parts_n<16>(part, R, stride, ix); });
    } else if (held) {
        for (int i = tid; i < n; i += blockDim.x) {
            const float h = sum_parts(part, R, stride, (size_t)t * n + i);
            hrow[i] = h;
            wrow[i] = w[i];
            ss += (double)h * (double)h;
        }
    } else {
        for (int i = tid; i < n; i += blockDim.x) {
            const float h = sum_parts(part, R, stride, (size_t)t * n + i);
            ss += (double)h * (double)h;
        }
    }
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) partial[tid >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += partial[i];
    const double r = 1.0 / sqrt(tot / (double)n + (double)eps);
    for (int i = tid; i < n; i += blockDim.x) {
        const double h = held ? (double)hrow[i] : (double)sum_parts(part, R, stride, (size_t)t * n + i);
        const uint16_t wi = held ? wrow[i] : w[i];
        store(i, bf16_from_f64(h * r * (double)bf16_f32(wi)));
    }
}

__global__ void __launch_bounds__(kNormThreads) rmsnorm_kernel(const float* __restrict__ part, int R, int m,
                                                               const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ out, int n, float eps)
{
    extern __shared__ float hrow[];   // [n] summed row, then [n] bf16 weight
    __shared__ double partial[kNormThreads / 64];
    const int t = blockIdx.x;
    rmsnorm_row(part, R, m, w, n, eps, t, hrow, (uint16_t*)(hrow + n), partial,
                [&](int i, uint16_t v) { out[(size_t)t * n + i] = v; });
}

// Dense tails after a K-split down projection: raw residual add
// ([llama/dense.rs] encode_residual_add), the sigmoid scalar gate
// ([qwen/moe_batch.rs] encode_sigmoid_scalar_mul) or a plain bf16 store.
__global__ void __launch_bounds__(256) ksum_tail_kernel(const float* __restrict__ part, int R, int m, int n, int tail,
                                                        uint16_t* __restrict__ out, const float* __restrict__ logit)
{
    const size_t total = (size_t)m * n;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
        const double h = (double)sum_parts(part, R, total, idx);
        if (tail == 1) {
            out[idx] = bf16_from_f64((double)bf16_f32(out[idx]) + h);
        } else if (tail == 3) {
            const double sg = 1.0 / (1.0 + exp(-(double)logit[idx / n]));
            out[idx] = bf16_from_f64(h * sg);
        } else {
            out[idx] = bf16_from_f64(h);
        }
    }
}

// Ranks of one token in batches of KB: the batch's ids, weights and partials
// are loaded before any add (ranks past k re-read rank k-1 and are not added);
// the adds keep rank order.
template <int KB>
__device__ __forceinline__ float moe_ranks(const float* __restrict__ part, int R, size_t stride,
                                           const float* __restrict__ topk_w, const int32_t* __restrict__ topk_ids,
                                           int n_experts, int t, int k, int n, int i, float acc)
{
    for (int r0 = 0; r0 < k; r0 += KB) {
        int e[KB];
        float wt[KB], d[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int p = t * k + min(r0 + j, k - 1);
            e[j] = topk_ids[p];
            wt[j] = topk_w[p];
            d[j] = R <= 8 ? sum_parts8(part, R, stride, (size_t)p * n + i) : sum_parts(part, R, stride, (size_t)p * n + i);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j)
            if (r0 + j < k && e[j] >= 0 && e[j] < n_experts) acc = __fadd_rn(acc, __fmul_rn(wt[j], d[j]));
    }
    return acc;
}

// The seeded phase-2 reduction and the raw residual add of the routed half
// ([qwen/moe_batch.rs]: moe_phase2_down_reduce_k8 starts its fp32
// accumulator at the gated shared expert, then adds the ranks in order; the
// tail is one residual add, no norm).  d = down_e(act_p) per pair p comes from
// the grouped down kernel.  Product and sum are each rounded to fp32
// (no fused multiply-add), in rank order.
// The seed is either a bf16 row (seed) or made here from the shared expert's
// fp32 K-range partials (shpart, shR ranges) and its gate logits: the same
// bf16(h * sigmoid(logit)) in double that the shared expert's own tail writes.
__global__ void __launch_bounds__(256) moe_reduce_kernel(const float* __restrict__ part, int R,
                                                         const float* __restrict__ topk_w,
                                                         const int32_t* __restrict__ topk_ids, int n_experts,
                                                         const uint16_t* __restrict__ seed, uint16_t* __restrict__ resid,
                                                         int m, int k, int n, const float* __restrict__ shpart,
                                                         int shR, const float* __restrict__ logit)
{
    const size_t total = (size_t)m * n;
    const size_t stride = (size_t)m * k * n;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx / n), i = (int)(idx - (size_t)t * n);
        float acc = 0.0f;
        if (shpart) {
            const double h = (double)sum_parts(shpart, shR, total, idx);
            const double sg = 1.0 / (1.0 + exp(-(double)logit[t]));
            acc = bf16_f32(bf16_from_f64(h * sg));
        } else if (seed) {
            acc = bf16_f32(seed[idx]);
        }
        const float rs = bf16_f32(resid[idx]);
        if (k <= 2)
            acc = moe_ranks<2>(part, R, stride, topk_w, topk_ids, n_experts, t, k, n, i, acc);
        else if (k <= 4)
            acc = moe_ranks<4>(part, R, stride, topk_w, topk_ids, n_experts, t, k, n, i, acc);
        else
            acc = moe_ranks<8>(part, R, stride, topk_w, topk_ids, n_experts, t, k, n, i, acc);
        resid[idx] = bf16_from_f64((double)rs + (double)acc);
    }
}

// Zero fill of n bf16 values (a kernel rather than a memset node, so that a
// caller may capture the call in a graph).
__global__ void __launch_bounds__(256) zero_u16_kernel(uint16_t* __restrict__ p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

// The Gemma-style sandwich tail ([qwen/moe_batch.rs] module doc, first
// bullet: the routed sum starts from zero and the shared branch, normed by
// its own post-FFN RMSNorm, joins in the layer's sandwich tail), with that
// RMSNorm in the same launch.  Per token t (one workgroup of kNormThreads):
// h1 = the shared expert's RMSNorm row from its down projection's partials
// (rmsnorm_row, the arithmetic of rmsnorm_kernel, so h1 is bit for bit what
// ffnq_shared_expert writes), kept in LDS; z = h1 + r (the bf16 shared row and
// the bf16 routed row, added in double, exactly), n = bf16(z / sqrt(mean(z^2)
// + eps) * w) with the sum of squares, the scale and the product in double,
// and one raw residual add resid = bf16(resid + n).  Dynamic LDS: n * 8 bytes
// when n <= kRowLds (the summed row, the weight, h1), else n * 2 (h1).
__global__ void __launch_bounds__(kNormThreads) sandwich_norm_tail_kernel(
    const float* __restrict__ part, int R, int m, const uint16_t* __restrict__ shared_w, const uint16_t* __restrict__ r,
    const uint16_t* __restrict__ w, int n, float eps, uint16_t* __restrict__ resid)
{
    extern __shared__ float hrow[];
    const bool held = n <= kRowLds;
    uint16_t* wrow = (uint16_t*)(hrow + (held ? n : 0));
    uint16_t* h1 = held ? wrow + n : (uint16_t*)hrow;
    __shared__ double partial[kNormThreads / 64];
    const int t = blockIdx.x, tid = threadIdx.x;
    rmsnorm_row(part, R, m, shared_w, n, eps, t, hrow, wrow, partial, [&](int i, uint16_t v) { h1[i] = v; });
    __syncthreads();   // h1 is in; partial is free again
    const uint16_t* rt = r + (size_t)t * n;
    double ss = 0.0;
    for (int i = tid; i < n; i += kNormThreads) {
        const double z = (double)bf16_f32(h1[i]) + (double)bf16_f32(rt[i]);
        ss += z * z;
    }
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) partial[tid >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int i = 0; i < kNormThreads / 64; ++i) tot += partial[i];
    const double inv = 1.0 / sqrt(tot / (double)n + (double)eps);
    uint16_t* o = resid + (size_t)t * n;
    for (int i = tid; i < n; i += kNormThreads) {
        const double z = (double)bf16_f32(h1[i]) + (double)bf16_f32(rt[i]);
        const uint16_t nb = bf16_from_f64(z * inv * (double)bf16_f32(w[i]));
        o[i] = bf16_from_f64((double)bf16_f32(o[i]) + (double)bf16_f32(nb));
    }
}

}  // namespace ffnq
