// route.h -- router top-k and the expert-union plan, on the device.
//
// The pages read the whole batch's router logits back to the host and run the
// top-k per token there ([qwen/moe_batch.rs], encode_qwen_layer_moe_batched:
// read_f32_buffer_at + router_topk_gemma4), then plan sub-batches whose expert
// union fits the slot cap (next_routed_sub_batch / plan_and_stream_union).
// Here both steps run in one workgroup so the layer has no host round trip:
// the tokens' experts are selected in parallel (a thread per (token, expert)
// key when a token has few experts, else a wave per token), then the greedy
// union plan is built -- in parallel when the whole batch's union fits the cap
// (one sub-batch), else by wave 0 walking the tokens in order.  The router GEMV
// that produces the logits (router_gemv_kernel) is a launch of its own.
#pragma once
#include "device.h"

namespace ffnq {

constexpr int kMaxExperts = 1024;   // logits per token held in registers: 16 per lane
constexpr int kMaxSlots = 32;
constexpr int kIdsCache = 4096;      // pairs whose expert ids the plan pass reads from LDS
constexpr int kRankMax = 256;        // experts up to which the top-k is found by ranking in LDS
constexpr int kLgCache = 4096;       // logits (m * E) staged in LDS before the top-k
constexpr int kParPlan = 64;         // pairs from which the one-sub-batch plan is built in parallel
constexpr int kPairPlan = 64;        // pairs up to which it is built one pair per thread, CSR included
#ifndef FFNQ_KEY_RANK_MAX_E
#define FFNQ_KEY_RANK_MAX_E 32
#endif
constexpr int kKeyRankMaxE = FFNQ_KEY_RANK_MAX_E;   // experts up to which the top-k takes a thread per key
constexpr long long kKeyRankWeightWork = 16384;      // m * k * k bound of its thread-per-pair weights

struct RouteParams {
    const float* logits;    // [m][E]
    const float* scale;     // [E] or null
    int m, E, k, cap;
    int32_t* ids;           // [m][k]
    float* w;               // [m][k]
    int32_t* plan;
};

// Orderable key: larger logit first, then lower index; NaN ranks as -inf and
// -0 as +0.  Zero is below every real key.
__device__ __forceinline__ uint64_t route_key(float l, int e)
{
    uint32_t u = __float_as_uint(l);
    if (l != l) u = 0xFF800000u;
    if (l == 0.0f) u = 0u;
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// The logit a key was made from (NaN comes back as -inf and -0 as +0, which is
// how the weights treat them).
__device__ __forceinline__ float route_key_logit(uint64_t key)
{
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// v of lane `src` (uniform), by lane reads rather than a shuffle through LDS.
__device__ __forceinline__ double read_lane_f64(double v, int src)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off);
        v = o > v ? o : v;
    }
    return v;
}

// Router GEMV ([qwen/moe_batch.rs] encode_qwen_layer_moe_batched: the M
// router GEMVs run before the routed half, which reads their fp32 logits back):
// logits[t][e] = sum_i w[e][i] * x[t][i], bf16 operands (exact in fp32), fp32
// products and sums.  One wave per (token, expert): lane l takes inputs
// 8l .. 8l+7 of every 512 (16-byte loads of both rows, all issued before the
// adds), then the wave adds its lanes' sums.  hidden is a multiple of 8.
__global__ void __launch_bounds__(256) router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, int m, int hidden,
                                                          int n_experts, float* __restrict__ logits)
{
    const int wid = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wid >= m * n_experts) return;   // whole waves (wid is uniform in a wave)
    const int t = wid / n_experts, e = wid - t * n_experts;
    const uint16_t* xr = x + (size_t)t * hidden;
    const uint16_t* wr = w + (size_t)e * hidden;
    float acc = 0.0f;
    int i = lane * 8;
    for (; i + 3 * 512 < hidden; i += 4 * 512) {
        u32x4 xv[4], wv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xv[u] = *(const u32x4*)(xr + i + u * 512);
            wv[u] = *(const u32x4*)(wr + i + u * 512);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc = fmaf(bf16lo_f32(wv[u][j]), bf16lo_f32(xv[u][j]), acc);
                acc = fmaf(bf16hi_f32(wv[u][j]), bf16hi_f32(xv[u][j]), acc);
            }
    }
    for (; i < hidden; i += 512) {
        const u32x4 xv = *(const u32x4*)(xr + i), wv = *(const u32x4*)(wr + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc = fmaf(bf16lo_f32(wv[j]), bf16lo_f32(xv[j]), acc);
            acc = fmaf(bf16hi_f32(wv[j]), bf16hi_f32(xv[j]), acc);
        }
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) logits[(size_t)t * n_experts + e] = acc;
}

template <int N>
struct IntC {
    static constexpr int value = N;
};

// ---------------------------------------------------------------------------
// Routing of a small batch (m * E <= kSmallKeys keys, m * k <= 64 pairs) by
// one workgroup of nt >= 64 threads, entirely in LDS: the top-k of every token
// with its weights, and the plan.  The same selection, weights and plan as
// route_kernel (and as the definition: rank by key, weights exp(l_r - l_0)
// over their sum in rank order times the expert scale, greedy maximal
// sub-batches with first-appearance slots).  A thread per (token, expert) key
// counts the keys above it; a thread per pair forms its exponential, then its
// weight; wave 0 builds the plan with one lane per pair, walking the tokens
// in order for the greedy sub-batches.  Ends with a workgroup barrier; the
// results are in the LDS arrays of SmallRoute.
constexpr int kSmallKeys = 2048;
constexpr int kSmallPairs = 64;

struct SmallRoute {
    uint64_t* keys;   // [m][E]
    int* sel;         // [P] expert of pair p = t*k + r
    float* sell;      // [P] its logit (from its key: NaN as -inf, -0 as +0)
    double* ex;       // [P] exp(l_r - l_0)
    float* w;         // [P] route weight
    int* plan;        // [FFNQ_PLAN_INTS(m, k)]: the plan, -1 in unused entries
};

__host__ __device__ inline size_t small_route_lds(int m, int E, int k)
{
    const int P = m * k;
    return (size_t)m * E * 8 + (size_t)P * 8 + (size_t)P * 4 * 3 + (size_t)(2 * m + 4 + 4 * P) * 4 + 64;
}

__device__ inline SmallRoute small_route_layout(unsigned char* base, int m, int E, int k)
{
    const int P = m * k;
    SmallRoute L;
    L.keys = (uint64_t*)base;
    L.ex = (double*)(base + (size_t)m * E * 8);
    L.sel = (int*)(L.ex + P);
    L.sell = (float*)(L.sel + P);
    L.w = L.sell + P;
    L.plan = (int*)(L.w + P);
    return L;
}

__device__ void route_small(const float* __restrict__ logits, const float* __restrict__ scale, int m, int E, int k,
                            int cap, const SmallRoute& L)
{
    const int tid = threadIdx.x, nt = blockDim.x, P = m * k;
    for (int i = tid; i < m * E; i += nt) {
        const int t = i / E;
        L.keys[i] = route_key(logits[i], i - t * E);
    }
    const int total = 2 * m + 4 + 4 * P;
    for (int i = tid; i < total; i += nt) L.plan[i] = -1;
    __syncthreads();
    // rank of each key among its token's keys: the keys above it (keys are distinct)
    for (int i = tid; i < m * E; i += nt) {
        const int t = i / E;
        const uint64_t key = L.keys[i];
        const uint64_t* row = L.keys + (size_t)t * E;
        int rank = 0;
        for (int e2 = 0; e2 < E; ++e2) rank += row[e2] > key ? 1 : 0;
        if (rank < k) {
            L.sel[t * k + rank] = i - t * E;
            L.sell[t * k + rank] = route_key_logit(key);
        }
    }
    __syncthreads();
    for (int i = tid; i < P; i += nt) {
        const int t = i / k;
        const float l = L.sell[i], f0 = L.sell[t * k];
        const double lr = (l != l) ? -INFINITY : (double)l;
        const double l0 = (f0 != f0) ? -INFINITY : (double)f0;
        L.ex[i] = (lr == l0) ? 1.0 : exp(lr - l0);
    }
    __syncthreads();
    for (int i = tid; i < P; i += nt) {
        const int t = i / k;
        double sum = 0.0;
        for (int r = 0; r < k; ++r) sum += L.ex[t * k + r];
        const double sc = scale ? (double)scale[L.sel[i]] : 1.0;
        L.w[i] = (float)(L.ex[i] / sum * sc);
    }
    // the plan: wave 0, lane = pair
    if (tid < 64) {
        const int lane = tid;
        const bool valid = lane < P;
        const int id = valid ? L.sel[lane] : -1;
        const int tok = lane / k;
        int32_t* sub_tok = L.plan + 1;
        int32_t* sub_uni = L.plan + (m + 2);
        int32_t* uexp = L.plan + (2 * m + 3);
        int32_t* pslot = L.plan + (2 * m + 3 + P);
        int32_t* spb = L.plan + (2 * m + 3 + 2 * P);
        int32_t* sp = L.plan + (2 * m + 4 + 3 * P);
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        int S = 0, s = 0, usize = 0, base = 0;
        int my_sb = -1, my_first = 0, my_slot = -1, my_base = 0;
        for (int t = 0; t < m; ++t) {
            const bool in_t = valid && tok == t;
            bool seen = false;   // my expert already in the current sub-batch's earlier tokens
            for (int q = s * k; q < t * k; ++q) seen |= __builtin_amdgcn_readlane(id, q) == id;
            uint64_t fresh = __ballot(in_t && !seen);
            int nf = __popcll(fresh);
            if (usize + nf > cap) {   // close [s, t): the greedy sub-batch is maximal
                if (lane == 0) {
                    sub_tok[S] = s;
                    sub_uni[S] = base;
                }
                ++S;
                base += usize;
                usize = 0;
                s = t;
                fresh = __ballot(in_t);
                nf = __popcll(fresh);
            }
            if (in_t) {
                my_sb = S;
                my_base = base;
                my_first = (int)((fresh >> lane) & 1ull);
                if (my_first) my_slot = usize + __popcll(fresh & below);
            }
            usize += nf;
        }
        if (lane == 0) {
            sub_tok[S] = s;
            sub_uni[S] = base;
            sub_tok[S + 1] = m;
            sub_uni[S + 1] = base + usize;
            L.plan[0] = S + 1;
        }
        // a repeated expert takes the slot of its first pair in the sub-batch
        for (int q = 0; q < P; ++q) {
            const int qid = __builtin_amdgcn_readlane(id, q), qsb = __builtin_amdgcn_readlane(my_sb, q);
            const int qf = __builtin_amdgcn_readlane(my_first, q), qs = __builtin_amdgcn_readlane(my_slot, q);
            if (valid && !my_first && qf && qsb == my_sb && qid == id) my_slot = qs;
        }
        const int my_g = valid ? my_base + my_slot : 0x7FFFFFFF;
        int before = 0, same = 0;   // pairs of earlier entries; earlier pairs of my entry
        for (int q = 0; q < P; ++q) {
            const int qg = __builtin_amdgcn_readlane(my_g, q);
            before += qg < my_g ? 1 : 0;
            same += (q < lane && qg == my_g) ? 1 : 0;
        }
        if (valid) {
            pslot[lane] = my_slot;
            sp[before + same] = lane;
            if (my_first) {
                uexp[my_g] = id;
                spb[my_g] = before;
            }
        }
        if (lane == 0) spb[base + usize] = P;
    }
    __syncthreads();
}

// ffnq_moe_route for a small batch: route_small, then the outputs to global memory.
__global__ void __launch_bounds__(256) route_small_kernel(RouteParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const SmallRoute L = small_route_layout(smem, p.m, p.E, p.k);
    route_small(p.logits, p.scale, p.m, p.E, p.k, p.cap, L);
    const int P = p.m * p.k, total = 2 * p.m + 4 + 4 * P;
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
        p.ids[i] = L.sel[i];
        p.w[i] = L.w[i];
    }
    for (int i = threadIdx.x; i < total; i += blockDim.x) p.plan[i] = L.plan[i];
}

// SMALL: the batch's logits (m * E <= kLgCache) and chosen ids (m * k <=
// kIdsCache) are held in LDS; a compile-time choice, because a run-time select
// between an LDS and a global source compiles to one flat load, and a flat load
// waits for every global store of the wave before it returns.
template <bool SMALL>
__global__ void __launch_bounds__(256) route_kernel(RouteParams p)
{
    __shared__ int slot_of[kMaxExperts];
    __shared__ int cur_union[kMaxSlots];
    __shared__ int wsum_s[256 / 64];
    __shared__ int pl_s[kPairPlan];                   // per pair: first-appearance flag, then slot
    __shared__ int sst_s[kMaxSlots];                  // per slot: first position in the CSR
    __shared__ int ids_s[kIdsCache];
    __shared__ uint64_t keys_s[256 / 64][kRankMax];   // per wave: the token's keys
    __shared__ int sel_s[256 / 64][kRankMax];         // per wave: expert of each rank < k
    __shared__ float sell_s[256 / 64][kRankMax];      // per wave: logit of each rank < k
    __shared__ float lg_s[kLgCache];                  // the batch's logits, when they fit
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
    const int m = p.m, k = p.k, E = p.E;
    const int nj = (E + 63) >> 6;
    // the plan pass reads the chosen experts back: from LDS when they fit
    constexpr bool cached = SMALL;
    auto id_of = [&](int pp) {
        if constexpr (SMALL)
            return ids_s[pp];
        else
            return p.ids[pp];
    };

    // ---- top-k and weights, one token per wave ----
    // the batch's logits go to LDS in one round of coalesced loads when they fit,
    // so that a wave's tokens do not each wait for their own global loads
    if constexpr (SMALL) {
        for (int i = tid; i < m * E; i += blockDim.x) lg_s[i] = p.logits[i];
        __syncthreads();
    }
    if (SMALL && E <= kKeyRankMaxE && (long long)m * k * k <= kKeyRankWeightWork) {
        // Few experts per token: a thread per (token, expert) key counts the
        // keys of its token above it, so that every token is ranked at once
        // rather than a wave walking its tokens; ranks 0..k-1 name the top k.
        for (int i = tid; i < m * E; i += blockDim.x) {
            const int t = i / E, e = i - t * E;
            const uint64_t key = route_key(lg_s[i], e);
            const float* row = lg_s + t * E;
            int rank = 0;
            for (int e2 = 0; e2 < E; ++e2) rank += route_key(row[e2], e2) > key ? 1 : 0;
            if (rank < k) ids_s[t * k + rank] = e;
        }
        __syncthreads();
        // a thread per pair: the token's exponentials in rank order (NaN as
        // -inf, -0 as +0, as the keys read them), their sum, its weight
        for (int pp = tid; pp < m * k; pp += blockDim.x) {
            const int t = pp / k, r_me = pp - t * k;
            const float* row = lg_s + t * E;
            const int* sel = ids_s + t * k;
            auto logit = [&](int r) {
                const float l = route_key_logit(route_key(row[sel[r]], 0));
                return (l != l) ? -(double)INFINITY : (double)l;
            };
            const double l0 = logit(0);
            double sum = 0.0, ex_me = 0.0;
            for (int r = 0; r < k; ++r) {
                const double lr = logit(r);
                const double ex = (lr == l0) ? 1.0 : exp(lr - l0);
                sum += ex;
                if (r == r_me) ex_me = ex;
            }
            const int e = sel[r_me];
            const double sc = p.scale ? (double)p.scale[e] : 1.0;
            p.ids[pp] = e;
            p.w[pp] = (float)(ex_me / sum * sc);
        }
    } else
    for (int t = w; t < m; t += nw) {
        uint64_t key[kMaxExperts / 64];
#pragma unroll
        for (int j = 0; j < kMaxExperts / 64; ++j) {
            const int e = lane + 64 * j;
            float l = 0.0f;
            if (j < nj && e < E) {
                if constexpr (SMALL)
                    l = lg_s[t * E + e];
                else
                    l = p.logits[(size_t)t * E + e];
            }
            key[j] = (j < nj && e < E) ? route_key(l, e) : 0ull;
        }
        int my_e = -1;
        float my_l = 0.0f;   // its logit, from the key
        if (E <= kRankMax) {
            // rank of each key = number of keys above it (keys are distinct: they
            // carry the index); the keys of ranks 0..k-1 are the top k in order
#pragma unroll
            for (int j = 0; j < kRankMax / 64; ++j)
                if (lane + 64 * j < E) keys_s[w][lane + 64 * j] = key[j];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            // eight keys per pass, read before any compare; only the NJ key
            // registers that hold experts are ranked (the 64-bit compares are
            // the cost of this step)
            auto rank_keys = [&](auto njc) {
                constexpr int NJ = decltype(njc)::value;
                int rank[NJ] = {};
                int q = 0;
                for (; q + 8 <= E; q += 8) {
                    uint64_t o[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) o[u] = keys_s[w][q + u];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
#pragma unroll
                        for (int j = 0; j < NJ; ++j) rank[j] += o[u] > key[j] ? 1 : 0;
                }
                for (; q < E; ++q) {
                    const uint64_t o = keys_s[w][q];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) rank[j] += o > key[j] ? 1 : 0;
                }
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    if (lane + 64 * j < E && rank[j] < k) {
                        sel_s[w][rank[j]] = lane + 64 * j;
                        sell_s[w][rank[j]] = route_key_logit(key[j]);
                    }
            };
            if (nj <= 1)
                rank_keys(IntC<1>{});
            else if (nj == 2)
                rank_keys(IntC<2>{});
            else if (nj == 3)
                rank_keys(IntC<3>{});
            else
                rank_keys(IntC<4>{});
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            if (lane < k) {
                my_e = sel_s[w][lane];
                my_l = sell_s[w][lane];
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();   // the next token's writes come after these reads
        } else {
            for (int r = 0; r < k; ++r) {
                uint64_t best = 0;
#pragma unroll
                for (int j = 0; j < kMaxExperts / 64; ++j) best = key[j] > best ? key[j] : best;
                best = wave_max_u64(best);
#pragma unroll
                for (int j = 0; j < kMaxExperts / 64; ++j)
                    if (key[j] == best) key[j] = 0ull;
                if (lane == r) {
                    my_e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
                    my_l = route_key_logit(best);
                }
            }
        }
        double lr = -INFINITY;
        if (lane < k) lr = (my_l != my_l) ? -INFINITY : (double)my_l;
        const double l0 = read_lane_f64(lr, 0);
        const double ex = (lane < k) ? ((lr == l0) ? 1.0 : exp(lr - l0)) : 0.0;
        double sum = 0.0;
        for (int r = 0; r < k; ++r) sum += read_lane_f64(ex, r);
        if (lane < k) {
            const double sc = p.scale ? (double)p.scale[my_e] : 1.0;
            p.ids[(size_t)t * k + lane] = my_e;
            p.w[(size_t)t * k + lane] = (float)(ex / sum * sc);
            if (cached) ids_s[t * k + lane] = my_e;
        }
    }
    // Token t's ids were written by wave t % nw; the plan pass below reads
    // every pair's id from any thread, so all waves' writes must land first.
    __syncthreads();

    // ---- plan: unused entries are -1 ----
    const int total = 2 * m + 4 + 4 * m * k;
    const int P = m * k;
    for (int i = tid; i < total; i += blockDim.x) p.plan[i] = -1;
    int32_t* sub_tok = p.plan + 1;
    int32_t* sub_uni = p.plan + (m + 2);
    int32_t* uexp = p.plan + (2 * m + 3);
    int32_t* pslot = p.plan + (2 * m + 3 + m * k);
    int32_t* spb = p.plan + (2 * m + 3 + 2 * m * k);
    int32_t* sp = p.plan + (2 * m + 4 + 3 * m * k);

    // When the expert union of the whole batch fits the cap, the greedy plan is
    // one sub-batch of every token, with slots in first-appearance pair order;
    // that is found in parallel: up to kPairPlan pairs with one pair per thread
    // (CSR included), from kParPlan pairs on with each expert's first pair as an
    // LDS minimum and a scan over the pairs' first-appearance flags.  Otherwise
    // (or when the ids are not held in LDS) wave 0 walks the tokens in order.
    int U = kMaxSlots + 1;
    bool done = false;   // the whole plan is written (one sub-batch, pair-per-thread path)
    if (cached && P <= kPairPlan) {
        // one pair per thread; every count is a loop over earlier pairs in LDS
        // (the same address in every lane of a step)
        for (int i = tid; i < E; i += blockDim.x) slot_of[i] = -1;
        const int e = tid < P ? ids_s[tid] : -1;
        int first = tid < P ? 1 : 0;
#pragma unroll 8
        for (int q = 0; q < tid && q < P; ++q) first &= ids_s[q] != e;
        if (tid < kPairPlan) pl_s[tid] = first;
        U = __syncthreads_count(first);
        if (U <= p.cap) {
            if (first) {   // slot = first appearances before this pair
                int sl = 0;
#pragma unroll 8
                for (int q = 0; q < tid; ++q) sl += pl_s[q];
                slot_of[e] = sl;
                cur_union[sl] = e;
                uexp[sl] = e;
            }
            __syncthreads();
            const int my = tid < P ? slot_of[e] : -1;
            if (tid < P) {
                pslot[tid] = my;
                pl_s[tid] = my;
            }
            __syncthreads();
            if (tid < U) {   // slot starts: pairs in earlier slots
                int st = 0;
#pragma unroll 8
                for (int q = 0; q < P; ++q) st += pl_s[q] < tid ? 1 : 0;
                sst_s[tid] = st;
                spb[tid] = st;
            }
            __syncthreads();
            if (tid < P) {   // the pair's place among its slot's pairs, ascending
                int r = 0;
#pragma unroll 8
                for (int q = 0; q < tid; ++q) r += pl_s[q] == my ? 1 : 0;
                sp[sst_s[my] + r] = tid;
            }
            done = true;
        }
        __syncthreads();
        if (!done)
            for (int i = tid; i < E; i += blockDim.x) slot_of[i] = -1;
    } else if (cached && P >= kParPlan) {
        for (int i = tid; i < E; i += blockDim.x) slot_of[i] = 0x7FFFFFFF;
        __syncthreads();
        for (int pp = tid; pp < P; pp += blockDim.x) atomicMin(&slot_of[ids_s[pp]], pp);
        __syncthreads();
        const int C = (P + (int)blockDim.x - 1) / (int)blockDim.x;   // pairs per thread (<= 16)
        const int b0 = min(P, tid * C), b1 = min(P, b0 + C);
        unsigned firsts = 0u;
        int cnt = 0;
        for (int pp = b0; pp < b1; ++pp)
            if (slot_of[ids_s[pp]] == pp) {
                firsts |= 1u << (pp - b0);
                ++cnt;
            }
        int incl = cnt;   // inclusive scan over the wave, then over the waves
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wsum_s[w] = incl;
        __syncthreads();   // every flag is read before slot_of is overwritten below
        int wbase = 0;
        U = 0;
        for (int i = 0; i < nw; ++i) {
            wbase += i < w ? wsum_s[i] : 0;
            U += wsum_s[i];
        }
        if (U <= p.cap) {
            int sl = wbase + incl - cnt;
            for (int pp = b0; pp < b1; ++pp)
                if (firsts & (1u << (pp - b0))) {
                    const int e = ids_s[pp];
                    slot_of[e] = sl;
                    cur_union[sl] = e;
                    uexp[sl] = e;
                    ++sl;
                }
            __syncthreads();
            for (int pp = tid; pp < P; pp += blockDim.x) pslot[pp] = slot_of[ids_s[pp]];
        } else {
            __syncthreads();
            for (int i = tid; i < E; i += blockDim.x) slot_of[i] = -1;
        }
    } else {
        for (int i = tid; i < E; i += blockDim.x) slot_of[i] = -1;
    }
    __syncthreads();
    if (w != 0) return;

    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    int S = 0, base = 0, usize = 0, s_tok = 0, pos = 0;
    if (lane == 0) {
        sub_tok[0] = 0;
        sub_uni[0] = 0;
        if (done) {
            sub_tok[1] = m;
            sub_uni[1] = U;
            spb[U] = P;
            p.plan[0] = 1;
        }
    }
    if (done) return;

    // CSR of the sub-batch [t0, t1): pairs grouped by slot, ascending.
    auto close_sub = [&](int t0, int t1) {
        const int P0 = t0 * k, P1 = t1 * k;
        int cnt = 0;   // lane j < usize: pairs in slot j
        for (int c = P0; c < P1; c += 64) {
            const int pp = c + lane;
            const int sl = (pp < P1) ? slot_of[id_of(pp)] : -1;
            for (int j = 0; j < usize; ++j) {
                const uint64_t msk = __ballot(sl == j);
                if (lane == j) cnt += __popcll(msk);
            }
        }
        int excl = 0;   // exclusive prefix over lanes 0..usize-1 (lane reads, no LDS round trips)
        for (int j = 0, run = 0; j < usize; ++j) {
            if (lane == j) excl = run;
            run += __builtin_amdgcn_readlane(cnt, j);
        }
        int cur = pos + excl;
        if (lane < usize) spb[base + lane] = cur;
        for (int c = P0; c < P1; c += 64) {
            const int pp = c + lane;
            const int sl = (pp < P1) ? slot_of[id_of(pp)] : -1;
            for (int j = 0; j < usize; ++j) {
                const uint64_t msk = __ballot(sl == j);
                const int start = __builtin_amdgcn_readlane(cur, j);
                if (sl == j) sp[start + __popcll(msk & lt)] = pp;
                if (lane == j) cur += __popcll(msk);
            }
        }
        pos += P1 - P0;
        __builtin_amdgcn_wave_barrier();
        if (lane < usize) slot_of[cur_union[lane]] = -1;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };

    if (U <= p.cap) {   // one sub-batch, slots assigned above
        usize = U;
        s_tok = 0;
    } else {
    for (int t = 0; t < m; ++t) {
        const int e = (lane < k) ? id_of(t * k + lane) : 0;
        int cur = (lane < k) ? slot_of[e] : 0;
        bool fresh = (lane < k) && cur < 0;
        uint64_t fm = __ballot(fresh);
        int nf = __popcll(fm);
        if (usize + nf > p.cap) {
            close_sub(s_tok, t);
            ++S;
            if (lane == 0) {
                sub_tok[S] = t;
                sub_uni[S] = base + usize;
            }
            base += usize;
            usize = 0;
            s_tok = t;
            fresh = (lane < k);
            fm = __ballot(fresh);
            nf = __popcll(fm);
        }
        if (fresh) {
            cur = usize + __popcll(fm & lt);
            slot_of[e] = cur;
            cur_union[cur] = e;
            uexp[base + cur] = e;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (lane < k) pslot[(size_t)t * k + lane] = cur;
        usize += nf;
    }
    }
    close_sub(s_tok, m);
    ++S;
    if (lane == 0) {
        sub_tok[S] = m;
        sub_uni[S] = base + usize;
        spb[base + usize] = m * k;
        p.plan[0] = S;
    }
}

// ---------------------------------------------------------------------------
// One sub-batch of a routing plan as a plan of its own, over the experts held
// in a slot cache ([qwen/moe_batch.rs] `encode_qwen_layer_moe_batched`: each
// sub-batch's union is streamed into the expert slots, then its routed phases
// run on them).  Sub-batch tokens [t0, t1), union entries [u0, u1); union
// entry j is held by slot slot_of[j].  Writes ids (the slot holding each
// pair's expert, [m_b][k]) and the plan of m_b = t1 - t0 tokens with one
// sub-batch: union experts = the slots, pair slots unchanged, the union's pair
// lists shifted to the sub-batch's own pair numbers; unused entries -1, as
// ffnq_moe_route leaves them.  One workgroup; the host has checked the plan.
struct SubPlanParams {
    const int32_t* plan;   // the whole batch's plan (m tokens, k per token)
    int m, k;
    int t0, t1, u0, u1;
    int32_t slot_of[32];
    int32_t* ids_out;      // [m_b * k]
    int32_t* plan_out;     // FFNQ_PLAN_INTS(m_b, k) ints
};

__global__ void __launch_bounds__(256) sub_plan_kernel(SubPlanParams p)
{
    const int tid = threadIdx.x;
    const int mb = p.t1 - p.t0, Pb = mb * p.k, U = p.u1 - p.u0, P = p.m * p.k;
    const int32_t* pslot = p.plan + (2 * p.m + 3 + P);
    const int32_t* spb = p.plan + (2 * p.m + 3 + 2 * P);
    const int32_t* sp = p.plan + (2 * p.m + 4 + 3 * P);
    int32_t* o = p.plan_out;
    int32_t* o_tok = o + 1;
    int32_t* o_uni = o + (mb + 2);
    int32_t* o_uexp = o + (2 * mb + 3);
    int32_t* o_pslot = o + (2 * mb + 3 + Pb);
    int32_t* o_spb = o + (2 * mb + 3 + 2 * Pb);
    int32_t* o_sp = o + (2 * mb + 4 + 3 * Pb);
    const int s0 = spb[p.u0];
    for (int i = tid; i <= mb; i += blockDim.x) {
        o_tok[i] = i == 0 ? 0 : (i == 1 ? mb : -1);
        o_uni[i] = i == 0 ? 0 : (i == 1 ? U : -1);
    }
    for (int i = tid; i < Pb; i += blockDim.x) {
        const int pg = p.t0 * p.k + i;
        const int j = pslot[pg];
        o_pslot[i] = j;
        p.ids_out[i] = p.slot_of[j];
        o_uexp[i] = i < U ? p.slot_of[i] : -1;
        o_sp[i] = sp[s0 + i] - p.t0 * p.k;
    }
    for (int i = tid; i <= Pb; i += blockDim.x) o_spb[i] = i <= U ? spb[p.u0 + i] - s0 : -1;
    if (tid == 0) o[0] = 1;
}

}  // namespace ffnq
