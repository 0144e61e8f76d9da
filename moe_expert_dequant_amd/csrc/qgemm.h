// qgemm.h -- the dequant-fused small-M GEMM/GEMV kernels of libffnq (gfx950).
//
// One engine serves every projection of the quantized gated FFN
// ([llama/dense.rs] gate/up/down GEMVs; [gemma4/shared_expert.rs] the
// batched M-row GEMMs; [qwen/moe_batch.rs] the routed phase-1 and phase-2
// dispatches).  A wave owns a 16-row tile of one (or two) weight matrices and
// streams its packed codes from HBM with 16-byte loads, a few blocks ahead.
// Codes are widened in registers to bf16 "128 + code" (exact) and multiplied
// on the MFMA unit (v_mfma_f32_16x16x32_bf16) against up to 16 activation
// rows per token block; the code bias and the INT4 zero point are removed
// with a second MFMA against a ones operand (which yields sum(x) per group):
//     sum_k s (q - z) x_k = s * (sum_k (128 + q) x_k - (128 + z) sum_k x_k)
// INT4 groups (64 inputs) are kept apart by a lane permutation
// (v_permlane32_swap) so that each MFMA step sees one group only.
// Activations are staged once per workgroup in LDS, already in the order the
// MFMA consumes, so the weight stream is the only global traffic in the loop.
#pragma once
#include "device.h"

namespace ffnq {

enum { FMT_INT8 = 1, FMT_INT4 = 2 };

template <int FMT>
struct FmtT;
template <>
struct FmtT<FMT_INT4> { static constexpr int BK = 128; };   // inputs per 64-byte block row
template <>
struct FmtT<FMT_INT8> { static constexpr int BK = 64; };

// A quantized matrix on the device (expert 0 of a stack for routed calls).
struct MatDev {
    const uint8_t* q;
    const void* s;
    const uint16_t* z;
    int n, k;
    long long qe;   // bytes of codes per expert
    long long se;   // scale (and zero) elements per expert
};

// --------------------------------------------------------------------------
// Consumption order.  Within a block of BK inputs, the wave reads the 16-byte
// chunk c = 4*d + g for MFMA step d and lane group g (lanes 16g..16g+15).
// nat_run(c) is the natural index of the chunk's first input; inside an INT4
// chunk the eight inputs appear in the order [0,4,1,5,2,6,3,7].
template <int FMT>
__device__ __forceinline__ int nat_run(int c);
template <>
__device__ __forceinline__ int nat_run<FMT_INT4>(int c)
{
    const int d = c >> 2, g = c & 3;
    return 64 * (d >> 1) + 8 * (d & 1) + 32 * (g & 1) + 16 * (g >> 1);
}
template <>
__device__ __forceinline__ int nat_run<FMT_INT8>(int c)
{
    const int d = c >> 2, g = c & 3;
    return 16 * g + 8 * d;
}

// Position in consumption order of natural input r (0 <= r < BK).
template <int FMT>
__device__ __forceinline__ int cons_pos(int r);
template <>
__device__ __forceinline__ int cons_pos<FMT_INT4>(int r)
{
    const int a = (r >> 6) & 1, p = (r >> 5) & 1, q = (r >> 4) & 1, c = (r >> 3) & 1, j = r & 7;
    return (4 * (2 * a + c) + (p + 2 * q)) * 8 + 2 * (j & 3) + (j >> 2);
}
template <>
__device__ __forceinline__ int cons_pos<FMT_INT8>(int r)
{
    return (4 * ((r >> 3) & 1) + (r >> 4)) * 8 + (r & 7);
}

__device__ __forceinline__ int cons_index(int dfmt, int k)
{
    if (dfmt == FMT_INT4) return (k & ~127) + cons_pos<FMT_INT4>(k & 127);
    return (k & ~63) + cons_pos<FMT_INT8>(k & 63);
}

// --------------------------------------------------------------------------
// The streaming core.

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // two bf16 1.0

template <int FMT, int NMAT, int NT, int MT>
__device__ __forceinline__ void compute_block(const u32x4 (&cq)[NMAT], const uint32_t (&cs)[NMAT],
                                              const uint32_t (&cz)[NMAT], const uint16_t* const (&xl)[NT],
                                              int lb, f32x4 (&tot)[NMAT][NT], f32x4 (&one)[NT])
{
    constexpr int BK = FmtT<FMT>::BK;
    constexpr int MTC = (NT == 1) ? MT : 4;
    const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == FMT_INT4) {
        u32x4 xs[NT][4];
#pragma unroll
        for (int tb = 0; tb < NT; ++tb)
#pragma unroll
            for (int d = 0; d < 4; ++d) xs[tb][d] = *(const u32x4*)(xl[tb] + lb * BK + d * 32);
        u32x4 c[NMAT];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
            // lanes 0-31 hold inputs [0,64) of the block, lanes 32-63 [64,128):
            // swap so that steps 0,1 hold group 0 and steps 2,3 group 1
            auto a = __builtin_amdgcn_permlane32_swap(cq[mt][0], cq[mt][2], false, false);
            auto b = __builtin_amdgcn_permlane32_swap(cq[mt][1], cq[mt][3], false, false);
            c[mt][0] = a[0];
            c[mt][2] = a[1];
            c[mt][1] = b[0];
            c[mt][3] = b[1];
        }
#pragma unroll
        for (int jg = 0; jg < 2; ++jg) {
            f32x4 o[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
                o[tb] = mfma_bf16(xs[tb][2 * jg], ones, zero);
                o[tb] = mfma_bf16(xs[tb][2 * jg + 1], ones, o[tb]);
            }
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                const u32x4 b0 = unpack_int4_biased(c[mt][2 * jg]);
                const u32x4 b1 = unpack_int4_biased(c[mt][2 * jg + 1]);
                const float s = jg ? bf16hi_f32(cs[mt]) : bf16lo_f32(cs[mt]);
                const float zb = (jg ? bf16hi_f32(cz[mt]) : bf16lo_f32(cz[mt])) + 128.0f;
#pragma unroll
                for (int tb = 0; tb < NT; ++tb) {
                    f32x4 a = mfma_bf16(xs[tb][2 * jg], b0, zero);
                    a = mfma_bf16(xs[tb][2 * jg + 1], b1, a);
#pragma unroll
                    for (int i = 0; i < MTC; ++i) tot[mt][tb][i] = fmaf(s, fmaf(-zb, o[tb][i], a[i]), tot[mt][tb][i]);
                }
            }
        }
    } else {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            u32x4 xs[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
                xs[tb] = *(const u32x4*)(xl[tb] + lb * BK + d * 32);
                one[tb] = mfma_bf16(xs[tb], ones, one[tb]);
            }
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                const u32x2 p0 = unpack_int8_biased(cq[mt][2 * d]);
                const u32x2 p1 = unpack_int8_biased(cq[mt][2 * d + 1]);
                const u32x4 b = {p0[0], p0[1], p1[0], p1[1]};
#pragma unroll
                for (int tb = 0; tb < NT; ++tb) tot[mt][tb] = mfma_bf16(xs[tb], b, tot[mt][tb]);
            }
        }
    }
}

// Streams blocks gb = gb0 + j*step (j < nb) of a 16-row tile of NMAT matrices.
// wq: per lane, code row base + 16*lane_group; wsp/wzp: per lane, INT4 scale
// and zero rows as bf16 pairs (one dword per block).  xl: per lane and token
// block, the LDS row of activations (+ 8*lane_group); block gb is at local
// block lb = lb0 + j*step.  PF blocks of codes are kept in flight.
template <int FMT, int NMAT, int NT, int MT, int PF>
__device__ __forceinline__ void stream_tile(const uint8_t* const (&wq)[NMAT], const uint32_t* const (&wsp)[NMAT],
                                            const uint32_t* const (&wzp)[NMAT], const uint16_t* const (&xl)[NT],
                                            int nb, int gb0, int lb0, int step, f32x4 (&tot)[NMAT][NT],
                                            f32x4 (&one)[NT])
{
    u32x4 rq[PF][NMAT];
    uint32_t rs[PF][NMAT], rz[PF][NMAT];
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        if (s < nb) {
            const int gb = gb0 + s * step;
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                rq[s][mt] = __builtin_nontemporal_load((const u32x4*)(wq[mt] + (size_t)gb * 64));
                if constexpr (FMT == FMT_INT4) {
                    rs[s][mt] = wsp[mt][gb];
                    rz[s][mt] = wzp[mt][gb];
                }
            }
        }
    }
    for (int j0 = 0; j0 < nb; j0 += PF) {
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            const int j = j0 + s;
            if (j < nb) {
                u32x4 cq[NMAT];
                uint32_t cs[NMAT], cz[NMAT];
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) {
                    cq[mt] = rq[s][mt];
                    cs[mt] = rs[s][mt];
                    cz[mt] = rz[s][mt];
                }
                const int jn = j + PF;
                if (jn < nb) {
                    const int gb = gb0 + jn * step;
#pragma unroll
                    for (int mt = 0; mt < NMAT; ++mt) {
                        rq[s][mt] = __builtin_nontemporal_load((const u32x4*)(wq[mt] + (size_t)gb * 64));
                        if constexpr (FMT == FMT_INT4) {
                            rs[s][mt] = wsp[mt][gb];
                            rz[s][mt] = wzp[mt][gb];
                        }
                    }
                }
                compute_block<FMT, NMAT, NT, MT>(cq, cs, cz, xl, lb0 + j * step, tot, one);
            }
        }
    }
}

// --------------------------------------------------------------------------
// Plan access (layout of ffnq_moe_route's output), with device-side clamping
// so that a malformed plan cannot send a kernel out of bounds.

struct PlanView {
    const int32_t* p;
    int m, k;
    __device__ int n_sub() const { return min(max(p[0], 0), m); }
    __device__ int n_union() const { return min(max(p[m + 2 + n_sub()], 0), m * k); }
    __device__ int slot_begin(int u) const { return min(max(p[2 * m + 3 + 2 * m * k + u], 0), m * k); }
    __device__ int slot_pair(int i) const { return p[2 * m + 4 + 3 * m * k + i]; }
};

// --------------------------------------------------------------------------
// gate + up + activation.  One workgroup = KS waves on one 16-row tile; the
// waves split K (blocks w, w+KS, ...) and are reduced through LDS.  The
// activation f(gate)*up is computed in double, rounded to fp32, split into a
// bf16 hi/lo pair and written in the consumption order of the down matrix.

struct GUParams {
    MatDev gate, up;
    int N, K;                  // inter, hidden
    int act;                   // 1 SiLU, 2 GELU(tanh)
    int dfmt;                  // down matrix format: order of the act planes
    const uint16_t* x;         // [m][K] bf16
    int m;
    int rows_cap;              // activation rows staged per pass (<= 16*NT)
    // routed mode (plan != nullptr): items are (union entry, tile)
    const int32_t* plan;
    int top_k;
    const int32_t* topk_ids;
    int n_experts;
    uint16_t* act_hi;          // [rows][N]
    uint16_t* act_lo;
    int act_rows;              // rows of the act planes (m, or m*top_k)
    // dense shared-expert gate logit: logit[t] = <gate_vec, x_t>
    const uint16_t* gate_vec;
    float* logit;
    // counters of the next kernel, cleared here
    unsigned* zero_ptr;
    int zero_count;
};

template <int FMT, int NT, int MT>
__global__ void __launch_bounds__(512) gu_kernel(GUParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int BK = FmtT<FMT>::BK;
    const int KS = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int NB = p.K / BK;
    const int tiles = (p.N + 15) >> 4;
    const int xstride = p.K + 8;   // elements; +16 bytes spreads LDS banks
    uint16_t* xs = (uint16_t*)smem;
    float* red = (float*)(smem + (size_t)p.rows_cap * xstride * 2);

    for (int i = blockIdx.x * nthr + tid; i < p.zero_count; i += gridDim.x * nthr) p.zero_ptr[i] = 0u;

    if (p.gate_vec != nullptr && blockIdx.x == 0) {
        for (int t = w; t < p.m; t += KS) {
            double acc = 0.0;
            for (int i = lane; i < p.K; i += 64) acc += (double)bf16_f32(p.gate_vec[i]) * (double)bf16_f32(p.x[(size_t)t * p.K + i]);
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (lane == 0) p.logit[t] = (float)acc;
        }
    }

    PlanView pv{p.plan, p.m, p.top_k};
    const int n_items = p.plan ? pv.n_union() * tiles : tiles;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int tile = item % tiles;
        int R, pb = 0, e = 0;
        if (p.plan) {
            const int u = item / tiles;
            pb = pv.slot_begin(u);
            R = pv.slot_begin(u + 1) - pb;
            if (R <= 0) continue;
            const int p0 = pv.slot_pair(pb);
            if (p0 < 0 || p0 >= p.m * p.top_k) continue;
            e = p.topk_ids[p0];
            if (e < 0 || e >= p.n_experts) continue;
        } else {
            R = p.m;
        }
        const int row0 = tile * 16;
        const int wrow = min(row0 + lr, p.N - 1);
        const uint8_t* wq[2];
        const uint32_t* wsp[2];
        const uint32_t* wzp[2];
        const MatDev* mats[2] = {&p.gate, &p.up};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const MatDev& M = *mats[mt];
            if constexpr (FMT == FMT_INT4) {
                wq[mt] = M.q + (size_t)e * M.qe + (size_t)wrow * (p.K / 2) + 16 * g;
                wsp[mt] = (const uint32_t*)((const uint16_t*)M.s + (size_t)e * M.se + (size_t)wrow * (p.K / 64));
                wzp[mt] = (const uint32_t*)(M.z + (size_t)e * M.se + (size_t)wrow * (p.K / 64));
            } else {
                wq[mt] = M.q + (size_t)e * M.qe + (size_t)wrow * p.K + 16 * g;
                wsp[mt] = nullptr;
                wzp[mt] = nullptr;
            }
        }
        for (int c0 = 0; c0 < R; c0 += p.rows_cap) {
            const int Rc = min(p.rows_cap, R - c0);
            // stage activation rows c0..c0+Rc in consumption order
            const int chunks = NB * (BK / 8);
            for (int it = tid; it < Rc * chunks; it += nthr) {
                const int rr = it / chunks, ci = it - rr * chunks;
                const int lb = ci / (BK / 8), c = ci - lb * (BK / 8);
                int src_row;
                if (p.plan) {
                    const int pr = pv.slot_pair(pb + c0 + rr);
                    src_row = (pr >= 0 && pr < p.m * p.top_k) ? pr / p.top_k : 0;
                } else {
                    src_row = c0 + rr;
                }
                u32x4 v = *(const u32x4*)(p.x + (size_t)src_row * p.K + lb * BK + nat_run<FMT>(c));
                if constexpr (FMT == FMT_INT4) v = permute_0415(v);
                *(u32x4*)(xs + rr * xstride + lb * BK + c * 8) = v;
            }
            __syncthreads();

            f32x4 tot[2][NT], one[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
                one[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                tot[0][tb] = one[tb];
                tot[1][tb] = one[tb];
            }
            const uint16_t* xl[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) xl[tb] = xs + min(tb * 16 + lr, Rc - 1) * xstride + 8 * g;
            const int nb = (NB - w + KS - 1) / KS;
            stream_tile<FMT, 2, NT, MT, 4>(wq, wsp, wzp, xl, nb, w, w, KS, tot, one);

            // cross-wave reduction
            constexpr int PER = (FMT == FMT_INT8 ? 3 : 2) * NT * 4;   // floats per lane
#pragma unroll
            for (int tb = 0; tb < NT; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    red[((w * PER) + (0 * NT + tb) * 4 + i) * 64 + lane] = tot[0][tb][i];
                    red[((w * PER) + (1 * NT + tb) * 4 + i) * 64 + lane] = tot[1][tb][i];
                    if constexpr (FMT == FMT_INT8) red[((w * PER) + (2 * NT + tb) * 4 + i) * 64 + lane] = one[tb][i];
                }
            __syncthreads();
            for (int it = tid; it < Rc * 16; it += nthr) {
                const int rr = it >> 4, nl = it & 15, n = row0 + nl;
                if (n >= p.N) continue;
                const int tb = rr >> 4, rl = rr & 15;
                const int ln = ((rl >> 2) << 4) | nl, i = rl & 3;
                float gs = 0.f, us = 0.f, os = 0.f;
                for (int ww = 0; ww < KS; ++ww) {
                    gs += red[((ww * PER) + (0 * NT + tb) * 4 + i) * 64 + ln];
                    us += red[((ww * PER) + (1 * NT + tb) * 4 + i) * 64 + ln];
                    if constexpr (FMT == FMT_INT8) os += red[((ww * PER) + (2 * NT + tb) * 4 + i) * 64 + ln];
                }
                if constexpr (FMT == FMT_INT8) {
                    const float sg = ((const float*)p.gate.s)[(size_t)e * p.gate.se + n];
                    const float su = ((const float*)p.up.s)[(size_t)e * p.up.se + n];
                    gs = sg * fmaf(-128.0f, os, gs);
                    us = su * fmaf(-128.0f, os, us);
                }
                const float a = (float)(act_f64(p.act, (double)gs) * (double)us);
                uint16_t hi, lo;
                split_bf16(a, hi, lo);
                int orow;
                if (p.plan) {
                    orow = pv.slot_pair(pb + c0 + rr);
                    if (orow < 0 || orow >= p.act_rows) continue;
                } else {
                    orow = c0 + rr;
                }
                const size_t o = (size_t)orow * p.N + cons_index(p.dfmt, n);
                p.act_hi[o] = hi;
                p.act_lo[o] = lo;
            }
            __syncthreads();
        }
    }
}

// --------------------------------------------------------------------------
// down + tail.  One workgroup = WR waves, each on its own 16-row tile (the
// workgroup covers 16*WR rows), over the K range of grid row blockIdx.y.  The
// activation rows (hi and lo planes) of that range are staged in LDS.  With
// more than one K range the partial sums go to the workspace and the last
// workgroup of a row group (a counter cleared by the gate/up kernel) reduces
// them in a fixed order and applies the tail.

enum { TAIL_NONE = 0, TAIL_RESIDUAL = 1, TAIL_RMSNORM = 2, TAIL_SIGMOID = 3, TAIL_PAIR = 4 };

struct DownParams {
    MatDev down;
    int N, K;                  // hidden, inter
    const uint16_t* act_hi;    // [act_rows][K] consumption order
    const uint16_t* act_lo;
    int act_rows;
    int m;
    int rows_cap;              // X rows (hi + lo) staged per pass (<= 16*NT)
    const int32_t* plan;       // routed mode
    int top_k;
    const int32_t* topk_ids;
    int n_experts;
    float* partial;            // [KG][2*act_rows][N] fp32 (KG > 1)
    unsigned* counters;        // [n_items]
    int tail;
    uint16_t* out;             // [m][N] bf16
    float* hbuf;               // [m][N] fp32 (RMSNORM) or [act_rows][N] (PAIR)
    const float* logit;        // [m] (SIGMOID)
};

template <int FMT, int NT, int MT>
__device__ __forceinline__ void down_finish(const DownParams& p, int t, int n, float h)
{
    if (p.tail == TAIL_PAIR || p.tail == TAIL_RMSNORM) {
        p.hbuf[(size_t)t * p.N + n] = h;
    } else if (p.tail == TAIL_RESIDUAL) {
        uint16_t* o = p.out + (size_t)t * p.N + n;
        *o = bf16_from_f64((double)bf16_f32(*o) + (double)h);
    } else if (p.tail == TAIL_SIGMOID) {
        const double sg = 1.0 / (1.0 + exp(-(double)p.logit[t]));
        p.out[(size_t)t * p.N + n] = bf16_from_f64((double)h * sg);
    } else {
        p.out[(size_t)t * p.N + n] = bf16_from_f64((double)h);
    }
}

template <int FMT, int NT, int MT>
__global__ void __launch_bounds__(256) down_kernel(DownParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ unsigned s_last;
    constexpr int BK = FmtT<FMT>::BK;
    const int WR = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int NB = p.K / BK;
    const int KG = gridDim.y, kg = blockIdx.y;
    const int kb0 = (int)(((long long)NB * kg) / KG), kb1 = (int)(((long long)NB * (kg + 1)) / KG);
    const int nbl = kb1 - kb0;
    const int xstride = nbl * BK + 8;
    uint16_t* xs = (uint16_t*)smem;
    float* res = (float*)(smem + (size_t)p.rows_cap * xstride * 2);   // [rows_cap][16*WR] (KG == 1)
    const int rows_g = 16 * WR;
    const int groups = (p.N + rows_g - 1) / rows_g;

    PlanView pv{p.plan, p.m, p.top_k};
    const int n_items = p.plan ? pv.n_union() * groups : groups;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int grp = item % groups;
        int R, pb = 0, e = 0;
        if (p.plan) {
            const int u = item / groups;
            pb = pv.slot_begin(u);
            R = pv.slot_begin(u + 1) - pb;
            if (R <= 0) continue;
            const int p0 = pv.slot_pair(pb);
            if (p0 < 0 || p0 >= p.act_rows) continue;
            e = p.topk_ids[p0];
            if (e < 0 || e >= p.n_experts) continue;
        } else {
            R = p.m;
        }
        const int R2 = 2 * R;                  // hi rows then lo rows
        const int row0 = grp * rows_g + w * 16;
        const int wrow = min(row0 + lr, p.N - 1);
        const MatDev& M = p.down;
        const uint8_t* wq[1];
        const uint32_t* wsp[1];
        const uint32_t* wzp[1];
        if constexpr (FMT == FMT_INT4) {
            wq[0] = M.q + (size_t)e * M.qe + (size_t)wrow * (p.K / 2) + 16 * g;
            wsp[0] = (const uint32_t*)((const uint16_t*)M.s + (size_t)e * M.se + (size_t)wrow * (p.K / 64));
            wzp[0] = (const uint32_t*)(M.z + (size_t)e * M.se + (size_t)wrow * (p.K / 64));
        } else {
            wq[0] = M.q + (size_t)e * M.qe + (size_t)wrow * p.K + 16 * g;
            wsp[0] = nullptr;
            wzp[0] = nullptr;
        }
        for (int c0 = 0; c0 < R2; c0 += p.rows_cap) {
            const int Rc = min(p.rows_cap, R2 - c0);
            const int chunks = nbl * (BK / 8);
            for (int it = tid; it < Rc * chunks; it += nthr) {
                const int rr = it / chunks, ci = it - rr * chunks;
                const int xr = c0 + rr;
                const int li = xr < R ? xr : xr - R;
                int arow;
                if (p.plan) {
                    arow = pv.slot_pair(pb + li);
                    if (arow < 0 || arow >= p.act_rows) arow = 0;
                } else {
                    arow = li;
                }
                const uint16_t* src = (xr < R ? p.act_hi : p.act_lo) + (size_t)arow * p.K + kb0 * BK + ci * 8;
                *(u32x4*)(xs + rr * xstride + ci * 8) = *(const u32x4*)src;
            }
            __syncthreads();

            f32x4 tot[1][NT], one[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
                one[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                tot[0][tb] = one[tb];
            }
            const uint16_t* xl[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) xl[tb] = xs + min(tb * 16 + lr, Rc - 1) * xstride + 8 * g;
            if (row0 < p.N) stream_tile<FMT, 1, NT, MT, 6>(wq, wsp, wzp, xl, nbl, kb0, 0, 1, tot, one);

            // per-lane results: weight row row0 + lr, X rows c0 + tb*16 + 4g + i
            float sc = 1.0f;
            if constexpr (FMT == FMT_INT8) sc = ((const float*)M.s)[(size_t)e * M.se + wrow];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = tb * 16 + 4 * g + i;
                    if (rr >= Rc || row0 + lr >= p.N) continue;
                    float v = tot[0][tb][i];
                    if constexpr (FMT == FMT_INT8) v = sc * fmaf(-128.0f, one[tb][i], v);
                    const int xr = c0 + rr;
                    if (KG == 1) {
                        res[xr * rows_g + w * 16 + lr] = v;
                    } else {
                        int prow;   // partial row: hi rows [0, act_rows), lo rows [act_rows, 2*act_rows)
                        const int li = xr < R ? xr : xr - R;
                        if (p.plan) prow = pv.slot_pair(pb + li);
                        else prow = li;
                        if (prow < 0 || prow >= p.act_rows) continue;
                        if (xr >= R) prow += p.act_rows;
                        p.partial[((size_t)kg * 2 * p.act_rows + prow) * p.N + row0 + lr] = v;
                    }
                }
            __syncthreads();
        }
        // finish: sum the hi and lo rows (and the K ranges) and apply the tail
        bool finisher = (KG == 1);
        if (KG > 1) {
            __threadfence();
            __syncthreads();
            if (tid == 0) s_last = atomicAdd(&p.counters[item], 1u);
            __syncthreads();
            finisher = (s_last == (unsigned)(KG - 1));
            if (finisher) __threadfence();
        }
        if (finisher) {
            for (int it = tid; it < R * rows_g; it += nthr) {
                const int li = it / rows_g, nl = it - li * rows_g, n = grp * rows_g + nl;
                if (n >= p.N) continue;
                int trow;
                if (p.plan) {
                    trow = pv.slot_pair(pb + li);
                    if (trow < 0 || trow >= p.act_rows) continue;
                } else {
                    trow = li;
                }
                float h;
                if (KG == 1) {
                    h = res[li * rows_g + nl] + res[(R + li) * rows_g + nl];
                } else {
                    h = 0.f;
                    for (int q = 0; q < KG; ++q) {
                        const float* P = p.partial + (size_t)q * 2 * p.act_rows * p.N;
                        h += __builtin_nontemporal_load(P + (size_t)trow * p.N + n) +
                             __builtin_nontemporal_load(P + (size_t)(p.act_rows + trow) * p.N + n);
                    }
                }
                down_finish<FMT, NT, MT>(p, trow, n, h);
            }
        }
        __syncthreads();
    }
}

}  // namespace ffnq
