// stream.h -- burst kernels: the small-M dense projections with every weight
// load of a wave issued at once.
//
// At one to four tokens the gate/up and down GEMVs of a layer ([llama/dense.rs]
// encode_llama_layer_dense; [gemma4/shared_expert.rs] the shared-expert GEMVs)
// are bound by how many bytes the chip keeps in flight, not by arithmetic.
// Here a wave owns one 16-row tile over `upw` K units (INT4: a scale/zero step
// and up to 8 code blocks of 128 inputs; INT8: up to 8 code blocks of 64) and
// issues all of those 1 KB steps (per matrix) before it computes anything; the
// activation slice of its units goes to wave-private LDS by direct
// global->LDS loads issued just before them.  There is no ring to refill, no
// workgroup barrier until the tile's waves meet in one LDS reduction, and the
// code stays small enough to keep four waves per SIMD.
//
// Same arithmetic as the streaming kernels (tiled.h): codes widened to bf16
// 128 + q, contracted on v_mfma_f32_16x16x32_bf16 against the activation rows,
// bias and zero point removed through a ones-operand MFMA, INT4 group scales
// per 64 inputs, INT8 row scales after the sum.  The split of K among waves
// (and so the order of the fp32 partial sums) differs, and the INT8 code bias
// is removed per block of 64 inputs rather than once per K range.
#pragma once
#include "tiled.h"

namespace ffnq {

// One wave's K units and their activation rows.  R: activation rows used
// (gate/up: the m token rows; down: the 2m hi/lo rows), at most 4, so the
// results sit in lanes 0-15, register i = row i.  Lanes of MFMA row r >= R read
// row r % R: rows of D depend only on the same rows of A, and rows >= R are
// never read.
struct BurstArgs {
    const uint8_t* tq[2];     // tiled matrices
    int N, K;                 // output rows, inputs
    const uint16_t* src;      // activation rows [R][K] (x rows, or hi/lo act rows), row stride K
    int upw, ks;              // K units per wave, waves per workgroup
};

template <int FMT>
struct BurstGeo {
    static constexpr int BK = FmtT<FMT>::BK;                 // inputs per code block
    static constexpr int SZ = FMT == FMT_INT4 ? 1 : 0;       // scale/zero steps per unit
    static constexpr int UB = 8;                             // code blocks per unit
    static constexpr int USTEPS = SZ + UB;                   // 1 KB steps per unit
    static constexpr int UIN = UB * BK;                      // inputs per unit
    static constexpr int CHUNKS = UIN * 2 / 1024;            // 1 KB activation chunks per row and unit
    static constexpr int ROWB = UIN * 2 + 64;                // LDS bytes per staged row and unit (padded)
};

// LDS bytes of one wave (activation rows of its units, then their scale/zero
// steps) and of the workgroup (waves, then the reduction area).
__host__ __device__ inline int burst_wave_lds(int fmt, int nmat, int R, int upw)
{
    const int uin = fmt == FMT_INT4 ? 1024 : 512;
    return upw * (R * (uin * 2 + 64) + (fmt == FMT_INT4 ? nmat * 1024 : 0));
}
__host__ __device__ inline int burst_lds(int fmt, int nmat, int R, int upw, int ks)
{
    return ks * burst_wave_lds(fmt, nmat, R, upw) + ks * nmat * 4 * 16 * 4;
}

// The wave's contribution: acc[mt][i] for rows i < R in lanes 0-15 (lane = tile
// row).  INT8 returns the unscaled sum of q*x (the code bias removed block by
// block; the row scale is applied after the waves' sums meet).
template <int FMT, int NMAT, int R, int UPW>
__device__ __forceinline__ void burst_wave(const BurstArgs& a, int tile, int w, uint8_t* wl, float (&acc)[NMAT][4])
{
    using G = BurstGeo<FMT>;
    constexpr int NL = UPW * G::UB * NMAT;       // code-step loads of the wave
    constexpr int NX = UPW * R * G::CHUNKS;      // activation chunk loads
    const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    const TileGeo geo = tile_geo(FMT, a.N, a.K);
    const int nun = FMT == FMT_INT4 ? geo.ng : (geo.nbk + G::UB - 1) / G::UB;
    const int u0 = w * UPW;

    // activation slice: rows r < R, inputs of units u0 .. u0+UPW-1, 1 KB per
    // wave instruction; source addresses are clamped into the row (a chunk
    // past K lands in LDS slots that are never read)
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < G::CHUNKS; ++c) {
                const int k = min((u0 + uu) * G::UIN + c * 512 + lane * 8, a.K - 8);
                lds_dma16(a.src + (size_t)r * a.K + k, lds_addr(wl + (uu * R + r) * G::ROWB + c * 1024));
            }
    uint8_t* szl = wl + UPW * R * G::ROWB;
    // INT4 scale/zero steps: straight to the wave's LDS as well (1 KB per
    // matrix and unit, no registers held)
    if constexpr (FMT == FMT_INT4) {
#pragma unroll
        for (int uu = 0; uu < UPW; ++uu) {
            const int st = min((u0 + uu) * G::USTEPS, geo.steps - 1);
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
                lds_dma16(a.tq[mt] + (size_t)tile * geo.tile_bytes + (size_t)st * kStep + lane * 16,
                          lds_addr(szl + (uu * NMAT + mt) * 1024));
        }
    }
    // code steps: every one of the wave's units, clamped to the tile's last step
    u32x4 q[UPW][G::UB][NMAT];
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu)
#pragma unroll
        for (int s = 0; s < G::UB; ++s) {
            const int st = min((u0 + uu) * G::USTEPS + G::SZ + s, geo.steps - 1);
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
                q[uu][s][mt] = __builtin_nontemporal_load(
                    (const u32x4*)(a.tq[mt] + (size_t)tile * geo.tile_bytes + (size_t)st * kStep + lane * 16));
        }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<NL>();   // the activation chunks and scale/zero steps (issued first) have landed
    __builtin_amdgcn_sched_barrier(0);
    (void)NX;

    const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = 0.f;
    const int xrow = (lr % R) * G::ROWB;
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        const int u = u0 + uu;
        if (u >= nun) break;   // uniform
        const int nb = FMT == FMT_INT4 ? min(G::UB, geo.nbk - 8 * u) : min(G::UB, geo.nbk - G::UB * u);
#pragma unroll
        for (int bi = 0; bi < G::UB; ++bi) {
            if (bi >= nb) break;   // uniform
            __builtin_amdgcn_sched_barrier(0);   // one block's LDS reads at a time (register pressure)
            const uint8_t* xb = wl + (uu * R) * G::ROWB + xrow + bi * G::BK * 2 + g * 16;
            u32x4 xs[FmtT<FMT>::STEPS];
#pragma unroll
            for (int d = 0; d < FmtT<FMT>::STEPS; ++d) xs[d] = *(const u32x4*)(xb + d * 64);
            if constexpr (FMT == FMT_INT4) {
                f32x4 o[2];
#pragma unroll
                for (int jg = 0; jg < 2; ++jg) o[jg] = mfma_bf16(xs[2 * jg + 1], ones, mfma_bf16(xs[2 * jg], ones, zero));
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) {
                    const u32x2 sz = *(const u32x2*)(szl + (uu * NMAT + mt) * 1024 + bi * 128 + lr * 8);
                    const uint32_t w32[4] = {q[uu][bi][mt][0], q[uu][bi][mt][1], q[uu][bi][mt][2], q[uu][bi][mt][3]};
#pragma unroll
                    for (int jg = 0; jg < 2; ++jg) {
                        f32x4 m = mfma_bf16(xs[2 * jg], unpack_int4_biased(w32[2 * jg]), zero);
                        m = mfma_bf16(xs[2 * jg + 1], unpack_int4_biased(w32[2 * jg + 1]), m);
                        const float sg = jg ? bf16hi_f32(sz[0]) : bf16lo_f32(sz[0]);
                        const float zg = (jg ? bf16hi_f32(sz[1]) : bf16lo_f32(sz[1])) + 128.0f;
#pragma unroll
                        for (int i = 0; i < R; ++i) acc[mt][i] = fmaf(sg, fmaf(-zg, o[jg][i], m[i]), acc[mt][i]);
                    }
                }
            } else {
                // the code bias comes off per block, so that only the unbiased
                // sums of q*x accumulate across blocks
                const f32x4 o = mfma_bf16(xs[1], ones, mfma_bf16(xs[0], ones, zero));
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) {
                    f32x4 m = zero;
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const u32x2 p0 = unpack_int8_biased(q[uu][bi][mt][2 * d]);
                        const u32x2 p1 = unpack_int8_biased(q[uu][bi][mt][2 * d + 1]);
                        m = mfma_bf16(xs[d], u32x4{p0[0], p0[1], p1[0], p1[1]}, m);
                    }
#pragma unroll
                    for (int i = 0; i < R; ++i) acc[mt][i] += fmaf(-128.0f, o[i], m[i]);
                }
            }
        }
    }
}

// The workgroup of one tile: its ks waves take units w*upw ..; their sums meet
// in LDS in wave order; finish(i, n, v[NMAT]) gets row i, tile row n (< N).
template <int FMT, int NMAT, int R, int UPW, typename Finish>
__device__ __forceinline__ void burst_tile(const BurstArgs& a, int tile, Finish finish)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wlds = burst_wave_lds(FMT, NMAT, R, UPW);
    float acc[NMAT][4];
    burst_wave<FMT, NMAT, R, UPW>(a, tile, w, smem + w * wlds, acc);
    float* red = (float*)(smem + a.ks * wlds);   // [ks][NMAT][4][16]
    if (lane < 16) {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int i = 0; i < R; ++i) red[((w * NMAT + mt) * 4 + i) * 16 + lane] = acc[mt][i];
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < R * 16) {
        const int i = tid >> 4, nl = tid & 15, n = tile * 16 + nl;
        float v[NMAT];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
            float h = 0.f;
            for (int ww = 0; ww < a.ks; ++ww) h += red[((ww * NMAT + mt) * 4 + i) * 16 + nl];
            v[mt] = h;
        }
        if (FMT == FMT_INT8) {
            const TileGeo geo = tile_geo(FMT, a.N, a.K);
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) v[mt] *= ((const float*)(a.tq[mt] + geo.scale_off))[n];
        }
        if (n < a.N) finish(i, n, v);
    }
}

// gate + up + activation for m = R tokens (one workgroup per tile): the
// fp32 f(gate) * up as a bf16 hi/lo pair (act row 2t = hi, 2t+1 = lo), in the
// natural order of a tiled down matrix.  With gate_vec, workgroup 0 also
// forms the shared-expert gate logits <gate_vec, x_t>.
template <int FMT, int R>
__global__ void __launch_bounds__(1024) gu_burst_kernel(GUParams p)
{
    BurstArgs a{{p.tgate, p.tup}, p.N, p.K, p.x, p.upw, p.ks};
    const int tile = blockIdx.x;
    auto finish = [&](int i, int n, const float (&v)[2]) {
        const float y = act_f32(p.act, v[0]) * v[1];
        uint16_t hi, lo;
        split_bf16(y, hi, lo);
        p.act_out[(size_t)(2 * i) * p.N + n] = hi;
        p.act_out[(size_t)(2 * i + 1) * p.N + n] = lo;
    };
    burst_tile<FMT, 2, R, 1>(a, tile, finish);   // one K unit per wave (the host launches upw == 1)
    if (p.gate_vec != nullptr && tile == 0) {
        const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
        for (int t = w; t < p.m; t += a.ks) {
            double acc = 0.0;
            for (int i = lane; i < p.K; i += 64)
                acc += (double)bf16_f32(p.gate_vec[i]) * (double)bf16_f32(p.x[(size_t)t * p.K + i]);
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (lane == 0) p.logit[t] = (float)acc;
        }
    }
}

// down + tail for m = R / 2 tokens (act rows 2t, 2t+1 = the hi/lo pair of
// token t), one workgroup per tile over the whole K range, so the tail runs
// here (down_finish with one K range).
template <int FMT, int R>
__global__ void __launch_bounds__(1024) down_burst_kernel(DownParams p)
{
    static_assert(R % 2 == 0, "hi/lo row pairs");
    BurstArgs a{{p.tdown, nullptr}, p.N, p.K, p.act, p.upw, p.ks};
    const int tile = blockIdx.x;
    // the waves' sums meet in LDS; the hi and lo rows of token t are summed
    // separately in wave order, then added (hi + lo, as the streaming kernels
    // do), scaled (INT8) and finished by the tail
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    auto body = [&](auto upwc) {
        constexpr int UPW = decltype(upwc)::value;
        const int wlds = burst_wave_lds(FMT, 1, R, UPW);
        float acc[1][4];
        burst_wave<FMT, 1, R, UPW>(a, tile, w, smem + w * wlds, acc);
        float* red = (float*)(smem + a.ks * wlds);   // [ks][4][16]
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < R; ++i) red[(w * 4 + i) * 16 + lane] = acc[0][i];
        }
        __syncthreads();
        const int tid = threadIdx.x;
        if (tid < (R / 2) * 16) {
            const int t = tid >> 4, nl = tid & 15, n = tile * 16 + nl;
            float hh = 0.f, hl = 0.f;
            for (int ww = 0; ww < a.ks; ++ww) {
                hh += red[(ww * 4 + 2 * t) * 16 + nl];
                hl += red[(ww * 4 + 2 * t + 1) * 16 + nl];
            }
            float h = hh + hl;
            if (FMT == FMT_INT8) {
                const TileGeo geo = tile_geo(FMT, a.N, a.K);
                h *= ((const float*)(a.tq[0] + geo.scale_off))[n];
            }
            if (n < a.N) down_finish(p, 0, t, n, h);
        }
    };
    if (a.upw == 1)
        body(IntC<1>{});
    else
        body(IntC<2>{});
}

}  // namespace ffnq
