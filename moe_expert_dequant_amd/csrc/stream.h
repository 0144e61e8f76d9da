// stream.h -- burst kernels: the small-M projections with every weight load of
// a wave issued at once, and the fused down + seeded reduction of a MoE layer.
//
// At one to four tokens the gate/up and down GEMVs of a layer ([llama/dense.rs]
// encode_llama_layer_dense; [gemma4/shared_expert.rs] the shared-expert GEMVs;
// [qwen/moe_batch.rs] the routed phases) are bound by how many bytes the chip
// keeps in flight, not by arithmetic.  Here a wave streams one or two "units"
// -- one 16-row tile over one K unit (INT4: a scale/zero step and up to 8 code
// blocks of 128 inputs; INT8: up to 8 code blocks of 64) -- and issues all of
// their 1 KB steps (per matrix) before it computes anything; the activation
// rows of its units and the scale/zero steps go to wave-private LDS by direct
// global->LDS loads issued just before them.  There is no ring to refill and
// no workgroup barrier until the tile's partial sums meet in LDS.
//
// Same arithmetic as the streaming kernels (tiled.h): codes widened to bf16
// 128 + q, contracted on v_mfma_f32_16x16x32_bf16 against the activation rows,
// bias and zero point removed through a ones-operand MFMA, INT4 group scales
// per 64 inputs, INT8 row scales after the sum.  The split of K among waves
// (and so the order of the fp32 partial sums) differs, and the INT8 code bias
// is removed per block of 64 inputs rather than once per K range.
#pragma once
#include "route.h"
#include "tiled.h"

namespace ffnq {

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

// K units of a tiled matrix with k inputs.
__host__ __device__ inline int burst_units(int fmt, int n, int k)
{
    const TileGeo g = tile_geo(fmt, n, k);
    return fmt == FMT_INT4 ? g.ng : (g.nbk + 7) / 8;
}

// LDS bytes of one wave: the activation rows of its units, then their
// scale/zero steps.
__host__ __device__ inline int burst_wave_lds(int fmt, int nmat, int R, int upw)
{
    const int uin = fmt == FMT_INT4 ? 1024 : 512;
    return upw * (R * (uin * 2 + 64) + (fmt == FMT_INT4 ? nmat * 1024 : 0));
}
// Rows of a unit's sums kept in a reduction slot (R <= 8: MFMA rows 0-3 in
// lanes 0-15, rows 4-7 in lanes 16-31, register i = row 4 * (lane / 16) + i).
constexpr int kRedRows = 8;

// A workgroup of ks waves, each one unit, meeting in a [ks][nmat][8][16] reduction.
__host__ __device__ inline int burst_lds(int fmt, int nmat, int R, int upw, int ks)
{
    return ks * burst_wave_lds(fmt, nmat, R, upw) + ks * nmat * kRedRows * 16 * 4;
}

// Lanes 0..16*ceil(R/4)-1 hold a unit's sums: row 4 * (lane / 16) + i in
// register i.  Writes them to slot[row][16] (rows < R).
template <int R>
__device__ __forceinline__ void burst_store_rows(float* slot, const float (&acc)[4])
{
    const int lane = threadIdx.x & 63;
    if (lane < 16 * ((R + 3) / 4)) {
        const int rb = 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < (R < 4 ? R : 4); ++i)
            if (rb + i < R) slot[(rb + i) * 16 + (lane & 15)] = acc[i];
    }
}

// One unit: tile `tile` of the matrices at tq (expert offset applied), K unit
// u, against activation rows row[0..R) (each k bf16 long).  Lanes of MFMA row
// r >= R read row r % R: rows of D depend only on the same rows of A, and rows
// >= R are never read.
struct BUnit {
    const uint8_t* tq[2];
    int n, k;                 // matrix rows and inputs
    int tile, u;
    const uint16_t* row[8];
};

// UPW units of one wave; acc[uu][mt][i] = the unit's sum for row
// 4 * (lane / 16) + i, tile row lane % 16 (rows < R, at most 8).  INT4 applies the group scales; INT8 returns
// the unscaled sum of q*x (the code bias removed block by block; the row
// scale is applied by the caller).  The first nvalid (uniform) units are
// real; the code loads of the others repeat unit 0's, so that the number of
// loads after the direct-to-LDS ones is a constant.
template <int FMT, int NMAT, int R, int UPW>
__device__ __forceinline__ void burst_wave(const BUnit (&un)[UPW], int nvalid, uint8_t* wl,
                                           float (&acc)[UPW][NMAT][4])
{
    using G = BurstGeo<FMT>;
    constexpr int NL = UPW * G::UB * NMAT;   // code-step loads of the wave
    const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    uint8_t* szl = wl + UPW * R * G::ROWB;

    // activation rows of each unit, 1 KB per wave instruction; source
    // addresses are clamped into the row (a chunk past k lands in LDS slots
    // that are never read)
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        if (uu >= nvalid) break;   // uniform
        const BUnit& U = un[uu];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < G::CHUNKS; ++c) {
                const int kk = min(U.u * G::UIN + c * 512 + lane * 8, U.k - 8);
                lds_dma16(U.row[r] + kk, lds_addr(wl + (uu * R + r) * G::ROWB + c * 1024));
            }
    }
    // INT4 scale/zero steps: straight to the wave's LDS as well
    if constexpr (FMT == FMT_INT4) {
#pragma unroll
        for (int uu = 0; uu < UPW; ++uu) {
            if (uu >= nvalid) break;
            const BUnit& U = un[uu];
            const TileGeo geo = tile_geo(FMT, U.n, U.k);
            const int st = min(U.u * G::USTEPS, geo.steps - 1);
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
                lds_dma16(U.tq[mt] + (size_t)U.tile * geo.tile_bytes + (size_t)st * kStep + lane * 16,
                          lds_addr(szl + (uu * NMAT + mt) * 1024));
        }
    }
    // code steps of every unit, clamped to the tile's last step
    u32x4 q[UPW][G::UB][NMAT];
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        const BUnit& U = un[uu < nvalid ? uu : 0];
        const TileGeo geo = tile_geo(FMT, U.n, U.k);
#pragma unroll
        for (int s = 0; s < G::UB; ++s) {
            const int st = min(U.u * G::USTEPS + G::SZ + s, geo.steps - 1);
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
                q[uu][s][mt] = __builtin_nontemporal_load(
                    (const u32x4*)(U.tq[mt] + (size_t)U.tile * geo.tile_bytes + (size_t)st * kStep + lane * 16));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<NL>();   // the activation chunks and scale/zero steps (issued first) have landed
    __builtin_amdgcn_sched_barrier(0);

    const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int xrow = (lr % R) * G::ROWB;
#pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[uu][mt][i] = 0.f;
        if (uu >= nvalid) continue;   // uniform
        const BUnit& U = un[uu];
        const int nbk = FMT == FMT_INT4 ? U.k / 128 : U.k / 64;
        const int nb = min(G::UB, nbk - G::UB * U.u);
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
                        for (int i = 0; i < (R < 4 ? R : 4); ++i)
                            acc[uu][mt][i] = fmaf(sg, fmaf(-zg, o[jg][i], m[i]), acc[uu][mt][i]);
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
                    for (int i = 0; i < (R < 4 ? R : 4); ++i) acc[uu][mt][i] += fmaf(-128.0f, o[i], m[i]);
                }
            }
        }
    }
}

// The fp32 row scale of tile row n of an INT8 tiled matrix (1 for INT4).
template <int FMT>
__device__ __forceinline__ float burst_row_scale(const uint8_t* tq, int n, int nrow, int k)
{
    if constexpr (FMT == FMT_INT8) {
        const TileGeo geo = tile_geo(FMT, nrow, k);
        return ((const float*)(tq + geo.scale_off))[n];
    }
    return 1.0f;
}

// ---------------------------------------------------------------------------
// A union entry of a routing plan (ffnq_moe_route's layout), for batches of
// at most 64 pairs: its expert and the mask of its pairs (bit p = pair p, in
// ascending order), from one round of independent loads -- the entry's
// expert, every pair's expert id and the sub-batch bounds -- and ballots,
// instead of walking the plan's arrays one dependent load after another.
// An entry past the plan's union, an expert id out of range or an entry with
// no pairs comes back with e = -1.  The pairs are those of the entry's
// sub-batch whose id is the entry's expert (the plan's slot lists for a plan
// that ffnq_moe_route wrote for these ids).
struct PlanEntry {
    int e;
    uint64_t pairs;
};

__device__ __forceinline__ PlanEntry plan_entry(const int32_t* __restrict__ plan, const int32_t* __restrict__ ids,
                                                int m, int k, int n_experts, int g)
{
    const int lane = threadIdx.x & 63, P = m * k;
    const int32_t* sub_tok = plan + 1;
    const int32_t* sub_uni = plan + (m + 2);
    const int32_t* uexp = plan + (2 * m + 3);
    const int n_sub = plan[0];
    const int e = uexp[min(max(g, 0), P - 1)];
    const int id = lane < P ? ids[lane] : -1;
    const int st = lane <= m ? sub_tok[lane] : 0x7FFFFFFF;
    const int su = lane <= m ? sub_uni[lane] : 0x7FFFFFFF;
    PlanEntry r{-1, 0ull};
    const int S = min(max(n_sub, 0), m);
    // sub-batch b: the last of [0, S) whose first union entry is <= g
    const uint64_t le = __ballot(lane < S && su <= g);
    const int b = __popcll(le) - 1;
    if (g < 0 || g >= P || e < 0 || e >= n_experts || b < 0) return r;
    const int t0 = __builtin_amdgcn_readlane(st, b), t1 = __builtin_amdgcn_readlane(st, b + 1);
    const int u1 = __builtin_amdgcn_readlane(su, b + 1);
    if (g >= u1 || t0 < 0 || t1 > m || t0 >= t1) return r;
    r.pairs = __ballot(lane < P && id == e && lane >= t0 * k && lane < t1 * k);
    if (r.pairs) r.e = e;
    return r;
}

// The index of the j-th set bit of a nonzero mask (j < popcount), or of the
// last one when j is past it.
__device__ __forceinline__ int nth_bit(uint64_t msk, int j)
{
    int b = __builtin_ctzll(msk);
    for (int i = 0; i < j; ++i) {
        const uint64_t rest = msk & (msk - 1);
        if (!rest) break;
        msk = rest;
        b = __builtin_ctzll(msk);
    }
    return b;
}

// ---------------------------------------------------------------------------
// gate + up + activation.  A job is a dense FFN (the m token rows, one
// workgroup per tile) or a routed phase 1 (one workgroup per (union entry,
// tile), its rows the entry's pairs); a launch runs one job or two (a layer's
// shared expert and its routed experts read the same x).  The waves of a
// workgroup take the tile's K units, one each, and their sums meet in LDS in
// wave order; f(gate) * up is written as the fp32 value's bf16 hi/lo pair
// (act rows 2r, 2r+1 of row r: token or pair), in the natural order of a
// tiled down matrix.  A job with gate_vec also forms the shared-expert gate
// logits <gate_vec, x_t> in its workgroup 0.
template <int FMT, int R>
__device__ __forceinline__ void gu_burst_job(const GUParams& p, int bx)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
    const TileGeo geo = tile_geo(FMT, p.N, p.K);
    const bool routed = p.plan != nullptr;
    const int item = routed ? bx / geo.T : 0, tile = routed ? bx - item * geo.T : bx;
    int e = 0, rows = p.m;
    uint64_t pairs = 0;
    if (routed && p.logits) {
        // route the batch here (every workgroup of the job, in LDS): the entry's
        // expert and pairs from the plan; workgroup 0 writes ids, weights and plan
        const int P = p.m * p.top_k;
        const SmallRoute L = small_route_layout(smem, p.m, p.n_experts, p.top_k);
        route_small(p.logits, p.escale, p.m, p.n_experts, p.top_k, p.cap, L);
        const int32_t* lplan = L.plan;
        const int U = lplan[p.m + 2 + lplan[0]];   // sub_union_begin[n_sub]: the union's size
        if (bx == 0) {
            const int total = 2 * p.m + 4 + 4 * P;
            for (int i = tid; i < P; i += blockDim.x) {
                p.ids_out[i] = L.sel[i];
                p.w_out[i] = L.w[i];
            }
            for (int i = tid; i < total; i += blockDim.x) p.plan_out[i] = lplan[i];
        }
        if (item < U) {
            e = lplan[2 * p.m + 3 + item];
            const int32_t* spb = lplan + (2 * p.m + 3 + 2 * P);
            const int32_t* sp = lplan + (2 * p.m + 4 + 3 * P);
            for (int i = spb[item]; i < spb[item + 1]; ++i) pairs |= 1ull << sp[i];
        }
        __syncthreads();   // the LDS is the burst's staging from here on
        if (item >= U || e < 0 || e >= p.n_experts || pairs == 0ull) return;   // uniform
        rows = min(__popcll(pairs), R);
    } else if (routed) {   // union entry `item`: its expert and its pairs (at most m, one per token)
        const PlanEntry pe = plan_entry(p.plan, p.topk_ids, p.m, p.top_k, p.n_experts, item);
        if (pe.e < 0) return;   // uniform: past this plan's union, or not a valid entry
        e = pe.e;
        pairs = pe.pairs;
        rows = min(__popcll(pairs), R);   // the host sizes R for every entry's rows
    }
    BUnit un[1];
    un[0].tq[0] = p.tgate + (size_t)e * p.tebytes;
    un[0].tq[1] = p.tup + (size_t)e * p.tebytes;
    un[0].n = p.N;
    un[0].k = p.K;
    un[0].tile = tile;
    un[0].u = w;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int rr = r < rows ? r : 0;
        const int tok = routed ? nth_bit(pairs, rr) / p.top_k : rr;
        un[0].row[r] = p.x + (size_t)tok * p.K;
    }
    const int wlds = burst_wave_lds(FMT, 2, R, 1);
    float acc[1][2][4];
    burst_wave<FMT, 2, R, 1>(un, 1, smem + w * wlds, acc);
    float* red = (float*)(smem + p.ks * wlds);   // [ks][2][8][16]
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) burst_store_rows<R>(red + (w * 2 + mt) * kRedRows * 16, acc[0][mt]);
    __syncthreads();
    for (int ti = tid; ti < rows * 16; ti += blockDim.x) {   // rows * 16 may exceed one wave's lanes
        const int i = ti >> 4, nl = ti & 15, n = tile * 16 + nl;
        float v[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            float h = 0.f;
            for (int ww = 0; ww < p.ks; ++ww) h += red[((ww * 2 + mt) * kRedRows + i) * 16 + nl];
            v[mt] = h * burst_row_scale<FMT>(un[0].tq[mt], n, p.N, p.K);
        }
        const int orow = routed ? nth_bit(pairs, i) : i;
        if (n < p.N) {
            const float y = act_f32(p.act, v[0]) * v[1];
            uint16_t hi, lo;
            split_bf16(y, hi, lo);
            p.act_out[(size_t)(2 * orow) * p.N + n] = hi;
            p.act_out[(size_t)(2 * orow + 1) * p.N + n] = lo;
        }
    }
    if (p.gate_vec != nullptr && bx == 0) {
        for (int t = w; t < p.m; t += p.ks) {
            double s = 0.0;
            for (int i = lane; i < p.K; i += 64)
                s += (double)bf16_f32(p.gate_vec[i]) * (double)bf16_f32(p.x[(size_t)t * p.K + i]);
            for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
            if (lane == 0) p.logit[t] = (float)s;
        }
    }
}

// One job (grid = its workgroups) or two (workgroups [0, na) job a, the rest
// job b; both with the same format, rows and waves per workgroup).
template <int FMT, int R>
__global__ void __launch_bounds__(1024) gu_burst_kernel(GUParams a, GUParams b, int na)
{
    const int bx = (int)blockIdx.x;
    if (bx < na)
        gu_burst_job<FMT, R>(a, bx);
    else
        gu_burst_job<FMT, R>(b, bx - na);
}

// ---------------------------------------------------------------------------
// Dense down + tail for m = R / 2 tokens (act rows 2t, 2t+1 = the hi/lo pair
// of token t): one workgroup per tile over the whole K range, so the tail runs
// here (down_finish with one K range).  The ks waves take the tile's K units
// w, w + ks, ... in passes of one; each unit's sums go to its own LDS slot.
// The hi and lo rows of a token are then summed separately in unit order,
// added (hi + lo, as the streaming kernels do), scaled (INT8) and finished.
__host__ __device__ inline int burst_down_lds(int fmt, int R, int ks, int units)
{
    return ks * burst_wave_lds(fmt, 1, R, 1) + units * kRedRows * 16 * 4;
}

template <int FMT, int R>
__global__ void __launch_bounds__(1024) down_burst_kernel(DownParams p)
{
    static_assert(R % 2 == 0, "hi/lo row pairs");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int w = uniform(threadIdx.x >> 6), tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int nu = burst_units(FMT, p.N, p.K);
    const int wlds = burst_wave_lds(FMT, 1, R, 1);
    float* red = (float*)(smem + p.ks * wlds);   // [nu][8][16]
    for (int q = w; q < nu; q += p.ks) {
        BUnit un[1];
        un[0].tq[0] = p.tdown;
        un[0].tq[1] = nullptr;
        un[0].n = p.N;
        un[0].k = p.K;
        un[0].tile = tile;
        un[0].u = q;
#pragma unroll
        for (int r = 0; r < R; ++r) un[0].row[r] = p.act + (size_t)min(r, 2 * p.m - 1) * p.K;
        float acc[1][1][4];
        burst_wave<FMT, 1, R, 1>(un, 1, smem + w * wlds, acc);
        burst_store_rows<R>(red + q * kRedRows * 16, acc[0][0]);
    }
    __syncthreads();
    if (tid < p.m * 16) {
        const int t = tid >> 4, nl = tid & 15, n = tile * 16 + nl;
        float hh = 0.f, hl = 0.f;
        for (int q = 0; q < nu; ++q) {
            hh += red[(q * kRedRows + 2 * t) * 16 + nl];
            hl += red[(q * kRedRows + 2 * t + 1) * 16 + nl];
        }
        const float h = (hh + hl) * burst_row_scale<FMT>(p.tdown, n, p.N, p.K);
        if (n < p.N) down_finish(p, 0, t, n, h);
    }
}

// ---------------------------------------------------------------------------
// The routed down projection fused with the seeded phase-2 reduction and the
// residual add ([qwen/moe_batch.rs] encode_qwen_layer_moe_batched: phase 2
// starts its fp32 accumulator at the gated shared expert, then adds the ranks
// in order; the tail is one raw residual add).  One workgroup per 16-row tile
// of the output; its units are the shared expert's K units of that tile (rows:
// the 2m hi/lo act rows) and, for each union entry of the plan, the expert's K
// units of that tile (rows: the hi/lo rows of the entry's pairs), so each union
// expert's tile is streamed once for all of its pairs.  A wave takes units w,
// w + ks, ... in passes of one (its LDS holds one unit's rows); the units'
// sums meet in LDS.  Then, per token and output row:
// the seed (the shared expert's h * sigmoid(logit) rounded to bf16, as its own
// tail writes it; or the caller's bf16 seed; or 0), acc += w_r * d_r for r =
// 0..k-1 with product and sum each rounded to fp32, and resid = bf16(resid +
// acc).  d_r and the shared h are (sum of the hi-row partials) + (sum of the
// lo-row partials) in unit order -- the arithmetic of down_burst_kernel, so the
// seed is bit for bit that of ffnq_shared_expert.  Pairs whose plan entry does
// not name their expert, or whose id is out of range, add nothing.
struct MoeDownParams {
    const uint8_t* tdown;     // routed experts, tiled (expert 0)
    long long tebytes;
    int N, K;                 // hidden, moe_inter
    const uint16_t* act;      // routed act rows [2 * act_rows][K]
    int act_rows;             // m * top_k
    const int32_t* plan;
    const int32_t* topk_ids;
    const float* topk_w;
    int m, top_k, n_experts;
    const uint8_t* sh_tdown;  // shared expert's tiled down [N][sh_K], or null
    int sh_K;
    const uint16_t* sh_act;   // its act rows [2m][sh_K]
    const float* sh_logit;    // its gate logits [m]
    const uint16_t* seed;     // bf16 [m][N] (no shared expert), or null for a zero seed
    uint16_t* resid;          // bf16 [m][N], in/out
    int resid_zero;           // 1: resid is written as bf16(+0 + acc); its contents on entry are not read
    int ks;                   // waves per workgroup
    int max_units;            // reduction slots: units of the largest union the plan can hold
};

// LDS of moe_down_kernel: ks waves' staging (UPP units each), the
// reduction slots, and the pair table (entry, place, weight; 64 pairs).
__host__ __device__ inline int moe_down_lds(int fmt, int R, int upp, int ks, int max_units)
{
    return ks * burst_wave_lds(fmt, 1, R, upp) + max_units * kRedRows * 16 * 4 + 64 * 12;
}

template <int FMT, int R, int UPP>
__global__ void __launch_bounds__(1024) moe_down_kernel(MoeDownParams p)
{
    static_assert(R % 2 == 0, "hi/lo row pairs");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int P = p.m * p.top_k;   // <= 64 (host)
    const int ns = p.sh_tdown ? burst_units(FMT, p.N, p.sh_K) : 0;
    const int nr = burst_units(FMT, p.N, p.K);
    const int Q = p.max_units;     // ns + nr * (largest possible union)
    const int wlds = burst_wave_lds(FMT, 1, R, UPP);
    float* red = (float*)(smem + p.ks * wlds);         // [Q][8][16]
    int* tg = (int*)(red + (size_t)Q * kRedRows * 16); // per pair: union entry (-1: adds nothing)
    int* tj = tg + 64;                                 // its place among the entry's pairs
    float* tw = (float*)(tj + 64);                     // its route weight

    // the wave's units q = w + (pass * UPP + uu) * ks, UPP at a time; routed
    // units of entries past the plan's union are skipped (uniform)
    for (int q0 = w; q0 < Q; q0 += UPP * p.ks) {
        BUnit un[UPP];
        int qs[UPP];
        int nvalid = 0;
#pragma unroll
        for (int uu = 0; uu < UPP; ++uu) {
            const int q = q0 + uu * p.ks;
            qs[uu] = -1;
            BUnit& B = un[uu];
            B.tile = tile;
            B.n = p.N;
            B.tq[1] = nullptr;
            B.tq[0] = p.tdown;
            B.k = p.K;
            B.u = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) B.row[r] = p.act;
            if (q >= Q || nvalid < uu) continue;   // units stay in order: valid ones first
            if (q < ns) {   // the shared expert's unit q
                B.tq[0] = p.sh_tdown;
                B.k = p.sh_K;
                B.u = q;
#pragma unroll
                for (int r = 0; r < R; ++r) B.row[r] = p.sh_act + (size_t)min(r, 2 * p.m - 1) * p.sh_K;
            } else {        // union entry g, unit j
                const int g = (q - ns) / nr;
                const PlanEntry pe = plan_entry(p.plan, p.topk_ids, p.m, p.top_k, p.n_experts, g);
                if (pe.e < 0) continue;
                B.tq[0] = p.tdown + (size_t)pe.e * p.tebytes;
                B.u = (q - ns) - g * nr;
                const int npr = min(__popcll(pe.pairs), R / 2);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    B.row[r] = p.act + (size_t)(2 * nth_bit(pe.pairs, min(r >> 1, npr - 1)) + (r & 1)) * p.K;
            }
            qs[uu] = q;
            nvalid = uu + 1;
        }
        if (nvalid == 0) break;   // uniform: the rest of this wave's units are past the union
        float acc[UPP][1][4];
        burst_wave<FMT, 1, R, UPP>(un, nvalid, smem + w * wlds, acc);
#pragma unroll
        for (int uu = 0; uu < UPP; ++uu)
            if (uu < nvalid) burst_store_rows<R>(red + qs[uu] * kRedRows * 16, acc[uu][0]);
    }
    // the pair table, by wave 0 (one lane per pair): entry g of pair p is the
    // entry of its token's sub-batch whose expert is the pair's; its place is
    // the count of earlier pairs of that sub-batch with the same expert
    if (w == 0) {
        const int32_t* sub_tok = p.plan + 1;
        const int32_t* sub_uni = p.plan + (p.m + 2);
        const int32_t* uexp = p.plan + (2 * p.m + 3);
        const int S = min(max(p.plan[0], 0), p.m);
        const int id = lane < P ? p.topk_ids[lane] : -1;
        const float wt = lane < P ? p.topk_w[lane] : 0.0f;
        const int st = lane <= p.m ? sub_tok[lane] : 0x7FFFFFFF;
        const int su = lane <= p.m ? sub_uni[lane] : 0x7FFFFFFF;
        const int ue = lane < P ? uexp[lane] : -1;
        const int t = lane / max(p.top_k, 1);
        // sub-batch of token t: the last b < S with sub_tok[b] <= t
        int b = -1;
        for (int i = 0; i < S; ++i) b = __builtin_amdgcn_readlane(st, i) <= t ? i : b;
        int g = -1, j = 0;
        if (b >= 0 && id >= 0 && id < p.n_experts) {
            int u0 = 0, u1 = 0, t0 = 0;
            for (int i = 0; i < S + 1; ++i) {   // lane reads of the sub-batch bounds
                const int sui = __builtin_amdgcn_readlane(su, i), sti = __builtin_amdgcn_readlane(st, i);
                if (i == b) {
                    u0 = sui;
                    t0 = sti;
                }
                if (i == b + 1) u1 = sui;
            }
            for (int gg = 0; gg < P; ++gg) {
                const int eg = __builtin_amdgcn_readlane(ue, gg);
                if (gg >= u0 && gg < u1 && eg == id) g = gg;
            }
            for (int qq = 0; qq < P; ++qq) {
                const int iq = __builtin_amdgcn_readlane(id, qq);
                if (qq >= t0 * p.top_k && qq < lane && iq == id) ++j;
            }
        }
        if (g >= 0 && (ns + (g + 1) * nr > Q || j >= R / 2)) g = -1;
        if (lane < 64) {
            tg[lane] = g;
            tj[lane] = j;
            tw[lane] = wt;
        }
    }
    __syncthreads();
    if (tid >= p.m * 16) return;
    const int t = tid >> 4, nl = tid & 15, n = tile * 16 + nl;
    if (n >= p.N) return;
    // (sum of the units' rows 2j) + (sum of their rows 2j + 1) over units [q0, q0 + nu)
    auto pair_sum = [&](int q0, int nu, int j) {
        float hh = 0.f, hl = 0.f;
        for (int q = q0; q < q0 + nu; ++q) {
            hh += red[(q * kRedRows + 2 * j) * 16 + nl];
            hl += red[(q * kRedRows + 2 * j + 1) * 16 + nl];
        }
        return hh + hl;
    };
    float acc0 = 0.0f;
    if (ns > 0) {
        const float h = pair_sum(0, ns, t) * burst_row_scale<FMT>(p.sh_tdown, n, p.N, p.sh_K);
        const double sg = 1.0 / (1.0 + exp(-(double)p.sh_logit[t]));
        acc0 = bf16_f32(bf16_from_f64((double)h * sg));
    } else if (p.seed) {
        acc0 = bf16_f32(p.seed[(size_t)t * p.N + n]);
    }
    for (int r = 0; r < p.top_k; ++r) {
        const int pr = t * p.top_k + r;
        const int g = tg[pr];
        if (g < 0) continue;
        const float d = pair_sum(ns + g * nr, nr, tj[pr]) *
                        burst_row_scale<FMT>(p.tdown + (size_t)p.topk_ids[pr] * p.tebytes, n, p.N, p.K);
        acc0 = __fadd_rn(acc0, __fmul_rn(tw[pr], d));
    }
    uint16_t* o = p.resid + (size_t)t * p.N + n;
    *o = bf16_from_f64((p.resid_zero ? 0.0 : (double)bf16_f32(*o)) + (double)acc0);
}

}  // namespace ffnq
