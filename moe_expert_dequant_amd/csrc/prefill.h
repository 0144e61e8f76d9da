// prefill.h -- the routed phases at prefill sizes: a grouped GEMM over the
// union experts, each weight tile streamed once for all of its expert's rows.
//
// [gemma4/shared_expert.rs] `encode_shared_expert_branch_batched` (the
// M-row GEMMs are where the weight amortisation lives) and [qwen/moe_batch.rs]
// `encode_qwen_layer_moe_batched` (phase 1 per union expert over its pairs,
// phase 2 down per pair, then the rank-ordered reduction).  With tens of rows
// per expert (8 experts, 64 tokens, top 2: 11-23 pairs each) the activation
// rows of an expert no longer fit the LDS over the whole K range, so:
//
//  * a workgroup of W waves (12 for gate/up, 8 for down) owns one union entry
//    and a run of tiles; each wave streams one matrix over TPW tiles with its
//    own accumulators over its K range (no reduction inside the workgroup);
//    gate/up splits the waves between the two matrices on the same tiles;
//    down may split K into ranges whose fp32 partials the reduction adds;
//  * K goes in chunks of CHB code blocks (128 inputs each); the chunk's rows of
//    every pair of the entry (up to 16*RB rows per pass) are staged into LDS by
//    direct global->LDS loads, double-buffered: chunk c+1 lands while chunk c
//    is multiplied.  Each chunk opens with a barrier (its rows are in, the
//    other buffer is free), then the workgroup forms every row's sum over each
//    64-input group of the chunk (the zero point's term) and meets a second
//    barrier;
//  * every wave keeps D steps (a tile's scale/zero step and SPS code steps per
//    tile) of weights in flight beyond the one it multiplies; scale/zero steps
//    go to wave-private LDS slots (their entries are read by row, which is not
//    how the lanes hold them).
//
// Same arithmetic as the other INT4 kernels: codes widened to bf16 128 + q, the
// contraction on v_mfma_f32_16x16x32_bf16 with the activation rows as A, bias
// and zero point removed with the rows' group sums, group scales per 64
// inputs, fp32 accumulation over K in increasing K order.
// gate/up: f(g) * u is written as the bf16 hi/lo pair of each pair's act rows.
// down: the rows are the pairs' hi/lo act rows; d = (hi-row sum) + (lo-row
// sum) is written as the fp32 partial of the pair, summed by the reduction.
#pragma once
#include "qgemm.h"
#include "tiled.h"

namespace ffnq {


// s_waitcnt vmcnt(N) as a hard boundary: neither the compiler nor the
// scheduler moves a memory access across it in either direction (the LDS
// written by direct global->LDS loads is invisible to the compiler, so reads of
// it must not be hoisted above the wait, nor the next loads sunk below it).
template <int N>
__device__ __forceinline__ void pf_wait()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    wait_vmcnt<N>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

struct PrefillParams {
    const uint8_t* tq[2];     // tiled INT4 matrices of expert 0: gate, up (gate/up) or down
    long long tebytes;        // bytes per expert of one matrix
    int N, K;
    const uint16_t* src;      // gate/up: x [m][K]; down: act rows [2 * m * top_k][K]
    const int32_t* plan;
    const int32_t* topk_ids;
    int m, top_k, n_experts;
    int act;
    uint16_t* act_out;        // gate/up: [2 * m * top_k][N] bf16 hi/lo
    float* part;              // down: [kg][m * top_k][N] fp32, one slice per K range
    int tpw;                  // tiles per wave (== TPW)
    int kg;                   // K ranges (down; 1 for gate/up): chunks split evenly among them
};

// LDS: two activation buffers of 16*RB rows (CHB blocks each; rows padded by
// 16 bytes so that the 16 rows of one MFMA operand column fall in distinct
// banks), per wave (D + 1) * TPW scale/zero slots, the row table, the staged chunk's
// per-row sums over each 64-input group.  gate/up hands u
// from the up waves to the gate waves through the activation buffers after
// the K loop.
__host__ __device__ inline int prefill_row_bytes(int chb) { return chb * 256 + 16; }
__host__ __device__ inline int prefill_lds(int waves, int rb, int chb, int d, int tpw)
{
    return 2 * 16 * rb * prefill_row_bytes(chb) + waves * (d + 1) * tpw * 1024 + 16 * rb * 12 + 16 * rb * chb * 2 * 4;
}

__host__ __device__ constexpr int pf_lcm(int a, int b)
{
    int x = a, y = b;
    while (y) {
        const int t = x % y;
        x = y;
        y = t;
    }
    return a / x * b;
}

// NMW matrices per workgroup (2: gate and up, 1: down); every wave streams one
// matrix over TPW tiles (waves [0, 8/NMW) the first matrix, the rest the
// second, on the same tiles).
template <int W, int NMW, int RB, int CHB, int TPW, int D, int SPS>
__global__ void __launch_bounds__(64 * W) prefill_kernel(PrefillParams p)
{
    constexpr int kPfWaves = W;                      // waves per workgroup
    static_assert(CHB == 4 || CHB == 8, "chunk of 4 or 8 blocks");
    static_assert(D >= 1 && D <= 8, "prefetch distance");
    static_assert(NMW == 1 || NMW == 2, "one or two matrices");
    static_assert(CHB % SPS == 0, "steps split a chunk evenly");
    constexpr int SPC = CHB / SPS;                   // steps per chunk (each over all TPW tiles)
    constexpr int NS = D + 1;                        // weight register sets
    constexpr int U = pf_lcm(SPC, NS);               // steps per unrolled loop body
    constexpr int RP = 16 * RB;                      // rows per pass
    constexpr int ROWB = CHB * 256 + 16;             // LDS bytes per staged row
    constexpr int NPC = RP * (CHB / 4);              // 1 KB pieces of a staged chunk
    constexpr int L = TPW * (1 + SPS);               // weight loads per wave and step
    constexpr int WPM = kPfWaves / NMW;              // waves per matrix
    constexpr bool DOWN = NMW == 1;
    static_assert(kPfWaves % NMW == 0, "waves split between the matrices");
    static_assert(2 * RP * ROWB >= WPM * TPW * RP * 16 * 4, "u hand-over fits the activation buffers");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char* xbuf = smem;                                         // [2][RP][ROWB]
    unsigned char* szbase = smem + 2 * RP * ROWB;                       // [waves][NS][TPW][1 KB]
    long long* roff = (long long*)(szbase + kPfWaves * NS * TPW * 1024); // [RP] source element offsets
    int* rpair = (int*)(roff + RP);                                     // [RP] output pair (-1: none)
    float* osum = (float*)(rpair + RP);                                 // [CHB * 2 groups][RP]: sums of x

    const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, tid = threadIdx.x;
    const int g = lane >> 4, lr = lane & 15;
    const int mt = w / WPM, wm = w - mt * WPM;     // this wave's matrix, and its place among that matrix's waves
    const TileGeo geo = tile_geo(FMT_INT4, p.N, p.K);
    const int P = p.m * p.top_k;
    const PlanView pv{p.plan, p.m, p.top_k};
    const int n_union = pv.n_union();
    const int per_unit = WPM * TPW;                  // tiles per work unit
    const int groups = (geo.T + per_unit - 1) / per_unit;
    const int nch_all = (geo.nbk + CHB - 1) / CHB;
    const int kg = max(p.kg, 1);
    const int cpr = (nch_all + kg - 1) / kg;        // chunks per K range
    uint8_t* szw = szbase + (size_t)w * NS * TPW * 1024;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    for (int unit = blockIdx.x; unit < n_union * groups * kg; unit += gridDim.x) {
        const int kr = unit % kg, ug = unit / kg;
        const int u = ug / groups, grp = ug - u * groups;
        const int cbase = kr * cpr;                               // first chunk of this K range
        const int nch = max(0, min(cpr, nch_all - cbase));        // chunks of this K range
        const Item it = resolve_item(pv, true, u, p.m, P, p.topk_ids, p.n_experts);
        if (!it.ok) continue;   // uniform
        const uint8_t* eq = p.tq[mt] + (size_t)it.e * p.tebytes;
        const int nrows = DOWN ? 2 * it.R : it.R;
        int tl[TPW];   // this wave's tiles (clamped; tv: real)
        bool tv[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = grp * per_unit + j * WPM + wm;
            tv[j] = t < geo.T;
            tl[j] = min(t, geo.T - 1);
        }

        for (int r0 = 0; r0 < nrows; r0 += RP) {   // passes of RP rows (one when the entry has <= RP rows)
            const int nr = min(RP, nrows - r0);
            __syncthreads();   // the previous pass's LDS reads are done
            for (int r = tid; r < RP; r += blockDim.x) {
                int pr = -1;
                long long off = 0;
                if (r < nr) {
                    const int li = r0 + r;
                    pr = item_pair(pv, it, DOWN ? li >> 1 : li, P);
                    if (pr >= 0) off = (long long)(DOWN ? 2 * pr + (li & 1) : pr / p.top_k) * p.K;
                }
                roff[r] = off;     // rows past the entry's read row 0 and are never stored
                rpair[r] = pr;
            }
            __syncthreads();

            f32x4 acc[TPW][RB];
#pragma unroll
            for (int j = 0; j < TPW; ++j)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) acc[j][rb] = zero;

            // staging of (range-relative) chunk c into buffer c & 1: 1 KB wave
            // loads, pieces w, w + waves, ... of the chunk's real rows (rows past
            // the pass's rows are not loaded: their MFMA rows are never stored)
            auto stage = [&](int c) {
                unsigned char* dst = xbuf + (size_t)(c & 1) * RP * ROWB;
                for (int q = w; q < NPC; q += kPfWaves) {
                    const int r = q / (CHB / 4), h = q - r * (CHB / 4);
                    if (r >= nr) break;                       // uniform
                    const int kk = min((cbase + c) * CHB * 128 + h * 512 + lane * 8, p.K - 8);
                    lds_dma16(p.src + roff[r] + kk, lds_addr(dst + (size_t)r * ROWB + h * 1024));
                }
            };
            // weights of step s -- chunk s / SPC, blocks SPS * (s % SPC) .. of it --
            // for every tile of the wave: the unit's scale/zero step (direct to the
            // wave's LDS slot (set, tile): a lane needs its tile row's entries,
            // which other lanes would hold) and SPS code steps into register set
            // `set`
            u32x4 wq[NS][TPW][SPS];
            auto load = [&](int st_s, int set, u32x4 (&dq)[TPW][SPS]) {
                const int c = cbase + st_s / SPC, sub = st_s % SPC;
                const int unitk = (c * CHB) >> 3;             // K unit of the chunk (8 blocks)
                const int b0 = ((c * CHB) & 7) + sub * SPS;
#pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    const uint8_t* tb = eq + (size_t)tl[j] * geo.tile_bytes;
                    lds_dma16(tb + (size_t)min(unitk * 9, geo.steps - 1) * kStep + lane * 16,
                              lds_addr(szw + (set * TPW + j) * 1024));
                }
#pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    const uint8_t* tb = eq + (size_t)tl[j] * geo.tile_bytes;
#pragma unroll
                    for (int sb = 0; sb < SPS; ++sb) {
                        const int st = min(unitk * 9 + 1 + b0 + sb, geo.steps - 1);
                        dq[j][sb] = __builtin_nontemporal_load((const u32x4*)(tb + (size_t)st * kStep + lane * 16));
                    }
                }
            };
            auto compute = [&](int c, int sub, int set, const u32x4 (&q)[TPW][SPS], f32x4 (&a)[TPW][RB]) {
                const unsigned char* xb = xbuf + (size_t)(c & 1) * RP * ROWB;
                const int b0 = ((cbase + c) * CHB) & 7;
                // the scale/zero DMAs were issued before this step's code loads and
                // loads retire in order: once the first code register is usable, the
                // slots are written.  The empty asm consumes it (so the compiler's
                // wait for it comes first) and no memory access moves above it.
                asm volatile("" ::"v"(q[0][0][0]) : "memory");
#pragma unroll
                for (int bb = 0; bb < SPS; ++bb) {
                    const int b = sub * SPS + bb;            // block of the chunk
                    if ((cbase + c) * CHB + b >= geo.nbk) break;   // uniform: past K
                    u32x2 sz[TPW];
#pragma unroll
                    for (int j = 0; j < TPW; ++j)
                        sz[j] = *(const u32x2*)(szw + (set * TPW + j) * 1024 + (b0 + b) * 128 + lr * 8);
                    // one 64-input group at a time: the weights of every tile, then per
                    // row block its two MFMA steps of activations (read once for all
                    // tiles) and the group's row sums
#pragma unroll
                    for (int jg = 0; jg < 2; ++jg) {
                        u32x4 lo[TPW], hi[TPW];
                        float sg[TPW], zg[TPW];
#pragma unroll
                        for (int j = 0; j < TPW; ++j) {
                            lo[j] = unpack_int4_biased(q[j][bb][2 * jg]);
                            hi[j] = unpack_int4_biased(q[j][bb][2 * jg + 1]);
                            sg[j] = jg ? bf16hi_f32(sz[j][0]) : bf16lo_f32(sz[j][0]);
                            zg[j] = (jg ? bf16hi_f32(sz[j][1]) : bf16lo_f32(sz[j][1])) + 128.0f;
                        }
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            if (rb * 16 >= nr) break;   // uniform: no rows in this block
                            const unsigned char* xr = xb + (size_t)(rb * 16 + lr) * ROWB + b * 256 + 2 * jg * 64 + g * 16;
                            const u32x4 x0 = *(const u32x4*)xr, x1 = *(const u32x4*)(xr + 64);
                            const f32x4 o = *(const f32x4*)(osum + (b * 2 + jg) * RP + rb * 16 + 4 * g);
#pragma unroll
                            for (int j = 0; j < TPW; ++j) {
                                f32x4 mm = mfma_bf16(x0, lo[j], zero);
                                mm = mfma_bf16(x1, hi[j], mm);
#pragma unroll
                                for (int i = 0; i < 4; ++i) a[j][rb][i] = fmaf(sg[j], fmaf(-zg[j], o[i], mm[i]), a[j][rb][i]);
                            }
                        }
                    }
                }
            };

            // steps s = 0 .. S-1 of this K range (chunk s / SPC, SPC steps each, every
            // step over all TPW tiles); step s + D's weights are requested while step
            // s is multiplied (NS = D + 1 register sets).  Chunk c + 1's rows are
            // requested right after the barrier that opens chunk c, so the wait that
            // opens chunk c + 1 has the SPC steps' loads issued after them still in
            // flight (0 near the end, where fewer were issued); the loads issued
            // before them belong to steps up to D - 1 ahead, so with D - 1 <= SPC
            // that wait holds nothing back that is not needed by then.  The loop is
            // unrolled over U = lcm(SPC, NS) steps so that every register set and
            // block index is known at compile time.  With D >= 2 the compiler's own
            // wait for a step's code registers never waits for rows staged after
            // them.
            const int S = nch * SPC;
            if (S > 0) {   // uniform
            stage(0);
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (d < S) load(d, d % NS, wq[d % NS]);
            for (int s0 = 0; s0 < S; s0 += U) {
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const int st = s0 + k;
                    if (st >= S) break;   // uniform
                    const int c = st / SPC;
                    if (k % SPC == 0) {
                        if (c > 0 && st - 1 + D < S)
                            pf_wait<SPC * L>();
                        else
                            pf_wait<0>();
                        __syncthreads();   // chunk c's rows are in for every wave; chunk c - 1's buffer is free
                        if (c + 1 < nch) stage(c + 1);
                        // each row's sum over each 64-input group of the chunk, once for
                        // every wave (the zero point's term): two threads per sum, 32
                        // inputs each, added in fp32
                        {
                            const unsigned char* xb = xbuf + (size_t)(c & 1) * RP * ROWB;
                            for (int t = tid; t < RP * CHB * 4; t += 64 * W) {
                                const int h = t & 1, gr = (t >> 1) % (CHB * 2), r = (t >> 1) / (CHB * 2);
                                const unsigned char* src = xb + (size_t)r * ROWB + gr * 128 + h * 64;
                                float v = 0.f;
#pragma unroll
                                for (int d4 = 0; d4 < 4; ++d4) {
                                    const u32x4 x4 = *(const u32x4*)(src + d4 * 16);
#pragma unroll
                                    for (int e = 0; e < 4; ++e) v += bf16lo_f32(x4[e]) + bf16hi_f32(x4[e]);
                                }
                                v += __shfl_xor(v, 1);
                                if (h == 0) osum[gr * RP + r] = v;
                            }
                        }
                        __syncthreads();
                    }
                    if (st + D < S) load(st + D, (k + D) % NS, wq[(k + D) % NS]);
                    compute(c, k % SPC, k % NS, wq[k % NS], acc);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            }

            // epilogue: each wave its own tiles
            if constexpr (DOWN) {
#pragma unroll
                for (int j = 0; j < TPW; ++j) {
                    const int n = tl[j] * 16 + lr;
                    if (!tv[j] || n >= p.N) continue;
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        if (rb * 16 >= nr) break;
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const int r = rb * 16 + 4 * g + 2 * h2;   // the hi row of a pair
                            const int pr = r < nr ? rpair[r] : -1;
                            if (pr >= 0)
                                p.part[((size_t)kr * P + pr) * p.N + n] = acc[j][rb][2 * h2] + acc[j][rb][2 * h2 + 1];
                        }
                    }
                }
            } else {
                // u from the up waves to the gate waves of the same tiles, through
                // the (now idle) activation buffers: [tile slot][row][16] fp32
                float* xch = (float*)xbuf;
                __syncthreads();   // every wave is done with the staged rows
                if (mt == 1) {
#pragma unroll
                    for (int j = 0; j < TPW; ++j)
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            if (rb * 16 >= nr) break;
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                xch[((size_t)(j * WPM + wm) * RP + rb * 16 + 4 * g + i) * 16 + lr] = acc[j][rb][i];
                        }
                }
                __syncthreads();
                if (mt == 0) {
#pragma unroll
                    for (int j = 0; j < TPW; ++j) {
                        const int n = tl[j] * 16 + lr;
                        if (!tv[j] || n >= p.N) continue;
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            if (rb * 16 >= nr) break;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int r = rb * 16 + 4 * g + i;
                                const int pr = r < nr ? rpair[r] : -1;
                                if (pr < 0) continue;
                                const float uu = xch[((size_t)(j * WPM + wm) * RP + r) * 16 + lr];
                                const float y = act_f32(p.act, acc[j][rb][i]) * uu;
                                uint16_t hi, lo;
                                split_bf16(y, hi, lo);
                                p.act_out[(size_t)(2 * pr) * p.N + n] = hi;
                                p.act_out[(size_t)(2 * pr + 1) * p.N + n] = lo;
                            }
                        }
                    }
                }
            }
        }
    }
}

}  // namespace ffnq
