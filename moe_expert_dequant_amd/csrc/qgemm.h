// qgemm.h -- the dequant-fused small-M GEMM/GEMV kernels of libffnq (gfx950).
//
// One engine serves every projection of the quantized gated FFN
// ([llama/dense.rs] gate/up/down GEMVs; [gemma4/shared_expert.rs] the
// batched M-row GEMMs; [qwen/moe_batch.rs] the routed phase-1 and phase-2
// dispatches).  A wave owns a 16-row tile of one (or two) weight matrices and
// streams its packed codes from HBM with 16-byte loads, several blocks ahead.
// Codes are widened in registers to bf16 "128 + code" (exact) and multiplied
// on the MFMA unit (v_mfma_f32_16x16x32_bf16) against up to 16 activation
// rows per token block; the code bias and the INT4 zero point are removed
// with a second MFMA against a ones operand (which yields sum(x) per group):
//     sum_k s (q - z) x_k = s * (sum_k (128 + q) x_k - (128 + z) sum_k x_k)
// INT4 groups (64 inputs) are kept apart by a lane permutation
// (v_permlane32_swap) so that each MFMA step sees one group only.
//
// Activations reach the MFMA in "consumption order" (see nat_run/cons_pos):
// gate/up stage x in LDS in that order; the activation written by gate/up
// for the down projection is already in that order, so the down kernel reads
// it straight from L2 (decode sizes) or stages it in LDS (prefill sizes).
#pragma once
#include "device.h"

namespace ffnq {

enum { FMT_NATURAL = 0, FMT_INT8 = 1, FMT_INT4 = 2 };

template <int FMT>
struct FmtT;
template <>
struct FmtT<FMT_INT4> { static constexpr int BK = 128, STEPS = 4; };   // inputs per 64-byte block row
template <>
struct FmtT<FMT_INT8> { static constexpr int BK = 64, STEPS = 2; };

// A quantized matrix on the device (expert 0 of a stack for routed calls).
struct MatDev {
    const uint8_t* q;
    const void* s;
    const uint16_t* z;
    int n, k;
    long long qe;   // bytes of codes per expert
    long long se;   // scale (and zero) elements per expert
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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

// dfmt 0 (FMT_NATURAL): the tiled formats consume activations in natural order.
__device__ __forceinline__ int cons_index(int dfmt, int k)
{
    if (dfmt == FMT_INT4) return (k & ~127) + cons_pos<FMT_INT4>(k & 127);
    if (dfmt == FMT_INT8) return (k & ~63) + cons_pos<FMT_INT8>(k & 63);
    return k;
}

// --------------------------------------------------------------------------
// The streaming engine.
//
// A workgroup owns one 16-row tile of NMAT weight matrices and a range of K
// blocks; its KS waves split the range (wave ks takes local blocks ks,
// ks+KS, ...).  The only global loads inside the K loop are the 16-byte code
// loads, kept PF blocks ahead in a register ring.  Everything else comes from
// LDS, staged once per item: the tile's INT4 scale/zero pairs and the
// activation rows of the range (the host splits K across workgroups so that
// they fit).  The ring is primed before the staging so that the first weight
// loads overlap it.

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // two bf16 1.0
constexpr int kSX = 8;                          // 16-byte activation pieces per thread per staging batch
constexpr int kSZ = 4;                          // scale/zero pairs per thread and matrix per staging batch
constexpr int kPfGU = 4;                        // code blocks in flight, gate/up kernel
constexpr int kPfDN = 6;                        // code blocks in flight, down kernel

template <int NMAT>
struct TileW {
    const uint8_t* q[NMAT];   // uniform: codes of row 0 of the tile, block kb0
    uint32_t vq;              // lane: row offset + 16 * lane group
};

struct KRange {
    int kb0, nbk;   // first block and number of blocks of the workgroup's K range
    int KS, ks;     // waves splitting the range, this wave
};

// The waves of a workgroup split the range in pairs of consecutive blocks
// (pair p goes to wave p % KS): a lane's 16-byte loads of blocks 2p and 2p+1
// are the two halves of one 128-byte line of its row, so each line is fetched
// by one wave in consecutive loads.  Returns the number of blocks of wave ks;
// its q-th block is pair_block(ks, KS, q) and every such block is < nbk.
__device__ __forceinline__ int pair_count(int nbk, int KS, int ks)
{
    const int np = (nbk + 1) >> 1;
    if (ks >= np) return 0;
    const int npw = (np - ks + KS - 1) / KS;
    const bool odd_tail = (nbk & 1) && ((np - 1) % KS == ks);
    return 2 * npw - (odd_tail ? 1 : 0);
}
__device__ __forceinline__ int pair_block(int ks, int KS, int q) { return 2 * (ks + (q >> 1) * KS) + (q & 1); }

struct Lds {
    uint8_t* x;             // activation slots [Rc][per_row] of 16 bytes, swizzled within each row
    int per_row;            // 16-byte pieces per row (nbk * BK / 8)
    int swz_mask, swz_shift;  // piece swizzle of row r: s(r) = (r >> swz_shift) & swz_mask
    uint8_t* sz;            // INT4 scale/zero dword pairs [NMAT][16][zstride] (8 bytes each)
    int zstride;            // odd, >= nbk
    const long long* roff;  // element offset of each staged activation row in its source array
};

// Piece swizzle: piece j of row r sits at slot r*per_row + (j ^ s(r)).  For
// INT4 (16 pieces per block) s(r) = r & 15 puts the 16 rows read by one
// ds_read_b128 on 16 distinct bank groups; INT8 keeps the swizzle inside its
// 8-piece blocks.
template <int FMT>
__device__ __forceinline__ void set_swizzle(Lds& L)
{
    if constexpr (FMT == FMT_INT4) {
        L.swz_mask = 15;
        L.swz_shift = 0;
    } else {
        L.swz_mask = 7;
        L.swz_shift = (L.per_row & 15) ? 1 : 0;
    }
}


// One K block of the tile: the codes cq of NMAT matrices (this lane's 16
// bytes each) against NT token blocks of activations, read per token block
// by xl(tb, xs) so that only one block's activations are live at a time.
template <int FMT, int NMAT, int NT, int MT, typename XLoad>
__device__ __forceinline__ void compute_block(const u32x4 (&cq)[NMAT], const uint32_t (&cs)[NMAT],
                                              const uint32_t (&cz)[NMAT], XLoad&& xl, f32x4 (&tot)[NMAT][NT],
                                              f32x4 (&one)[NT])
{
    constexpr int MTC = (NT == 1) ? MT : 4;
    constexpr int STEPS = FmtT<FMT>::STEPS;
    const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == FMT_INT4) {
        u32x4 bw[NMAT][4];
        float sg[NMAT][2], zg[NMAT][2];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
            // lanes 0-31 hold inputs [0,64) of the block, lanes 32-63 [64,128):
            // swap so that steps 0,1 hold group 0 and steps 2,3 group 1
            auto a = __builtin_amdgcn_permlane32_swap(cq[mt][0], cq[mt][2], false, false);
            auto b = __builtin_amdgcn_permlane32_swap(cq[mt][1], cq[mt][3], false, false);
            bw[mt][0] = unpack_int4_biased(a[0]);
            bw[mt][1] = unpack_int4_biased(b[0]);
            bw[mt][2] = unpack_int4_biased(a[1]);
            bw[mt][3] = unpack_int4_biased(b[1]);
            sg[mt][0] = bf16lo_f32(cs[mt]);
            sg[mt][1] = bf16hi_f32(cs[mt]);
            zg[mt][0] = bf16lo_f32(cz[mt]) + 128.0f;
            zg[mt][1] = bf16hi_f32(cz[mt]) + 128.0f;
        }
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
            u32x4 xs[STEPS];
            xl(tb, xs);
#pragma unroll
            for (int jg = 0; jg < 2; ++jg) {
                f32x4 o = mfma_bf16(xs[2 * jg], ones, zero);
                o = mfma_bf16(xs[2 * jg + 1], ones, o);
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) {
                    f32x4 a = mfma_bf16(xs[2 * jg], bw[mt][2 * jg], zero);
                    a = mfma_bf16(xs[2 * jg + 1], bw[mt][2 * jg + 1], a);
#pragma unroll
                    for (int i = 0; i < MTC; ++i)
                        tot[mt][tb][i] = fmaf(sg[mt][jg], fmaf(-zg[mt][jg], o[i], a[i]), tot[mt][tb][i]);
                }
            }
        }
    } else {
        u32x4 bw[NMAT][2];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const u32x2 p0 = unpack_int8_biased(cq[mt][2 * d]);
                const u32x2 p1 = unpack_int8_biased(cq[mt][2 * d + 1]);
                bw[mt][d] = u32x4{p0[0], p0[1], p1[0], p1[1]};
            }
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
            u32x4 xs[STEPS];
            xl(tb, xs);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                one[tb] = mfma_bf16(xs[d], ones, one[tb]);
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) tot[mt][tb] = mfma_bf16(xs[d], bw[mt][d], tot[mt][tb]);
            }
        }
    }
}

// Issues the staging of activation rows 0..Rc-1 of the K range (and, with
// SZ, the INT4 scale/zero pairs of the tile) as direct global->LDS loads: one
// wave instruction fills 64 consecutive LDS slots, lane i slot base+i.  Wave
// w issues instructions w, w+KS, ...  Nothing waits here; the caller waits on
// the vector memory counter and then on a barrier.  NATX: the source rows are
// natural-order x and the chunks are gathered in consumption order (INT4
// chunks are permuted when read); otherwise the source is already in
// consumption order.
template <int FMT, bool NATX, int NMAT>
__device__ __forceinline__ void stage_issue(const Lds& L, const uint16_t* __restrict__ src, int Rc, int kb0, int nbk,
                                            bool SZ, const MatDev (&mats)[NMAT], int e, int row0, int n, int KS,
                                            int w)
{
    constexpr int BK = FmtT<FMT>::BK, CPB = BK / 8;
    const int lane = threadIdx.x & 63;
    const int per_row = L.per_row;
    const int xslots = Rc * per_row;
    const int nxi = uniform((xslots + 63) >> 6);
    for (int i = w; i < nxi; i += KS) {
        const int slot = (i << 6) + lane;
        if (slot < xslots) {
            const int rr = slot / per_row, jp = slot - rr * per_row;
            const int lb = jp / CPB, ci = (jp - lb * CPB) ^ ((rr >> L.swz_shift) & L.swz_mask);
            const uint16_t* g = src + L.roff[rr] + (kb0 + lb) * BK + (NATX ? nat_run<FMT>(ci) : ci * 8);
            lds_dma16(g, lds_addr(L.x + (i << 10)));
        }
    }
    if constexpr (FMT == FMT_INT4) {
        if (SZ) {
            const int K = mats[0].k;
            const int zs = L.zstride;
            const int zslots = 2 * NMAT * 16 * zs;
            const int nzi = uniform((zslots + 63) >> 6);
            for (int i = w; i < nzi; i += KS) {
                const int slot = (i << 6) + lane;
                const int q = slot >> 1;
                const int mt = q / (16 * zs), rem = q - mt * 16 * zs;
                const int r = rem / zs, lb = rem - r * zs;
                if (slot < zslots && lb < nbk) {
                    const bool m1 = NMAT > 1 && mt != 0;
                    const uint16_t* zb = m1 ? mats[NMAT - 1].z : mats[0].z;
                    const uint16_t* sb = (const uint16_t*)(m1 ? mats[NMAT - 1].s : mats[0].s);
                    const long long se = m1 ? mats[NMAT - 1].se : mats[0].se;
                    const uint16_t* g = ((slot & 1) ? zb : sb) + (size_t)e * se + (size_t)min(row0 + r, n - 1) * (K / 64) +
                                        2 * (kb0 + lb);
                    lds_dma4(g, lds_addr(L.sz + (i << 8)));
                }
            }
        }
    }
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The K loop of this wave.  `stage` issues the staging loads (no waits);
// the ring is primed after it, so that waiting for the staging
// (vmcnt <= PF*NMAT) leaves the primed code loads in flight.
template <int FMT, int NMAT, int NT, int MT, int PF, bool NATX, typename Stage>
__device__ __forceinline__ void run_tile(const TileW<NMAT>& t, const KRange& kr, const Lds& L, int Rc, Stage stage,
                                         f32x4 (&tot)[NMAT][NT], f32x4 (&one)[NT])
{
    constexpr int BK = FmtT<FMT>::BK, STEPS = FmtT<FMT>::STEPS;
    const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    const int nbw = pair_count(kr.nbk, kr.KS, kr.ks);

    // LDS addresses of this lane's activation pieces: row base, and the
    // swizzled position of chunk 4d+g inside a block
    uint32_t xrow[NT];
    uint32_t xoff_b[NT], xoff_a[NT];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
        const int row = min(tb * 16 + lr, Rc - 1);
        const int sw = (row >> L.swz_shift) & L.swz_mask;
        xrow[tb] = (uint32_t)(row * L.per_row) * 16u;
        xoff_a[tb] = (uint32_t)((sw >> 2) & (STEPS - 1));
        xoff_b[tb] = 16u * (uint32_t)((g ^ sw) & 3);
    }
    const uint8_t* szrow = L.sz + (size_t)lr * L.zstride * 8;

    u32x4 rq[PF][NMAT];
    auto issue = [&](int slot, int q) {
        q = q < nbw ? q : nbw - 1;
        const int lb = pair_block(kr.ks, kr.KS, q);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
            rq[slot][mt] = __builtin_nontemporal_load((const u32x4*)(t.q[mt] + (size_t)lb * 64 + t.vq));
    };
    auto consume = [&](int slot, int q) {
        const int lb = pair_block(kr.ks, kr.KS, q);
        auto xl = [&](int tb, u32x4 (&xs)[STEPS]) {
            const uint8_t* xb = L.x + xrow[tb] + (uint32_t)lb * (BK * 2) + xoff_b[tb];
#pragma unroll
            for (int d = 0; d < STEPS; ++d) {
                xs[d] = *(const u32x4*)(xb + 64u * ((uint32_t)d ^ xoff_a[tb]));
                if constexpr (NATX && FMT == FMT_INT4) xs[d] = permute_0415(xs[d]);
            }
        };
        uint32_t cs[NMAT], cz[NMAT];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
            if constexpr (FMT == FMT_INT4) {
                const u32x2 v = *(const u32x2*)(szrow + ((size_t)mt * 16 * L.zstride + lb) * 8);
                cs[mt] = v[0];
                cz[mt] = v[1];
            } else {
                cs[mt] = 0u;
                cz[mt] = 0u;
            }
        }
        compute_block<FMT, NMAT, NT, MT>(rq[slot], cs, cz, xl, tot, one);
    };

    stage();
    __builtin_amdgcn_sched_barrier(0);
    if (nbw > 0) {
#pragma unroll
        for (int s = 0; s < PF; ++s) issue(s, s);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (nbw > 0)
        wait_vmcnt<PF * NMAT>();
    else
        wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");   // no LDS read moves above the barrier
    __builtin_amdgcn_sched_barrier(0);
    int q = 0;
    for (; q + PF <= nbw; q += PF) {
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            consume(s, q + s);
            __builtin_amdgcn_sched_barrier(0);
            issue(s, q + s + PF);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int s = 0; s < PF - 1; ++s)
        if (q + s < nbw) consume(s, q + s);
}

// Lane-level code addressing for rows row0..row0+15 (clamped to n-1) from block kb0.
template <int FMT, int NMAT>
__device__ __forceinline__ void tile_weights(TileW<NMAT>& t, const MatDev (&mats)[NMAT], int e, int row0, int n,
                                             int K, int kb0)
{
    const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    const int wrow = min(row0 + lr, n - 1) - row0;
    const size_t qrow = FMT == FMT_INT4 ? (size_t)K / 2 : (size_t)K;
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) {
        const MatDev& M = mats[mt];
        t.q[mt] = M.q + (size_t)e * M.qe + (size_t)row0 * qrow + (size_t)kb0 * 64;
    }
    t.vq = (uint32_t)(wrow * qrow + 16 * g);
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

struct Item {
    int e, R, pb;
    bool ok;
};

// Work item: union entry u (routed) or the whole batch (dense).
__device__ __forceinline__ Item resolve_item(const PlanView& pv, bool routed, int u, int m, int act_rows,
                                             const int32_t* topk_ids, int n_experts)
{
    Item it{0, m, 0, true};
    if (!routed) return it;
    it.pb = pv.slot_begin(u);
    it.R = pv.slot_begin(u + 1) - it.pb;
    if (it.R <= 0) {
        it.ok = false;
        return it;
    }
    const int p0 = pv.slot_pair(it.pb);
    if (p0 < 0 || p0 >= act_rows) {
        it.ok = false;
        return it;
    }
    it.e = topk_ids[p0];
    it.ok = it.e >= 0 && it.e < n_experts;
    return it;
}

// Pair index of row li of an item (-1 if the plan entry is out of range).
__device__ __forceinline__ int item_pair(const PlanView& pv, const Item& it, int li, int act_rows)
{
    const int pr = pv.slot_pair(it.pb + li);
    return (pr >= 0 && pr < act_rows) ? pr : -1;
}

// Dynamic LDS layout shared by the kernels (the host computes the same sizes).
struct LdsLayout {
    int per_row, zstride;
    size_t sz, rows, red, total;
};

__host__ __device__ inline LdsLayout lds_layout(int nmat, int fmt, int nbk, int rows_cap, int KS,
                                                int red_floats_per_lane)
{
    LdsLayout l;
    const int BK = fmt == FMT_INT4 ? 128 : 64;
    l.per_row = nbk * BK / 8;
    l.zstride = nbk | 1;
    l.sz = (size_t)rows_cap * l.per_row * 16;
    l.rows = l.sz + (fmt == FMT_INT4 ? (size_t)nmat * 16 * l.zstride * 8 : 0);
    l.rows = (l.rows + 15) & ~(size_t)15;
    l.red = l.rows + (size_t)rows_cap * 8;
    l.red = (l.red + 15) & ~(size_t)15;
    l.total = l.red + (size_t)KS * red_floats_per_lane * 64 * 4;
    return l;
}

// --------------------------------------------------------------------------
// gate + up + activation.  One workgroup = KS waves on one 16-row tile over
// the whole of K.  The activation f(gate)*up is computed in double, rounded
// to fp32, split into a bf16 hi/lo pair and written in the consumption order
// of the down matrix: act row 2r holds hi, row 2r+1 lo, of activation row r
// (token or pair).

struct GUParams {
    MatDev gate, up;
    int N, K;                  // inter, hidden
    int act;                   // 1 SiLU, 2 GELU(tanh)
    int dfmt;                  // down matrix format: order of the act rows
    const uint16_t* x;         // [m][K] bf16
    int m;
    int rows_cap;              // activation rows per pass (<= 16*NT)
    const int32_t* plan;       // routed mode: items are (union entry, tile)
    int top_k;
    const int32_t* topk_ids;
    int n_experts;
    uint16_t* act_out;         // [2*act_rows][N]
    int act_rows;              // m, or m*top_k
    const uint16_t* gate_vec;  // dense shared-expert gate: logit[t] = <gate_vec, x_t>
    float* logit;
    const uint8_t* tgate;      // tiled formats: packed gate / up (expert 0)
    const uint8_t* tup;
    long long tebytes;         // tiled bytes per expert
    int ks, grid;              // tiled kernels: waves per workgroup and gridDim.x, as launched
    // routed burst job that routes its own batch (the plan is then written by it):
    const float* logits;       // [m][n_experts] router logits, or null (plan given)
    const float* escale;       // [n_experts] per-expert scale, or null
    int cap;                   // slot cap of the sub-batches
    int32_t* ids_out;          // [m][top_k] route ids, written by the job's workgroup 0
    float* w_out;              // [m][top_k] route weights, likewise
    int32_t* plan_out;         // the plan, likewise (plan == plan_out)
};

template <int FMT, int NT, int MT>
__global__ void __launch_bounds__(512) gu_kernel(GUParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int BK = FmtT<FMT>::BK;
    constexpr int PER = 2 * NT * 4;   // reduction floats per lane and wave
    const int KS = uniform(blockDim.x >> 6);
    const int w = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lr = lane & 15;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int NB = p.K / BK;
    const int tiles = (p.N + 15) >> 4;
    const LdsLayout LL = lds_layout(2, FMT, NB, p.rows_cap, KS, PER);
    Lds L;
    L.x = smem;
    L.per_row = NB * (BK / 8);
    set_swizzle<FMT>(L);
    L.sz = smem + LL.sz;
    L.zstride = NB | 1;
    long long* roff = (long long*)(smem + LL.rows);
    L.roff = roff;
    float* red = (float*)(smem + LL.red);
    const KRange kr{0, NB, KS, w};

    if (p.gate_vec != nullptr && blockIdx.x == 0) {
        for (int t = w; t < p.m; t += KS) {
            double acc = 0.0;
            for (int i = lane; i < p.K; i += 64)
                acc += (double)bf16_f32(p.gate_vec[i]) * (double)bf16_f32(p.x[(size_t)t * p.K + i]);
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (lane == 0) p.logit[t] = (float)acc;
        }
    }

    const bool routed = p.plan != nullptr;
    PlanView pv{p.plan, p.m, p.top_k};
    const int n_items = routed ? pv.n_union() * tiles : tiles;
    const MatDev mats[2] = {p.gate, p.up};
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int tile = item % tiles;
        const Item it = resolve_item(pv, routed, item / tiles, p.m, p.act_rows, p.topk_ids, p.n_experts);
        if (!it.ok) continue;
        const int row0 = tile * 16;
        TileW<2> t;
        tile_weights<FMT, 2>(t, mats, it.e, row0, p.N, p.K, 0);
        for (int c0 = 0; c0 < it.R; c0 += p.rows_cap) {
            const int Rc = min(p.rows_cap, it.R - c0);
            if (tid < Rc) {
                int tok = c0 + tid;
                if (routed) {
                    const int pr = item_pair(pv, it, c0 + tid, p.act_rows);
                    tok = pr < 0 ? 0 : pr / p.top_k;
                }
                roff[tid] = (long long)tok * p.K;
            }
            __syncthreads();
            auto stage = [&]() {
                stage_issue<FMT, true, 2>(L, p.x, Rc, 0, NB, c0 == 0, mats, it.e, row0, p.N, KS, w);
            };
            f32x4 tot[2][NT], one[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
                one[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                tot[0][tb] = one[tb];
                tot[1][tb] = one[tb];
            }
            run_tile<FMT, 2, NT, MT, kPfGU, true>(t, kr, L, Rc, stage, tot, one);

            // per-wave partials (INT8: row scale and code bias applied)
            float sc[2] = {1.0f, 1.0f};
            if constexpr (FMT == FMT_INT8) {
                const int n = min(row0 + lr, p.N - 1);
                sc[0] = ((const float*)p.gate.s)[(size_t)it.e * p.gate.se + n];
                sc[1] = ((const float*)p.up.s)[(size_t)it.e * p.up.se + n];
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int tb = 0; tb < NT; ++tb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = tot[mt][tb][i];
                        if constexpr (FMT == FMT_INT8) v = sc[mt] * fmaf(-128.0f, one[tb][i], v);
                        red[((w * PER) + (mt * NT + tb) * 4 + i) * 64 + lane] = v;
                    }
            __syncthreads();
            for (int ii = tid; ii < Rc * 16; ii += nthr) {
                const int rr = ii >> 4, nl = ii & 15, n = row0 + nl;
                if (n >= p.N) continue;
                const int tb = rr >> 4, rl = rr & 15;
                const int ln = ((rl >> 2) << 4) | nl, i = rl & 3;
                float gs = 0.f, us = 0.f;
                for (int ww = 0; ww < KS; ++ww) {
                    gs += red[((ww * PER) + (0 * NT + tb) * 4 + i) * 64 + ln];
                    us += red[((ww * PER) + (1 * NT + tb) * 4 + i) * 64 + ln];
                }
                const float a = (float)(act_f64(p.act, (double)gs) * (double)us);
                uint16_t hi, lo;
                split_bf16(a, hi, lo);
                int orow = c0 + rr;
                if (routed) {
                    orow = item_pair(pv, it, c0 + rr, p.act_rows);
                    if (orow < 0) continue;
                }
                const size_t o = (size_t)(2 * orow) * p.N + cons_index(p.dfmt, n);
                p.act_out[o] = hi;
                p.act_out[o + p.N] = lo;
            }
            __syncthreads();
        }
    }
}

// --------------------------------------------------------------------------
// down + tail.  One workgroup = KS waves on one 16-row tile over the K range
// of grid row blockIdx.y.  The activation rows are the interleaved hi/lo act
// rows of the item's tokens (or pairs), so a lane holds the hi and lo sums of
// one token in registers i and i+1.  With one K range the tail is applied
// here; otherwise (and for the RMSNORM and routed tails) the workgroup writes
// its fp32 partial h to part[range][row][n] for the kernel that follows.

enum { TAIL_NONE = 0, TAIL_RESIDUAL = 1, TAIL_RMSNORM = 2, TAIL_SIGMOID = 3, TAIL_PAIR = 4,
       TAIL_PART = 5 };   // TAIL_PART: fp32 partials only, for a later kernel to finish

struct DownParams {
    MatDev down;
    int N, K;                  // hidden, inter
    const uint16_t* act;       // [2*act_rows][K] consumption order, hi/lo interleaved
    int act_rows;
    int m;
    int rows_cap;              // act rows per pass (even, <= 16*NT)
    int KG;                    // K ranges (gridDim.y)
    const int32_t* plan;       // routed mode
    int top_k;
    const int32_t* topk_ids;
    int n_experts;
    int tail;
    uint16_t* out;             // [m][N] bf16
    float* part;               // [KG][rows][N] fp32 partial h (rows: m tokens or act_rows pairs)
    const float* logit;        // [m] (SIGMOID)
    const uint8_t* tdown;      // tiled formats: packed down (expert 0)
    long long tebytes;         // tiled bytes per expert
    int ks, grid;              // tiled kernels: waves per workgroup and gridDim.x, as launched
};

// by: the K range whose partial sum h is.
__device__ __forceinline__ void down_finish(const DownParams& p, int by, int t, int n, float h)
{
    if (p.KG > 1 || p.tail == TAIL_PAIR || p.tail == TAIL_RMSNORM || p.tail == TAIL_PART) {
        const size_t rows = p.tail == TAIL_PAIR ? (size_t)p.act_rows : (size_t)p.m;
        p.part[((size_t)by * rows + t) * p.N + n] = h;
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
__global__ void __launch_bounds__(512) down_kernel(DownParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int PER = NT * 2;   // token sums per lane and wave
    const int KS = uniform(blockDim.x >> 6);
    const int w = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lr = lane & 15;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int NB = p.K / FmtT<FMT>::BK;
    const int kb0 = (int)(((long long)NB * blockIdx.y) / p.KG), kb1 = (int)(((long long)NB * (blockIdx.y + 1)) / p.KG);
    const int nbk = kb1 - kb0;
    const int nbk_max = (NB + p.KG - 1) / p.KG;
    const int tiles = (p.N + 15) >> 4;
    const LdsLayout LL = lds_layout(1, FMT, nbk_max, p.rows_cap, KS, PER);
    Lds L;
    L.x = smem;
    L.per_row = nbk * (FmtT<FMT>::BK / 8);   // this range; the layout is sized for the longest
    set_swizzle<FMT>(L);
    L.sz = smem + LL.sz;
    L.zstride = nbk | 1;
    long long* roff = (long long*)(smem + LL.rows);
    L.roff = roff;
    float* red = (float*)(smem + LL.red);
    const KRange kr{kb0, nbk, KS, w};

    const bool routed = p.plan != nullptr;
    PlanView pv{p.plan, p.m, p.top_k};
    const int n_items = routed ? pv.n_union() * tiles : tiles;
    const MatDev mats[1] = {p.down};
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int tile = item % tiles;
        const Item it = resolve_item(pv, routed, item / tiles, p.m, p.act_rows, p.topk_ids, p.n_experts);
        if (!it.ok) continue;
        const int row0 = tile * 16;
        TileW<1> t;
        tile_weights<FMT, 1>(t, mats, it.e, row0, p.N, p.K, kb0);
        float sc = 1.0f;
        if constexpr (FMT == FMT_INT8) sc = ((const float*)p.down.s)[(size_t)it.e * p.down.se + min(row0 + lr, p.N - 1)];
        const int R2 = 2 * it.R;
        for (int c0 = 0; c0 < R2; c0 += p.rows_cap) {
            const int Rc = min(p.rows_cap, R2 - c0);   // even
            if (tid < Rc) {
                const int xr = c0 + tid, li = xr >> 1;
                int arow = li;
                if (routed) {
                    arow = item_pair(pv, it, li, p.act_rows);
                    if (arow < 0) arow = 0;
                }
                roff[tid] = (long long)(2 * arow + (xr & 1)) * p.K;
            }
            __syncthreads();
            auto stage = [&]() {
                stage_issue<FMT, false, 1>(L, p.act, Rc, kb0, nbk, c0 == 0, mats, it.e, row0, p.N, KS, w);
            };
            f32x4 tot[1][NT], one[NT];
#pragma unroll
            for (int tb = 0; tb < NT; ++tb) {
                one[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                tot[0][tb] = one[tb];
            }
            run_tile<FMT, 1, NT, MT, (NT >= 4 ? 4 : kPfDN), false>(t, kr, L, Rc, stage, tot, one);

            // lane: weight row row0+lr, act rows tb*16 + 4g + i; hi (i even) + lo (i odd)
#pragma unroll
            for (int tb = 0; tb < NT; ++tb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    float vh = tot[0][tb][2 * h2], vl = tot[0][tb][2 * h2 + 1];
                    if constexpr (FMT == FMT_INT8) {
                        vh = sc * fmaf(-128.0f, one[tb][2 * h2], vh);
                        vl = sc * fmaf(-128.0f, one[tb][2 * h2 + 1], vl);
                    }
                    red[((w * PER) + tb * 2 + h2) * 64 + lane] = vh + vl;
                }
            __syncthreads();
            const int Tc = Rc >> 1;   // tokens in this pass
            for (int ii = tid; ii < Tc * 16; ii += nthr) {
                const int tr = ii >> 4, nl = ii & 15, n = row0 + nl;
                if (n >= p.N) continue;
                const int xr = 2 * tr;                 // hi row within the pass
                const int tb = xr >> 4, rl = xr & 15;
                const int ln = ((rl >> 2) << 4) | nl, h2 = (rl & 3) >> 1;
                float h = 0.f;
                for (int ww = 0; ww < KS; ++ww) h += red[((ww * PER) + tb * 2 + h2) * 64 + ln];
                const int li = (c0 >> 1) + tr;
                int trow = li;
                if (routed) {
                    trow = item_pair(pv, it, li, p.act_rows);
                    if (trow < 0) continue;
                }
                down_finish(p, blockIdx.y, trow, n, h);
            }
            __syncthreads();
        }
    }
}

}  // namespace ffnq
