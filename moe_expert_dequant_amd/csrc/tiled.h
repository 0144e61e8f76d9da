// tiled.h -- the tiled weight formats of libffnq and the kernels that stream them.
//
// A tiled matrix stores each 16-row tile as a sequence of 1 KB "steps", so that
// every load of the K loop is one wave-wide 16-byte load of 1 KB of
// contiguous memory (full 128-byte lines, one DRAM page run) instead of 16
// rows x 64 bytes.  The row-major formats ([qwen/moe_batch.rs] Affine layout,
// [gemma4/shared_expert.rs] INT8 rows) are converted once by ffnq_pack.
//
//   INT4 affine g64 (K % 128 == 0, nbk = K/128 code blocks of 128 inputs):
//     for each group j of up to 8 code blocks:
//       step 9j      : scale/zero step -- block bi (0..7) of the group, row r:
//                      8 bytes at bi*128 + r*8 = (s pair, z pair) as two
//                      bf16x2 words (groups 2b and 2b+1 of the row)
//       step 9j+1+bi : code block b = 8j+bi -- lane l = 16g + r, dword d
//                      (d = 0..3) holds the codes of row r for inputs
//                      128b + 32d + 8g + e (e = 0..7), code e = 2v in nibble
//                      v and e = 2v+1 in nibble v+4 (the order in which one
//                      shift-and-mask per register widens them)
//   INT8 per-row (K % 64 == 0, nbk = K/64 blocks of 64 inputs):
//     step b : code block b -- lane l = 16g + r, dword 2d+h (d, h = 0..1)
//              holds the codes of row r for inputs 64b + 32d + 8g + 4h + i
//              (i = 0..3) in byte order; after all tiles, the fp32 row
//              scales [T*16] (rows >= N are 0)
//   With these lane layouts MFMA step d of a block reads the inputs
//   [32d, 32d+32) of the block in natural order (lane group g holds
//   32d + 8g .. +7), and for INT4 steps 0-1 and 2-3 each see one group of 64
//   inputs: activations are staged and handed on in natural order.
//   Rows >= N of the last tile are zero codes with zero scales.
//   Experts of a stack follow each other, expert_bytes apart.
//
// Kernels (gu_tiled_kernel: gate and up; down_tiled_kernel: down and tail):
// the waves of a workgroup split a tile's K range by scale/zero groups (INT4)
// or blocks (INT8) and meet in one LDS reduction per tile; they share the
// activation rows staged in LDS; scale/zero steps land in wave-private LDS.
// The register ring of code steps runs across tile boundaries.
#pragma once
#include "qgemm.h"

namespace ffnq {

constexpr int kStep = 1024;   // bytes per matrix and ring step
constexpr int kPfT = 4;       // steps in flight per matrix, tiled kernels

struct TileGeo {
    int T;                  // 16-row tiles
    int nbk;                // code blocks per row
    int ng;                 // INT4 scale/zero groups (0 for INT8)
    int steps;              // 1 KB steps per tile
    long long tile_bytes;
    long long scale_off;    // INT8: offset of the fp32 row scales
    long long expert_bytes;
};

__host__ __device__ inline TileGeo tile_geo(int fmt, int n, int k)
{
    TileGeo g;
    g.T = (n + 15) / 16;
    if (fmt == FMT_INT4) {
        g.nbk = k / 128;
        g.ng = (g.nbk + 7) / 8;
    } else {
        g.nbk = k / 64;
        g.ng = 0;
    }
    g.steps = g.ng + g.nbk;
    g.tile_bytes = (long long)g.steps * kStep;
    g.scale_off = (long long)g.T * g.tile_bytes;
    g.expert_bytes = g.scale_off + (fmt == FMT_INT8 ? ((long long)g.T * 64 + 255) / 256 * 256 : 0);
    return g;
}

// --------------------------------------------------------------------------
// Packing (row-major -> tiled).  One thread per 16-byte chunk of the output.

struct PackParams {
    int fmt, n, k, n_experts;
    const uint8_t* q;       // row-major codes, expert 0
    const void* s;          // INT4: bf16 [N][K/64]; INT8: fp32 [N]
    const uint16_t* z;      // INT4: bf16 [N][K/64]
    long long qe, se;       // per-expert strides: code bytes, scale elements
    uint8_t* dst;
};

__global__ void __launch_bounds__(256) pack_kernel(PackParams p)
{
    const TileGeo geo = tile_geo(p.fmt, p.n, p.k);
    const long long chunks = (long long)p.n_experts * (geo.expert_bytes / 16);
    const long long per_e = geo.expert_bytes / 16;
    const int rowb = p.fmt == FMT_INT4 ? p.k / 2 : p.k;   // code bytes per row
    const int gs = p.k / 64;                               // INT4 scale/zero entries per row
    for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
         c += (long long)gridDim.x * blockDim.x) {
        const int e = (int)(c / per_e);
        const long long off = (c - (long long)e * per_e) * 16;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (off < geo.scale_off) {
            const int tile = (int)(off / geo.tile_bytes);
            const int rem = (int)(off - (long long)tile * geo.tile_bytes);
            const int st = rem >> 10, lane = (rem & 1023) >> 4;
            bool szs = false;
            int blk = st;
            if (p.fmt == FMT_INT4) {
                const int j = st / 9, r = st - 9 * j;
                szs = r == 0;
                blk = szs ? 8 * j + (lane >> 3) : 8 * j + r - 1;
            }
            if (szs) {
                const uint16_t* s = (const uint16_t*)p.s + (size_t)e * p.se;
                const uint16_t* z = p.z + (size_t)e * p.se;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = tile * 16 + 2 * (lane & 7) + h;
                    if (row < p.n && blk < geo.nbk) {
                        const size_t o = (size_t)row * gs + 2 * blk;
                        v[2 * h] = (uint32_t)s[o] | ((uint32_t)s[o + 1] << 16);
                        v[2 * h + 1] = (uint32_t)z[o] | ((uint32_t)z[o + 1] << 16);
                    }
                }
            } else {
                const int row = tile * 16 + (lane & 15), g = lane >> 4;
                if (row < p.n) {
                    const uint8_t* rp = p.q + (size_t)e * p.qe + (size_t)row * rowb;
                    if (p.fmt == FMT_INT4) {
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            // codes 128*blk + 32d + 8g .. +7: four source bytes, each (even code, odd code)
                            const uint32_t sw = *(const uint32_t*)(rp + (size_t)blk * 64 + 16 * d + 4 * g);
                            uint32_t o = 0u;
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                const uint32_t by = (sw >> (8 * b)) & 0xFFu;
                                o |= (by & 0xFu) << (4 * b);
                                o |= (by >> 4) << (4 * b + 16);
                            }
                            v[d] = o;
                        }
                    } else {
#pragma unroll
                        for (int d = 0; d < 2; ++d)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                v[2 * d + h] = *(const uint32_t*)(rp + (size_t)blk * 64 + 32 * d + 8 * g + 4 * h);
                    }
                }
            }
        } else {
            const int row0 = (int)((off - geo.scale_off) / 4);
            const float* s8 = (const float*)p.s + (size_t)e * p.se;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int row = row0 + h;
                v[h] = row < p.n ? __float_as_uint(s8[row]) : 0u;
            }
        }
        *(u32x4*)(p.dst + (size_t)e * geo.expert_bytes + (size_t)off) = v;
    }
}

// --------------------------------------------------------------------------
// LDS layout of the tiled kernels (the host computes the same sizes).

struct TLdsLayout {
    int per_row;
    size_t wsz, rows, orow, red, total;
};

// Lanes of a wave whose accumulators hold staged rows: with one 16-row MFMA
// block and at most 4 staged rows only lanes 0-15 (D rows 0-3) do, and the
// cross-wave reduction keeps just those.
__host__ __device__ inline int red_lanes(int nt, int rows_cap) { return (nt == 1 && rows_cap <= 4) ? 16 : 64; }

__host__ __device__ inline TLdsLayout tiled_lds(int nmat, int fmt, int nbk, int rows_cap, int nwaves,
                                                int red_floats_per_wave)
{
    TLdsLayout l;
    const int BK = fmt == FMT_INT4 ? 128 : 64;
    l.per_row = nbk * BK / 8;
    l.wsz = (size_t)rows_cap * l.per_row * 16;
    l.rows = l.wsz + (fmt == FMT_INT4 ? (size_t)nwaves * nmat * kStep : 0);
    l.orow = l.rows + (size_t)rows_cap * 8;   // int32 output row of each staged row
    l.red = l.orow + (size_t)rows_cap * 4;
    l.red = (l.red + 15) & ~(size_t)15;
    l.total = l.red + (size_t)2 * nwaves * red_floats_per_wave * 4;
    return l;
}

// The layout of a tiled kernel launch, from the launch parameters alone; the
// host sizes the dynamic LDS with this same function.  K is split into KG
// ranges of whole K units (INT4: groups of 8 code blocks; INT8: blocks), so the
// staged activation rows hold at most 8*ceil(ng/KG) (INT4) or ceil(nbk/KG)
// (INT8) blocks.
__host__ __device__ inline int tiled_nbk_max(int fmt, int n, int k, int KG)
{
    const TileGeo g = tile_geo(fmt, n, k);
    return fmt == FMT_INT4 ? 8 * ((g.ng + KG - 1) / KG) : (g.nbk + KG - 1) / KG;
}

__host__ __device__ inline TLdsLayout tiled_launch_lds(int nmat, int fmt, int n, int k, int KG, int rows_cap, int KS,
                                                       int red_floats_per_wave)
{
    return tiled_lds(nmat, fmt, tiled_nbk_max(fmt, n, k, KG), rows_cap, KS, red_floats_per_wave);
}

// Sixteen fp32 row scales of an INT8 tile through the scalar cache (a
// wave-uniform 64-byte read), then the lane's own row.  Issued from inline asm
// with its own lgkmcnt wait, so the vector-memory counter bookkeeping of the
// ring is not involved.
__device__ __forceinline__ float tile_row_scale(const uint8_t* p, int lr)
{
    typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint64_t au = ((uint64_t)hi << 32) | lo;
    u32x16 v;
    asm volatile("s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(au) : "memory");
    uint32_t r = v[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) r = lr == k ? v[k] : r;
    return __uint_as_float(r);
}

// --------------------------------------------------------------------------
// Staging of activation rows 0..Rc-1, blocks [kb0, kb0+nbk), into the
// swizzled slot layout (slot r*per_row + (j ^ s(r)) holds piece j of row r),
// with coalesced 16-byte loads through registers.  Pieces are handed out in
// batches of kSR per thread; every batch issues all of its loads before its
// stores, and the last batch's stores are deferred to finish(), so that the
// caller can issue the weight ring in between and one wait covers both.
// Row r's source offset is direct0 + r*rstride when direct0 >= 0 (rows that
// follow each other in the source: no row table needed, so staging can start
// before the table is written), else the row table L.roff[r].
constexpr int kSR = 8;

template <int FMT>
struct RegStager {
    const Lds& L;
    const uint16_t* src;
    int Rc, kb0, xslots, nthr;
    long long direct0, rstride;
    u32x4 v[kSR];
    int slot[kSR];

    __device__ __forceinline__ RegStager(const Lds& l, const uint16_t* s, int rc, int k0, int nt, long long d0,
                                         long long rs)
        : L(l), src(s), Rc(rc), kb0(k0), xslots(rc * l.per_row), nthr(nt), direct0(d0), rstride(rs) {}

    __device__ __forceinline__ void load(int base)
    {
        constexpr int BK = FmtT<FMT>::BK, CPB = BK / 8;
        const int per_row = L.per_row;
#pragma unroll
        for (int i = 0; i < kSR; ++i) {
            const int sl = min(base + (int)threadIdx.x + i * nthr, xslots - 1);
            const int rr = sl / per_row, jp = sl - rr * per_row;
            const int lb = jp / CPB, ci = (jp - lb * CPB) ^ ((rr >> L.swz_shift) & L.swz_mask);
            const long long ro = direct0 >= 0 ? direct0 + rr * rstride : L.roff[rr];
            v[i] = *(const u32x4*)(src + ro + (kb0 + lb) * BK + ci * 8);
            slot[i] = sl;
        }
    }
    __device__ __forceinline__ void store()
    {
#pragma unroll
        for (int i = 0; i < kSR; ++i) *(u32x4*)(L.x + (size_t)slot[i] * 16) = v[i];
    }
    // all batches but the last, then the last batch's loads.  The K range must
    // not be empty (per_row > 0): the host never splits K into more ranges than
    // it has K units.
    __device__ __forceinline__ void begin()
    {
        const int step = kSR * nthr;
        int base = 0;
        for (; base + step < xslots; base += step) {
            load(base);
            store();
        }
        load(base);
    }
    __device__ __forceinline__ void finish() { store(); }
};

// --------------------------------------------------------------------------
// One code step of tiled matrices (natural input order, see the layout
// above): widen() turns the ring slot's codes (and the step's scale/zero
// pair) into MFMA operands; contract() runs the matrix-core work.  (Refilling
// the slot between the two halves keeps more loads in flight but holds the
// widened operands across the refill; measured, the lower occupancy costs
// more than the overlap gains.)  INT4 accumulates per
// element in `acc` (fp32 scalars, so that a partial-row update does not
// rebuild a vector); INT8 accumulates on the MFMA in `tot`/`one`.
template <int FMT, int NMAT>
struct Widened;
template <int NMAT>
struct Widened<FMT_INT4, NMAT> {
    u32x4 bw[NMAT][4];
    float sg[NMAT][2], zg[NMAT][2];
};
template <int NMAT>
struct Widened<FMT_INT8, NMAT> {
    u32x4 bw[NMAT][2];
};

template <int FMT, int NMAT>
__device__ __forceinline__ void widen(const u32x4 (&cq)[NMAT], const uint32_t (&cs)[NMAT], const uint32_t (&cz)[NMAT],
                                      Widened<FMT, NMAT>& W)
{
    if constexpr (FMT == FMT_INT4) {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
#pragma unroll
            for (int d = 0; d < 4; ++d) W.bw[mt][d] = unpack_int4_biased(cq[mt][d]);
            W.sg[mt][0] = bf16lo_f32(cs[mt]);
            W.sg[mt][1] = bf16hi_f32(cs[mt]);
            W.zg[mt][0] = bf16lo_f32(cz[mt]) + 128.0f;
            W.zg[mt][1] = bf16hi_f32(cz[mt]) + 128.0f;
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const u32x2 p0 = unpack_int8_biased(cq[mt][2 * d]);
                const u32x2 p1 = unpack_int8_biased(cq[mt][2 * d + 1]);
                W.bw[mt][d] = u32x4{p0[0], p0[1], p1[0], p1[1]};
            }
    }
}

template <int FMT, int NMAT, int NT, int MT, typename XLoad>
__device__ __forceinline__ void contract(const Widened<FMT, NMAT>& W, XLoad&& xl, float (&acc)[NMAT][NT][4],
                                         f32x4 (&tot)[NMAT][NT], f32x4 (&one)[NT])
{
    constexpr int MTC = (NT == 1) ? MT : 4;
    constexpr int STEPS = FmtT<FMT>::STEPS;
    const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
        u32x4 xs[STEPS];
        xl(tb, xs);
        if constexpr (FMT == FMT_INT4) {
#pragma unroll
            for (int jg = 0; jg < 2; ++jg) {
                f32x4 o = mfma_bf16(xs[2 * jg], ones, zero);
                o = mfma_bf16(xs[2 * jg + 1], ones, o);
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) {
                    f32x4 a = mfma_bf16(xs[2 * jg], W.bw[mt][2 * jg], zero);
                    a = mfma_bf16(xs[2 * jg + 1], W.bw[mt][2 * jg + 1], a);
#pragma unroll
                    for (int i = 0; i < MTC; ++i)
                        acc[mt][tb][i] = fmaf(W.sg[mt][jg], fmaf(-W.zg[mt][jg], o[i], a[i]), acc[mt][tb][i]);
                }
            }
        } else {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                one[tb] = mfma_bf16(xs[d], ones, one[tb]);
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) tot[mt][tb] = mfma_bf16(xs[d], W.bw[mt][d], tot[mt][tb]);
            }
        }
    }
}

// --------------------------------------------------------------------------
// The register ring of one wave: `ntiles` tiles, steps [s0, s1) of each, NMAT
// matrices, PF steps in flight.  base(i, mt) is the (uniform) address of tile
// i of matrix mt.  prime() issues the first PF steps; it runs before anything
// else the workgroup does for these tiles (row tables, barrier, activation
// staging), so that HBM is busy from the start of the kernel.
template <int NMAT, int PF, typename Base>
struct TRing {
    Base base;
    int ntiles, s0, len;
    int it = 0, is = 0;       // issue cursor: tile, step (relative to s0)
    const uint8_t* ib[NMAT];
    u32x4 rq[PF][NMAT];

    __device__ __forceinline__ TRing(Base b, int nt, int first, int last)
        : base(b), ntiles(nt), s0(first), len(last - first) {}

    __device__ __forceinline__ void set_base(int t)
    {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) ib[mt] = base(t, mt) + (size_t)s0 * kStep + (threadIdx.x & 63) * 16;
    }
    __device__ __forceinline__ void issue(int slot)
    {
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
            rq[slot][mt] = __builtin_nontemporal_load((const u32x4*)(ib[mt] + (size_t)is * kStep));
        if (is + 1 < len) {
            ++is;
        } else if (it + 1 < ntiles) {
            ++it;
            is = 0;
            set_base(it);
        }   // past the last step: the last step is loaded again (never consumed)
    }
    __device__ __forceinline__ void prime()
    {
        if (ntiles * len > 0) {
            set_base(0);
#pragma unroll
            for (int s = 0; s < PF; ++s) issue(s);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
};

// The tiled stream of one wave over the ring's tiles.  The ring is primed and
// stage.begin() has issued the activation staging; stage.finish() stores the
// last staged batch and a barrier publishes it.  end(i, tot, one) runs after the
// last step of tile i (every wave of the workgroup calls it the same number
// of times, also a wave whose step range is empty).
template <int FMT, int NMAT, int NT, int MT, int PF, typename Ring, typename Stage, typename End>
__device__ __forceinline__ void tiled_stream(Ring& ring, int kb0, const Lds& L, int Rc, uint8_t* wsz, Stage stage,
                                             End end)
{
    constexpr int BK = FmtT<FMT>::BK, STEPS = FmtT<FMT>::STEPS;
    const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15;
    const int ntiles = ring.ntiles, s0 = ring.s0, len = ring.len;
    const int total = ntiles * len;

    uint32_t xrow[NT], xoff_b[NT], xoff_a[NT];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
        const int row = min(tb * 16 + lr, Rc - 1);
        const int sw = (row >> L.swz_shift) & L.swz_mask;
        xrow[tb] = (uint32_t)(row * L.per_row) * 16u;
        xoff_a[tb] = (uint32_t)((sw >> 2) & (STEPS - 1));
        xoff_b[tb] = 16u * (uint32_t)((g ^ sw) & 3);
    }

    f32x4 tot[NMAT][NT], one[NT];
    float acc[NMAT][NT][4];
    auto zero_acc = [&]() {
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
            one[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                tot[mt][tb] = one[tb];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][tb][i] = 0.f;
            }
        }
    };
    zero_acc();

    // consume cursor
    int ct = 0, cs = 0;
    auto consume = [&](int slot) {
        const int s = s0 + cs;
        int b = s;
        bool szs = false;
        if constexpr (FMT == FMT_INT4) {
            const int j = s / 9, r = s - 9 * j;
            szs = r == 0;
            b = 8 * j + r - 1;
        }
        if (szs) {   // scale/zero step: to the wave's LDS
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) *(u32x4*)(wsz + mt * kStep + lane * 16) = ring.rq[slot][mt];
        } else {
            const int lb = b - kb0;
            uint32_t cs_[NMAT], cz_[NMAT];
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                if constexpr (FMT == FMT_INT4) {
                    const u32x2 v = *(const u32x2*)(wsz + mt * kStep + (b & 7) * 128 + lr * 8);
                    cs_[mt] = v[0];
                    cz_[mt] = v[1];
                } else {
                    cs_[mt] = 0u;
                    cz_[mt] = 0u;
                }
            }
            Widened<FMT, NMAT> W;
            widen<FMT, NMAT>(ring.rq[slot], cs_, cz_, W);
            auto xl = [&](int tb, u32x4 (&xs)[STEPS]) {
                const uint8_t* xb = L.x + xrow[tb] + (uint32_t)lb * (BK * 2) + xoff_b[tb];
#pragma unroll
                for (int d = 0; d < STEPS; ++d) xs[d] = *(const u32x4*)(xb + 64u * ((uint32_t)d ^ xoff_a[tb]));
            };
            contract<FMT, NMAT, NT, MT>(W, xl, acc, tot, one);
        }
        if (++cs == len) {
            if constexpr (FMT == FMT_INT4) {
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                    for (int tb = 0; tb < NT; ++tb)
                        tot[mt][tb] = f32x4{acc[mt][tb][0], acc[mt][tb][1], acc[mt][tb][2], acc[mt][tb][3]};
            }
            end(ct, tot, one);
            zero_acc();
            cs = 0;
            ++ct;
        }
    };

    stage.finish();
    __syncthreads();

    if (len <= 0) {
        for (int i = 0; i < ntiles; ++i) end(i, tot, one);
        return;
    }
    int p = 0;
    for (; p + PF <= total; p += PF) {
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            consume(s);
            __builtin_amdgcn_sched_barrier(0);
            ring.issue(s);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int s = 0; s < PF - 1; ++s)
        if (p + s < total) consume(s);
}

// --------------------------------------------------------------------------
// The workgroup body shared by the tiled kernels.  Work units are
// (item, tile): an item is the whole batch (dense) or one union entry of the
// plan (routed: one expert with its pairs).  A workgroup walks units
// blockIdx.x, +gridDim.x, ...; consecutive units of the same item form a run,
// for which the activation rows stay staged and the ring runs on from tile to
// tile.  Grid row blockIdx.y takes a range of K (whole scale/zero groups for
// INT4, blocks for INT8).  Two ways to share it among the KS waves:
//   K split (!TS): the waves split the K range of every tile; at each
//     tile end their partial sums meet in LDS (double-buffered by tile parity)
//     and the tile's outputs are finished.
//   tile split (TS): every wave covers the whole K range and the waves
//     take turns over the run's tiles; each wave finishes its own tiles from
//     its accumulators, with no reduction or barrier.  The staged activation
//     rows then serve KS tiles at once.
//
// HILO: the staged rows are hi/lo pairs of one activation row (the down
// projection): row 2r + 1 is added to row 2r before the finish.
// rows(it, c0, tid, roff, orows): writes the source offset of staged row tid
//   (tid < Rc) and, for the first row of each output row, its output row.
// finish(orow, n, v): output row orow, matrix row n, the fp32 sums v[NMAT].

struct TiledJob {
    const uint8_t* tq[2];     // tiled matrices (expert 0)
    long long tebytes;
    int N, K, KG;
    const uint16_t* src;      // staged rows' source array
    int rows_cap;             // staged rows per pass
    int rows_per_item_mul;    // staged rows per item row (2 with HILO)
    bool routed;
    PlanView pv;
    int m, act_rows;
    const int32_t* topk_ids;
    int n_experts;
    int KS, G;                // waves per workgroup, workgroups along x
    int bx, by;               // this workgroup (the kernel may run several jobs side by side)
};

template <int FMT, int NMAT, int NT, int MT, bool HILO, bool TS, typename Rows, typename Finish>
__device__ __forceinline__ void tiled_body(const TiledJob& J, Rows rows, Finish finish)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int PER = HILO ? NT * 2 : NMAT * NT * 4;   // reduction floats per lane and wave
    const int KS = J.KS;
    const int w = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x, nthr = 64 * KS;
    const TileGeo geo = tile_geo(FMT, J.N, J.K);
    const int T = geo.T;
    const int nun = FMT == FMT_INT4 ? geo.ng : geo.nbk;   // K units: groups or blocks
    // K range of this grid row and of this wave (32-bit: nun * KG is small)
    const int U0 = nun * J.by / J.KG, U1 = nun * (J.by + 1) / J.KG;
    const int kb0 = FMT == FMT_INT4 ? 8 * U0 : U0;
    const int kb1 = FMT == FMT_INT4 ? min(8 * U1, geo.nbk) : U1;
    const int u0w = TS ? U0 : U0 + (U1 - U0) * w / KS, u1w = TS ? U1 : U0 + (U1 - U0) * (w + 1) / KS;
    const int s0 = FMT == FMT_INT4 ? 9 * u0w : u0w;
    const int s1 = FMT == FMT_INT4 ? min(9 * u1w, geo.steps) : u1w;

    const int n_units = (J.routed ? J.pv.n_union() : 1) * T;
    const int G = J.G;
    const int RL = red_lanes(NT, J.rows_cap);   // lanes kept by the reduction (uniform)
    for (int u0 = J.bx; u0 < n_units;) {
        int item = 0, run;
        if (!J.routed) {
            run = (n_units - u0 + G - 1) / G;   // every unit belongs to the one item
        } else {
            item = u0 / T;
            run = 0;
            while (u0 + run * G < n_units && (u0 + run * G) / T == item) ++run;
        }
        const Item it = resolve_item(J.pv, J.routed, item, J.m, J.act_rows, J.topk_ids, J.n_experts);
        if (it.ok) {
            const uint8_t* eq[NMAT];
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) eq[mt] = J.tq[mt] + (size_t)it.e * J.tebytes;
            const int t0 = u0 - item * T;   // tile of the run's first unit; later ones are G tiles apart
            // this wave's units of the run: all (K split) or w, w + KS, ... (tile split)
            const int wi0 = TS ? w : 0, wstep = TS ? KS : 1;
            const int nrun = TS ? (run > w ? (run - w + KS - 1) / KS : 0) : run;
            auto tile_at = [&](int i) { return t0 + (wi0 + i * wstep) * G; };
            auto base = [&](int i, int mt) { return eq[mt] + (size_t)tile_at(i) * geo.tile_bytes; };
            const int RR = J.rows_per_item_mul * it.R;
            for (int c0 = 0; c0 < RR; c0 += J.rows_cap) {
                TRing<NMAT, kPfT, decltype(base)> ring(base, nrun, s0, s1);
                const TLdsLayout LL = tiled_launch_lds(NMAT, FMT, J.N, J.K, J.KG, J.rows_cap, KS, TS ? 0 : PER * RL);
                Lds L;
                L.x = smem;
                L.per_row = (kb1 - kb0) * (FmtT<FMT>::BK / 8);
                set_swizzle<FMT>(L);
                L.sz = nullptr;
                L.zstride = 1;
                long long* roff = (long long*)(smem + LL.rows);
                L.roff = roff;
                int* orows = (int*)(smem + LL.orow);
                uint8_t* wsz = smem + LL.wsz + (size_t)w * NMAT * kStep;
                float* red = (float*)(smem + LL.red);
                const size_t red_half = (size_t)KS * PER * RL;
                const int Rc = min(J.rows_cap, RR - c0);
                auto end = [&](int i, f32x4 (&tot)[NMAT][NT], f32x4 (&one)[NT]) {
                    const int tile = tile_at(i);
                    const int row0 = tile * 16;
                    if constexpr (TS) {   // this wave's own tile: finish from the accumulators
                        constexpr int MTC = (NT == 1) ? MT : 4;
                        const int l16 = lane >> 4, nl = lane & 15, n = row0 + nl;
                        float sc[NMAT];
#pragma unroll
                        for (int mt = 0; mt < NMAT; ++mt)
                            sc[mt] = FMT == FMT_INT8 ? tile_row_scale(eq[mt] + geo.scale_off + (size_t)tile * 64, nl) : 1.0f;
                        if (n < J.N) {
#pragma unroll
                            for (int tb = 0; tb < NT; ++tb) {
                                if constexpr (HILO) {
#pragma unroll
                                    for (int h2 = 0; h2 < 2; ++h2) {
                                        const int xr = tb * 16 + 4 * l16 + 2 * h2;   // hi row of a hi/lo pair
                                        if (xr >= Rc) continue;
                                        const int orow = orows[xr >> 1];
                                        if (orow < 0) continue;
                                        float vh = tot[0][tb][2 * h2], vl = tot[0][tb][2 * h2 + 1];
                                        if constexpr (FMT == FMT_INT8) {
                                            vh = fmaf(-128.0f, one[tb][2 * h2], vh);
                                            vl = fmaf(-128.0f, one[tb][2 * h2 + 1], vl);
                                        }
                                        float v[NMAT];
                                        v[0] = sc[0] * (vh + vl);
                                        finish(orow, n, v);
                                    }
                                } else {
#pragma unroll
                                    for (int i2 = 0; i2 < MTC; ++i2) {
                                        const int xr = tb * 16 + 4 * l16 + i2;
                                        if (xr >= Rc) continue;
                                        const int orow = orows[xr];
                                        if (orow < 0) continue;
                                        float v[NMAT];
#pragma unroll
                                        for (int mt = 0; mt < NMAT; ++mt) {
                                            float h = tot[mt][tb][i2];
                                            if constexpr (FMT == FMT_INT8) h = fmaf(-128.0f, one[tb][i2], h);
                                            v[mt] = sc[mt] * h;
                                        }
                                        finish(orow, n, v);
                                    }
                                }
                            }
                        }
                        return;
                    }
                    float* rb = red + (size_t)(i & 1) * red_half;
#pragma unroll
                    for (int tb = 0; tb < NT; ++tb) {
                        if constexpr (HILO) {
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                float vh = tot[0][tb][2 * h2], vl = tot[0][tb][2 * h2 + 1];
                                if constexpr (FMT == FMT_INT8) {
                                    vh = fmaf(-128.0f, one[tb][2 * h2], vh);
                                    vl = fmaf(-128.0f, one[tb][2 * h2 + 1], vl);
                                }
                                if (lane < RL) rb[((w * PER) + tb * 2 + h2) * RL + lane] = vh + vl;
                            }
                        } else {
#pragma unroll
                            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                                for (int i2 = 0; i2 < 4; ++i2) {
                                    float v = tot[mt][tb][i2];
                                    if constexpr (FMT == FMT_INT8) v = fmaf(-128.0f, one[tb][i2], v);
                                    if (lane < RL) rb[((w * PER) + (mt * NT + tb) * 4 + i2) * RL + lane] = v;
                                }
                        }
                    }
                    __syncthreads();
                    float sc[NMAT];
                    const int Tc = HILO ? Rc >> 1 : Rc;   // output rows of this pass
                    for (int ii = tid; ii < Tc * 16; ii += nthr) {
                        const int tr = ii >> 4, nl = ii & 15, n = row0 + nl;
                        if constexpr (FMT == FMT_INT8) {
#pragma unroll
                            for (int mt = 0; mt < NMAT; ++mt)
                                sc[mt] = tile_row_scale(eq[mt] + geo.scale_off + (size_t)tile * 64, nl);
                        }
                        if (n >= J.N) continue;
                        const int orow = orows[tr];
                        if (orow < 0) continue;
                        float v[NMAT];
                        const int xr = HILO ? 2 * tr : tr;
                        const int tb = xr >> 4, rl = xr & 15;
                        const int ln = ((rl >> 2) << 4) | nl;
#pragma unroll
                        for (int mt = 0; mt < NMAT; ++mt) {
                            float h = 0.f;
                            for (int ww = 0; ww < KS; ++ww) {
                                const int slot = HILO ? (ww * PER + tb * 2 + ((rl & 3) >> 1))
                                                      : (ww * PER + (mt * NT + tb) * 4 + (rl & 3));
                                h += rb[slot * RL + ln];
                            }
                            v[mt] = FMT == FMT_INT8 ? sc[mt] * h : h;
                        }
                        finish(orow, n, v);
                    }
                };
                if (!J.routed) {
                    // dense: staged row r is source row c0 + r, so the activation loads go out
                    // first (ahead of the weight burst), then the ring, then the row table
                    RegStager<FMT> stage(L, J.src, Rc, kb0, nthr, (long long)c0 * J.K, J.K);
                    stage.begin();
                    __builtin_amdgcn_sched_barrier(0);
                    ring.prime();
                    if (tid < Rc) rows(it, c0, tid, roff, orows);
                    tiled_stream<FMT, NMAT, NT, MT, kPfT>(ring, kb0, L, Rc, wsz, stage, end);
                } else {
                    ring.prime();
                    if (tid < Rc) rows(it, c0, tid, roff, orows);
                    __syncthreads();
                    RegStager<FMT> stage(L, J.src, Rc, kb0, nthr, -1, 0);
                    stage.begin();
                    __builtin_amdgcn_sched_barrier(0);
                    tiled_stream<FMT, NMAT, NT, MT, kPfT>(ring, kb0, L, Rc, wsz, stage, end);
                }
                __syncthreads();
            }
        }
        u0 += run * G;
    }
}

// gate + up + activation: f(gate)*up per (token or pair, inter row) in fp32,
// written as the bf16 hi/lo pair (act row 2r = hi, 2r+1 = lo) in the order the
// down kernel reads (natural for tiled down weights).
//
// Both tiled kernels read the kernel arguments they use into SGPRs at entry:
// an empty asm statement takes them all as inputs, so they are fetched up
// front instead of in the block that first needs each (dependent round trips
// that would delay the first weight loads of every wave).  Inputs only: the
// values, and what the compiler knows of the pointers, are unchanged.  The
// launch shape comes in the arguments too (ks, grid) rather than from the
// dispatch packet.
template <int FMT, int NT, int MT, bool TS>
__device__ __forceinline__ void gu_tiled_run(const GUParams& p, int bx, int by)
{
    asm volatile("" ::"s"(p.tgate), "s"(p.tup), "s"(p.tebytes), "s"(p.N), "s"(p.K), "s"(p.x), "s"(p.rows_cap),
                 "s"(p.plan), "s"(p.m), "s"(p.top_k), "s"(p.act_rows), "s"(p.topk_ids), "s"(p.n_experts), "s"(p.act),
                 "s"(p.dfmt), "s"(p.act_out), "s"(p.gate_vec), "s"(p.logit), "s"(p.ks), "s"(p.grid));
    TiledJob J;
    J.tq[0] = p.tgate;
    J.tq[1] = p.tup;
    J.tebytes = p.tebytes;
    J.N = p.N;
    J.K = p.K;
    J.KG = 1;
    J.src = p.x;
    J.rows_cap = p.rows_cap;
    J.rows_per_item_mul = 1;
    const int32_t* plan = p.plan;
    J.routed = plan != nullptr;
    J.m = p.m;
    const int top_k = p.top_k;
    J.pv = PlanView{plan, J.m, top_k};
    J.act_rows = p.act_rows;
    J.topk_ids = p.topk_ids;
    J.n_experts = p.n_experts;
    J.KS = p.ks;
    J.G = p.grid;
    J.bx = bx;
    J.by = by;
    const int act = p.act, dfmt = p.dfmt;
    uint16_t* const act_out = p.act_out;
    const uint16_t* const gate_vec = p.gate_vec;
    float* const logit = p.logit;
    auto rows = [&](const Item& it, int c0, int t, long long* roff, int* orows) {
        int tok = c0 + t, orow = c0 + t;
        if (J.routed) {
            orow = item_pair(J.pv, it, c0 + t, J.act_rows);
            tok = orow < 0 ? 0 : orow / top_k;
        }
        roff[t] = (long long)tok * J.K;
        orows[t] = orow;
    };
    auto finish = [&](int orow, int n, const float (&v)[2]) {
        const float a = act_f32(act, v[0]) * v[1];
        uint16_t hi, lo;
        split_bf16(a, hi, lo);
        const size_t o = (size_t)(2 * orow) * J.N + cons_index(dfmt, n);
        act_out[o] = hi;
        act_out[o + J.N] = lo;
    };
    tiled_body<FMT, 2, NT, MT, false, TS>(J, rows, finish);
    // shared-expert gate logits (read by the down kernel's tail): one
    // workgroup, after its tiles
    if (gate_vec != nullptr && bx == 0 && by == 0) {
        const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, nw = J.KS;
        for (int t = w; t < J.m; t += nw) {
            double acc = 0.0;
            for (int i = lane; i < J.K; i += 64)
                acc += (double)bf16_f32(gate_vec[i]) * (double)bf16_f32(J.src[(size_t)t * J.K + i]);
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (lane == 0) logit[t] = (float)acc;
        }
    }
}

template <int FMT, int NT, int MT, bool TS>
__global__ void __launch_bounds__(512) gu_tiled_kernel(GUParams p)
{
    gu_tiled_run<FMT, NT, MT, TS>(p, blockIdx.x, blockIdx.y);
}

// Two gate/up jobs in one launch (e.g. a layer's shared expert and its routed
// experts, both reading x): grid row 0 runs job a, row 1 job b, each over its
// own p.grid workgroups along x.  The jobs share the template shape and the
// waves per workgroup; each lays out its own LDS within the launch's allocation.
template <int FMT, int NT, int MT>
__global__ void __launch_bounds__(512) gu_tiled_kernel2(GUParams a, GUParams b)
{
    const bool jb = blockIdx.y != 0;
    const GUParams& p = jb ? b : a;
    if ((int)blockIdx.x >= p.grid) return;
    gu_tiled_run<FMT, NT, MT, false>(p, blockIdx.x, 0);
}

// down + tail: h per (token or pair, hidden row), finished by down_finish
// (tail, or fp32 partials when K is split or for the routed and RMSNorm tails).
// bx, by: the workgroup's position along x (tiles) and y (K range).
template <int FMT, int NT, int MT, bool TS>
__device__ __forceinline__ void down_tiled_run(const DownParams& p, int bx, int by)
{
    asm volatile("" ::"s"(p.tdown), "s"(p.tebytes), "s"(p.N), "s"(p.K), "s"(p.KG), "s"(p.act), "s"(p.rows_cap),
                 "s"(p.plan), "s"(p.m), "s"(p.top_k), "s"(p.act_rows), "s"(p.topk_ids), "s"(p.n_experts), "s"(p.tail),
                 "s"(p.out), "s"(p.part), "s"(p.logit), "s"(p.ks), "s"(p.grid));
    TiledJob J;
    J.tq[0] = p.tdown;
    J.tq[1] = nullptr;
    J.tebytes = p.tebytes;
    J.N = p.N;
    J.K = p.K;
    J.KG = p.KG;
    J.src = p.act;
    J.rows_cap = p.rows_cap;
    J.rows_per_item_mul = 2;
    const int32_t* plan = p.plan;
    J.routed = plan != nullptr;
    J.m = p.m;
    J.pv = PlanView{plan, J.m, p.top_k};
    J.act_rows = p.act_rows;
    J.topk_ids = p.topk_ids;
    J.n_experts = p.n_experts;
    J.KS = p.ks;
    J.G = p.grid;
    J.bx = bx;
    J.by = by;
    auto rows = [&](const Item& it, int c0, int t, long long* roff, int* orows) {
        const int xr = c0 + t, li = xr >> 1;
        int arow = li;
        if (J.routed) arow = item_pair(J.pv, it, li, J.act_rows);
        roff[t] = (long long)(2 * (arow < 0 ? 0 : arow) + (xr & 1)) * J.K;
        if ((t & 1) == 0) orows[t >> 1] = arow;
    };
    auto finish = [&](int orow, int n, const float (&v)[1]) { down_finish(p, by, orow, n, v[0]); };
    tiled_body<FMT, 1, NT, MT, true, TS>(J, rows, finish);
}

template <int FMT, int NT, int MT, bool TS>
__global__ void __launch_bounds__(512) down_tiled_kernel(DownParams p)
{
    down_tiled_run<FMT, NT, MT, TS>(p, blockIdx.x, blockIdx.y);
}

// Two down jobs in one launch (a layer's shared expert and its routed experts),
// both with the K split: workgroups [0, na) run job a, laid out as a.grid
// workgroups along x for each of its K ranges; the rest run job b likewise.
// The jobs share the template shape and the waves per workgroup; each lays out
// its own LDS within the launch's allocation.
template <int FMT, int NT, int MT>
__global__ void __launch_bounds__(512) down_tiled_kernel2(DownParams a, DownParams b, int na)
{
    const int bid = (int)blockIdx.x;
    if (bid < na) {
        down_tiled_run<FMT, NT, MT, false>(a, bid % a.grid, bid / a.grid);
    } else {
        const int r = bid - na;
        down_tiled_run<FMT, NT, MT, false>(b, r % b.grid, r / b.grid);
    }
}

}  // namespace ffnq
