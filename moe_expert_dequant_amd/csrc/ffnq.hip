// ffnq.hip -- the C ABI of libffnq: argument checks, workspace layout, launch
// configuration and kernel launches.  Every check runs on the host before the
// first launch; the library allocates nothing and synchronises nothing.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "ffnq.h"
#include "device.h"
#include "qgemm.h"
#include "prefill.h"
#include "route.h"
#include "stream.h"
#include "tail.h"
#include "tiled.h"

namespace {

using namespace ffnq;

constexpr size_t kLdsBudget = 80 * 1024;   // two workgroups per CU (160 KB of LDS)
constexpr size_t kLdsBig = 152 * 1024;     // one workgroup per CU (prefill-sized items)
constexpr size_t kLdsMax = 160 * 1024;     // LDS of one gfx950 CU (one workgroup per CU)
constexpr int kBigRows = 12;               // activation rows per item from which the prefill shapes apply

// Rows per work item: every token (dense), or the pairs of one expert of the
// union on average (routed; an estimate: a plan of one sub-batch has at most
// min(pairs, experts) union entries, one split by the slot cap may have more).
int rows_per_item(bool dense, int m, int top_k, int n_experts)
{
    if (dense) return m;
    const long long P = (long long)m * top_k;
    const long long u = std::max<long long>(1, std::min<long long>(P, n_experts));
    return (int)((P + u - 1) / u);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Per-thread timing switch (ffnq_set_phase_events): start/stop events of the
// gate/up kernel (ev[0], ev[1]) and of the down kernel (ev[2], ev[3]),
// recorded by the kernel dispatch itself (hipExtLaunchKernel).
thread_local hipEvent_t* t_phase_ev = nullptr;

hipEvent_t phase_event(int i) { return t_phase_ev ? t_phase_ev[i] : nullptr; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool is_tiled(int f) { return f == FFNQ_FMT_INT8_ROW_TILED || f == FFNQ_FMT_INT4_AFFINE_G64_TILED; }
bool is_int4(int f) { return f == FFNQ_FMT_INT4_AFFINE_G64 || f == FFNQ_FMT_INT4_AFFINE_G64_TILED; }

int block_k(int fmt) { return is_int4(fmt) ? 128 : 64; }

// library format code -> kernel format code
int to_fmt(int f) { return is_int4(f) ? ffnq::FMT_INT4 : ffnq::FMT_INT8; }
int to_fmt_dev(int f) { return to_fmt(f); }

// Compute units of the current device, cached per device ordinal.
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int check_mat(const ffnq_qmat& w, bool* unsupported)
{
    if (w.fmt != FFNQ_FMT_INT8_ROW && w.fmt != FFNQ_FMT_INT4_AFFINE_G64 && !is_tiled(w.fmt)) {
        *unsupported = true;
        return FFNQ_ERR_UNSUPPORTED;
    }
    if (w.n <= 0 || w.k <= 0 || w.k % 64 != 0) return FFNQ_ERR_INVALID;
    if (!w.q) return FFNQ_ERR_INVALID;
    if (misaligned(w.q)) return FFNQ_ERR_INVALID;
    if (!is_tiled(w.fmt)) {
        if (!w.s) return FFNQ_ERR_INVALID;
        if (w.fmt == FFNQ_FMT_INT4_AFFINE_G64 && !w.z) return FFNQ_ERR_INVALID;
        if (misaligned(w.s) || (w.z && misaligned(w.z))) return FFNQ_ERR_INVALID;
    }
    if (is_int4(w.fmt) && w.k % 128 != 0) {
        *unsupported = true;
        return FFNQ_ERR_UNSUPPORTED;
    }
    return FFNQ_OK;
}

int check_ffn(const ffnq_ffn* f, int hidden, int inter)
{
    if (!f) return FFNQ_ERR_INVALID;
    if (hidden <= 0 || inter <= 0) return FFNQ_ERR_INVALID;
    bool uns = false;
    int worst = FFNQ_OK;
    for (const ffnq_qmat* w : {&f->gate, &f->up, &f->down}) {
        const int rc = check_mat(*w, &uns);
        if (rc == FFNQ_ERR_INVALID) return rc;
        if (rc != FFNQ_OK) worst = rc;
    }
    if (f->gate.n != inter || f->up.n != inter || f->gate.k != hidden || f->up.k != hidden) return FFNQ_ERR_INVALID;
    if (f->down.n != hidden || f->down.k != inter) return FFNQ_ERR_INVALID;
    if (worst != FFNQ_OK) return worst;
    if (f->gate.fmt != f->up.fmt) return FFNQ_ERR_UNSUPPORTED;
    if (is_tiled(f->gate.fmt) != is_tiled(f->down.fmt)) return FFNQ_ERR_UNSUPPORTED;
    return FFNQ_OK;
}

long long tiled_expert_bytes(const ffnq_qmat& w)
{
    return tile_geo(to_fmt(w.fmt), w.n, w.k).expert_bytes;
}

MatDev mat_dev(const ffnq_qmat& w)
{
    MatDev d;
    d.q = static_cast<const uint8_t*>(w.q);
    d.s = w.s;
    d.z = static_cast<const uint16_t*>(w.z);
    d.n = w.n;
    d.k = w.k;
    if (w.fmt == FFNQ_FMT_INT4_AFFINE_G64) {
        d.qe = (long long)w.n * (w.k / 2);
        d.se = (long long)w.n * (w.k / 64);
    } else {
        d.qe = (long long)w.n * w.k;
        d.se = w.n;
    }
    return d;
}

// ---------------------------------------------------------------------------
// launch configuration

constexpr int kRefCUs = 256;       // K-split heuristic reference (keeps workspace sizes device-independent)
constexpr int kKSMax = 8;          // waves per workgroup (upper bound used for LDS sizing)

struct KConfig {
    int nt, mt, ks, rows_cap, kg;
    size_t lds;
    int grid;   // tiled kernels: workgroups along x
    int ts;     // tiled kernels: waves take turns over tiles (1) or split K (0)
};

KConfig gu_config(int fmt, int K, int N, long long items_est, int rows_total, int cus)
{
    KConfig c{};
    const int NB = K / block_k(fmt);
    const int rp = std::max(1, std::min(rows_total, 32));
    c.nt = rp <= 16 ? 1 : 2;
    c.mt = c.nt == 2 ? 4 : (rp <= 1 ? 1 : (rp <= 2 ? 2 : 4));
    c.rows_cap = std::min(rp, 16 * c.nt);
    c.kg = 1;
    const long long tiles = (N + 15) / 16;
    const long long target = (long long)cus * 12;
    int ks = 1;
    while (ks < kKSMax && items_est * tiles * ks * 2 <= target && ks * 2 <= NB) ks *= 2;
    c.ks = ks;
    for (;;) {
        c.lds = lds_layout(2, to_fmt_dev(fmt), NB, c.rows_cap, c.ks, 2 * c.nt * 4).total;
        if (c.lds <= kLdsBudget || c.rows_cap <= 1) break;
        --c.rows_cap;
    }
    return c;
}

// K ranges of the down projection: enough for the activation slice of a
// range to fit LDS, and enough workgroups when the matrix has few row tiles.
int down_kg(int fmt, int K, int N, int rows_total)
{
    const int NB = K / block_k(fmt);
    const int r2 = 2 * std::max(1, rows_total);
    const int nt = std::min(r2, 64) <= 16 ? 1 : (std::min(r2, 64) <= 32 ? 2 : 4);
    const int rows_cap = std::min(std::min(r2, 64), 16 * nt);
    const long long tiles = (N + 15) / 16;
    int kg = (int)std::max<long long>(1, (kRefCUs + tiles - 1) / tiles);
    kg = std::min(kg, NB);
    while (kg < NB && lds_layout(1, to_fmt_dev(fmt), (NB + kg - 1) / kg, rows_cap, kKSMax, 2 * nt).total > kLdsBudget)
        ++kg;
    return kg;
}

KConfig down_config(int fmt, int K, int N, long long items_est, int rows_total, int cus)
{
    KConfig c{};
    const int NB = K / block_k(fmt);
    const int r2 = 2 * std::max(1, rows_total);
    const int rp = std::min(r2, 64);
    c.nt = rp <= 16 ? 1 : (rp <= 32 ? 2 : 4);
    c.mt = c.nt > 1 ? 4 : (rp <= 2 ? 2 : 4);
    c.rows_cap = std::min(rp, 16 * c.nt);
    c.kg = down_kg(fmt, K, N, rows_total);
    const int nbk = (NB + c.kg - 1) / c.kg;
    const long long tiles = (N + 15) / 16;
    const long long target = (long long)cus * 12;
    int ks = 1;
    while (ks < kKSMax && items_est * tiles * c.kg * ks * 2 <= target && ks * 2 <= nbk) ks *= 2;
    c.ks = ks;
    c.lds = lds_layout(1, to_fmt_dev(fmt), nbk, c.rows_cap, c.ks, 2 * c.nt).total;
    return c;
}

// ---------------------------------------------------------------------------
// kernel dispatch over the template parameters

#define FFNQ_GU_CASE(F, NT_, MT_)                                                              \
    if (fmt == F && c.nt == NT_ && c.mt == MT_) {                                              \
        hipExtLaunchKernelGGL((gu_kernel<F, NT_, MT_>), grid, block, c.lds, stream, phase_event(0), \
                              phase_event(1), 0, prm);                                          \
        return true;                                                                           \
    }

bool launch_gu(int fmt, const KConfig& c, long long items, int N, hipStream_t stream, const GUParams& prm)
{
    const long long tiles = (N + 15) / 16;
    const dim3 grid((unsigned)std::min<long long>(items * tiles, 65535)), block(64 * c.ks);
    FFNQ_GU_CASE(FMT_INT4, 1, 1) FFNQ_GU_CASE(FMT_INT4, 1, 2) FFNQ_GU_CASE(FMT_INT4, 1, 4)
    FFNQ_GU_CASE(FMT_INT4, 2, 4) FFNQ_GU_CASE(FMT_INT8, 1, 1) FFNQ_GU_CASE(FMT_INT8, 1, 2)
    FFNQ_GU_CASE(FMT_INT8, 1, 4) FFNQ_GU_CASE(FMT_INT8, 2, 4)
    return false;
}

#define FFNQ_DOWN_CASE(F, NT_, MT_)                                                            \
    if (fmt == F && c.nt == NT_ && c.mt == MT_) {                                              \
        hipExtLaunchKernelGGL((down_kernel<F, NT_, MT_>), grid, block, c.lds, stream, phase_event(2), \
                              phase_event(3), 0, prm);                                            \
        return true;                                                                           \
    }

bool launch_down(int fmt, const KConfig& c, long long items, int N, hipStream_t stream, const DownParams& prm)
{
    const long long tiles = (N + 15) / 16;
    const dim3 grid((unsigned)std::min<long long>(items * tiles, 65535), c.kg), block(64 * c.ks);
    FFNQ_DOWN_CASE(FMT_INT4, 1, 2) FFNQ_DOWN_CASE(FMT_INT4, 1, 4) FFNQ_DOWN_CASE(FMT_INT4, 2, 4)
    FFNQ_DOWN_CASE(FMT_INT4, 4, 4) FFNQ_DOWN_CASE(FMT_INT8, 1, 2) FFNQ_DOWN_CASE(FMT_INT8, 1, 4)
    FFNQ_DOWN_CASE(FMT_INT8, 2, 4) FFNQ_DOWN_CASE(FMT_INT8, 4, 4)
    return false;
}

// ---------------------------------------------------------------------------
// tiled kernels: configuration and dispatch

// Waves per workgroup splitting a tile's K units (scale/zero groups or
// blocks): about `per_cu` waves per CU, not more (rounded down: a grid of one
// workgroup per tile that overflows the resident waves leaves a second
// generation to start late), while every wave keeps the smallest possible
// number of units, all waves equal if possible.
int tiled_ks(int units, long long tiles_total, int cus, int per_cu, int max_ks)
{
    long long want = ((long long)cus * per_cu) / std::max<long long>(1, tiles_total);
    int ks = (int)std::max<long long>(1, std::min<long long>({want, (long long)units, (long long)max_ks}));
    const int per = (units + ks - 1) / ks;
    return (units + per - 1) / per;
}

KConfig gu_tiled_config(int fmt, int K, int N, long long items_est, int rows_total, int cus, int rows_item)
{
    KConfig c{};
    const int F = to_fmt(fmt);
    const TileGeo geo = tile_geo(F, N, K);
    if (rows_item >= kBigRows) {
        // prefill-sized items: one 16-row block per pass with the whole K range of
        // its rows staged (one workgroup per CU), the waves splitting K, and one
        // resident workgroup per CU so that each walks runs of tiles of an item
        const int nun = is_int4(fmt) ? geo.ng : geo.nbk;
        c.nt = 1;
        c.mt = 4;
        c.rows_cap = std::min(std::max(1, rows_total), 16);
        c.kg = 1;
        c.ks = is_int4(fmt) ? std::min(nun, 8) : std::max(1, std::min(8, nun / 4));
        for (;;) {
            c.lds = tiled_launch_lds(2, F, N, K, 1, c.rows_cap, c.ks, 2 * c.nt * 4 * red_lanes(c.nt, c.rows_cap)).total;
            if (c.lds <= kLdsBig || c.rows_cap <= 1) break;
            --c.rows_cap;
        }
        c.grid = (int)std::max<long long>(1, std::min<long long>(items_est * geo.T, (long long)cus));
        return c;
    }
    const int nun = is_int4(fmt) ? geo.ng : geo.nbk;
    const int rp = std::max(1, std::min(rows_total, 32));
    c.nt = rp <= 16 ? 1 : 2;
    c.mt = c.nt == 2 ? 4 : (rp <= 1 ? 1 : (rp <= 2 ? 2 : 4));
    c.rows_cap = std::min(rp, 16 * c.nt);
    c.kg = 1;
    const int max_units_per_wave_int8 = 4;   // INT8: at least this many blocks per wave
    c.ks = is_int4(fmt) ? tiled_ks(nun, items_est * geo.T, cus, 8, 8)
                        : tiled_ks(std::max(1, nun / max_units_per_wave_int8), items_est * geo.T, cus, 8, 8);
    for (;;) {
        c.lds = tiled_launch_lds(2, F, N, K, 1, c.rows_cap, c.ks, c.ts ? 0 : 2 * c.nt * 4 * red_lanes(c.nt, c.rows_cap)).total;
        if (c.lds <= kLdsBudget || c.rows_cap <= 1) break;
        --c.rows_cap;
    }
    c.grid = (int)std::max<long long>(1, std::min<long long>(items_est * geo.T, (long long)cus * 16));
    return c;
}

// Split of the tiled down projection (device independent, so that the
// workspace size is too): K ranges across workgroups (kg), and either K
// ranges across the ks waves (K split) or tiles across them (ts, tile split).
// Dense calls with two or more tokens take the tile split: staging 2 rows per
// token over a whole K range for a single tile would move more bytes from L2
// than the tile's weights; with four tiles per workgroup and K cut into
// about 7 ranges the staged rows serve four tiles and the grid still fills
// the chip.  The fp32 partials of the K ranges are summed by the tail kernel.
struct DSplit {
    int kg, ks, rows_cap, nt, ts, gx;
};

DSplit down_tiled_split(int fmt, int K, int N, int rows_total, bool dense, int rows_item, bool tail_sums)
{
    const int F = to_fmt(fmt);
    const TileGeo geo = tile_geo(F, N, K);
    const int nun = is_int4(fmt) ? geo.ng : geo.nbk;   // K units: scale/zero groups or blocks
    const int r2 = 2 * std::max(1, rows_total);
    const int rp = std::min(r2, 64);
    DSplit d{};
    d.nt = rp <= 16 ? 1 : (rp <= 32 ? 2 : 4);
    d.rows_cap = std::min(rp, 16 * d.nt);
    int kg = std::max(1, (kRefCUs + geo.T - 1) / geo.T);
    kg = std::min(kg, nun);
    while (kg < nun && tiled_launch_lds(1, F, N, K, kg, d.rows_cap, 8, 2 * d.nt * 64).total > kLdsBudget) ++kg;
    d.kg = std::min(kg, nun);   // every K range holds at least one K unit (the kernels rely on it)
    const int upw = (nun + kg - 1) / kg;   // K units of the longest range
    if (is_int4(fmt)) {
        // fewest waves that give every wave the minimal number of groups
        const int best = (upw + 7) / 8;
        d.ks = std::max(1, (upw + best - 1) / best);
    } else {
        d.ks = std::max(1, std::min(8, upw / 4));
    }
    if (!dense && rows_item >= kBigRows) {
        // prefill-sized routed items: tile split over runs of 16 tiles of one item
        // (2 per wave; gx = T/16 workgroups along x walk the union), the staged
        // rows' K range sized to fill one workgroup per CU
        d.ts = 1;
        d.ks = 8;
        d.gx = (geo.T + 2 * d.ks - 1) / (2 * d.ks);
        int tk = 1;
        while (tk < nun && tiled_launch_lds(1, F, N, K, tk, d.rows_cap, d.ks, 0).total > kLdsBig) ++tk;
        d.kg = tk;
    } else if (dense && (rows_total >= 2 || tail_sums || d.kg > 1)) {
        // (one token: only when fp32 partials are summed anyway -- by the RMSNorm
        // tail, or because the K split above already cuts K -- otherwise one K
        // range keeps the residual add in the down kernel)
        d.ts = 1;
        d.ks = 4;
        d.gx = (geo.T + d.ks - 1) / d.ks;
        const long long per_range = (long long)d.ks * d.gx;   // waves of one K range
        int tk = (int)((7LL * kRefCUs + per_range / 2) / per_range);   // ~7 waves per CU in all
        tk = std::max(1, std::min(tk, nun));
        while (tk < nun && tiled_launch_lds(1, F, N, K, tk, d.rows_cap, d.ks, 0).total > kLdsBudget) ++tk;
        d.kg = tk;
    }
    return d;
}

KConfig down_tiled_config(int fmt, int K, int N, long long items_est, int rows_total, int cus, bool dense,
                          int rows_item, bool tail_sums)
{
    const DSplit d = down_tiled_split(fmt, K, N, rows_total, dense, rows_item, tail_sums);
    const int F = to_fmt(fmt);
    const TileGeo geo = tile_geo(F, N, K);
    KConfig c{};
    c.nt = d.nt;
    c.mt = c.nt > 1 ? 4 : (std::min(2 * std::max(1, rows_total), 64) <= 2 ? 2 : 4);
    c.rows_cap = d.rows_cap;
    c.kg = d.kg;
    c.ks = d.ks;
    c.ts = d.ts;
    c.lds = tiled_launch_lds(1, F, N, K, d.kg, c.rows_cap, c.ks, c.ts ? 0 : 2 * c.nt * red_lanes(c.nt, c.rows_cap)).total;
    c.grid = c.ts ? d.gx : (int)std::max<long long>(1, std::min<long long>(items_est * geo.T, (long long)cus * 16));
    return c;
}

// gate/up runs the K split only (the tile split measured slower for it).
#define FFNQ_GUT_CASE(F, NT_, MT_)                                                                           \
    if (fmt == F && c.nt == NT_ && c.mt == MT_ && !c.ts) {                                                   \
        hipExtLaunchKernelGGL((gu_tiled_kernel<F, NT_, MT_, false>), dim3(c.grid), dim3(64 * c.ks), c.lds,    \
                              stream, phase_event(0), phase_event(1), 0, q);                                 \
        return true;                                                                                         \
    }

bool launch_gu_tiled(int fmt, const KConfig& c, hipStream_t stream, const GUParams& prm)
{
    GUParams q = prm;   // the kernels take the launch shape as arguments (cheaper than reading it back)
    q.ks = c.ks;
    q.grid = c.grid;
    FFNQ_GUT_CASE(FMT_INT4, 1, 1) FFNQ_GUT_CASE(FMT_INT4, 1, 2) FFNQ_GUT_CASE(FMT_INT4, 1, 4)
    FFNQ_GUT_CASE(FMT_INT4, 2, 4) FFNQ_GUT_CASE(FMT_INT8, 1, 1) FFNQ_GUT_CASE(FMT_INT8, 1, 2)
    FFNQ_GUT_CASE(FMT_INT8, 1, 4) FFNQ_GUT_CASE(FMT_INT8, 2, 4)
    return false;
}

#define FFNQ_DNT_CASE(F, NT_, MT_)                                                                           \
    if (fmt == F && c.nt == NT_ && c.mt == MT_) {                                                            \
        if (c.ts)                                                                                            \
            hipExtLaunchKernelGGL((down_tiled_kernel<F, NT_, MT_, true>), dim3(c.grid, c.kg), dim3(64 * c.ks), \
                                  c.lds, stream, phase_event(2), phase_event(3), 0, q);                      \
        else                                                                                                 \
            hipExtLaunchKernelGGL((down_tiled_kernel<F, NT_, MT_, false>), dim3(c.grid, c.kg), dim3(64 * c.ks), \
                                  c.lds, stream, phase_event(2), phase_event(3), 0, q);                      \
        return true;                                                                                         \
    }

bool launch_down_tiled(int fmt, const KConfig& c, hipStream_t stream, const DownParams& prm)
{
    DownParams q = prm;
    q.ks = c.ks;
    q.grid = c.grid;
    FFNQ_DNT_CASE(FMT_INT4, 1, 2) FFNQ_DNT_CASE(FMT_INT4, 1, 4) FFNQ_DNT_CASE(FMT_INT4, 2, 4)
    FFNQ_DNT_CASE(FMT_INT4, 4, 4) FFNQ_DNT_CASE(FMT_INT8, 1, 2) FFNQ_DNT_CASE(FMT_INT8, 1, 4)
    FFNQ_DNT_CASE(FMT_INT8, 2, 4) FFNQ_DNT_CASE(FMT_INT8, 4, 4)
    return false;
}

// K ranges of the down projection for a format (row-major or tiled).
int down_ranges(int fmt, int K, int N, int rows_total, bool dense, int rows_item, bool tail_sums)
{
    return is_tiled(fmt) ? down_tiled_split(fmt, K, N, rows_total, dense, rows_item, tail_sums).kg
                         : down_kg(fmt, K, N, rows_total);
}

// ---------------------------------------------------------------------------
// burst kernels (stream.h): gate/up at 1..4 rows and down at 1..2 tokens on
// tiled weights.  A workgroup takes one 16-row tile; its ks waves take the
// tile's K units (gate/up: one each; down: in passes of one).  FFNQ_BURST=0
// at build time turns them off (the streaming kernels then run every shape).

#ifndef FFNQ_BURST
#define FFNQ_BURST 1
#endif

struct BurstCfg {
    bool ok;
    int ks, R;
    size_t lds;
};

// gate/up: one K unit per wave, all of a tile's units in one workgroup.
BurstCfg burst_gu_cfg(int fmt, int K, int N, int m)
{
    const int R = m <= 4 ? m : 8;   // activation rows of the kernel (rows past m repeat row 0)
    BurstCfg c{false, 1, R, 0};
    if (!FFNQ_BURST || !is_tiled(fmt) || m < 1 || m > 8) return c;
    const int F = to_fmt(fmt);
    c.ks = burst_units(F, N, K);
    if (c.ks > 16) return c;
    c.lds = (size_t)burst_lds(F, 2, R, 1, c.ks);
    c.ok = c.lds <= kLdsBudget;
    return c;
}

// down (m tokens: 2m hi/lo rows, R = 2, 4 or 8): the most waves, up to 16, whose
// staging fits one CU's LDS take the tile's K units in passes of one.
BurstCfg burst_down_cfg(int fmt, int K, int N, int m)
{
    const int R = m == 1 ? 2 : (m == 2 ? 4 : 8);
    BurstCfg c{false, 1, R, 0};
    if (!FFNQ_BURST || !is_tiled(fmt) || m < 1 || m > 4) return c;
    const int F = to_fmt(fmt);
    const int nu = burst_units(F, N, K);
    if (nu > 64) return c;
    for (c.ks = std::min(nu, 16); c.ks >= 1; --c.ks) {
        c.lds = (size_t)burst_down_lds(F, R, c.ks, nu);
        if (c.lds <= kLdsMax) break;
    }
    c.ok = c.ks >= 1 && (nu + c.ks - 1) / c.ks <= 4;   // at most four passes
    return c;
}

BurstCfg dense_gu_burst(const ffnq_ffn* ffn, int hidden, int inter, int m)
{
    return burst_gu_cfg(ffn->gate.fmt, hidden, inter, m);
}

BurstCfg dense_down_burst(int fmt_down, int hidden, int inter, int m)
{
    return burst_down_cfg(fmt_down, inter, hidden, m);
}

#define FFNQ_GUB_CASE(F, R_)                                                                                  \
    if (F_ == F && R == R_) {                                                                                 \
        hipExtLaunchKernelGGL((gu_burst_kernel<F, R_>), dim3(na + nb), dim3(64 * ks), lds, stream, phase_event(0), \
                              phase_event(1), 0, qa, qb, na);                                                 \
        return true;                                                                                          \
    }

// One or two gate/up jobs (dense or routed GUParams) in one burst launch: job a
// on workgroups [0, na), job b (if any) on the next nb; both with R activation
// rows, ks waves per workgroup (one K unit each) and the same format.
bool launch_gu_burst_jobs(int fmt, int R, int ks, size_t lds, const GUParams& a, int na, const GUParams* b, int nb,
                          hipStream_t stream)
{
    GUParams qa = a, qb = b ? *b : a;
    qa.ks = qb.ks = ks;
    if (!b) nb = 0;
    const int F_ = to_fmt(fmt);
    FFNQ_GUB_CASE(FMT_INT4, 1) FFNQ_GUB_CASE(FMT_INT4, 2) FFNQ_GUB_CASE(FMT_INT4, 3) FFNQ_GUB_CASE(FMT_INT4, 4)
    FFNQ_GUB_CASE(FMT_INT4, 8) FFNQ_GUB_CASE(FMT_INT8, 1) FFNQ_GUB_CASE(FMT_INT8, 2) FFNQ_GUB_CASE(FMT_INT8, 3)
    FFNQ_GUB_CASE(FMT_INT8, 4) FFNQ_GUB_CASE(FMT_INT8, 8)
    return false;
}

bool launch_gu_burst(int fmt, const BurstCfg& c, int N, hipStream_t stream, const GUParams& prm)
{
    return launch_gu_burst_jobs(fmt, c.R, c.ks, c.lds, prm, (N + 15) / 16, nullptr, 0, stream);
}

#define FFNQ_DNB_CASE(F, R_)                                                                                     \
    if (F_ == F && c.R == R_) {                                                                                  \
        hipExtLaunchKernelGGL((down_burst_kernel<F, R_>), dim3(T), dim3(64 * c.ks), c.lds, stream, phase_event(2), \
                              phase_event(3), 0, q);                                                             \
        return true;                                                                                             \
    }

bool launch_down_burst(int fmt, const BurstCfg& c, int N, hipStream_t stream, const DownParams& prm)
{
    DownParams q = prm;
    q.ks = c.ks;
    q.KG = 1;
    const int F_ = to_fmt(fmt);
    const int T = (N + 15) / 16;
    FFNQ_DNB_CASE(FMT_INT4, 2) FFNQ_DNB_CASE(FMT_INT4, 4) FFNQ_DNB_CASE(FMT_INT4, 8) FFNQ_DNB_CASE(FMT_INT8, 2)
    FFNQ_DNB_CASE(FMT_INT8, 4) FFNQ_DNB_CASE(FMT_INT8, 8)
    return false;
}

// ---------------------------------------------------------------------------
// dense FFN (ffnq_dense and ffnq_shared_expert)

struct DenseWs {
    size_t act, part, logit, total;
};

DenseWs dense_ws(int fmt_down, int hidden, int inter, int m, int tail, bool shared)
{
    DenseWs w{};
    size_t o = 0;
    const int kg = dense_down_burst(fmt_down, hidden, inter, m).ok
                       ? 1
                       : down_ranges(fmt_down, inter, hidden, m, true, m, tail == TAIL_RMSNORM);
    w.act = o; o += align_up((size_t)2 * m * inter * 2, 256);
    w.part = o; o += align_up((size_t)kg * m * hidden * sizeof(float), 256);
    w.logit = o; o += align_up((size_t)m * sizeof(float), 256);
    w.total = m == 0 ? 0 : o;
    return w;
}

// Gate/up parameters and configuration of a dense FFN (all m rows, one item).
// gate_vec/logit: the sigmoid-gate logits, computed by the same launch.
GUParams dense_gu_params(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, const uint16_t* x,
                         const KConfig& gc, uint16_t* act_out, const uint16_t* gate_vec, float* logit)
{
    GUParams gp{};
    gp.gate = mat_dev(ffn->gate);
    gp.up = mat_dev(ffn->up);
    gp.N = inter;
    gp.K = hidden;
    gp.act = act;
    gp.dfmt = to_fmt(ffn->down.fmt);
    gp.x = x;
    gp.m = m;
    gp.rows_cap = gc.rows_cap;
    gp.plan = nullptr;
    gp.act_out = act_out;
    gp.act_rows = m;
    gp.gate_vec = gate_vec;
    gp.logit = logit;
    if (is_tiled(ffn->gate.fmt)) {
        gp.tgate = static_cast<const uint8_t*>(ffn->gate.q);
        gp.tup = static_cast<const uint8_t*>(ffn->up.q);
        gp.tebytes = tiled_expert_bytes(ffn->gate);
        gp.dfmt = FMT_NATURAL;   // a tiled down matrix reads the activation in natural order
    }
    return gp;
}

// wide (ffnq_dense, two or more rows, tiled): twice the waves per workgroup over
// runs of two tiles, the same waves in all, so that the staged activation rows
// serve two tiles (Llama-shaped gate/up at M = 4: 20.9 -> 19.7 us).  Not for
// the shared expert: ffnq_moe_layer matches its launch shape, and its results,
// to those of ffnq_shared_expert.
KConfig dense_gu_config(const ffnq_ffn* ffn, int hidden, int inter, int m, int cus, bool wide = false)
{
    if (!is_tiled(ffn->gate.fmt)) return gu_config(ffn->gate.fmt, hidden, inter, 1, m, cus);
    KConfig c = gu_tiled_config(ffn->gate.fmt, hidden, inter, 1, m, cus, m);
    if (wide && m >= 2 && m < kBigRows && !c.ts) {
        const int F = to_fmt(ffn->gate.fmt);
        const TileGeo geo = tile_geo(F, inter, hidden);
        const int units = is_int4(ffn->gate.fmt) ? geo.ng : std::max(1, geo.nbk / 4);   // K units a wave may take
        if (2 * c.ks <= std::min(units, 8) && geo.T >= 2) {
            KConfig w = c;
            w.ks = 2 * c.ks;
            w.grid = (geo.T + 1) / 2;
            w.lds = tiled_launch_lds(2, F, inter, hidden, 1, w.rows_cap, w.ks, 2 * w.nt * 4 * red_lanes(w.nt, w.rows_cap)).total;
            if (w.lds <= kLdsBudget) c = w;
        }
    }
    return c;
}

KConfig dense_down_config(const ffnq_ffn* ffn, int hidden, int inter, int m, int cus, int tail)
{
    return is_tiled(ffn->down.fmt)
               ? down_tiled_config(ffn->down.fmt, inter, hidden, 1, m, cus, true, m, tail == FFNQ_TAIL_RMSNORM)
               : down_config(ffn->down.fmt, inter, hidden, 1, m, cus);
}

DownParams dense_down_params(const ffnq_ffn* ffn, int hidden, int inter, int m, const KConfig& dc,
                             const uint16_t* act, uint16_t* out, float* part, const float* logit, int dtail)
{
    DownParams dp{};
    dp.down = mat_dev(ffn->down);
    dp.N = hidden;
    dp.K = inter;
    dp.act = act;
    dp.act_rows = m;
    dp.m = m;
    dp.rows_cap = dc.rows_cap;
    dp.KG = dc.kg;
    dp.plan = nullptr;
    dp.out = out;
    dp.part = part;
    dp.logit = logit;
    dp.tail = dtail;
    if (is_tiled(ffn->down.fmt)) {
        dp.tdown = static_cast<const uint8_t*>(ffn->down.q);
        dp.tebytes = tiled_expert_bytes(ffn->down);
    }
    return dp;
}

// With norm_part (RMSNorm tail only): the down projection's fp32 partials and
// their count are handed back instead of launching the RMSNorm, for a caller
// that folds the norm into a kernel of its own.
int run_dense(bool shared, const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x,
              uint16_t* out, const uint16_t* aux, float eps, void* ws, hipStream_t stream,
              const float** norm_part = nullptr, int* norm_R = nullptr)
{
    const int cus = device_cus();
    unsigned char* base = static_cast<unsigned char*>(ws);
    const DenseWs L = dense_ws(ffn->down.fmt, hidden, inter, m, tail, shared);
    const int gfmt = to_fmt(ffn->gate.fmt), dfmt = to_fmt(ffn->down.fmt);
    const bool tiled = is_tiled(ffn->gate.fmt);

    const KConfig gc = dense_gu_config(ffn, hidden, inter, m, cus, !shared);
    const bool sg = tail == FFNQ_TAIL_SIGMOID_GATE;
    const GUParams gp = dense_gu_params(ffn, hidden, inter, m, act, x, gc, reinterpret_cast<uint16_t*>(base + L.act),
                                        sg ? aux : nullptr, sg ? reinterpret_cast<float*>(base + L.logit) : nullptr);
    const BurstCfg gb = dense_gu_burst(ffn, hidden, inter, m);
    if (gb.ok) {
        if (!launch_gu_burst(ffn->gate.fmt, gb, inter, stream, gp)) return FFNQ_ERR_UNSUPPORTED;
    } else if (!(tiled ? launch_gu_tiled(gfmt, gc, stream, gp) : launch_gu(gfmt, gc, 1, inter, stream, gp))) {
        return FFNQ_ERR_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    const KConfig dc = dense_down_config(ffn, hidden, inter, m, cus, tail);
    int dtail = TAIL_NONE;
    switch (tail) {
        case FFNQ_TAIL_RESIDUAL: dtail = TAIL_RESIDUAL; break;
        case FFNQ_TAIL_RMSNORM: dtail = TAIL_RMSNORM; break;
        case FFNQ_TAIL_SIGMOID_GATE: dtail = TAIL_SIGMOID; break;
        default: break;
    }
    DownParams dp = dense_down_params(ffn, hidden, inter, m, dc, gp.act_out, out,
                                      reinterpret_cast<float*>(base + L.part),
                                      reinterpret_cast<const float*>(base + L.logit), dtail);
    const BurstCfg db = dense_down_burst(ffn->down.fmt, hidden, inter, m);
    const int kg = db.ok ? 1 : dc.kg;
    if (db.ok) {
        dp.KG = 1;
        if (!launch_down_burst(ffn->down.fmt, db, hidden, stream, dp)) return FFNQ_ERR_UNSUPPORTED;
    } else if (!(tiled ? launch_down_tiled(dfmt, dc, stream, dp) : launch_down(dfmt, dc, 1, hidden, stream, dp))) {
        return FFNQ_ERR_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    if (tail == FFNQ_TAIL_RMSNORM && norm_part) {
        *norm_part = dp.part;
        *norm_R = kg;
    } else if (tail == FFNQ_TAIL_RMSNORM) {
        const size_t row_lds = hidden <= kRowLds ? (size_t)hidden * 6 : 0;
        hipLaunchKernelGGL(rmsnorm_kernel, dim3(m), dim3(kNormThreads), row_lds, stream, dp.part, kg, m, aux, out, hidden,
                           eps);
        if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;
    } else if (kg > 1) {
        const long long total = (long long)m * hidden;
        const int grid = (int)std::min<long long>((total + 255) / 256, (long long)cus * 8);
        hipLaunchKernelGGL(ksum_tail_kernel, dim3(grid), dim3(256), 0, stream, dp.part, kg, m, hidden, dp.tail, out,
                           dp.logit);
        if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;
    }
    return FFNQ_OK;
}

int dense_common(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x,
                 uint16_t* out, const uint16_t* aux, float eps, void* ws, size_t* ws_bytes, hipStream_t stream,
                 bool shared)
{
    if (!ws_bytes) return FFNQ_ERR_INVALID;
    if (m < 0) return FFNQ_ERR_INVALID;
    const int rc = check_ffn(ffn, hidden, inter);
    if (rc != FFNQ_OK) return rc;
    if (act != FFNQ_ACT_SILU && act != FFNQ_ACT_GELU_TANH) return FFNQ_ERR_UNSUPPORTED;
    if (shared) {
        if (tail != FFNQ_TAIL_NONE && tail != FFNQ_TAIL_RMSNORM && tail != FFNQ_TAIL_SIGMOID_GATE)
            return FFNQ_ERR_UNSUPPORTED;
    } else if (tail != FFNQ_TAIL_RESIDUAL && tail != FFNQ_TAIL_RMSNORM) {
        return FFNQ_ERR_UNSUPPORTED;
    }
    if (!x || !out) return FFNQ_ERR_INVALID;
    if (misaligned(x) || misaligned(out)) return FFNQ_ERR_INVALID;
    const size_t rows_bytes = (size_t)m * hidden * 2;
    if (m > 0 && overlap(x, rows_bytes, out, rows_bytes)) return FFNQ_ERR_INVALID;
    if (tail == FFNQ_TAIL_RMSNORM || tail == FFNQ_TAIL_SIGMOID_GATE) {
        if (!aux || misaligned(aux)) return FFNQ_ERR_INVALID;
    }
    if (tail == FFNQ_TAIL_RMSNORM && !(eps >= 0.0f && std::isfinite(eps))) return FFNQ_ERR_INVALID;
    const DenseWs L = dense_ws(ffn->down.fmt, hidden, inter, m, tail, shared);
    if (!ws) {
        *ws_bytes = L.total;
        return FFNQ_OK;
    }
    if (*ws_bytes < L.total) return FFNQ_ERR_WORKSPACE;
    if (misaligned(ws)) return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;
    return run_dense(shared, ffn, hidden, inter, m, act, tail, x, out, aux, eps, ws, stream);
}

// ---------------------------------------------------------------------------
// routed half

struct RoutedWs {
    size_t act, part, seed, total;
};

int prefill_down_kg(int hidden, int moe_inter, long long u_est);

RoutedWs routed_ws(int fmt, int hidden, int moe_inter, int m, int k, int n_experts)
{
    RoutedWs w{};
    const size_t P = (size_t)m * k;
    int kg = down_ranges(fmt, moe_inter, hidden, m, false, rows_per_item(false, m, k, n_experts), false);
    if (is_tiled(fmt) && is_int4(fmt) && rows_per_item(false, m, k, n_experts) >= kBigRows)
        kg = std::max(kg, prefill_down_kg(hidden, moe_inter, std::min<long long>((long long)P, n_experts)));
    size_t o = 0;
    w.act = o; o += align_up(2 * P * moe_inter * 2, 256);
    w.part = o; o += align_up((size_t)kg * P * hidden * sizeof(float), 256);
    w.seed = o; o += align_up((size_t)m * hidden * 2, 256);   // a layer's shared-expert seed
    w.total = m == 0 ? 0 : o;
    return w;
}

// The shared expert of a MoE layer when it runs fused with the routed half
// (ffnq_moe_layer): its gate/up shares the routed gate/up launch when their
// launch shapes agree, its down leaves fp32 partials, and the routed reduction
// makes the seed from them.  Same arithmetic as ffnq_shared_expert followed by
// ffnq_moe_routed_batched.
struct LayerShared {
    const ffnq_ffn* ffn;
    int inter;
    const uint16_t* gate_vec;
    unsigned char* base;   // its workspace (dense_ws with the sigmoid-gate tail)
};

#define FFNQ_GUT2_CASE(NT_, MT_)                                                                       \
    if (a.nt == NT_ && a.mt == MT_) {                                                                  \
        hipExtLaunchKernelGGL((gu_tiled_kernel2<FMT_INT4, NT_, MT_>), grid, dim3(64 * a.ks), lds, stream, \
                              phase_event(0), phase_event(1), 0, qa, qb);                              \
        return true;                                                                                   \
    }

// Shared and routed tiled INT4 gate/up in one launch (grid rows 0 and 1).
bool launch_gu_tiled2(const KConfig& a, const GUParams& pa, const KConfig& b, const GUParams& pb, hipStream_t stream)
{
    if (a.nt != b.nt || a.mt != b.mt || a.ks != b.ks || a.ts || b.ts) return false;
    GUParams qa = pa, qb = pb;
    qa.ks = a.ks;
    qa.grid = a.grid;
    qb.ks = b.ks;
    qb.grid = b.grid;
    const dim3 grid((unsigned)std::max(a.grid, b.grid), 2);
    const size_t lds = std::max(a.lds, b.lds);
    FFNQ_GUT2_CASE(1, 1) FFNQ_GUT2_CASE(1, 2) FFNQ_GUT2_CASE(1, 4) FFNQ_GUT2_CASE(2, 4)
    return false;
}

#define FFNQ_DNT2_CASE(NT_, MT_)                                                                             \
    if (a.nt == NT_ && a.mt == MT_) {                                                                        \
        hipExtLaunchKernelGGL((down_tiled_kernel2<FMT_INT4, NT_, MT_>), dim3(na + nb), dim3(64 * a.ks), lds, stream, \
                              phase_event(2), phase_event(3), 0, qa, qb, na);                                \
        return true;                                                                                         \
    }

// Shared and routed tiled INT4 down in one launch (both with the K split).
bool launch_down_tiled2(const KConfig& a, const DownParams& pa, const KConfig& b, const DownParams& pb,
                        hipStream_t stream)
{
    if (a.nt != b.nt || a.mt != b.mt || a.ks != b.ks || a.ts || b.ts) return false;
    DownParams qa = pa, qb = pb;
    qa.ks = a.ks;
    qa.grid = a.grid;
    qb.ks = b.ks;
    qb.grid = b.grid;
    const int na = a.grid * a.kg, nb = b.grid * b.kg;
    const size_t lds = std::max(a.lds, b.lds);
    FFNQ_DNT2_CASE(1, 2) FFNQ_DNT2_CASE(1, 4) FFNQ_DNT2_CASE(2, 4) FFNQ_DNT2_CASE(4, 4)
    return false;
}

// The fused routed down (stream.h moe_down_kernel): configuration.  One
// workgroup per 16-row output tile; its units are the shared expert's K units
// and those of every possible union entry (at most min(m*k, E)); ks waves take
// them in passes of one.  For m <= 2 tokens (2m activation rows per unit).
struct MoeDownCfg {
    bool ok;
    int R, ks, upp, max_units;
    size_t lds;
};

// Units a wave of moe_down_kernel stages per pass: one.  (Two per pass, with
// both units' loads in flight together, gave NaN outputs on the Mixtral-shaped
// layer -- 28 units per tile -- for a reason not yet found; that path is off.)
#ifndef FFNQ_MOE_DOWN_UPP
#define FFNQ_MOE_DOWN_UPP 1
#endif

MoeDownCfg moe_down_cfg(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k,
                        const ffnq_ffn* shared, int shared_inter)
{
    MoeDownCfg c{false, m == 1 ? 2 : (m == 2 ? 4 : 8), 1, 1, 0, 0};
    if (!FFNQ_BURST || m > 4 || (long long)m * top_k > 64 || !is_tiled(experts->down.fmt) ||
        !is_int4(experts->down.fmt))
        return c;
    int ns = 0;
    if (shared) {
        if (!is_tiled(shared->down.fmt) || !is_int4(shared->down.fmt)) return c;
        if (!dense_down_burst(shared->down.fmt, hidden, shared_inter, m).ok) return c;
        ns = burst_units(FMT_INT4, hidden, shared_inter);
    }
    const int nr = burst_units(FMT_INT4, hidden, moe_inter);
    // a plan's union has at most one entry per pair; it can hold more entries
    // than there are experts when the slot cap splits the batch
    const long long umax = (long long)m * top_k;
    const long long units = ns + umax * nr;
    if (units > 64) return c;
    c.max_units = (int)units;
    // fewest passes (then most waves) among one or two units per pass that fit LDS
    int best_passes = 1 << 30;
    for (int upp = 1; upp <= FFNQ_MOE_DOWN_UPP; ++upp) {
        for (int ks = (int)std::min<long long>(16, (units + upp - 1) / upp); ks >= 1; --ks) {
            const size_t lds = (size_t)moe_down_lds(FMT_INT4, c.R, upp, ks, c.max_units);
            if (lds > kLdsMax) continue;
            const int passes = (int)((units + (long long)upp * ks - 1) / ((long long)upp * ks));
            if (passes < best_passes) {
                best_passes = passes;
                c.upp = upp;
                c.ks = ks;
                c.lds = lds;
                c.ok = true;
            }
            break;   // the most waves that fit for this upp
        }
    }
    return c;
}

#define FFNQ_MDN_CASE(R_, UPP_)                                                                                 \
    if (c.R == R_ && c.upp == UPP_) {                                                                           \
        hipExtLaunchKernelGGL((moe_down_kernel<FMT_INT4, R_, UPP_>), dim3((N + 15) / 16), dim3(64 * c.ks), c.lds,  \
                              stream, phase_event(2), phase_event(3), 0, q);                                    \
        return true;                                                                                            \
    }

bool launch_moe_down(const MoeDownCfg& c, int N, hipStream_t stream, const MoeDownParams& prm)
{
    MoeDownParams q = prm;
    q.ks = c.ks;
    q.max_units = c.max_units;
    FFNQ_MDN_CASE(2, 1) FFNQ_MDN_CASE(4, 1) FFNQ_MDN_CASE(8, 1)
    return false;
}

// Gate/up of a layer's shared expert in ffnq_moe_layer: the kernel that
// ffnq_shared_expert runs for it (burst or streaming), so that its activation,
// and from it the seed, are bit for bit the same.
int launch_shared_gu(const LayerShared* sh, int hidden, int m, int act, const uint16_t* x, const GUParams& gps,
                     const KConfig& gcs, const BurstCfg& sb, hipStream_t stream)
{
    if (sb.ok) return launch_gu_burst(sh->ffn->gate.fmt, sb, sh->inter, stream, gps) ? FFNQ_OK : FFNQ_ERR_UNSUPPORTED;
    const int sfmt = to_fmt(sh->ffn->gate.fmt);
    (void)hidden;
    (void)m;
    (void)act;
    (void)x;
    return (is_tiled(sh->ffn->gate.fmt) ? launch_gu_tiled(sfmt, gcs, stream, gps)
                                        : launch_gu(sfmt, gcs, 1, sh->inter, stream, gps))
               ? FFNQ_OK
               : FFNQ_ERR_UNSUPPORTED;
}

// The routed half on a checked call (m > 0; the routed workspace at base).
//   m <= 4 and tiled experts: phase 1 is a burst launch (with the shared
//     expert's gate/up as a second job when their shapes agree);
//   m <= 2 and tiled INT4 (shared expert too, if any): phase 2, the shared
//     expert's down, the seeded reduction and the residual add are one launch
//     (moe_down_kernel);
//   otherwise the streaming kernels, fp32 per-pair partials and
//     moe_reduce_kernel.
// Routing done inside the routed gate/up launch (ffnq_moe_layer_logits): the
// logits, the expert scale and the slot cap; the ids, weights and plan are
// written to the call's topk_ids / topk_w / plan.
struct RouteIn {
    const float* logits;
    const float* scale;
    int cap;
};

// Prefill-sized routed items (prefill.h): the grouped kernels for the routed
// gate/up and down when the experts are tiled INT4 and the pairs per union
// entry reach kBigRows.  Rows per pass: 32 pairs for gate/up, 24 pairs (48
// hi/lo rows) for down -- entries with more take further passes, row blocks
// an entry leaves empty cost no MFMA; 4 code blocks per staged chunk (the
// double-buffered rows then fit one CU's LDS); one tile per wave for gate/up,
// and for down 2 where that keeps the grid's last round as full as 1 does.
#ifndef FFNQ_PREFILL
#define FFNQ_PREFILL 1
#endif

// Prefetch distance (steps of weights in flight per wave beyond the one being
// multiplied), at least two, so that the wait for a step's weights never waits
// for the activation rows staged after the previous step's loads.
#ifndef FFNQ_PF_D_GU
#define FFNQ_PF_D_GU 3
#endif
#ifndef FFNQ_PF_D_DN
#define FFNQ_PF_D_DN 2   // two tiles per step: its scale/zero slots must fit the LDS beside 48 staged rows
#endif

// Waves per workgroup: 12 for gate/up (6 per matrix), 8 for down (at 4096
// outputs, 12 would leave CUs without a unit).
#ifndef FFNQ_PF_WAVES_GU
#define FFNQ_PF_WAVES_GU 12
#endif
#ifndef FFNQ_PF_WAVES_DN
#define FFNQ_PF_WAVES_DN 8
#endif
constexpr int kPfWavesGU = FFNQ_PF_WAVES_GU, kPfWavesDN = FFNQ_PF_WAVES_DN;
#ifndef FFNQ_PF_TPW_GU
#define FFNQ_PF_TPW_GU 1   // most tiles per gate/up wave (the registers of 12-wave workgroups hold one)
#endif

struct PrefillCfg {
    bool ok;
    int tpw_gu, tpw_dn, grid_gu, grid_dn, kg_dn;
    size_t lds_gu, lds_dn;
};

// K ranges of the prefill down: enough (tile group, range) units for every CU
// of a reference 256-CU part (device independent, so that the workspace size
// is), at least 4 chunks of 512 inputs per range.
constexpr int kPfTpwDn = 2;
int prefill_down_kg(int hidden, int moe_inter, long long u_est)
{
    const TileGeo gd = tile_geo(FMT_INT4, hidden, moe_inter);
    const long long units = u_est * ((gd.T + kPfWavesDN * kPfTpwDn - 1) / (kPfWavesDN * kPfTpwDn));
    const int nch = (gd.nbk + 3) / 4;
    int kg = (int)std::max<long long>(1, (kRefCUs + units - 1) / std::max<long long>(units, 1));
    return std::max(1, std::min(kg, nch / 4));
}

// Tiles per wave: the most (up to `most`) for which the grid's last round is as
// full as with fewer -- more tiles per unit amortise the staged rows.
int prefill_tpw(int tiles, int waves_per_matrix, long long items, int cus, int most)
{
    auto eff = [&](int tpw) {
        const long long per = (long long)waves_per_matrix * tpw;
        const long long units = items * ((tiles + per - 1) / per);
        const long long rounds = (units + cus - 1) / cus;
        return (double)units / (double)(rounds * cus);
    };
    int best = 1;
    for (int t = 2; t <= most; t *= 2)
        if (eff(t) >= eff(best) - 1e-9) best = t;
    return best;
}

PrefillCfg prefill_cfg(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k, int cus)
{
    PrefillCfg c{};
    const int tf = FFNQ_FMT_INT4_AFFINE_G64_TILED;
    if (!FFNQ_PREFILL || experts->gate.fmt != tf || experts->up.fmt != tf || experts->down.fmt != tf) return c;
    if (rows_per_item(false, m, top_k, n_experts) < kBigRows) return c;
    const long long u_est = std::min<long long>((long long)m * top_k, n_experts);
    const TileGeo gg = tile_geo(FMT_INT4, moe_inter, hidden), gd = tile_geo(FMT_INT4, hidden, moe_inter);
    c.tpw_gu = prefill_tpw(gg.T, kPfWavesGU / 2, u_est, cus, FFNQ_PF_TPW_GU);
    c.tpw_dn = kPfTpwDn;
    c.kg_dn = prefill_down_kg(hidden, moe_inter, u_est);
    auto grid = [&](int tiles, int per, int kg) {
        const long long units = u_est * ((tiles + per - 1) / per) * kg;
        return (int)std::max<long long>(1, std::min<long long>(units, cus));
    };
    c.grid_gu = grid(gg.T, kPfWavesGU / 2 * c.tpw_gu, 1);
    c.grid_dn = grid(gd.T, kPfWavesDN * c.tpw_dn, c.kg_dn);
    c.lds_gu = (size_t)prefill_lds(kPfWavesGU, 2, 4, FFNQ_PF_D_GU, c.tpw_gu);
    c.lds_dn = (size_t)prefill_lds(kPfWavesDN, 3, 4, FFNQ_PF_D_DN, c.tpw_dn);
    c.ok = c.lds_gu <= kLdsMax && c.lds_dn <= kLdsMax;
    return c;
}

#ifndef FFNQ_PF_SPS
#define FFNQ_PF_SPS 2   // code blocks per step: two steps per 4-block chunk and tile
#endif

#define FFNQ_PF_CASE(DOWN_, W_, NMW_, RB_, TPW_, D_, EV)                                                     \
    if (down == DOWN_ && tpw == TPW_) {                                                                       \
        hipExtLaunchKernelGGL((prefill_kernel<W_, NMW_, RB_, 4, TPW_, D_, FFNQ_PF_SPS>), dim3(grid),          \
                              dim3(64 * W_), lds, stream, phase_event(EV), phase_event(EV + 1), 0, q);       \
        return hipGetLastError() == hipSuccess;                                                               \
    }

bool launch_prefill(bool down, int tpw, int grid, size_t lds, hipStream_t stream, const PrefillParams& prm)
{
    PrefillParams q = prm;
    q.tpw = tpw;
    FFNQ_PF_CASE(false, kPfWavesGU, 2, 2, 1, FFNQ_PF_D_GU, 0)
#if FFNQ_PF_TPW_GU >= 2
    FFNQ_PF_CASE(false, kPfWavesGU, 2, 2, 2, FFNQ_PF_D_GU, 0)
#endif
    FFNQ_PF_CASE(true, kPfWavesDN, 1, 3, kPfTpwDn, FFNQ_PF_D_DN, 2)
    return false;
}

// Whether the routed gate/up launch routes the batch itself: every one of its
// workgroups repeats the routing (ranking m * E keys), so only for batches
// with few keys, where that costs less than a launch of its own.
#ifndef FFNQ_ROUTE_IN_GU_KEYS
#define FFNQ_ROUTE_IN_GU_KEYS 128   // measured: Qwen-shaped M = 1 (128 keys) gains ~4 us; M = 2 (256) does not
#endif

bool route_in_gu(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k)
{
    const long long P = (long long)m * top_k;
    if (!FFNQ_BURST || !is_tiled(experts->gate.fmt) || !is_int4(experts->gate.fmt)) return false;
    if (P > kSmallPairs || (long long)m * n_experts > std::min(kSmallKeys, FFNQ_ROUTE_IN_GU_KEYS)) return false;
    const BurstCfg rb = burst_gu_cfg(experts->gate.fmt, hidden, moe_inter, m);
    return rb.ok && small_route_lds(m, n_experts, top_k) <= kLdsBudget;
}

int run_routed(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k, int act,
               const uint16_t* x, const int32_t* topk_ids, const float* topk_w, const int32_t* plan,
               const uint16_t* seed, uint16_t* resid, unsigned char* base, hipStream_t stream, const LayerShared* sh,
               const RouteIn* rin = nullptr, bool out_zero = false)
{
    // out_zero: the rows are written as the sum on +0 (their contents on entry
    // do not matter) -- in the fused down directly, else by zeroing them first
    if (out_zero && !moe_down_cfg(experts, n_experts, hidden, moe_inter, m, top_k, sh ? sh->ffn : nullptr,
                                  sh ? sh->inter : 0).ok) {
        const size_t nrow = (size_t)m * hidden;
        hipLaunchKernelGGL(zero_u16_kernel, dim3((unsigned)std::min<size_t>((nrow + 255) / 256, 1024)), dim3(256), 0,
                           stream, resid, nrow);
        if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;
        out_zero = false;
    }
    const RoutedWs L = routed_ws(experts->down.fmt, hidden, moe_inter, m, top_k, n_experts);
    const int cus = device_cus();
    const int P = m * top_k;
    const long long u_est = std::min<long long>(P, n_experts);

    // phase 1: gate/up + activation per union entry and tile
    const bool tiled = is_tiled(experts->gate.fmt);
    const KConfig gc = tiled ? gu_tiled_config(experts->gate.fmt, hidden, moe_inter, u_est, m, cus,
                                               rows_per_item(false, m, top_k, n_experts))
                             : gu_config(experts->gate.fmt, hidden, moe_inter, u_est, m, cus);
    GUParams gp{};
    gp.gate = mat_dev(experts->gate);
    gp.up = mat_dev(experts->up);
    gp.N = moe_inter;
    gp.K = hidden;
    gp.act = act;
    gp.dfmt = FMT_INT4;
    gp.x = x;
    gp.m = m;
    gp.rows_cap = gc.rows_cap;
    gp.plan = plan;
    gp.top_k = top_k;
    gp.topk_ids = topk_ids;
    gp.n_experts = n_experts;
    gp.act_out = reinterpret_cast<uint16_t*>(base + L.act);
    gp.act_rows = P;
    if (tiled) {
        gp.tgate = static_cast<const uint8_t*>(experts->gate.q);
        gp.tup = static_cast<const uint8_t*>(experts->up.q);
        gp.tebytes = tiled_expert_bytes(experts->gate);
        gp.dfmt = FMT_NATURAL;
    }
    // the routed gate/up burst: every union entry holds at most m pairs (one per token)
    BurstCfg rb = burst_gu_cfg(experts->gate.fmt, hidden, moe_inter, m);
    rb.ok = rb.ok && P <= 64;   // the burst kernel reads a plan entry's pairs with one ballot
    if (rin) {   // the caller checked route_in_gu: the routed job routes the batch first
        gp.logits = rin->logits;
        gp.escale = rin->scale;
        gp.cap = rin->cap;
        gp.ids_out = const_cast<int32_t*>(topk_ids);
        gp.w_out = const_cast<float*>(topk_w);
        gp.plan_out = const_cast<int32_t*>(plan);
        rb.lds = std::max(rb.lds, small_route_lds(m, n_experts, top_k));
        if (!rb.ok) return FFNQ_ERR_UNSUPPORTED;
    }
    KConfig gcs{};
    GUParams gps{};
    DenseWs Ls{};
    BurstCfg sb{};
    if (sh) {
        Ls = dense_ws(sh->ffn->down.fmt, hidden, sh->inter, m, FFNQ_TAIL_SIGMOID_GATE, true);
        gcs = dense_gu_config(sh->ffn, hidden, sh->inter, m, cus);
        gps = dense_gu_params(sh->ffn, hidden, sh->inter, m, act, x, gcs,
                              reinterpret_cast<uint16_t*>(sh->base + Ls.act), sh->gate_vec,
                              reinterpret_cast<float*>(sh->base + Ls.logit));
        sb = dense_gu_burst(sh->ffn, hidden, sh->inter, m);
    }
    // burst workgroups: one per (union entry, tile) for every entry the plan can
    // hold (one per pair; several sub-batches may repeat an expert), those past
    // the plan's union return at once
    const int nr_items = P * ((moe_inter + 15) / 16);
    const PrefillCfg pf = rb.ok ? PrefillCfg{} : prefill_cfg(experts, n_experts, hidden, moe_inter, m, top_k, cus);
    PrefillParams pp{};
    if (pf.ok) {
        pp.tebytes = gp.tebytes;
        pp.plan = plan;
        pp.topk_ids = topk_ids;
        pp.m = m;
        pp.top_k = top_k;
        pp.n_experts = n_experts;
        pp.act = act;
    }
    if (pf.ok) {
        if (sh) {
            const int rc = launch_shared_gu(sh, hidden, m, act, x, gps, gcs, sb, stream);
            if (rc != FFNQ_OK) return rc;
        }
        PrefillParams q = pp;
        q.tq[0] = gp.tgate;
        q.tq[1] = gp.tup;
        q.N = moe_inter;
        q.K = hidden;
        q.src = x;
        q.act_out = gp.act_out;
        q.kg = 1;
        if (!launch_prefill(false, pf.tpw_gu, pf.grid_gu, pf.lds_gu, stream, q)) return FFNQ_ERR_HIP;
    } else if (rb.ok) {
        if (sh && sb.ok && to_fmt(sh->ffn->gate.fmt) == FMT_INT4 && sb.ks == rb.ks && sb.R == rb.R) {
            // shared and routed gate/up in one burst launch
            if (!launch_gu_burst_jobs(experts->gate.fmt, rb.R, rb.ks, std::max(sb.lds, rb.lds), gps,
                                      (sh->inter + 15) / 16, &gp, nr_items, stream))
                return FFNQ_ERR_UNSUPPORTED;
        } else {
            if (sh) {
                const int rc = launch_shared_gu(sh, hidden, m, act, x, gps, gcs, sb, stream);
                if (rc != FFNQ_OK) return rc;
            }
            if (!launch_gu_burst_jobs(experts->gate.fmt, rb.R, rb.ks, rb.lds, gp, nr_items, nullptr, 0, stream))
                return FFNQ_ERR_UNSUPPORTED;
        }
    } else if (sh && !sb.ok && tiled && is_tiled(sh->ffn->gate.fmt) && is_int4(sh->ffn->gate.fmt) &&
               launch_gu_tiled2(gcs, gps, gc, gp, stream)) {
        // shared and routed gate/up in one streaming launch
    } else {
        if (sh) {
            const int rc = launch_shared_gu(sh, hidden, m, act, x, gps, gcs, sb, stream);
            if (rc != FFNQ_OK) return rc;
        }
        if (!(tiled ? launch_gu_tiled(FMT_INT4, gc, stream, gp) : launch_gu(FMT_INT4, gc, u_est, moe_inter, stream, gp)))
            return FFNQ_ERR_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    // phase 2, fused: the shared expert's down, the routed down, the seeded
    // reduction and the residual add in one launch
    const MoeDownCfg md = moe_down_cfg(experts, n_experts, hidden, moe_inter, m, top_k, sh ? sh->ffn : nullptr,
                                       sh ? sh->inter : 0);
    if (md.ok) {
        MoeDownParams q{};
        q.tdown = static_cast<const uint8_t*>(experts->down.q);
        q.tebytes = tiled_expert_bytes(experts->down);
        q.N = hidden;
        q.K = moe_inter;
        q.act = gp.act_out;
        q.act_rows = P;
        q.plan = plan;
        q.topk_ids = topk_ids;
        q.topk_w = topk_w;
        q.m = m;
        q.top_k = top_k;
        q.n_experts = n_experts;
        if (sh) {
            q.sh_tdown = static_cast<const uint8_t*>(sh->ffn->down.q);
            q.sh_K = sh->inter;
            q.sh_act = gps.act_out;
            q.sh_logit = gps.logit;
        } else {
            q.seed = seed;
        }
        q.resid = resid;
        q.resid_zero = out_zero ? 1 : 0;
        if (!launch_moe_down(md, hidden, stream, q)) return FFNQ_ERR_UNSUPPORTED;
        return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
    }

    // the shared expert's down: as ffnq_shared_expert runs it -- the burst
    // kernel with its sigmoid-gate tail writing the bf16 seed, or fp32 K-range
    // partials from which the routed reduction makes the seed
    KConfig dcs{};
    DownParams dps{};
    const uint16_t* seed_rows = seed;
    bool sh_part = false;
    if (sh) {
        dcs = dense_down_config(sh->ffn, hidden, sh->inter, m, cus, FFNQ_TAIL_SIGMOID_GATE);
        const BurstCfg sdb = dense_down_burst(sh->ffn->down.fmt, hidden, sh->inter, m);
        if (sdb.ok) {
            uint16_t* sbuf = reinterpret_cast<uint16_t*>(base + L.seed);
            dps = dense_down_params(sh->ffn, hidden, sh->inter, m, dcs, gps.act_out, sbuf,
                                    reinterpret_cast<float*>(sh->base + Ls.part),
                                    reinterpret_cast<const float*>(sh->base + Ls.logit), TAIL_SIGMOID);
            dps.KG = 1;
            if (!launch_down_burst(sh->ffn->down.fmt, sdb, hidden, stream, dps)) return FFNQ_ERR_UNSUPPORTED;
            if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;
            seed_rows = sbuf;
        } else {
            dps = dense_down_params(sh->ffn, hidden, sh->inter, m, dcs, gps.act_out, nullptr,
                                    reinterpret_cast<float*>(sh->base + Ls.part),
                                    reinterpret_cast<const float*>(sh->base + Ls.logit), TAIL_PART);
            sh_part = true;
        }
    }

    // phase 2: down per union entry and tile, d_p to pair_out
    const KConfig dc = tiled ? down_tiled_config(experts->down.fmt, moe_inter, hidden, u_est, m, cus, false,
                                                 rows_per_item(false, m, top_k, n_experts), false)
                             : down_config(experts->down.fmt, moe_inter, hidden, u_est, m, cus);

    // Both downs tiled INT4 and the routed one a K split with one wave per
    // workgroup: the shared down takes the same shape (its K ranges, and so its
    // partials, unchanged; one K range per workgroup) and both run in one launch.
    bool merged = false;
    KConfig dcs1 = dcs;
    if (!pf.ok && sh_part && tiled && is_tiled(sh->ffn->down.fmt) && is_int4(sh->ffn->down.fmt) && !dc.ts &&
        dc.ks == 1 && dcs.nt == dc.nt && dcs.mt == dc.mt) {
        const TileGeo gs = tile_geo(FMT_INT4, hidden, sh->inter);
        dcs1.ts = 0;
        dcs1.ks = 1;
        dcs1.grid = (int)std::min<long long>(gs.T, (long long)cus * 16);
        dcs1.lds = tiled_launch_lds(1, FMT_INT4, hidden, sh->inter, dcs1.kg, dcs1.rows_cap, 1,
                                    2 * dcs1.nt * red_lanes(dcs1.nt, dcs1.rows_cap)).total;
        merged = dcs1.lds <= kLdsBudget;
    }
    if (sh_part && !merged) {
        const int sdfmt = to_fmt(sh->ffn->down.fmt);
        if (!(is_tiled(sh->ffn->down.fmt) ? launch_down_tiled(sdfmt, dcs, stream, dps)
                                          : launch_down(sdfmt, dcs, 1, hidden, stream, dps)))
            return FFNQ_ERR_UNSUPPORTED;
        if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;
    }
    DownParams dp{};
    dp.down = mat_dev(experts->down);
    dp.N = hidden;
    dp.K = moe_inter;
    dp.act = gp.act_out;
    dp.act_rows = P;
    dp.m = m;
    dp.rows_cap = dc.rows_cap;
    dp.KG = dc.kg;
    dp.plan = plan;
    dp.top_k = top_k;
    dp.topk_ids = topk_ids;
    dp.n_experts = n_experts;
    dp.tail = TAIL_PAIR;
    dp.part = reinterpret_cast<float*>(base + L.part);
    if (tiled) {
        dp.tdown = static_cast<const uint8_t*>(experts->down.q);
        dp.tebytes = tiled_expert_bytes(experts->down);
    }
    int part_ranges = dc.kg;
    if (pf.ok) {   // the grouped down: every pair's d as fp32 partials over kg K ranges
        PrefillParams q = pp;
        q.tq[0] = dp.tdown;
        q.tebytes = dp.tebytes;   // the down matrices' own expert stride
        q.N = hidden;
        q.K = moe_inter;
        q.src = gp.act_out;
        q.part = dp.part;
        q.kg = pf.kg_dn;
        if (!launch_prefill(true, pf.tpw_dn, pf.grid_dn, pf.lds_dn, stream, q)) return FFNQ_ERR_HIP;
        part_ranges = pf.kg_dn;
    } else if (merged) {
        if (!launch_down_tiled2(dcs1, dps, dc, dp, stream)) return FFNQ_ERR_UNSUPPORTED;
    } else if (!(tiled ? launch_down_tiled(FMT_INT4, dc, stream, dp)
                       : launch_down(FMT_INT4, dc, u_est, hidden, stream, dp))) {
        return FFNQ_ERR_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    // seeded rank-ordered reduce + residual
    const long long total = (long long)m * hidden;
    const int rgrid = (int)std::min<long long>((total + 255) / 256, (long long)cus * 8);
    hipLaunchKernelGGL(moe_reduce_kernel, dim3(rgrid), dim3(256), 0, stream, dp.part, part_ranges, topk_w, topk_ids,
                       n_experts, sh_part ? nullptr : seed_rows, resid, m, top_k, hidden, sh_part ? dps.part : nullptr,
                       sh_part ? dcs.kg : 0, sh_part ? dps.logit : nullptr);
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;
    return FFNQ_OK;
}

// ---------------------------------------------------------------------------
// router top-k and plan (ffnq_moe_route, and ffnq_moe_layer_logits when it
// cannot route inside the gate/up launch)

int check_route(const float* logits, const float* expert_scale, int m, int n_experts, int top_k, int slot_cap,
                const int32_t* topk_ids, const float* topk_w, const int32_t* plan, size_t plan_bytes)
{
    if (m < 0 || n_experts <= 0 || top_k < 1 || top_k > n_experts) return FFNQ_ERR_INVALID;
    if (!logits || !topk_ids || !topk_w || !plan) return FFNQ_ERR_INVALID;
    if (misaligned(logits) || misaligned(topk_ids) || misaligned(topk_w) || misaligned(plan) ||
        (expert_scale && misaligned(expert_scale)))
        return FFNQ_ERR_INVALID;
    if (n_experts > FFNQ_MAX_EXPERTS) return FFNQ_ERR_UNSUPPORTED;
    if (slot_cap > FFNQ_MAX_SLOTS) return FFNQ_ERR_UNSUPPORTED;
    if (slot_cap < top_k) return FFNQ_ERR_CAPACITY;
    if ((long long)m * top_k > (1 << 28)) return FFNQ_ERR_INVALID;
    if (plan_bytes < (size_t)FFNQ_PLAN_INTS((size_t)m, (size_t)top_k) * 4) return FFNQ_ERR_WORKSPACE;
    return FFNQ_OK;
}

// A checked route with m > 0: the small-batch kernel when the batch has at most
// 256 keys (one workgroup, a thread per key; measured faster there, slower
// than route_kernel at 512 keys), else route_kernel.
constexpr int kSmallRouteKeys = 256;
int launch_route(const float* logits, const float* expert_scale, int m, int n_experts, int top_k, int slot_cap,
                 int32_t* topk_ids, float* topk_w, int32_t* plan, hipStream_t stream)
{
    RouteParams p{logits, expert_scale, m, n_experts, top_k, slot_cap, topk_ids, topk_w, plan};
    const long long P = (long long)m * top_k;
    const size_t slds = small_route_lds(m, n_experts, top_k);
    if (P <= kSmallPairs && (long long)m * n_experts <= kSmallRouteKeys && slds <= kLdsBudget) {
        hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(256), slds, stream, p);
    } else if (P <= kIdsCache && (long long)m * n_experts <= kLgCache) {
        hipLaunchKernelGGL(route_kernel<true>, dim3(1), dim3(256), 0, stream, p);
    } else {
        hipLaunchKernelGGL(route_kernel<false>, dim3(1), dim3(256), 0, stream, p);
    }
    return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
}

// ffnq_moe_layer, and ffnq_moe_layer_logits (rin: route the batch first; in
// the routed gate/up launch when it can, else with its own launch).
int moe_layer_common(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k, int act,
                     const ffnq_ffn* shared, int shared_inter, const uint16_t* shared_gate, const uint16_t* x,
                     const int32_t* topk_ids, const float* topk_w, const int32_t* plan, size_t plan_bytes,
                     uint16_t* resid, void* ws, size_t* ws_bytes, hipStream_t stream, const RouteIn* rin)
{
    if (!ws_bytes) return FFNQ_ERR_INVALID;
    if (m < 0 || n_experts <= 0 || top_k < 1 || top_k > n_experts) return FFNQ_ERR_INVALID;
    int rc = check_ffn(experts, hidden, moe_inter);
    if (rc != FFNQ_OK) return rc;
    if (!is_int4(experts->gate.fmt) || !is_int4(experts->up.fmt) || !is_int4(experts->down.fmt))
        return FFNQ_ERR_UNSUPPORTED;
    if (shared) {
        rc = check_ffn(shared, hidden, shared_inter);
        if (rc != FFNQ_OK) return rc;
        if (!shared_gate || misaligned(shared_gate)) return FFNQ_ERR_INVALID;
    }
    if (act != FFNQ_ACT_SILU && act != FFNQ_ACT_GELU_TANH) return FFNQ_ERR_UNSUPPORTED;
    if (!x || !topk_ids || !topk_w || !plan || !resid) return FFNQ_ERR_INVALID;
    if (misaligned(x) || misaligned(topk_ids) || misaligned(topk_w) || misaligned(plan) || misaligned(resid))
        return FFNQ_ERR_INVALID;
    if ((long long)m * top_k > (1 << 28)) return FFNQ_ERR_INVALID;
    const size_t rows_bytes = (size_t)m * hidden * 2;
    if (m > 0 && overlap(x, rows_bytes, resid, rows_bytes)) return FFNQ_ERR_INVALID;
    if (rin) {
        rc = check_route(rin->logits, rin->scale, m, n_experts, top_k, rin->cap, topk_ids, topk_w, plan, plan_bytes);
        if (rc != FFNQ_OK) return rc;
    }
    const RoutedWs L = routed_ws(experts->down.fmt, hidden, moe_inter, m, top_k, n_experts);
    const size_t shared_off = align_up(L.total, 256);
    const size_t total = m == 0 ? 0
                                : shared_off + (shared ? dense_ws(shared->down.fmt, hidden, shared_inter, m,
                                                                  FFNQ_TAIL_SIGMOID_GATE, true).total
                                                       : 0);
    if (!ws) {
        *ws_bytes = total;
        return FFNQ_OK;
    }
    if (*ws_bytes < total) return FFNQ_ERR_WORKSPACE;
    if (misaligned(ws)) return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;
    if (rin && !route_in_gu(experts, n_experts, hidden, moe_inter, m, top_k)) {
        rc = launch_route(rin->logits, rin->scale, m, n_experts, top_k, rin->cap, const_cast<int32_t*>(topk_ids),
                          const_cast<float*>(topk_w), const_cast<int32_t*>(plan), stream);
        if (rc != FFNQ_OK) return rc;
        rin = nullptr;
    }
    unsigned char* base = static_cast<unsigned char*>(ws);
    const LayerShared lsh{shared, shared_inter, shared_gate, base + shared_off};
    return run_routed(experts, n_experts, hidden, moe_inter, m, top_k, act, x, topk_ids, topk_w, plan, nullptr, resid,
                      base, stream, shared ? &lsh : nullptr, rin);
}

// ---------------------------------------------------------------------------
// The Gemma-style routed layer (ffnq_moe_layer_sandwich): route with the
// per-expert scale; the shared branch with its own RMSNorm tail into the bf16
// row h1; the routed half unseeded into the bf16 row r (the routed call on a
// zeroed row: its sum starts from nothing); the sandwich tail.  Workspace:
// h1 and r, then the shared branch's workspace, then the routed half's.
struct SandwichWs {
    size_t h1, r, sh, routed, total;
};

SandwichWs sandwich_ws(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k,
                       const ffnq_ffn* shared, int shared_inter)
{
    SandwichWs w{};
    const size_t rows = align_up((size_t)m * hidden * 2, 256);
    size_t o = 0;
    w.h1 = o; o += rows;
    w.r = o; o += rows;
    w.sh = o; o += align_up(dense_ws(shared->down.fmt, hidden, shared_inter, m, FFNQ_TAIL_RMSNORM, true).total, 256);
    w.routed = o; o += routed_ws(experts->down.fmt, hidden, moe_inter, m, top_k, n_experts).total;
    w.total = m == 0 ? 0 : o;
    return w;
}

int moe_layer_sandwich(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k, int act,
                       const ffnq_ffn* shared, int shared_inter, const uint16_t* shared_norm_w,
                       const uint16_t* post_norm_w, float eps, const uint16_t* x, const float* logits,
                       const float* expert_scale, int slot_cap, int32_t* topk_ids, float* topk_w, int32_t* plan,
                       size_t plan_bytes, uint16_t* resid, void* ws, size_t* ws_bytes, hipStream_t stream)
{
    if (!ws_bytes) return FFNQ_ERR_INVALID;
    if (m < 0 || n_experts <= 0 || top_k < 1 || top_k > n_experts) return FFNQ_ERR_INVALID;
    int rc = check_ffn(experts, hidden, moe_inter);
    if (rc != FFNQ_OK) return rc;
    if (!is_int4(experts->gate.fmt) || !is_int4(experts->up.fmt) || !is_int4(experts->down.fmt))
        return FFNQ_ERR_UNSUPPORTED;
    if (!shared) return FFNQ_ERR_INVALID;
    rc = check_ffn(shared, hidden, shared_inter);
    if (rc != FFNQ_OK) return rc;
    if (act != FFNQ_ACT_SILU && act != FFNQ_ACT_GELU_TANH) return FFNQ_ERR_UNSUPPORTED;
    if (!x || !resid || !shared_norm_w || !post_norm_w) return FFNQ_ERR_INVALID;
    if (misaligned(x) || misaligned(resid) || misaligned(shared_norm_w) || misaligned(post_norm_w))
        return FFNQ_ERR_INVALID;
    if (!(eps >= 0.0f && std::isfinite(eps))) return FFNQ_ERR_INVALID;
    if ((long long)m * top_k > (1 << 28)) return FFNQ_ERR_INVALID;
    const size_t rows_bytes = (size_t)m * hidden * 2;
    if (m > 0 && overlap(x, rows_bytes, resid, rows_bytes)) return FFNQ_ERR_INVALID;
    rc = check_route(logits, expert_scale, m, n_experts, top_k, slot_cap, topk_ids, topk_w, plan, plan_bytes);
    if (rc != FFNQ_OK) return rc;
    const SandwichWs L = sandwich_ws(experts, n_experts, hidden, moe_inter, m, top_k, shared, shared_inter);
    if (!ws) {
        *ws_bytes = L.total;
        return FFNQ_OK;
    }
    if (*ws_bytes < L.total) return FFNQ_ERR_WORKSPACE;
    if (misaligned(ws)) return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;
    unsigned char* base = static_cast<unsigned char*>(ws);
    uint16_t* h1 = reinterpret_cast<uint16_t*>(base + L.h1);
    uint16_t* r = reinterpret_cast<uint16_t*>(base + L.r);

    const RouteIn rin_v{logits, expert_scale, slot_cap};
    const RouteIn* rin = &rin_v;
    if (!route_in_gu(experts, n_experts, hidden, moe_inter, m, top_k)) {
        rc = launch_route(logits, expert_scale, m, n_experts, top_k, slot_cap, topk_ids, topk_w, plan, stream);
        if (rc != FFNQ_OK) return rc;
        rin = nullptr;
    }
    // the shared branch up to its down projection's partials; its RMSNorm runs
    // in the tail kernel
    const float* sh_part = nullptr;
    int sh_R = 0;
    rc = run_dense(true, shared, hidden, shared_inter, m, act, FFNQ_TAIL_RMSNORM, x, h1, shared_norm_w, eps,
                   base + L.sh, stream, &sh_part, &sh_R);
    if (rc != FFNQ_OK) return rc;
    // the routed sum from +0 into r
    rc = run_routed(experts, n_experts, hidden, moe_inter, m, top_k, act, x, topk_ids, topk_w, plan, nullptr, r,
                    base + L.routed, stream, nullptr, rin, true);
    if (rc != FFNQ_OK) return rc;
    const size_t tail_lds = hidden <= kRowLds ? (size_t)hidden * 8 : (size_t)hidden * 2;
    hipLaunchKernelGGL(sandwich_norm_tail_kernel, dim3(m), dim3(kNormThreads), tail_lds, stream, sh_part, sh_R, m,
                       shared_norm_w, r, post_norm_w, hidden, eps, resid);
    return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Routed experts streamed from host memory through a slot cache
// (ffnq_moe_routed_streamed).

// Whether the host copy of a plan and its ids (m tokens, k per token) is one
// that ffnq_moe_route could write: sub-batch bounds in order and covering the
// tokens, unions of 1..min(32, n_slots) distinct valid experts, every pair's
// slot inside its sub-batch's union and naming its id's expert, and the pair
// lists a permutation of each sub-batch's pairs by slot.  FFNQ_OK,
// FFNQ_ERR_CAPACITY (a union larger than the cache) or FFNQ_ERR_INVALID.
int check_host_plan(const int32_t* plan, const int32_t* ids, int m, int k, int n_experts, int n_slots)
{
    const int P = m * k;
    const int32_t* tok = plan + 1;
    const int32_t* uni = plan + (m + 2);
    const int32_t* uexp = plan + (2 * m + 3);
    const int32_t* pslot = plan + (2 * m + 3 + P);
    const int32_t* spb = plan + (2 * m + 3 + 2 * P);
    const int32_t* sp = plan + (2 * m + 4 + 3 * P);
    const int S = plan[0];
    if (S < 1 || S > m || tok[0] != 0 || uni[0] != 0 || tok[S] != m) return FFNQ_ERR_INVALID;
    std::vector<char> seen((size_t)P, 0);
    for (int b = 0; b < S; ++b) {
        const int t0 = tok[b], t1 = tok[b + 1], u0 = uni[b], u1 = uni[b + 1];
        if (t1 <= t0 || t1 > m || u1 <= u0 || u1 > P) return FFNQ_ERR_INVALID;
        if (u1 - u0 > std::min(FFNQ_MAX_SLOTS, n_slots)) return FFNQ_ERR_CAPACITY;
        for (int j = u0; j < u1; ++j) {
            if (uexp[j] < 0 || uexp[j] >= n_experts) return FFNQ_ERR_INVALID;
            for (int j2 = u0; j2 < j; ++j2)
                if (uexp[j2] == uexp[j]) return FFNQ_ERR_INVALID;
        }
        for (int p = t0 * k; p < t1 * k; ++p) {
            const int j = pslot[p];
            if (j < 0 || j >= u1 - u0 || uexp[u0 + j] != ids[p]) return FFNQ_ERR_INVALID;
        }
        if (spb[u0] < 0 || spb[u1] - spb[u0] != (t1 - t0) * k || spb[u1] > P) return FFNQ_ERR_INVALID;
        for (int j = u0; j < u1; ++j) {
            if (spb[j + 1] < spb[j]) return FFNQ_ERR_INVALID;
            for (int i = spb[j]; i < spb[j + 1]; ++i) {
                if (sp[i] < t0 * k || sp[i] >= t1 * k || pslot[sp[i]] != j - u0 || seen[sp[i]]) return FFNQ_ERR_INVALID;
                seen[sp[i]] = 1;
            }
        }
    }
    if (uni[S] > P) return FFNQ_ERR_INVALID;
    return FFNQ_OK;
}

struct StreamWs {
    size_t ids, plan, routed, total;
};

StreamWs stream_ws(const ffnq_ffn* experts, int n_slots, int hidden, int moe_inter, int m, int k)
{
    StreamWs w{};
    size_t o = 0;
    w.ids = o; o += align_up((size_t)m * k * 4, 256);
    w.plan = o; o += align_up((size_t)FFNQ_PLAN_INTS((size_t)m, (size_t)k) * 4, 256);
    w.routed = o; o += routed_ws(experts->down.fmt, hidden, moe_inter, m, k, n_slots).total;
    w.total = m == 0 ? 0 : o;
    return w;
}

int moe_routed_streamed(const ffnq_ffn* hx, int n_experts, int hidden, int moe_inter, int m, int top_k, int act,
                        const uint16_t* x, const int32_t* topk_ids, const float* topk_w, const int32_t* plan,
                        const uint16_t* seed, uint16_t* resid, ffnq_slot_cache* cache, int32_t* host_staging,
                        void* ws, size_t* ws_bytes, hipStream_t stream)
{
    if (!ws_bytes || !cache) return FFNQ_ERR_INVALID;
    if (m < 0 || n_experts <= 0 || n_experts > FFNQ_MAX_EXPERTS || top_k < 1 || top_k > n_experts)
        return FFNQ_ERR_INVALID;
    int rc = check_ffn(hx, hidden, moe_inter);
    if (rc != FFNQ_OK) return rc;
    const int tf = FFNQ_FMT_INT4_AFFINE_G64_TILED;
    if (hx->gate.fmt != tf || hx->up.fmt != tf || hx->down.fmt != tf) return FFNQ_ERR_UNSUPPORTED;
    if (act != FFNQ_ACT_SILU && act != FFNQ_ACT_GELU_TANH) return FFNQ_ERR_UNSUPPORTED;
    if (!x || !topk_ids || !topk_w || !plan || !resid || !host_staging) return FFNQ_ERR_INVALID;
    if (misaligned(x) || misaligned(topk_ids) || misaligned(topk_w) || misaligned(plan) || misaligned(resid) ||
        (seed && misaligned(seed)))
        return FFNQ_ERR_INVALID;
    if ((long long)m * top_k > (1 << 28)) return FFNQ_ERR_INVALID;
    const size_t rows_bytes = (size_t)m * hidden * 2;
    if (m > 0 && overlap(x, rows_bytes, resid, rows_bytes)) return FFNQ_ERR_INVALID;
    const int ns = cache->n_slots;
    if (ns < 1 || ns > FFNQ_MAX_EXPERTS || !cache->slots || misaligned(cache->slots) || !cache->expert ||
        !cache->last_use)
        return FFNQ_ERR_INVALID;
    const size_t gb = (size_t)tiled_expert_bytes(hx->gate), db = (size_t)tiled_expert_bytes(hx->down);
    if (cache->slots_bytes < (size_t)ns * (2 * gb + db)) return FFNQ_ERR_INVALID;
    for (int s = 0; s < ns; ++s)
        if (cache->expert[s] < -1 || cache->expert[s] >= n_experts) return FFNQ_ERR_INVALID;
    const StreamWs L = stream_ws(hx, ns, hidden, moe_inter, m, top_k);
    if (!ws) {
        *ws_bytes = L.total;
        return FFNQ_OK;
    }
    if (*ws_bytes < L.total) return FFNQ_ERR_WORKSPACE;
    if (misaligned(ws)) return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;

    // the host's read-back of the routes
    const int P = m * top_k;
    const size_t pints = (size_t)FFNQ_PLAN_INTS((size_t)m, (size_t)top_k);
    int32_t* hplan = host_staging;
    int32_t* hids = host_staging + pints;
    if (hipMemcpyAsync(hplan, plan, pints * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(hids, topk_ids, (size_t)P * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return FFNQ_ERR_HIP;
    rc = check_host_plan(hplan, hids, m, top_k, n_experts, ns);
    if (rc != FFNQ_OK) return rc;

    // the slots as a stacked tiled expert tensor of ns experts
    unsigned char* sbase = static_cast<unsigned char*>(cache->slots);
    ffnq_ffn sx = *hx;
    sx.gate.q = sbase;
    sx.up.q = sbase + (size_t)ns * gb;
    sx.down.q = sbase + (size_t)ns * 2 * gb;
    const unsigned char* hg = static_cast<const unsigned char*>(hx->gate.q);
    const unsigned char* hu = static_cast<const unsigned char*>(hx->up.q);
    const unsigned char* hd = static_cast<const unsigned char*>(hx->down.q);
    unsigned char* base = static_cast<unsigned char*>(ws);
    int32_t* sub_ids = reinterpret_cast<int32_t*>(base + L.ids);
    int32_t* sub_plan = reinterpret_cast<int32_t*>(base + L.plan);

    const int S = hplan[0];
    const int32_t* tok = hplan + 1;
    const int32_t* uni = hplan + (m + 2);
    const int32_t* uexp = hplan + (2 * m + 3);
    std::vector<char> in_use(ns);
    for (int b = 0; b < S; ++b) {
        const int t0 = tok[b], t1 = tok[b + 1], u0 = uni[b], u1 = uni[b + 1], U = u1 - u0;
        SubPlanParams sp{};
        sp.plan = plan;
        sp.m = m;
        sp.k = top_k;
        sp.t0 = t0;
        sp.t1 = t1;
        sp.u0 = u0;
        sp.u1 = u1;
        sp.ids_out = sub_ids;
        sp.plan_out = sub_plan;
        std::fill(in_use.begin(), in_use.end(), 0);
        // hits first, so that no miss evicts an expert this union still needs
        for (int j = 0; j < U; ++j) {
            sp.slot_of[j] = -1;
            for (int s = 0; s < ns; ++s)
                if (cache->expert[s] == uexp[u0 + j]) {
                    sp.slot_of[j] = s;
                    in_use[s] = 1;
                    break;
                }
        }
        for (int j = 0; j < U; ++j) {
            if (sp.slot_of[j] >= 0) continue;
            int v = -1;
            for (int s = 0; s < ns; ++s) {
                if (in_use[s]) continue;
                if (v < 0 || (cache->expert[s] < 0 && cache->expert[v] >= 0) ||
                    ((cache->expert[s] < 0) == (cache->expert[v] < 0) && cache->last_use[s] < cache->last_use[v]))
                    v = s;
            }
            const size_t e = (size_t)uexp[u0 + j];
            if (hipMemcpyAsync(sbase + (size_t)v * gb, hg + e * gb, gb, hipMemcpyHostToDevice, stream) != hipSuccess ||
                hipMemcpyAsync(sbase + (size_t)(ns + v) * gb, hu + e * gb, gb, hipMemcpyHostToDevice, stream) !=
                    hipSuccess ||
                hipMemcpyAsync(sbase + (size_t)ns * 2 * gb + (size_t)v * db, hd + e * db, db, hipMemcpyHostToDevice,
                               stream) != hipSuccess) {
                cache->expert[v] = -1;   // its contents are unknown now
                return FFNQ_ERR_HIP;
            }
            cache->expert[v] = (int32_t)e;
            ++cache->copied;
            sp.slot_of[j] = v;
            in_use[v] = 1;
        }
        for (int j = 0; j < U; ++j) cache->last_use[sp.slot_of[j]] = ++cache->clock;
        hipLaunchKernelGGL(sub_plan_kernel, dim3(1), dim3(256), 0, stream, sp);
        if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;
        rc = run_routed(&sx, ns, hidden, moe_inter, t1 - t0, top_k, act, x + (size_t)t0 * hidden, sub_ids,
                        topk_w + (size_t)t0 * top_k, sub_plan, seed ? seed + (size_t)t0 * hidden : nullptr,
                        resid + (size_t)t0 * hidden, base + L.routed, stream, nullptr);
        if (rc != FFNQ_OK) return rc;
    }
    return FFNQ_OK;
}

// ---------------------------------------------------------------------------
// The allocation-free dense call (ffnq_dense_noalloc) keeps its workspace in
// this file-scope device array: every GPU the library runs on holds one copy,
// for the life of the process.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address); it asks the
// runtime once per device for that device's address and uses only that.
__device__ __align__(256) unsigned char scratch[FFNQ_NOALLOC_SCRATCH_BYTES];

// The device address of `scratch` on the current device, looked up on the
// first call made with that device current and kept; nullptr if the lookup
// fails (the caller then returns FFNQ_ERR_HIP).
void* scratch_address()
{
    constexpr int kMaxDev = 64;
    static std::atomic<void*> addr[kMaxDev];
    static std::mutex mu;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    addr[dev].store(q, std::memory_order_release);
    return q;
}

// A plain streaming read (16-byte loads, four in flight per thread, grid-stride)
// that only folds what it reads into a value it almost never stores: the
// practical HBM read rate of this GPU, which the weight-streaming kernels are
// held against beside the published peak.
constexpr int kReadWGs = 256, kReadThreads = 512, kReadUnroll = 4;

__global__ void __launch_bounds__(kReadThreads) stream_read_kernel(const uint4* __restrict__ p, size_t n,
                                                                    unsigned* sink)
{
    unsigned acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) atomicXor(sink, acc);   // keeps the loads; the value itself means nothing
}

}  // namespace

extern "C" {

const char* ffnq_status_string(int status)
{
    switch (status) {
        case FFNQ_OK: return "ok";
        case FFNQ_ERR_INVALID: return "invalid argument";
        case FFNQ_ERR_UNSUPPORTED: return "unsupported";
        case FFNQ_ERR_CAPACITY: return "capacity: slot_cap < top_k";
        case FFNQ_ERR_WORKSPACE: return "workspace too small";
        case FFNQ_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

size_t ffnq_packed_bytes(int fmt, int n, int k)
{
    if (fmt != FFNQ_FMT_INT8_ROW && fmt != FFNQ_FMT_INT4_AFFINE_G64 && !is_tiled(fmt)) return 0;
    if (n <= 0 || k <= 0 || k % 64 != 0 || (is_int4(fmt) && k % 128 != 0)) return 0;
    return (size_t)tile_geo(to_fmt(fmt), n, k).expert_bytes;
}

int ffnq_pack(const ffnq_qmat* src, int n_experts, void* dst, size_t dst_bytes, hipStream_t stream)
{
    if (!src || !dst || n_experts <= 0) return FFNQ_ERR_INVALID;
    if (src->fmt != FFNQ_FMT_INT8_ROW && src->fmt != FFNQ_FMT_INT4_AFFINE_G64) return FFNQ_ERR_UNSUPPORTED;
    bool uns = false;
    const int rc = check_mat(*src, &uns);
    if (rc != FFNQ_OK) return rc;
    if (misaligned(dst)) return FFNQ_ERR_INVALID;
    const long long eb = tile_geo(to_fmt(src->fmt), src->n, src->k).expert_bytes;
    if ((long long)n_experts > (1LL << 40) / eb) return FFNQ_ERR_INVALID;
    const size_t need = (size_t)eb * (size_t)n_experts;
    if (dst_bytes < need) return FFNQ_ERR_WORKSPACE;
    const MatDev d = mat_dev(*src);
    const size_t qbytes = (size_t)d.qe * n_experts;
    const size_t sbytes = (size_t)d.se * n_experts * (is_int4(src->fmt) ? 2 : 4);
    if (overlap(dst, need, src->q, qbytes) || overlap(dst, need, src->s, sbytes) ||
        (src->z && overlap(dst, need, src->z, sbytes)))
        return FFNQ_ERR_INVALID;
    PackParams p{};
    p.fmt = to_fmt(src->fmt);
    p.n = src->n;
    p.k = src->k;
    p.n_experts = n_experts;
    p.q = static_cast<const uint8_t*>(src->q);
    p.s = src->s;
    p.z = static_cast<const uint16_t*>(src->z);
    p.qe = d.qe;
    p.se = d.se;
    p.dst = static_cast<uint8_t*>(dst);
    const long long chunks = (long long)need / 16;
    const int grid = (int)std::min<long long>((chunks + 255) / 256, (long long)device_cus() * 16);
    hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
}

int ffnq_set_phase_events(hipEvent_t* ev)
{
    t_phase_ev = ev;
    return FFNQ_OK;
}

int ffnq_stream_read(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream)
{
    if (!buf || !sink || misaligned(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0 || bytes % 16 != 0)
        return FFNQ_ERR_INVALID;
    if (bytes == 0) return FFNQ_OK;
    hipExtLaunchKernelGGL(stream_read_kernel, dim3(kReadWGs), dim3(kReadThreads), 0, stream, phase_event(0),
                          phase_event(1), 0, static_cast<const uint4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
}

int ffnq_dense(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x, uint16_t* out,
               const uint16_t* norm_w, float eps, void* ws, size_t* ws_bytes, hipStream_t stream)
{
    return dense_common(ffn, hidden, inter, m, act, tail, x, out, norm_w, eps, ws, ws_bytes, stream, false);
}

int ffnq_dense_noalloc(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x,
                       uint16_t* out, const uint16_t* norm_w, float eps, hipStream_t stream)
{
    // the checks and the size query of ffnq_dense; then its launches on the device's scratch array
    size_t need = 0;
    const int rc = dense_common(ffn, hidden, inter, m, act, tail, x, out, norm_w, eps, nullptr, &need, stream, false);
    if (rc != FFNQ_OK) return rc;
    if (need > (size_t)FFNQ_NOALLOC_SCRATCH_BYTES) return FFNQ_ERR_WORKSPACE;
    if (m == 0) return FFNQ_OK;
    void* ws = scratch_address();
    if (!ws) return FFNQ_ERR_HIP;
    return dense_common(ffn, hidden, inter, m, act, tail, x, out, norm_w, eps, ws, &need, stream, false);
}

int ffnq_shared_expert(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x,
                       uint16_t* h_out, const uint16_t* aux, float eps, void* ws, size_t* ws_bytes,
                       hipStream_t stream)
{
    return dense_common(ffn, hidden, inter, m, act, tail, x, h_out, aux, eps, ws, ws_bytes, stream, true);
}

int ffnq_router_logits(const uint16_t* x, const uint16_t* w, int m, int hidden, int n_experts, float* logits,
                       hipStream_t stream)
{
    if (!x || !w || !logits) return FFNQ_ERR_INVALID;
    if (m < 0 || hidden <= 0 || hidden % 8 != 0 || n_experts <= 0) return FFNQ_ERR_INVALID;
    if (misaligned(x) || misaligned(w) || misaligned(logits)) return FFNQ_ERR_INVALID;
    if ((long long)m * n_experts > (1LL << 30) || (long long)n_experts * hidden > (1LL << 40)) return FFNQ_ERR_INVALID;
    const size_t lbytes = (size_t)m * n_experts * 4;
    if (m > 0 && (overlap(logits, lbytes, x, (size_t)m * hidden * 2) ||
                  overlap(logits, lbytes, w, (size_t)n_experts * hidden * 2)))
        return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;
    const long long waves = (long long)m * n_experts;
    hipLaunchKernelGGL(router_gemv_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, x, w, m, hidden,
                       n_experts, logits);
    return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
}

int ffnq_moe_route(const float* logits, const float* expert_scale, int m, int n_experts, int top_k, int slot_cap,
                   int32_t* topk_ids, float* topk_w, int32_t* plan, size_t plan_bytes, hipStream_t stream)
{
    const int rc = check_route(logits, expert_scale, m, n_experts, top_k, slot_cap, topk_ids, topk_w, plan, plan_bytes);
    if (rc != FFNQ_OK || m == 0) return rc;
    return launch_route(logits, expert_scale, m, n_experts, top_k, slot_cap, topk_ids, topk_w, plan, stream);
}

int ffnq_moe_routed_batched(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k,
                            int act, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                            const int32_t* plan, const uint16_t* seed, uint16_t* resid, void* ws,
                            size_t* ws_bytes, hipStream_t stream)
{
    if (!ws_bytes) return FFNQ_ERR_INVALID;
    if (m < 0 || n_experts <= 0 || top_k < 1 || top_k > n_experts) return FFNQ_ERR_INVALID;
    const int rc = check_ffn(experts, hidden, moe_inter);
    if (rc != FFNQ_OK) return rc;
    if (!is_int4(experts->gate.fmt) || !is_int4(experts->up.fmt) || !is_int4(experts->down.fmt))
        return FFNQ_ERR_UNSUPPORTED;
    if (act != FFNQ_ACT_SILU && act != FFNQ_ACT_GELU_TANH) return FFNQ_ERR_UNSUPPORTED;
    if (!x || !topk_ids || !topk_w || !plan || !resid) return FFNQ_ERR_INVALID;
    if (misaligned(x) || misaligned(topk_ids) || misaligned(topk_w) || misaligned(plan) || misaligned(resid) ||
        (seed && misaligned(seed)))
        return FFNQ_ERR_INVALID;
    if ((long long)m * top_k > (1 << 28)) return FFNQ_ERR_INVALID;
    const size_t rows_bytes = (size_t)m * hidden * 2;
    if (m > 0 && overlap(x, rows_bytes, resid, rows_bytes)) return FFNQ_ERR_INVALID;
    const RoutedWs L = routed_ws(experts->down.fmt, hidden, moe_inter, m, top_k, n_experts);
    if (!ws) {
        *ws_bytes = L.total;
        return FFNQ_OK;
    }
    if (*ws_bytes < L.total) return FFNQ_ERR_WORKSPACE;
    if (misaligned(ws)) return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;

    return run_routed(experts, n_experts, hidden, moe_inter, m, top_k, act, x, topk_ids, topk_w, plan, seed, resid,
                      static_cast<unsigned char*>(ws), stream, nullptr);
}

int ffnq_moe_layer(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k, int act,
                   const ffnq_ffn* shared, int shared_inter, const uint16_t* shared_gate, const uint16_t* x,
                   const int32_t* topk_ids, const float* topk_w, const int32_t* plan, uint16_t* resid, void* ws,
                   size_t* ws_bytes, hipStream_t stream)
{
    return moe_layer_common(experts, n_experts, hidden, moe_inter, m, top_k, act, shared, shared_inter, shared_gate,
                            x, topk_ids, topk_w, plan, 0, resid, ws, ws_bytes, stream, nullptr);
}

int ffnq_moe_layer_logits(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k,
                          int act, const ffnq_ffn* shared, int shared_inter, const uint16_t* shared_gate,
                          const uint16_t* x, const float* logits, const float* expert_scale, int slot_cap,
                          int32_t* topk_ids, float* topk_w, int32_t* plan, size_t plan_bytes, uint16_t* resid,
                          void* ws, size_t* ws_bytes, hipStream_t stream)
{
    const RouteIn rin{logits, expert_scale, slot_cap};
    return moe_layer_common(experts, n_experts, hidden, moe_inter, m, top_k, act, shared, shared_inter, shared_gate,
                            x, topk_ids, topk_w, plan, plan_bytes, resid, ws, ws_bytes, stream, &rin);
}

int ffnq_moe_layer_sandwich(const ffnq_ffn* experts, int n_experts, int hidden, int moe_inter, int m, int top_k,
                            int act, const ffnq_ffn* shared, int shared_inter, const uint16_t* shared_norm_w,
                            const uint16_t* post_norm_w, float eps, const uint16_t* x, const float* logits,
                            const float* expert_scale, int slot_cap, int32_t* topk_ids, float* topk_w,
                            int32_t* plan, size_t plan_bytes, uint16_t* resid, void* ws, size_t* ws_bytes,
                            hipStream_t stream)
{
    return moe_layer_sandwich(experts, n_experts, hidden, moe_inter, m, top_k, act, shared, shared_inter,
                              shared_norm_w, post_norm_w, eps, x, logits, expert_scale, slot_cap, topk_ids, topk_w,
                              plan, plan_bytes, resid, ws, ws_bytes, stream);
}

int ffnq_moe_routed_streamed(const ffnq_ffn* host_experts, int n_experts, int hidden, int moe_inter, int m,
                             int top_k, int act, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                             const int32_t* plan, const uint16_t* seed, uint16_t* resid, ffnq_slot_cache* cache,
                             int32_t* host_staging, void* ws, size_t* ws_bytes, hipStream_t stream)
{
    return moe_routed_streamed(host_experts, n_experts, hidden, moe_inter, m, top_k, act, x, topk_ids, topk_w, plan,
                               seed, resid, cache, host_staging, ws, ws_bytes, stream);
}

}  // extern "C"
