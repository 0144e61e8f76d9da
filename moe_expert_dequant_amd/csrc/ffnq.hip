// ffnq.hip -- the C ABI of libffnq: argument checks, workspace layout, launch
// configuration and kernel launches.  Every check runs on the host before the
// first launch; the library allocates nothing and synchronises nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "ffnq.h"
#include "device.h"
#include "qgemm.h"
#include "route.h"
#include "tail.h"

namespace {

using namespace ffnq;

constexpr int kKGMax = 16;            // largest K split of the down kernel
constexpr size_t kLdsBudget = 64 * 1024;
constexpr int kDownWaves = 4;         // row tiles per down workgroup

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int block_k(int fmt) { return fmt == FFNQ_FMT_INT4_AFFINE_G64 ? 128 : 64; }

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
    if (w.fmt != FFNQ_FMT_INT8_ROW && w.fmt != FFNQ_FMT_INT4_AFFINE_G64) {
        *unsupported = true;
        return FFNQ_ERR_UNSUPPORTED;
    }
    if (w.n <= 0 || w.k <= 0 || w.k % 64 != 0) return FFNQ_ERR_INVALID;
    if (!w.q || !w.s) return FFNQ_ERR_INVALID;
    if (w.fmt == FFNQ_FMT_INT4_AFFINE_G64 && !w.z) return FFNQ_ERR_INVALID;
    if (misaligned(w.q) || misaligned(w.s) || (w.z && misaligned(w.z))) return FFNQ_ERR_INVALID;
    if (w.fmt == FFNQ_FMT_INT4_AFFINE_G64 && w.k % 128 != 0) {
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
    return FFNQ_OK;
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

struct GUConfig {
    int nt, mt, ks, rows_cap;
    size_t lds;
};

GUConfig gu_config(int fmt, int K, int N, long long items_est, int rows_total, int cus)
{
    GUConfig c;
    const int rp = std::max(1, std::min(rows_total, 32));
    c.nt = rp <= 16 ? 1 : 2;
    c.mt = c.nt == 2 ? 4 : (rp <= 1 ? 1 : (rp <= 2 ? 2 : 4));
    const int NB = K / block_k(fmt);
    const long long target = (long long)cus * 12;
    int ks = 1;
    while (ks < 8 && items_est * ks * 2 <= target && ks * 2 <= NB) ks *= 2;
    c.ks = ks;
    const size_t per = (size_t)(fmt == FFNQ_FMT_INT8_ROW ? 3 : 2) * c.nt * 4;
    const size_t red = (size_t)ks * per * 64 * sizeof(float);
    const size_t row_bytes = (size_t)(K + 8) * 2;
    int cap = std::min(rp, 16 * c.nt);
    while (cap > 1 && red + cap * row_bytes > kLdsBudget) --cap;
    c.rows_cap = cap;
    c.lds = red + cap * row_bytes;
    (void)N;
    return c;
}

struct DownConfig {
    int nt, mt, kg, rows_cap;
    size_t lds;
};

DownConfig down_config(int fmt, int K, int N, long long items_est, int rows_total, int cus)
{
    DownConfig c;
    const int r2 = 2 * std::max(1, rows_total);
    const int rp = std::min(r2, 64);
    c.nt = rp <= 16 ? 1 : (rp <= 32 ? 2 : 4);
    c.mt = c.nt > 1 ? 4 : (rp <= 2 ? 2 : 4);
    const int BK = block_k(fmt);
    const int NB = K / BK;
    const long long target = (long long)cus * 16;
    int kg = 1;
    while (kg < kKGMax && kg < NB && items_est * kDownWaves * kg < target) ++kg;
    c.rows_cap = std::min(r2, 16 * c.nt);
    for (;;) {
        const int nbl = (NB + kg - 1) / kg;
        const size_t xb = (size_t)c.rows_cap * (nbl * BK + 8) * 2;
        const size_t resb = kg == 1 ? (size_t)r2 * 16 * kDownWaves * sizeof(float) : 0;
        c.lds = xb + resb;
        if (c.lds <= kLdsBudget) break;
        if (kg < std::min(kKGMax, NB)) {
            ++kg;
        } else if (c.rows_cap > 1) {
            --c.rows_cap;
        } else {
            break;
        }
    }
    c.kg = kg;
    (void)N;
    return c;
}

// ---------------------------------------------------------------------------
// kernel dispatch over the template parameters

#define FFNQ_GU_CASE(F, NT_, MT_)                                                              \
    if (fmt == F && c.nt == NT_ && c.mt == MT_) {                                              \
        hipLaunchKernelGGL((gu_kernel<F, NT_, MT_>), grid, block, c.lds, stream, prm);         \
        return true;                                                                           \
    }

bool launch_gu(int fmt, const GUConfig& c, dim3 grid, dim3 block, hipStream_t stream, const GUParams& prm)
{
    FFNQ_GU_CASE(FMT_INT4, 1, 1) FFNQ_GU_CASE(FMT_INT4, 1, 2) FFNQ_GU_CASE(FMT_INT4, 1, 4)
    FFNQ_GU_CASE(FMT_INT4, 2, 4) FFNQ_GU_CASE(FMT_INT8, 1, 1) FFNQ_GU_CASE(FMT_INT8, 1, 2)
    FFNQ_GU_CASE(FMT_INT8, 1, 4) FFNQ_GU_CASE(FMT_INT8, 2, 4)
    return false;
}

#define FFNQ_DOWN_CASE(F, NT_, MT_)                                                            \
    if (fmt == F && c.nt == NT_ && c.mt == MT_) {                                              \
        hipLaunchKernelGGL((down_kernel<F, NT_, MT_>), grid, block, c.lds, stream, prm);       \
        return true;                                                                           \
    }

bool launch_down(int fmt, const DownConfig& c, dim3 grid, dim3 block, hipStream_t stream, const DownParams& prm)
{
    FFNQ_DOWN_CASE(FMT_INT4, 1, 2) FFNQ_DOWN_CASE(FMT_INT4, 1, 4) FFNQ_DOWN_CASE(FMT_INT4, 2, 4)
    FFNQ_DOWN_CASE(FMT_INT4, 4, 4) FFNQ_DOWN_CASE(FMT_INT8, 1, 2) FFNQ_DOWN_CASE(FMT_INT8, 1, 4)
    FFNQ_DOWN_CASE(FMT_INT8, 2, 4) FFNQ_DOWN_CASE(FMT_INT8, 4, 4)
    return false;
}

int to_fmt(int f) { return f == FFNQ_FMT_INT4_AFFINE_G64 ? FMT_INT4 : FMT_INT8; }

// ---------------------------------------------------------------------------
// dense FFN (ffnq_dense and ffnq_shared_expert)

struct DenseWs {
    size_t act_hi, act_lo, partial, counters, hbuf, logit, total;
};

DenseWs dense_ws(int hidden, int inter, int m)
{
    DenseWs w{};
    size_t o = 0;
    const size_t plane = align_up((size_t)m * inter * 2, 256);
    w.act_hi = o; o += plane;
    w.act_lo = o; o += plane;
    w.partial = o; o += align_up((size_t)kKGMax * 2 * m * hidden * sizeof(float), 256);
    const int groups = (hidden + 16 * kDownWaves - 1) / (16 * kDownWaves);
    w.counters = o; o += align_up((size_t)groups * sizeof(unsigned), 256);
    w.hbuf = o; o += align_up((size_t)m * hidden * sizeof(float), 256);
    w.logit = o; o += align_up((size_t)m * sizeof(float), 256);
    w.total = m == 0 ? 0 : o;
    return w;
}

int run_dense(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x,
              uint16_t* out, const uint16_t* aux, float eps, void* ws, hipStream_t stream)
{
    const int cus = device_cus();
    unsigned char* base = static_cast<unsigned char*>(ws);
    const DenseWs L = dense_ws(hidden, inter, m);
    const int gfmt = to_fmt(ffn->gate.fmt), dfmt = to_fmt(ffn->down.fmt);
    const int groups = (hidden + 16 * kDownWaves - 1) / (16 * kDownWaves);

    const int tiles = (inter + 15) / 16;
    const GUConfig gc = gu_config(ffn->gate.fmt, hidden, inter, tiles, m, cus);
    GUParams gp{};
    gp.gate = mat_dev(ffn->gate);
    gp.up = mat_dev(ffn->up);
    gp.N = inter;
    gp.K = hidden;
    gp.act = act;
    gp.dfmt = dfmt;
    gp.x = x;
    gp.m = m;
    gp.rows_cap = gc.rows_cap;
    gp.plan = nullptr;
    gp.act_hi = reinterpret_cast<uint16_t*>(base + L.act_hi);
    gp.act_lo = reinterpret_cast<uint16_t*>(base + L.act_lo);
    gp.act_rows = m;
    if (tail == FFNQ_TAIL_SIGMOID_GATE) {
        gp.gate_vec = aux;
        gp.logit = reinterpret_cast<float*>(base + L.logit);
    }
    gp.zero_ptr = reinterpret_cast<unsigned*>(base + L.counters);
    gp.zero_count = groups;
    if (!launch_gu(gfmt, gc, dim3(tiles), dim3(64 * gc.ks), stream, gp)) return FFNQ_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    const DownConfig dc = down_config(ffn->down.fmt, inter, hidden, groups, m, cus);
    DownParams dp{};
    dp.down = mat_dev(ffn->down);
    dp.N = hidden;
    dp.K = inter;
    dp.act_hi = gp.act_hi;
    dp.act_lo = gp.act_lo;
    dp.act_rows = m;
    dp.m = m;
    dp.rows_cap = dc.rows_cap;
    dp.plan = nullptr;
    dp.partial = reinterpret_cast<float*>(base + L.partial);
    dp.counters = reinterpret_cast<unsigned*>(base + L.counters);
    dp.out = out;
    dp.hbuf = reinterpret_cast<float*>(base + L.hbuf);
    dp.logit = reinterpret_cast<const float*>(base + L.logit);
    switch (tail) {
        case FFNQ_TAIL_RESIDUAL: dp.tail = TAIL_RESIDUAL; break;
        case FFNQ_TAIL_RMSNORM: dp.tail = TAIL_RMSNORM; break;
        case FFNQ_TAIL_SIGMOID_GATE: dp.tail = TAIL_SIGMOID; break;
        default: dp.tail = TAIL_NONE; break;
    }
    if (!launch_down(dfmt, dc, dim3(groups, dc.kg), dim3(64 * kDownWaves), stream, dp)) return FFNQ_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    if (tail == FFNQ_TAIL_RMSNORM) {
        hipLaunchKernelGGL(rmsnorm_kernel, dim3(m), dim3(256), 0, stream, dp.hbuf, aux, out, hidden, eps);
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
    const DenseWs L = dense_ws(hidden, inter, m);
    if (!ws) {
        *ws_bytes = L.total;
        return FFNQ_OK;
    }
    if (*ws_bytes < L.total) return FFNQ_ERR_WORKSPACE;
    if (misaligned(ws)) return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;
    return run_dense(ffn, hidden, inter, m, act, tail, x, out, aux, eps, ws, stream);
}

// ---------------------------------------------------------------------------
// routed half

struct RoutedWs {
    size_t act_hi, act_lo, partial, counters, pair_out, total;
};

RoutedWs routed_ws(int hidden, int moe_inter, int m, int k)
{
    RoutedWs w{};
    const size_t P = (size_t)m * k;
    size_t o = 0;
    const size_t plane = align_up(P * moe_inter * 2, 256);
    w.act_hi = o; o += plane;
    w.act_lo = o; o += plane;
    w.partial = o; o += align_up((size_t)kKGMax * 2 * P * hidden * sizeof(float), 256);
    const int groups = (hidden + 16 * kDownWaves - 1) / (16 * kDownWaves);
    w.counters = o; o += align_up(P * groups * sizeof(unsigned), 256);
    w.pair_out = o; o += align_up(P * hidden * sizeof(float), 256);
    w.total = m == 0 ? 0 : o;
    return w;
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

int ffnq_dense(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x, uint16_t* out,
               const uint16_t* norm_w, float eps, void* ws, size_t* ws_bytes, hipStream_t stream)
{
    return dense_common(ffn, hidden, inter, m, act, tail, x, out, norm_w, eps, ws, ws_bytes, stream, false);
}

int ffnq_shared_expert(const ffnq_ffn* ffn, int hidden, int inter, int m, int act, int tail, const uint16_t* x,
                       uint16_t* h_out, const uint16_t* aux, float eps, void* ws, size_t* ws_bytes,
                       hipStream_t stream)
{
    return dense_common(ffn, hidden, inter, m, act, tail, x, h_out, aux, eps, ws, ws_bytes, stream, true);
}

int ffnq_moe_route(const float* logits, const float* expert_scale, int m, int n_experts, int top_k, int slot_cap,
                   int32_t* topk_ids, float* topk_w, int32_t* plan, size_t plan_bytes, hipStream_t stream)
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
    if (m == 0) return FFNQ_OK;
    RouteParams p{logits, expert_scale, m, n_experts, top_k, slot_cap, topk_ids, topk_w, plan};
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
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
    if (experts->gate.fmt != FFNQ_FMT_INT4_AFFINE_G64 || experts->up.fmt != FFNQ_FMT_INT4_AFFINE_G64 ||
        experts->down.fmt != FFNQ_FMT_INT4_AFFINE_G64)
        return FFNQ_ERR_UNSUPPORTED;
    if (act != FFNQ_ACT_SILU && act != FFNQ_ACT_GELU_TANH) return FFNQ_ERR_UNSUPPORTED;
    if (!x || !topk_ids || !topk_w || !plan || !resid) return FFNQ_ERR_INVALID;
    if (misaligned(x) || misaligned(topk_ids) || misaligned(topk_w) || misaligned(plan) || misaligned(resid) ||
        (seed && misaligned(seed)))
        return FFNQ_ERR_INVALID;
    if ((long long)m * top_k > (1 << 28)) return FFNQ_ERR_INVALID;
    const size_t rows_bytes = (size_t)m * hidden * 2;
    if (m > 0 && overlap(x, rows_bytes, resid, rows_bytes)) return FFNQ_ERR_INVALID;
    const RoutedWs L = routed_ws(hidden, moe_inter, m, top_k);
    if (!ws) {
        *ws_bytes = L.total;
        return FFNQ_OK;
    }
    if (*ws_bytes < L.total) return FFNQ_ERR_WORKSPACE;
    if (misaligned(ws)) return FFNQ_ERR_INVALID;
    if (m == 0) return FFNQ_OK;

    const int cus = device_cus();
    unsigned char* base = static_cast<unsigned char*>(ws);
    const int P = m * top_k;
    const long long u_est = std::min<long long>(P, n_experts);
    const int groups = (hidden + 16 * kDownWaves - 1) / (16 * kDownWaves);
    const int tiles = (moe_inter + 15) / 16;

    // phase 1: gate/up + activation per union entry and tile
    const GUConfig gc = gu_config(FFNQ_FMT_INT4_AFFINE_G64, hidden, moe_inter, u_est * tiles, m, cus);
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
    gp.act_hi = reinterpret_cast<uint16_t*>(base + L.act_hi);
    gp.act_lo = reinterpret_cast<uint16_t*>(base + L.act_lo);
    gp.act_rows = P;
    gp.zero_ptr = reinterpret_cast<unsigned*>(base + L.counters);
    gp.zero_count = P * groups;
    const long long gu_items = u_est * tiles;
    const int gu_grid = (int)std::min<long long>(gu_items, 65535);
    if (!launch_gu(FMT_INT4, gc, dim3(gu_grid), dim3(64 * gc.ks), stream, gp)) return FFNQ_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    // phase 2: down per union entry and row group, d_p to pair_out
    const DownConfig dc = down_config(FFNQ_FMT_INT4_AFFINE_G64, moe_inter, hidden, u_est * groups, m, cus);
    DownParams dp{};
    dp.down = mat_dev(experts->down);
    dp.N = hidden;
    dp.K = moe_inter;
    dp.act_hi = gp.act_hi;
    dp.act_lo = gp.act_lo;
    dp.act_rows = P;
    dp.m = m;
    dp.rows_cap = dc.rows_cap;
    dp.plan = plan;
    dp.top_k = top_k;
    dp.topk_ids = topk_ids;
    dp.n_experts = n_experts;
    dp.partial = reinterpret_cast<float*>(base + L.partial);
    dp.counters = reinterpret_cast<unsigned*>(base + L.counters);
    dp.tail = TAIL_PAIR;
    dp.hbuf = reinterpret_cast<float*>(base + L.pair_out);
    const int dn_grid = (int)std::min<long long>(u_est * groups, 65535);
    if (!launch_down(FMT_INT4, dc, dim3(dn_grid, dc.kg), dim3(64 * kDownWaves), stream, dp))
        return FFNQ_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return FFNQ_ERR_HIP;

    // seeded rank-ordered reduce + residual
    const long long total = (long long)m * hidden;
    const int rgrid = (int)std::min<long long>((total + 255) / 256, (long long)cus * 8);
    hipLaunchKernelGGL(moe_reduce_kernel, dim3(rgrid), dim3(256), 0, stream, dp.hbuf, topk_w, topk_ids, n_experts,
                       seed, resid, m, top_k, hidden);
    return hipGetLastError() == hipSuccess ? FFNQ_OK : FFNQ_ERR_HIP;
}

}  // extern "C"
