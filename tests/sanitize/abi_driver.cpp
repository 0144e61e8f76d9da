// Host-side exercise of the libffnq C ABI under AddressSanitizer and UBSan
// (built by tests/test_sanitizers.py from the library's own source, host code
// only).  Every call here is refused, or is a workspace query or an m == 0
// no-op, before any pointer is dereferenced or any GPU work is queued: the
// fake device addresses are never touched.  Checks the status codes.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "ffnq.h"

namespace {

const void* addr(int i) { return reinterpret_cast<const void*>(static_cast<uintptr_t>(0x10000) * (i + 1)); }
template <class T>
T* mut(int i) { return reinterpret_cast<T*>(const_cast<void*>(addr(i))); }

ffnq_qmat mat(int fmt, int n, int k, int base)
{
    const bool tiled = fmt == FFNQ_FMT_INT8_ROW_TILED || fmt == FFNQ_FMT_INT4_AFFINE_G64_TILED;
    const bool int4 = fmt == FFNQ_FMT_INT4_AFFINE_G64 || fmt == FFNQ_FMT_INT4_AFFINE_G64_TILED;
    return ffnq_qmat{fmt, n, k, addr(base), tiled ? nullptr : addr(base + 1), (int4 && !tiled) ? addr(base + 2) : nullptr};
}

ffnq_ffn ffn(int fg, int fd, int hidden, int inter)
{
    return ffnq_ffn{mat(fg, inter, hidden, 0), mat(fg, inter, hidden, 10), mat(fd, hidden, inter, 20)};
}

int failures = 0;
void expect(int got, int want, int line)
{
    if (got != want) {
        std::fprintf(stderr, "line %d: status %d, expected %d\n", line, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), __LINE__)

}  // namespace

int main()
{
    const int I8 = FFNQ_FMT_INT8_ROW, I4 = FFNQ_FMT_INT4_AFFINE_G64, T4 = FFNQ_FMT_INT4_AFFINE_G64_TILED;
    size_t n = 0;
    ffnq_ffn f = ffn(I4, I4, 256, 512);
    // dense: query, no-op, refusals
    EXPECT(ffnq_dense(&f, 256, 512, 2, FFNQ_ACT_SILU, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40), mut<uint16_t>(50), nullptr,
                      1e-6f, nullptr, &n, nullptr), FFNQ_OK);
    size_t z = 0;
    EXPECT(ffnq_dense(&f, 256, 512, 0, FFNQ_ACT_SILU, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40), mut<uint16_t>(50), nullptr,
                      1e-6f, nullptr, &z, nullptr), FFNQ_OK);
    EXPECT(ffnq_dense(nullptr, 256, 512, 2, FFNQ_ACT_SILU, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40), mut<uint16_t>(50),
                      nullptr, 1e-6f, nullptr, &n, nullptr), FFNQ_ERR_INVALID);
    EXPECT(ffnq_dense(&f, 256, 512, 2, 9, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40), mut<uint16_t>(50), nullptr, 1e-6f,
                      nullptr, &n, nullptr), FFNQ_ERR_UNSUPPORTED);
    EXPECT(ffnq_dense(&f, 256, 512, 2, FFNQ_ACT_SILU, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40), mut<uint16_t>(40),
                      nullptr, 1e-6f, nullptr, &n, nullptr), FFNQ_ERR_INVALID);        // x aliases out
    EXPECT(ffnq_dense(&f, 256, 512, 2, FFNQ_ACT_SILU, FFNQ_TAIL_RMSNORM, mut<uint16_t>(40), mut<uint16_t>(50), nullptr,
                      1e-6f, nullptr, &n, nullptr), FFNQ_ERR_INVALID);                 // no norm weight
    size_t small = n - 256;
    EXPECT(ffnq_dense(&f, 256, 512, 2, FFNQ_ACT_SILU, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40), mut<uint16_t>(50),
                      nullptr, 1e-6f, mut<void>(60), &small, nullptr), FFNQ_ERR_WORKSPACE);
    ffnq_ffn odd = ffn(I4, I4, 320, 512);   // INT4 with K % 128 == 64
    EXPECT(ffnq_dense(&odd, 320, 512, 2, FFNQ_ACT_SILU, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40), mut<uint16_t>(50),
                      nullptr, 1e-6f, nullptr, &n, nullptr), FFNQ_ERR_UNSUPPORTED);
    EXPECT(ffnq_dense_noalloc(&f, 256, 512, 0, FFNQ_ACT_SILU, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40),
                              mut<uint16_t>(50), nullptr, 1e-6f, nullptr), FFNQ_OK);
    // shared expert tails
    ffnq_ffn f8 = ffn(I8, I8, 256, 512);
    for (int tail : {FFNQ_TAIL_NONE, FFNQ_TAIL_RMSNORM, FFNQ_TAIL_SIGMOID_GATE})
        EXPECT(ffnq_shared_expert(&f8, 256, 512, 3, FFNQ_ACT_GELU_TANH, tail, mut<uint16_t>(40), mut<uint16_t>(50),
                                  mut<uint16_t>(60), 1e-6f, nullptr, &n, nullptr), FFNQ_OK);
    EXPECT(ffnq_shared_expert(&f8, 256, 512, 3, FFNQ_ACT_GELU_TANH, FFNQ_TAIL_RESIDUAL, mut<uint16_t>(40),
                              mut<uint16_t>(50), mut<uint16_t>(60), 1e-6f, nullptr, &n, nullptr), FFNQ_ERR_UNSUPPORTED);
    // route
    const int m = 3, k = 2;
    const size_t pb = 4 * (size_t)FFNQ_PLAN_INTS(m, k);
    EXPECT(ffnq_moe_route(mut<float>(46), nullptr, 0, 8, k, 8, mut<int32_t>(41), mut<float>(42), mut<int32_t>(43), pb,
                          nullptr), FFNQ_OK);
    EXPECT(ffnq_moe_route(nullptr, nullptr, m, 8, k, 8, mut<int32_t>(41), mut<float>(42), mut<int32_t>(43), pb,
                          nullptr), FFNQ_ERR_INVALID);
    EXPECT(ffnq_moe_route(mut<float>(46), nullptr, m, 8, k, 33, mut<int32_t>(41), mut<float>(42), mut<int32_t>(43),
                          pb, nullptr), FFNQ_ERR_UNSUPPORTED);
    EXPECT(ffnq_moe_route(mut<float>(46), nullptr, m, 8, 4, 3, mut<int32_t>(41), mut<float>(42), mut<int32_t>(43), pb,
                          nullptr), FFNQ_ERR_CAPACITY);
    EXPECT(ffnq_moe_route(mut<float>(46), nullptr, m, 8, k, 8, mut<int32_t>(41), mut<float>(42), mut<int32_t>(43),
                          pb - 4, nullptr), FFNQ_ERR_WORKSPACE);
    // routed half, layers
    ffnq_ffn ex = ffn(I4, I4, 256, 256), sh = ffn(I4, I4, 256, 512);
    EXPECT(ffnq_moe_routed_batched(&ex, 8, 256, 256, m, k, FFNQ_ACT_SILU, mut<uint16_t>(40), mut<int32_t>(41),
                                   mut<float>(42), mut<int32_t>(43), nullptr, mut<uint16_t>(50), nullptr, &n, nullptr),
           FFNQ_OK);
    EXPECT(ffnq_moe_routed_batched(&f8, 8, 256, 512, m, k, FFNQ_ACT_SILU, mut<uint16_t>(40), mut<int32_t>(41),
                                   mut<float>(42), mut<int32_t>(43), nullptr, mut<uint16_t>(50), nullptr, &n, nullptr),
           FFNQ_ERR_UNSUPPORTED);
    EXPECT(ffnq_moe_layer(&ex, 8, 256, 256, m, k, FFNQ_ACT_SILU, &sh, 512, mut<uint16_t>(45), mut<uint16_t>(40),
                          mut<int32_t>(41), mut<float>(42), mut<int32_t>(43), mut<uint16_t>(50), nullptr, &n, nullptr),
           FFNQ_OK);
    EXPECT(ffnq_moe_layer(&ex, 8, 256, 256, m, k, FFNQ_ACT_SILU, &sh, 512, nullptr, mut<uint16_t>(40),
                          mut<int32_t>(41), mut<float>(42), mut<int32_t>(43), mut<uint16_t>(50), nullptr, &n, nullptr),
           FFNQ_ERR_INVALID);
    EXPECT(ffnq_moe_layer_logits(&ex, 8, 256, 256, m, k, FFNQ_ACT_SILU, &sh, 512, mut<uint16_t>(45),
                                 mut<uint16_t>(40), mut<float>(46), nullptr, 8, mut<int32_t>(41), mut<float>(42),
                                 mut<int32_t>(43), pb, mut<uint16_t>(50), nullptr, &n, nullptr), FFNQ_OK);
    EXPECT(ffnq_moe_layer_sandwich(&ex, 8, 256, 256, m, k, FFNQ_ACT_GELU_TANH, &f8, 512, mut<uint16_t>(47),
                                   mut<uint16_t>(48), 1e-6f, mut<uint16_t>(40), mut<float>(46), nullptr, 8,
                                   mut<int32_t>(41), mut<float>(42), mut<int32_t>(43), pb, mut<uint16_t>(50), nullptr,
                                   &n, nullptr), FFNQ_OK);
    EXPECT(ffnq_moe_layer_sandwich(&ex, 8, 256, 256, m, k, FFNQ_ACT_GELU_TANH, nullptr, 512, mut<uint16_t>(47),
                                   mut<uint16_t>(48), 1e-6f, mut<uint16_t>(40), mut<float>(46), nullptr, 8,
                                   mut<int32_t>(41), mut<float>(42), mut<int32_t>(43), pb, mut<uint16_t>(50), nullptr,
                                   &n, nullptr), FFNQ_ERR_INVALID);
    // streamed routed half: a query and refusals (the slot table is host memory)
    ffnq_ffn tx = ffn(T4, T4, 256, 256);
    std::vector<int32_t> expert(4, -1);
    std::vector<uint64_t> last(4, 0);
    const size_t per = 3 * ffnq_packed_bytes(T4, 256, 256);
    ffnq_slot_cache cache{mut<void>(80), 4 * per, 4, expert.data(), last.data(), 0, 0};
    EXPECT(ffnq_moe_routed_streamed(&tx, 8, 256, 256, m, k, FFNQ_ACT_SILU, mut<uint16_t>(40), mut<int32_t>(41),
                                    mut<float>(42), mut<int32_t>(43), nullptr, mut<uint16_t>(50), &cache,
                                    mut<int32_t>(70), nullptr, &n, nullptr), FFNQ_OK);
    cache.slots_bytes = 4 * per - 1;
    EXPECT(ffnq_moe_routed_streamed(&tx, 8, 256, 256, m, k, FFNQ_ACT_SILU, mut<uint16_t>(40), mut<int32_t>(41),
                                    mut<float>(42), mut<int32_t>(43), nullptr, mut<uint16_t>(50), &cache,
                                    mut<int32_t>(70), nullptr, &n, nullptr), FFNQ_ERR_INVALID);
    cache.slots_bytes = 4 * per;
    expert[2] = 8;
    EXPECT(ffnq_moe_routed_streamed(&tx, 8, 256, 256, m, k, FFNQ_ACT_SILU, mut<uint16_t>(40), mut<int32_t>(41),
                                    mut<float>(42), mut<int32_t>(43), nullptr, mut<uint16_t>(50), &cache,
                                    mut<int32_t>(70), nullptr, &n, nullptr), FFNQ_ERR_INVALID);
    // router GEMV, packing, strings
    EXPECT(ffnq_router_logits(mut<uint16_t>(40), mut<uint16_t>(44), m, 250, 8, mut<float>(46), nullptr),
           FFNQ_ERR_INVALID);
    EXPECT(ffnq_router_logits(mut<uint16_t>(40), mut<uint16_t>(44), 0, 256, 8, mut<float>(46), nullptr), FFNQ_OK);
    if (ffnq_packed_bytes(I4, 16, 320) != 0) ++failures;
    ffnq_qmat src = mat(I4, 32, 256, 0);
    EXPECT(ffnq_pack(&src, 1, mut<void>(90), 1, nullptr), FFNQ_ERR_WORKSPACE);
    for (int s = 0; s >= -5; --s)
        if (!ffnq_status_string(s)) ++failures;
    if (failures) return 1;
    std::printf("abi sanitizer run: ok\n");
    return 0;
}
