"""Host-side checks of the C ABI: the library loads, exports every entry
point include/ffnq.h declares, and refuses bad arguments with the documented
status codes before touching the GPU.  No compute call is made."""
import ctypes as C
import os
import re

import pytest

import moe_expert_dequant_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fake, 16-byte aligned "device" addresses: every call below is refused (or is a
# workspace query / m == 0 no-op) before any pointer is dereferenced
A = 0x10000


def addr(i):
    return A * (i + 1)


def header_decls():
    with open(os.path.join(ROOT, "include", "ffnq.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"FFNQ_API\s+[\w\s\*]+?\b(ffnq_\w+)\s*\(", src)))


def test_exports_match_header():
    names = header_decls()
    assert set(names) == set(fq.EXPORTS)
    L = fq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = fq.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.ffnq_status_string(code)


def mat(fmt, n, k, base):
    return fq.QMat(fmt, n, k, addr(base), addr(base + 1), addr(base + 2) if fmt == fq.FMT_INT4_AFFINE_G64 else None)


def ffn(fmt_gu, fmt_d, hidden, inter):
    return fq.Ffn(mat(fmt_gu, inter, hidden, 0), mat(fmt_gu, inter, hidden, 10), mat(fmt_d, hidden, inter, 20))


def call_dense(f, hidden=256, inter=512, m=2, act=fq.ACT_SILU, tail=fq.TAIL_RESIDUAL, x=addr(40), out=addr(50),
               norm=addr(60), eps=1e-6, ws=None, ws_bytes=None, shared=False):
    L = fq.lib()
    size = C.c_size_t(ws_bytes or 0)
    fn = L.ffnq_shared_expert if shared else L.ffnq_dense
    rc = fn(C.byref(f) if f is not None else None, hidden, inter, m, act, tail, x, out, norm, eps, ws,
            C.byref(size), None)
    return rc, size.value


I8, I4 = fq.FMT_INT8_ROW, fq.FMT_INT4_AFFINE_G64


def test_dense_workspace_query_and_noop():
    f = ffn(I4, I4, 256, 512)
    rc, n = call_dense(f)
    assert rc == 0 and n > 0
    rc, n0 = call_dense(f, m=0)
    assert rc == 0 and n0 == 0
    # m == 0 with a (fake) workspace: a no-op
    rc, _ = call_dense(f, m=0, ws=addr(70), ws_bytes=0)
    assert rc == 0
    # too small a workspace
    rc, _ = call_dense(f, ws=addr(70), ws_bytes=n - 1)
    assert rc == -4


@pytest.mark.parametrize("case,expect", [
    (dict(hidden=0), -1), (dict(inter=0), -1), (dict(m=-1), -1),
    (dict(x=None), -1), (dict(out=None), -1),
    (dict(x=addr(40) + 8), -1),                   # misaligned
    (dict(out=addr(40) + 256), -1),               # overlaps x
    (dict(act=7), -2), (dict(tail=fq.TAIL_SIGMOID_GATE), -2), (dict(tail=9), -2),
    (dict(tail=fq.TAIL_RMSNORM, norm=None), -1),
    (dict(tail=fq.TAIL_RMSNORM, eps=-1.0), -1),
    (dict(tail=fq.TAIL_RMSNORM, eps=float("nan")), -1),
])
def test_dense_refusals(case, expect):
    f = ffn(I8, I4, 256, 512)
    rc, _ = call_dense(f, **case)
    assert rc == expect


def test_dense_shape_and_format_refusals():
    assert call_dense(None)[0] == -1
    bad = ffn(I4, I4, 256, 512)
    bad.down.n = 128                                     # down rows != hidden
    assert call_dense(bad)[0] == -1
    bad = ffn(I4, I4, 256, 512)
    bad.gate.k = 200                                     # k not a multiple of 64
    assert call_dense(bad)[0] == -1
    bad = ffn(I4, I4, 192, 512)                          # INT4 k % 128 == 64
    assert call_dense(bad, hidden=192)[0] == -2
    bad = ffn(I4, I4, 256, 512)
    bad.up.fmt = I8                                      # gate/up formats differ
    assert call_dense(bad)[0] == -2
    bad = ffn(I4, I4, 256, 512)
    bad.gate.fmt = 5                                     # unknown format
    assert call_dense(bad)[0] == -2
    bad = ffn(I4, I4, 256, 512)
    bad.gate.z = None                                    # INT4 without zero points
    assert call_dense(bad)[0] == -1
    bad = ffn(I4, I4, 256, 512)
    bad.down.q = addr(20) + 4                            # misaligned weights
    assert call_dense(bad)[0] == -1


def test_shared_expert_tails():
    f = ffn(I8, I8, 256, 704)
    for tail in (fq.TAIL_NONE, fq.TAIL_RMSNORM, fq.TAIL_SIGMOID_GATE):
        rc, n = call_dense(f, inter=704, tail=tail, shared=True)
        assert rc == 0 and n > 0
    assert call_dense(f, inter=704, tail=fq.TAIL_RESIDUAL, shared=True)[0] == -2
    assert call_dense(f, inter=704, tail=fq.TAIL_SIGMOID_GATE, norm=None, shared=True)[0] == -1


def call_route(m=4, E=16, k=4, cap=8, plan_bytes=None, logits=addr(1), ids=addr(2), w=addr(3), plan=addr(4),
               scale=None):
    L = fq.lib()
    pb = 4 * fq.plan_ints(m, k) if plan_bytes is None else plan_bytes
    return L.ffnq_moe_route(logits, scale, m, E, k, cap, ids, w, plan, pb, None)


def test_route_refusals():
    assert call_route(m=0) == 0                               # no-op
    assert call_route(k=0) == -1
    assert call_route(k=17) == -1
    assert call_route(E=0) == -1
    assert call_route(m=-1) == -1
    assert call_route(logits=None) == -1
    assert call_route(plan=addr(4) + 4) == -1
    assert call_route(E=2048, k=4) == -2                      # more experts than the router holds
    assert call_route(cap=33) == -2                           # above the 32-slot ceiling
    assert call_route(k=4, cap=3) == -3                       # not even one token fits
    assert call_route(plan_bytes=4 * fq.plan_ints(4, 4) - 4) == -4


def call_routed(f, E=8, hidden=256, inter=256, m=3, k=2, act=fq.ACT_SILU, x=addr(40), ids=addr(41), w=addr(42),
                plan=addr(43), seed=addr(44), resid=addr(50), ws=None, ws_bytes=0):
    L = fq.lib()
    size = C.c_size_t(ws_bytes)
    rc = L.ffnq_moe_routed_batched(C.byref(f), E, hidden, inter, m, k, act, x, ids, w, plan, seed, resid, ws,
                                   C.byref(size), None)
    return rc, size.value


def test_routed_refusals_and_query():
    f = ffn(I4, I4, 256, 256)
    rc, n = call_routed(f)
    assert rc == 0 and n > 0
    assert call_routed(f, seed=None)[0] == 0
    assert call_routed(f, m=0)[0] == 0 and call_routed(f, m=0)[1] == 0
    assert call_routed(ffn(I8, I4, 256, 256))[0] == -2        # routed experts must be INT4-affine
    assert call_routed(ffn(I4, I8, 256, 256))[0] == -2
    assert call_routed(f, k=9)[0] == -1
    assert call_routed(f, act=3)[0] == -2
    assert call_routed(f, plan=None)[0] == -1
    assert call_routed(f, resid=addr(40) + 64)[0] == -1       # overlaps x
    assert call_routed(f, ws=addr(60), ws_bytes=n - 256)[0] == -4


def call_layer(f, sh, E=8, hidden=256, inter=256, sh_inter=512, m=3, k=2, act=fq.ACT_SILU, gate=addr(45), x=addr(40),
               ids=addr(41), w=addr(42), plan=addr(43), resid=addr(50), ws=None, ws_bytes=0):
    L = fq.lib()
    size = C.c_size_t(ws_bytes)
    rc = L.ffnq_moe_layer(C.byref(f), E, hidden, inter, m, k, act, None if sh is None else C.byref(sh), sh_inter, gate,
                          x, ids, w, plan, resid, ws, C.byref(size), None)
    return rc, size.value


def test_layer_refusals_and_query():
    f, sh = ffn(I4, I4, 256, 256), ffn(I4, I4, 256, 512)
    rc, n = call_layer(f, sh)
    assert rc == 0
    rc0, n0 = call_layer(f, None)
    assert rc0 == 0
    # the workspace holds the routed half's (as ffnq_moe_routed_batched sizes it) and then the shared expert's
    assert n0 == call_routed(f)[1]
    assert n > n0
    assert call_layer(f, sh, m=0) == (0, 0)
    assert call_layer(ffn(I8, I4, 256, 256), sh)[0] == -2      # routed experts must be INT4-affine
    assert call_layer(f, sh, gate=None)[0] == -1               # the shared expert needs its gate vector
    assert call_layer(f, sh, gate=addr(45) + 2)[0] == -1       # misaligned
    assert call_layer(f, sh, sh_inter=256)[0] != 0             # shared matrices disagree with shared_inter
    assert call_layer(f, sh, k=9)[0] == -1
    assert call_layer(f, sh, act=3)[0] == -2
    assert call_layer(f, sh, resid=addr(40) + 64)[0] == -1     # overlaps x
    assert call_layer(f, sh, ws=addr(60), ws_bytes=n - 256)[0] == -4


# ---------------------------------------------------------------------------
# tiled formats and ffnq_pack (refusals only: no launch)

T8, T4 = fq.FMT_INT8_ROW_TILED, fq.FMT_INT4_AFFINE_G64_TILED


def test_packed_bytes():
    # INT4 4096 inputs: 32 code blocks in 4 groups -> 36 KB per 16-row tile; no padding at 14336 rows
    assert fq.packed_bytes(I4, 14336, 4096) == 896 * 36 * 1024 == 14336 * 2048 + 4 * 14336 * 4096 // 64
    assert fq.packed_bytes(T4, 14336, 4096) == fq.packed_bytes(I4, 14336, 4096)
    # short last group (6 blocks) and a ragged tile: 2 tiles of (1 + 6) steps
    assert fq.packed_bytes(I4, 20, 768) == 2 * 7 * 1024
    # INT8: 16-row tiles of K/64 steps, then 16 fp32 scales per tile padded to 256 bytes
    assert fq.packed_bytes(I8, 37, 320) == 3 * 5 * 1024 + 256
    assert fq.packed_bytes(I8, 2816, 11264) == 176 * 176 * 1024 + 176 * 64
    for bad in ((I4, 16, 192), (I8, 16, 100), (I4, 0, 128), (99, 16, 128), (I8, 16, -64)):
        assert fq.packed_bytes(*bad) == 0, bad


def test_pack_refusals():
    L = fq.lib()
    src = mat(I4, 32, 256, 0)
    need = fq.packed_bytes(I4, 32, 256)
    assert L.ffnq_pack(None, 1, addr(100), need, None) == -1
    assert L.ffnq_pack(C.byref(src), 0, addr(100), need, None) == -1
    assert L.ffnq_pack(C.byref(src), 1, None, need, None) == -1
    assert L.ffnq_pack(C.byref(src), 1, addr(100), need - 16, None) == -4
    assert L.ffnq_pack(C.byref(src), 2, addr(100), need, None) == -4
    assert L.ffnq_pack(C.byref(src), 1, addr(100) + 8, need, None) == -1          # misaligned dst
    assert L.ffnq_pack(C.byref(src), 1, addr(0), need, None) == -1                # dst overlaps src codes
    tiled = fq.QMat(T4, 32, 256, addr(0), None, None)
    assert L.ffnq_pack(C.byref(tiled), 1, addr(100), need, None) == -2            # already tiled
    odd = mat(I4, 32, 192, 0)
    assert L.ffnq_pack(C.byref(odd), 1, addr(100), need, None) == -2             # k % 128 != 0


def tiled_ffn(fmt_gu, fmt_d, hidden, inter):
    return fq.Ffn(fq.QMat(fmt_gu, inter, hidden, addr(0), None, None),
                  fq.QMat(fmt_gu, inter, hidden, addr(10), None, None),
                  fq.QMat(fmt_d, hidden, inter, addr(20), None, None))


def test_tiled_ffn_checks():
    rc, n = call_dense(tiled_ffn(T4, T4, 256, 512))
    assert rc == 0 and n > 0                                  # workspace query accepts tiled weights
    rc, _ = call_dense(tiled_ffn(T4, T8, 256, 512))
    assert rc == 0                                            # mixed tiled formats are fine
    mixed = fq.Ffn(fq.QMat(T4, 512, 256, addr(0), None, None), fq.QMat(T4, 512, 256, addr(10), None, None),
                   mat(I4, 256, 512, 20))
    rc, _ = call_dense(mixed)
    assert rc == -2                                           # tiled and row-major mixed: refused
    rc, _ = call_dense(fq.Ffn(fq.QMat(T4, 512, 256, None, None, None), fq.QMat(T4, 512, 256, addr(10), None, None),
                              fq.QMat(T4, 256, 512, addr(20), None, None)))
    assert rc == -1                                           # NULL packed buffer


def test_router_logits_refusals():
    L = fq.lib()
    x, w, lg = addr(70), addr(71), addr(72)
    assert L.ffnq_router_logits(None, w, 2, 256, 8, lg, None) == -1           # NULL
    assert L.ffnq_router_logits(x, w, 2, 250, 8, lg, None) == -1              # hidden not a multiple of 8
    assert L.ffnq_router_logits(x, w, 2, 256, 0, lg, None) == -1              # no experts
    assert L.ffnq_router_logits(x, w, -1, 256, 8, lg, None) == -1             # m < 0
    assert L.ffnq_router_logits(x + 4, w, 2, 256, 8, lg, None) == -1          # misaligned
    assert L.ffnq_router_logits(x, w, 2, 256, 8, x + 16, None) == -1          # logits overlap x
    assert L.ffnq_router_logits(x, w, 0, 256, 8, lg, None) == 0               # m == 0: no-op


def call_layer_logits(f, sh, E=8, hidden=256, inter=256, sh_inter=512, m=3, k=2, cap=8, plan_bytes=None,
                      logits=addr(46), ws=None, ws_bytes=0):
    L = fq.lib()
    size = C.c_size_t(ws_bytes)
    pb = 4 * fq.plan_ints(m, k) if plan_bytes is None else plan_bytes
    rc = L.ffnq_moe_layer_logits(C.byref(f), E, hidden, inter, m, k, fq.ACT_SILU,
                                 None if sh is None else C.byref(sh), sh_inter, addr(45), addr(40), logits, None, cap,
                                 addr(41), addr(42), addr(43), pb, addr(50), ws, C.byref(size), None)
    return rc, size.value


def test_layer_logits_refusals_and_query():
    # the checks of ffnq_moe_route and ffnq_moe_layer, and ffnq_moe_layer's workspace
    f, sh = ffn(I4, I4, 256, 256), ffn(I4, I4, 256, 512)
    rc, n = call_layer_logits(f, sh)
    assert rc == 0 and n == call_layer(f, sh)[1]
    assert call_layer_logits(f, sh, m=0) == (0, 0)
    assert call_layer_logits(f, sh, logits=None)[0] == -1
    assert call_layer_logits(f, sh, cap=33)[0] == -2
    assert call_layer_logits(f, sh, k=4, cap=3)[0] == -3
    assert call_layer_logits(f, sh, plan_bytes=4 * fq.plan_ints(3, 2) - 4)[0] == -4
    assert call_layer_logits(ffn(I8, I4, 256, 256), sh)[0] == -2
    assert call_layer_logits(f, sh, ws=addr(60), ws_bytes=n - 256)[0] == -4


def call_sandwich(f, sh, E=8, hidden=256, inter=256, sh_inter=512, m=3, k=2, cap=8, plan_bytes=None,
                  logits=addr(46), norm1=addr(47), norm2=addr(48), eps=1e-6, x=addr(40), ws=None, ws_bytes=0):
    L = fq.lib()
    size = C.c_size_t(ws_bytes)
    pb = 4 * fq.plan_ints(m, k) if plan_bytes is None else plan_bytes
    rc = L.ffnq_moe_layer_sandwich(C.byref(f), E, hidden, inter, m, k, fq.ACT_GELU_TANH,
                                   None if sh is None else C.byref(sh), sh_inter, norm1, norm2, eps, x, logits,
                                   addr(49), cap, addr(41), addr(42), addr(43), pb, addr(50), ws, C.byref(size), None)
    return rc, size.value


def test_layer_sandwich_refusals_and_query():
    f, sh = ffn(I4, I4, 256, 256), ffn(I8, I8, 256, 512)
    rc, n = call_sandwich(f, sh)
    assert rc == 0 and n > 0
    # workspace: the two bf16 rows, the shared expert's (RMSNorm tail) and the routed half's
    assert n >= 2 * 3 * 256 * 2 + call_dense(sh, 256, 512, 3, tail=fq.TAIL_RMSNORM, shared=True)[1]
    assert call_sandwich(f, sh, m=0) == (0, 0)
    assert call_sandwich(f, None)[0] == -1                      # the shared branch is required
    assert call_sandwich(f, sh, norm1=None)[0] == -1
    assert call_sandwich(f, sh, norm2=None)[0] == -1
    assert call_sandwich(f, sh, norm2=addr(48) + 2)[0] == -1    # misaligned
    assert call_sandwich(f, sh, eps=float("nan"))[0] == -1
    assert call_sandwich(f, sh, eps=-1.0)[0] == -1
    assert call_sandwich(f, sh, logits=None)[0] == -1
    assert call_sandwich(f, sh, x=addr(50))[0] == -1            # x overlaps resid
    assert call_sandwich(f, sh, cap=33)[0] == -2
    assert call_sandwich(f, sh, k=4, cap=3)[0] == -3
    assert call_sandwich(f, sh, plan_bytes=4 * fq.plan_ints(3, 2) - 4)[0] == -4
    assert call_sandwich(ffn(I8, I8, 256, 256), sh)[0] == -2    # INT4 experts only
    assert call_sandwich(f, ffn(I8, I8, 256, 384), sh_inter=512)[0] == -1   # shared shape mismatch
    assert call_sandwich(f, sh, ws=addr(60), ws_bytes=n - 256)[0] == -4


def call_streamed(f, cache, E=8, hidden=256, inter=256, m=3, k=2, staging=addr(70), ws=None, ws_bytes=0):
    L = fq.lib()
    size = C.c_size_t(ws_bytes)
    rc = L.ffnq_moe_routed_streamed(C.byref(f), E, hidden, inter, m, k, fq.ACT_SILU, addr(40), addr(41), addr(42),
                                    addr(43), None, addr(50), None if cache is None else C.byref(cache), staging, ws,
                                    C.byref(size), None)
    return rc, size.value


def test_streamed_refusals_and_query():
    import numpy as np
    T4 = fq.FMT_INT4_AFFINE_G64_TILED
    t = fq.Ffn(fq.QMat(T4, 256, 256, addr(0), None, None), fq.QMat(T4, 256, 256, addr(10), None, None),
               fq.QMat(T4, 256, 256, addr(20), None, None))
    per = 3 * fq.packed_bytes(T4, 256, 256)
    expert = np.full(4, -1, np.int32)
    last = np.zeros(4, np.uint64)

    def cache(n=4, nbytes=4 * per, slots=addr(80), table=True):
        return fq.SlotCacheC(slots, nbytes, n, expert.ctypes.data if table else None, last.ctypes.data, 0, 0)

    rc, n = call_streamed(t, cache())
    assert rc == 0 and n > 0
    assert call_streamed(t, cache(), m=0) == (0, 0)
    assert call_streamed(t, None)[0] == -1
    assert call_streamed(t, cache(), staging=None)[0] == -1
    assert call_streamed(t, cache(n=0))[0] == -1
    assert call_streamed(t, cache(nbytes=4 * per - 1))[0] == -1   # slots smaller than n_slots experts
    assert call_streamed(t, cache(slots=addr(80) + 4))[0] == -1   # misaligned
    assert call_streamed(t, cache(table=False))[0] == -1
    expert[1] = 8                                                 # a slot naming an expert past n_experts
    assert call_streamed(t, cache())[0] == -1
    expert[1] = -1
    assert call_streamed(ffn(I4, I4, 256, 256), cache())[0] == -2   # row-major experts: not streamed
    assert call_streamed(t, cache(), ws=addr(60), ws_bytes=n - 256)[0] == -4


def test_stream_read_refusals():
    L = fq.lib()
    vp = C.c_void_p
    assert L.ffnq_stream_read(None, 64, vp(addr(1)), None) == -1
    assert L.ffnq_stream_read(vp(addr(0)), 64, None, None) == -1
    assert L.ffnq_stream_read(vp(addr(0) + 8), 64, vp(addr(1)), None) == -1   # buf not 16-byte aligned
    assert L.ffnq_stream_read(vp(addr(0)), 72, vp(addr(1)), None) == -1       # not a multiple of 16
    assert L.ffnq_stream_read(vp(addr(0)), 64, vp(addr(1) + 2), None) == -1   # sink not 4-byte aligned
    assert L.ffnq_stream_read(vp(addr(0)), 0, vp(addr(1)), None) == fq.OK                 # nothing to read
