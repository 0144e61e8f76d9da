"""ffnq_dense_noalloc: ffnq_dense on the library's own per-GPU scratch array.

Called through the C ABI and compared bit for bit with ffnq_dense (same
kernels) on two calls in a row, the second with a smaller input, and with
the oracle within the float bar; a call that needs more than the array's
size is refused before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from helpers import rel_l2_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def ws_bytes(st, hidden, inter, m, act, tail, x, out, nw):
    size = C.c_size_t(0)
    rc = fq.lib().ffnq_dense(C.byref(st), hidden, inter, m, act, tail, x.data_ptr(), out.data_ptr(),
                             None if nw is None else nw.data_ptr(), 1e-6, None, C.byref(size), None)
    assert rc == 0
    return size.value


def run_pair(inp, hidden, inter, m, act, tail, st):
    x = dev16(inp["x"][:m])
    nw = dev16(inp["norm_w"]) if tail == gen.TAIL_RMSNORM else None
    start = inp["resid"][:m] if tail == gen.TAIL_RESIDUAL else np.zeros((m, hidden), np.uint16)
    a, b = dev16(start), dev16(start)
    need = ws_bytes(st, hidden, inter, m, act, tail, x, a, nw)
    assert 0 < need <= fq.NOALLOC_SCRATCH_BYTES
    fq.dense(st, hidden, inter, m, act, tail, x, a, nw)
    fq.dense_noalloc(st, hidden, inter, m, act, tail, x, b, nw)
    torch.cuda.synchronize()
    return host16(a), host16(b), need


@pytest.mark.parametrize("tiled", [True, False], ids=["tiled", "rowmajor"])
def test_noalloc_llama_shaped_two_calls(tiled):
    c = gen.CONFIGS[1]
    hidden, inter = c["hidden"], c["inter"]
    inp = gen.config_inputs(1, 4)
    d = {n: fq.to_device(inp["ffn"][n]) for n in ("gate", "up", "down")}
    if tiled:
        d = {n: fq.pack(d[n]) for n in d}
    st = fq.ffn_struct(d)
    for m in (4, 1):   # the second call smaller than the first
        say("noalloc llama", tiled, m)
        a, b, need = run_pair(inp, hidden, inter, m, c["act"], c["tail"], st)
        say(f"  workspace {need} bytes")
        assert np.array_equal(a, b)
    want = oracle.dense(inp["ffn"], hidden, inter, c["act"], c["tail"], inp["x"][:1], inp["resid"][:1])
    assert rel_l2_rows(b, want) <= 2e-3


@pytest.mark.parametrize("tiled", [True, False], ids=["tiled", "rowmajor"])
def test_noalloc_rmsnorm_two_calls(tiled):
    hidden, inter = 1024, 2816
    inp = gen.dense_inputs(hidden, inter, 8, gen.FMT_INT8_ROW, seed=8100, row_scales=True)
    d = {n: fq.to_device(inp["ffn"][n]) for n in ("gate", "up", "down")}
    if tiled:
        d = {n: fq.pack(d[n]) for n in d}
    st = fq.ffn_struct(d)
    for m in (8, 3):
        say("noalloc rmsnorm", tiled, m)
        a, b, _ = run_pair(inp, hidden, inter, m, gen.ACT_GELU_TANH, gen.TAIL_RMSNORM, st)
        assert np.array_equal(a, b)
        want = oracle.dense(inp["ffn"], hidden, inter, gen.ACT_GELU_TANH, gen.TAIL_RMSNORM, inp["x"][:m], None,
                            inp["norm_w"])
        assert rel_l2_rows(b, want) <= 2e-3


def test_noalloc_refuses_beyond_its_array():
    # the Llama-shaped layer at 64 tokens needs more workspace than the array holds:
    # refused on the host, nothing enqueued, the output untouched
    c = gen.CONFIGS[1]
    hidden, inter, m = c["hidden"], c["inter"], 64
    inp = gen.config_inputs(1, 1)
    d = {n: fq.pack(fq.to_device(inp["ffn"][n])) for n in ("gate", "up", "down")}
    st = fq.ffn_struct(d)
    x = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
    out = torch.full((m, hidden), 0x3F80, dtype=torch.int16, device="cuda")
    need = ws_bytes(st, hidden, inter, m, c["act"], c["tail"], x, out, None)
    say(f"noalloc refusal: needs {need} bytes, array {fq.NOALLOC_SCRATCH_BYTES}")
    assert need > fq.NOALLOC_SCRATCH_BYTES
    with pytest.raises(fq.FfnqError) as e:
        fq.dense_noalloc(st, hidden, inter, m, c["act"], c["tail"], x, out)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool(torch.all(out == 0x3F80))
