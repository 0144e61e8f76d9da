"""Seeded random shapes against the oracle.

ffnq_moe_layer_logits against the oracle's chain for the same layer:
oracle.moe_route (ids and plan bit for bit, weights within fp32 rounding), the
shared expert's sigmoid-gated seed, then the routed half seeded with it.  The
shapes are drawn so that every launch plan of the layer appears across the
cases: routing inside the gate/up launch or before it, the fused down
(m <= 4) or the per-pair partials and the reduction, caps that split the
batch, tiled and row-major weights, and the grouped prefill kernels (12 or
more pairs per expert).  Then ffnq_dense and ffnq_shared_expert over random
widths, token counts, format pairs, activations, tails and layouts, and
ffnq_moe_layer_sandwich over random shapes against the oracle's layer."""
import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from helpers import rel_l2_rows

pytestmark = pytest.mark.gpu

TOL = 2e-3
N_CASES = 24


def draw(i):
    r = np.random.default_rng(9000 + i)
    hidden = int(r.choice([256, 384, 512, 640, 1024]))
    inter = int(r.choice([128, 256, 384, 640]))
    if i % 6 == 5:   # prefill-sized: few experts, many tokens
        E, k, m = int(r.choice([4, 6, 8])), int(r.choice([1, 2])), int(r.integers(48, 97))
    else:
        E = int(r.integers(4, 41))
        k = int(r.integers(1, min(8, E) + 1))
        m = int(r.choice([1, 2, 3, 4, 5, 8, 13, 24]))
    cap = int(r.integers(k, 33))
    sh_inter = int(r.choice([0, 256, 384]))
    tiled = bool(r.integers(0, 4) > 0)
    act = int(r.choice([gen.ACT_SILU, gen.ACT_GELU_TANH]))
    scaled = bool(r.integers(0, 3) == 0)
    return hidden, inter, E, k, m, cap, sh_inter, tiled, act, scaled


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def mats(f, tiled, n_experts=1):
    d = {n: fq.to_device(f[n]) for n in ("gate", "up", "down")}
    if tiled:
        d = {n: fq.pack(d[n], n_experts) for n in d}
    return d, fq.ffn_struct(d)


@pytest.mark.parametrize("i", range(N_CASES))
def test_layer_logits_random(i):
    hidden, inter, E, k, m, cap, sh_inter, tiled, act, scaled = draw(i)
    print("[case] fuzz", i, dict(hidden=hidden, inter=inter, E=E, k=k, m=m, cap=cap, sh_inter=sh_inter,
                                 tiled=tiled, act=act, scaled=scaled), flush=True)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=9100 + i, shared_inter=sh_inter)
    scale = (0.5 + np.random.default_rng(9200 + i).random(E)).astype(np.float32) if scaled else None
    ex_d, ex = mats(inp["experts"], tiled, E)   # device tensors stay referenced while their structs are used
    sh_d, sh = mats(inp["shared"], tiled) if sh_inter else (None, None)
    gate = dev16(inp["gate_vec"]) if sh_inter else None
    resid = dev16(inp["resid"])
    ids = torch.full((m, k), -9, dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.full((fq.plan_ints(m, k),), -9, dtype=torch.int32, device="cuda")
    fq.moe_layer_logits(ex, E, hidden, inter, m, k, act, sh, sh_inter, gate, dev16(inp["x"]),
                        dev(inp["logits"].astype(np.float32)), cap, ids, w, plan, resid,
                        expert_scale=None if scale is None else dev(scale))
    torch.cuda.synchronize()

    rc, ids_o, w_o, plan_o = oracle.moe_route(inp["logits"], k, cap, scale)
    assert rc == 0
    assert np.array_equal(ids.cpu().numpy(), ids_o) and np.array_equal(plan.cpu().numpy(), plan_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=1e-6, atol=1e-30)
    seed = None
    if sh_inter:
        seed = oracle.shared_expert(inp["shared"], hidden, sh_inter, act, gen.TAIL_SIGMOID_GATE, inp["x"],
                                    inp["gate_vec"])
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, act, inp["x"], ids_o, w_o, seed, inp["resid"])
    got = resid.cpu().numpy().view(np.uint16)
    err = rel_l2_rows(got, want)
    assert err <= TOL, (i, err)


# ---------------------------------------------------------------------------
# the dense FFN and the shared expert: random widths, token counts, formats
# (gate/up and down independently), activations, tails and layouts, with a
# zero residual every other case so that the bar applies to h itself

def draw_dense(i):
    r = np.random.default_rng(9500 + i)
    hidden = int(r.choice([128, 256, 384, 640, 1024, 1536]))
    inter = int(r.choice([128, 256, 384, 896, 1408]))
    m = int(r.choice([1, 2, 3, 4, 5, 7, 8, 11, 16, 33]))
    fmt = int(r.choice([gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64]))
    fmt_down = int(r.choice([gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64]))
    act = int(r.choice([gen.ACT_SILU, gen.ACT_GELU_TANH]))
    shared = bool(r.integers(0, 2))
    tail = int(r.choice([gen.TAIL_NONE, gen.TAIL_RMSNORM, gen.TAIL_SIGMOID_GATE])) if shared else gen.TAIL_RESIDUAL
    tiled = bool(r.integers(0, 3) > 0)
    zero_resid = bool(i % 2)
    return hidden, inter, m, fmt, fmt_down, act, shared, tail, tiled, zero_resid


@pytest.mark.parametrize("i", range(N_CASES))
def test_dense_random(i):
    hidden, inter, m, fmt, fmt_down, act, shared, tail, tiled, zero_resid = draw_dense(i)
    print("[case] dense fuzz", i, dict(hidden=hidden, inter=inter, m=m, fmt=fmt, fmt_down=fmt_down, act=act,
                                       shared=shared, tail=tail, tiled=tiled, zero_resid=zero_resid), flush=True)
    inp = gen.dense_inputs(hidden, inter, m, fmt, seed=9600 + i, fmt_down=fmt_down, row_scales=True)
    if zero_resid:
        inp["resid"] = np.zeros_like(inp["resid"])
    aux = {gen.TAIL_NONE: None, gen.TAIL_RESIDUAL: None, gen.TAIL_RMSNORM: inp["norm_w"],
           gen.TAIL_SIGMOID_GATE: inp["gate_vec"]}[tail]
    d, st = mats(inp["ffn"], tiled)
    x = dev16(inp["x"])
    if shared:
        out = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
        fq.shared_expert(st, hidden, inter, m, act, tail, x, out, None if aux is None else dev16(aux), 1e-6)
        want = oracle.shared_expert(inp["ffn"], hidden, inter, act, tail, inp["x"], aux)
    else:
        out = dev16(inp["resid"])
        fq.dense(st, hidden, inter, m, act, tail, x, out, None, 1e-6)
        want = oracle.dense(inp["ffn"], hidden, inter, act, tail, inp["x"], inp["resid"])
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    err = rel_l2_rows(got, want)
    assert err <= TOL, (i, err)


# ---------------------------------------------------------------------------
# the Gemma-style sandwich layer: random shapes, shared-branch formats and
# expert scales, against the oracle's layer step by step

def draw_sandwich(i):
    r = np.random.default_rng(9800 + i)
    hidden = int(r.choice([256, 384, 512, 1024]))
    inter = int(r.choice([128, 256, 384]))
    sh_inter = int(r.choice([128, 256, 640]))
    E = int(r.integers(4, 33))
    k = int(r.integers(1, min(8, E) + 1))
    m = int(r.choice([1, 2, 3, 4, 6, 9, 17]))
    cap = int(r.integers(k, 33))
    sh_fmt = int(r.choice([gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64]))
    scaled = bool(r.integers(0, 2))
    tiled = bool(r.integers(0, 4) > 0)
    return hidden, inter, sh_inter, E, k, m, cap, sh_fmt, scaled, tiled


@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_sandwich_random(i):
    hidden, inter, sh_inter, E, k, m, cap, sh_fmt, scaled, tiled = draw_sandwich(i)
    print("[case] sandwich fuzz", i, dict(hidden=hidden, inter=inter, sh_inter=sh_inter, E=E, k=k, m=m, cap=cap,
                                          sh_fmt=sh_fmt, scaled=scaled, tiled=tiled), flush=True)
    act, eps = gen.ACT_GELU_TANH, 1e-6
    inp = gen.sandwich_inputs(hidden, E, inter, m, seed=9900 + i, shared_inter=sh_inter, shared_fmt=sh_fmt,
                              row_scales=True)
    sc = inp["expert_scale"] if scaled else None
    rc, ids_o, w_o, plan_o, h1_o, r_o, out_o = oracle.moe_sandwich_layer(
        inp["experts"], E, hidden, inter, act, inp["shared"], sh_inter, inp["shared_norm_w"], inp["post_norm_w"], eps,
        inp["x"], inp["logits"], sc, k, cap, inp["resid"])
    assert rc == 0
    ex_d, ex = mats(inp["experts"], tiled, E)
    sh_d, sh = mats(inp["shared"], tiled)
    resid = dev16(inp["resid"])
    ids = torch.full((m, k), -9, dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.full((fq.plan_ints(m, k),), -9, dtype=torch.int32, device="cuda")
    fq.moe_layer_sandwich(ex, E, hidden, inter, m, k, act, sh, sh_inter, dev16(inp["shared_norm_w"]),
                          dev16(inp["post_norm_w"]), eps, dev16(inp["x"]), dev(inp["logits"].astype(np.float32)), cap,
                          ids, w, plan, resid, expert_scale=None if sc is None else dev(sc))
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o) and np.array_equal(plan.cpu().numpy(), plan_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=1e-6, atol=1e-30)
    err = rel_l2_rows(resid.cpu().numpy().view(np.uint16), out_o)
    assert err <= TOL, (i, err)
