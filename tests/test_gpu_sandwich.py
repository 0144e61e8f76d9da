"""ffnq_moe_layer_sandwich, the Gemma-style routed layer: route with a learned
per-expert scale, the shared branch with its own RMSNorm, the routed sum from
zero, the sandwich tail.  Checked against the oracle's step-by-step layer
(routes and plans bit for bit, bf16 rows within the float bar, also with a
zero residual so that the bar applies to the layer's own output), and the tail
kernel alone against the oracle's tail on the GPU's own h1 and r rows."""
import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from test_gpu_parity import LAYOUTS, check, dev, dev16, host16, mats_dev, say, ulp_diag

pytestmark = pytest.mark.gpu
I8, I4 = gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64


def gpu_sandwich(inp, E, hidden, inter, sh_inter, m, k, cap, act, eps, tiled, resid, scale=True):
    ex_d = mats_dev(inp["experts"], tiled, E)       # device tensors stay referenced while their structs are used
    sh_d = mats_dev(inp["shared"], tiled)
    ex, sh = fq.ffn_struct(ex_d), fq.ffn_struct(sh_d)
    x = dev16(inp["x"])
    out = dev16(resid)
    ids = torch.full((m, k), -9, dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.full((fq.plan_ints(m, k),), -9, dtype=torch.int32, device="cuda")
    sc = dev(inp["expert_scale"]) if scale else None
    fq.moe_layer_sandwich(ex, E, hidden, inter, m, k, act, sh, sh_inter, dev16(inp["shared_norm_w"]),
                          dev16(inp["post_norm_w"]), eps, x, dev(inp["logits"].astype(np.float32)), cap, ids, w, plan,
                          out, expert_scale=sc)
    torch.cuda.synchronize()
    # the branch rows from the calls the layer composes: the shared expert with
    # its RMSNorm tail, the routed half unseeded on a zero row
    h1 = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
    fq.shared_expert(sh, hidden, sh_inter, m, act, gen.TAIL_RMSNORM, x, h1, dev16(inp["shared_norm_w"]), eps)
    r = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
    fq.moe_routed_batched(ex, E, hidden, inter, m, k, act, x, ids, w, plan, None, r)
    torch.cuda.synchronize()
    return host16(out), ids.cpu().numpy(), w.cpu().numpy(), plan.cpu().numpy(), host16(h1), host16(r)


def run_case(inp, E, hidden, inter, sh_inter, m, k, cap, tiled, label, scale=True):
    act, eps = gen.ACT_GELU_TANH, 1e-6
    sc = inp["expert_scale"] if scale else None
    rc, ids_o, w_o, plan_o, h1_o, r_o, out_o = oracle.moe_sandwich_layer(
        inp["experts"], E, hidden, inter, act, inp["shared"], sh_inter, inp["shared_norm_w"], inp["post_norm_w"], eps,
        inp["x"], inp["logits"], sc, k, cap, inp["resid"])
    assert rc == 0
    for resid, want, tag in ((inp["resid"], out_o, "resid"), (np.zeros_like(inp["resid"]), None, "zero resid")):
        got, ids, w, plan, h1, r = gpu_sandwich(inp, E, hidden, inter, sh_inter, m, k, cap, act, eps, tiled, resid,
                                                scale)
        assert np.array_equal(ids, ids_o) and np.array_equal(plan, plan_o)
        np.testing.assert_allclose(w, w_o, rtol=1e-6, atol=1e-30)
        if want is None:   # the layer's own output: the tail on the oracle's rows, added to +0
            want = oracle.sandwich_tail(h1_o, r_o, inp["post_norm_w"], eps, resid)
        check(got, want, f"{label} {tag}")
        # the branch rows against the oracle's, and the tail kernel on the GPU's own rows
        check(h1, h1_o, f"{label} h1")
        check(r, r_o, f"{label} routed row")
        tail = oracle.sandwich_tail(h1, r, inp["post_norm_w"], eps, resid)
        ulp, _ = ulp_diag(got, tail)
        assert ulp <= 1.0 and np.mean(got != tail) < 0.01, (label, tag, ulp)


@LAYOUTS
@pytest.mark.parametrize("m,E,k,cap,sh_fmt", [
    (1, 16, 4, 8, I8),      # router inside the gate/up launch (tiled)
    (3, 16, 4, 8, I4),      # an INT4 shared branch
    (5, 16, 4, 6, I8),      # a cap that splits the batch
    (8, 16, 8, 16, I8),     # 64 pairs
    (20, 16, 2, 16, I8),    # more rows per expert
])
def test_sandwich_small(m, E, k, cap, sh_fmt, tiled):
    hidden, inter, sh_inter = 512, 256, 384
    say("sandwich small", m, E, k, cap, sh_fmt, tiled)
    inp = gen.sandwich_inputs(hidden, E, inter, m, seed=5100 + m + k, shared_inter=sh_inter, shared_fmt=sh_fmt,
                              row_scales=True)
    run_case(inp, E, hidden, inter, sh_inter, m, k, cap, tiled, f"sandwich m {m} k {k} cap {cap} tiled {tiled}")


def test_sandwich_without_expert_scale():
    hidden, inter, sh_inter, E, m, k, cap = 512, 256, 384, 16, 2, 4, 8
    say("sandwich no expert scale")
    inp = gen.sandwich_inputs(hidden, E, inter, m, seed=5200, shared_inter=sh_inter)
    run_case(inp, E, hidden, inter, sh_inter, m, k, cap, True, "sandwich unscaled", scale=False)


@pytest.mark.parametrize("m", [1, 4])
def test_sandwich_workload(m):
    # the Gemma-style workload (hidden 2816; the shared branch of the INT8
    # shared-expert workload; 128 INT4 experts of width 768, top 8), every row
    c = gen.CONFIGS[5]
    say("sandwich workload", m)
    inp = gen.config_inputs(5, m, row_scales=True)
    run_case(inp, c["n_experts"], c["hidden"], c["moe_inter"], c["shared_inter"], m, c["top_k"], c["cap"], True,
             f"sandwich workload m {m}")


@pytest.mark.parametrize("m", [1, 5])
def test_sandwich_row_past_lds(m):
    # hidden 8320 > 8192: the fused tail holds only h1 in LDS and reads the
    # shared branch's partials twice; m = 5 takes the down path that zeroes r
    hidden, inter, sh_inter, E, k, cap = 8320, 256, 256, 8, 2, 8
    say("sandwich wide row", m)
    inp = gen.sandwich_inputs(hidden, E, inter, m, seed=5300 + m, shared_inter=sh_inter, shared_fmt=I8,
                              row_scales=True)
    run_case(inp, E, hidden, inter, sh_inter, m, k, cap, True, f"sandwich wide row m {m}")
