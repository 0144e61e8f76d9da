"""HIP-graph capture of the library's calls: a captured dense call, a
captured route + routed call and a captured route + whole MoE layer are
replayed several times, with eager work and synchronisation between the
replays; every replay must equal the eager result bit for bit (the calls
enqueue only kernels: no memset or copy nodes), and the replayed result is
checked against the CPU oracle."""
import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from test_gpu_parity import LAYOUTS, check, dev, dev16, ffn_dev, host16, mats_dev, say

pytestmark = pytest.mark.gpu


@LAYOUTS
def test_graph_replay_dense(tiled):
    hidden, inter, m = 512, 768, 3
    say("graph dense", tiled)
    inp = gen.dense_inputs(hidden, inter, m, gen.FMT_INT4_AFFINE_G64, seed=4242)
    d, st = ffn_dev(inp["ffn"], tiled)
    x, r0 = dev16(inp["x"]), dev16(inp["resid"])
    ws = fq.Workspace()
    want = r0.clone()
    fq.dense(st, hidden, inter, m, gen.ACT_SILU, gen.TAIL_RESIDUAL, x, want, ws=ws)
    torch.cuda.synchronize()
    r = r0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fq.dense(st, hidden, inter, m, gen.ACT_SILU, gen.TAIL_RESIDUAL, x, r, ws=ws)
    other = r0.clone()
    for rep in range(4):
        r.copy_(r0)
        fq.dense(st, hidden, inter, m, gen.ACT_SILU, gen.TAIL_RESIDUAL, x, other, ws=fq.Workspace())   # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, want), rep
    want_o = oracle.dense(inp["ffn"], hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, inp["x"], inp["resid"])
    check(host16(r), want_o, f"graph dense replay vs oracle tiled {tiled}")


@LAYOUTS
def test_graph_replay_routed(tiled):
    hidden, inter, E, m, k, cap = 512, 256, 16, 5, 4, 8
    say("graph routed", tiled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4343)
    d = mats_dev(inp["experts"], tiled, E)
    st = fq.ffn_struct(d)
    x, r0, lg = dev16(inp["x"]), dev16(inp["resid"]), dev(inp["logits"].astype(np.float32))
    seed_bits = gen.act_rows(gen.tensor_key(4344, m), m, hidden)
    seed = dev16(seed_bits)
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    ws = fq.Workspace()

    def layer(resid):
        fq.moe_route(lg, m, E, k, cap, ids, w, plan)
        fq.moe_routed_batched(st, E, hidden, inter, m, k, gen.ACT_SILU, x, ids, w, plan, seed, resid, ws=ws)

    want = r0.clone()
    layer(want)
    torch.cuda.synchronize()
    r = r0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(r)
    for rep in range(4):
        r.copy_(r0)
        ids.fill_(-7)
        plan.fill_(-7)                      # eager work that the replay must overwrite
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, want), rep
    rc, ids_o, w_o, plan_o = oracle.moe_route(inp["logits"], k, cap)
    assert rc == 0 and np.array_equal(ids.cpu().numpy(), ids_o) and np.array_equal(plan.cpu().numpy(), plan_o)
    want_o = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids_o, w_o, seed_bits,
                               inp["resid"])
    check(host16(r), want_o, f"graph routed replay vs oracle tiled {tiled}")


@LAYOUTS
def test_graph_replay_moe_layer(tiled):
    # route + ffnq_moe_layer with a gated shared expert, captured once and
    # replayed; the replays equal the eager layer and the oracle chain
    hidden, inter, E, m, k, cap, sh_inter = 512, 256, 32, 4, 8, 32, 384
    say("graph moe layer", tiled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4545, shared_inter=sh_inter)
    ex_d = mats_dev(inp["experts"], tiled, E)    # the device tensors stay referenced while they are used
    ex = fq.ffn_struct(ex_d)
    sh_d, sh = ffn_dev(inp["shared"], tiled)
    x, r0, lg, gv = dev16(inp["x"]), dev16(inp["resid"]), dev(inp["logits"].astype(np.float32)), dev16(inp["gate_vec"])
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    ws = fq.Workspace()

    def layer(resid):
        fq.moe_route(lg, m, E, k, cap, ids, w, plan)
        fq.moe_layer(ex, E, hidden, inter, m, k, gen.ACT_SILU, sh, sh_inter, gv, x, ids, w, plan, resid, ws=ws)

    want = r0.clone()
    layer(want)
    torch.cuda.synchronize()
    r = r0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(r)
    for rep in range(4):
        r.copy_(r0)
        ids.fill_(-7)
        plan.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, want), rep
    rc, ids_o, w_o, plan_o = oracle.moe_route(inp["logits"], k, cap)
    assert rc == 0 and np.array_equal(ids.cpu().numpy(), ids_o)
    seed_o = oracle.shared_expert(inp["shared"], hidden, sh_inter, gen.ACT_SILU, gen.TAIL_SIGMOID_GATE, inp["x"],
                                  inp["gate_vec"])
    want_o = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids_o, w_o, seed_o,
                               inp["resid"])
    check(host16(r), want_o, f"graph moe layer replay vs oracle tiled {tiled}")


@LAYOUTS
def test_graph_replay_moe_layer_logits(tiled):
    # ffnq_moe_layer_logits (the router inside the gate/up launch when tiled)
    # captured once and replayed; replays equal the eager call and the oracle
    hidden, inter, E, m, k, cap, sh_inter = 512, 256, 32, 2, 8, 32, 384
    say("graph moe layer logits", tiled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4646, shared_inter=sh_inter)
    ex_d = mats_dev(inp["experts"], tiled, E)
    ex = fq.ffn_struct(ex_d)
    sh_d, sh = ffn_dev(inp["shared"], tiled)
    x, r0, lg, gv = dev16(inp["x"]), dev16(inp["resid"]), dev(inp["logits"].astype(np.float32)), dev16(inp["gate_vec"])
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    ws = fq.Workspace()

    def layer(resid):
        fq.moe_layer_logits(ex, E, hidden, inter, m, k, gen.ACT_SILU, sh, sh_inter, gv, x, lg, cap, ids, w, plan,
                            resid, ws=ws)

    want = r0.clone()
    layer(want)
    torch.cuda.synchronize()
    r = r0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(r)
    for rep in range(4):
        r.copy_(r0)
        ids.fill_(-7)
        plan.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, want), rep
    rc, ids_o, w_o, plan_o = oracle.moe_route(inp["logits"], k, cap)
    assert rc == 0 and np.array_equal(ids.cpu().numpy(), ids_o) and np.array_equal(plan.cpu().numpy(), plan_o)
    seed_o = oracle.shared_expert(inp["shared"], hidden, sh_inter, gen.ACT_SILU, gen.TAIL_SIGMOID_GATE, inp["x"],
                                  inp["gate_vec"])
    want_o = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids_o, w_o, seed_o,
                               inp["resid"])
    check(host16(r), want_o, f"graph moe layer logits replay vs oracle tiled {tiled}")


@LAYOUTS
def test_graph_replay_moe_layer_sandwich(tiled):
    # the Gemma-style layer (route, shared branch, zero fill, routed half, sandwich
    # tail) captured once and replayed; replays equal the eager call and the oracle
    hidden, inter, E, m, k, cap, sh_inter, eps = 512, 256, 16, 3, 4, 8, 384, 1e-6
    say("graph moe layer sandwich", tiled)
    inp = gen.sandwich_inputs(hidden, E, inter, m, seed=4747, shared_inter=sh_inter)
    ex_d = mats_dev(inp["experts"], tiled, E)
    ex = fq.ffn_struct(ex_d)
    sh_d, sh = ffn_dev(inp["shared"], tiled)
    x, r0, lg = dev16(inp["x"]), dev16(inp["resid"]), dev(inp["logits"].astype(np.float32))
    n1, n2, sc = dev16(inp["shared_norm_w"]), dev16(inp["post_norm_w"]), dev(inp["expert_scale"])
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    ws = fq.Workspace()

    def layer(resid):
        fq.moe_layer_sandwich(ex, E, hidden, inter, m, k, gen.ACT_GELU_TANH, sh, sh_inter, n1, n2, eps, x, lg, cap,
                              ids, w, plan, resid, expert_scale=sc, ws=ws)

    want = r0.clone()
    layer(want)
    torch.cuda.synchronize()
    r = r0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(r)
    for rep in range(4):
        r.copy_(r0)
        ids.fill_(-7)
        plan.fill_(-7)
        ws.buf.fill_(0x7F)                  # eager work over the workspace the replay must rewrite (h1, r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, want), rep
    rc, ids_o, w_o, plan_o, h1_o, r_o, want_o = oracle.moe_sandwich_layer(
        inp["experts"], E, hidden, inter, gen.ACT_GELU_TANH, inp["shared"], sh_inter, inp["shared_norm_w"],
        inp["post_norm_w"], eps, inp["x"], inp["logits"], inp["expert_scale"], k, cap, inp["resid"])
    assert rc == 0 and np.array_equal(ids.cpu().numpy(), ids_o) and np.array_equal(plan.cpu().numpy(), plan_o)
    check(host16(r), want_o, f"graph moe layer sandwich replay vs oracle tiled {tiled}")
