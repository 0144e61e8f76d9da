"""ffnq_moe_layer: the gated shared expert and the routed half in one call.

Its contract is the two-call sequence ffnq_shared_expert(SIGMOID_GATE) ->
seed -> ffnq_moe_routed_batched(seed), bit for bit, whichever launch plan it
takes (shared and routed gate/up in one launch when both are tiled INT4 with
matching launch shapes, separate launches otherwise).  The two-call sequence
is checked against the oracle in test_gpu_parity; here the layer is compared
with it exactly, and once more with the oracle within the float bar."""
import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from helpers import rel_l2_rows

pytestmark = pytest.mark.gpu

TOL = 2e-3


def say(*a):
    print("[case]", *a, flush=True)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def mats(f, tiled, n_experts=1):
    d = {n: fq.to_device(f[n]) for n in ("gate", "up", "down")}
    if tiled:
        d = {n: fq.pack(d[n], n_experts) for n in d}
    return d, fq.ffn_struct(d)


def route(logits, k, cap):
    m, E = logits.shape
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    fq.moe_route(dev(logits.astype(np.float32)), m, E, k, cap, ids, w, plan)
    return ids, w, plan


def two_calls(ex, sh, E, hidden, inter, sh_inter, m, k, act, x, gate, ids, w, plan, resid0):
    resid = resid0.clone()
    seed = None
    if sh is not None:
        seed = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
        fq.shared_expert(sh, hidden, sh_inter, m, act, gen.TAIL_SIGMOID_GATE, x, seed, gate)
    fq.moe_routed_batched(ex, E, hidden, inter, m, k, act, x, ids, w, plan, seed, resid)
    torch.cuda.synchronize()
    return host16(resid), None if seed is None else host16(seed)


def one_call(ex, sh, E, hidden, inter, sh_inter, m, k, act, x, gate, ids, w, plan, resid0):
    resid = resid0.clone()
    fq.moe_layer(ex, E, hidden, inter, m, k, act, sh, sh_inter, gate, x, ids, w, plan, resid)
    torch.cuda.synchronize()
    return host16(resid)


def run_case(inp, E, hidden, inter, sh_inter, m, k, cap, act, tiled_ex, sh_fmt_tiled):
    ex_d, ex = mats(inp["experts"], tiled_ex, E)
    sh = None
    if sh_inter:
        sh_d, sh = mats(inp["shared"], sh_fmt_tiled)
    x = dev16(inp["x"])
    gate = dev16(inp["gate_vec"]) if sh_inter else None
    resid0 = dev16(inp["resid"])
    ids, w, plan = route(inp["logits"], k, cap)
    want, seed = two_calls(ex, sh, E, hidden, inter, sh_inter, m, k, act, x, gate, ids, w, plan, resid0)
    got = one_call(ex, sh, E, hidden, inter, sh_inter, m, k, act, x, gate, ids, w, plan, resid0)
    assert np.array_equal(got, want)
    return got, seed, ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("m", [1, 4])
def test_layer_config3_matches_two_calls(m):
    c = gen.CONFIGS[3]
    say("layer config3", m)
    inp = gen.config_inputs(3, m)
    hidden, E, inter, k = c["hidden"], c["n_experts"], c["moe_inter"], c["top_k"]
    got, seed, ids, w = run_case(inp, E, hidden, inter, c["shared_inter"], m, k, c["cap"], c["act"], True, True)
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, c["act"], inp["x"], ids, w, seed, inp["resid"])
    assert rel_l2_rows(got, want) <= TOL


@pytest.mark.parametrize("m,k,cap,tiled_ex,sh_tiled,sh_fmt", [
    (1, 4, 8, True, True, gen.FMT_INT4_AFFINE_G64),     # one gate/up launch for both
    (5, 4, 8, True, True, gen.FMT_INT4_AFFINE_G64),     # ragged rows, several sub-batches
    (3, 2, 8, False, False, gen.FMT_INT4_AFFINE_G64),   # row-major: separate launches
    (4, 4, 8, True, False, gen.FMT_INT8_ROW),           # INT8 row-major shared expert, tiled experts
    (20, 2, 16, True, True, gen.FMT_INT4_AFFINE_G64),   # more rows per expert
    (8, 8, 16, True, True, gen.FMT_INT4_AFFINE_G64),    # 64 pairs: eight activation rows per burst unit
])
def test_layer_small_matches_two_calls(m, k, cap, tiled_ex, sh_tiled, sh_fmt):
    hidden, inter, E, sh_inter = 512, 256, 16, 384
    say("layer small", m, k, cap, tiled_ex, sh_tiled, sh_fmt)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4600 + m + 10 * k)
    inp["shared"] = gen.ffn(sh_fmt, sh_fmt, hidden, sh_inter, gen.tensor_key(4700 + m, 1))
    inp["gate_vec"] = gen.gate_vector(gen.tensor_key(4701 + m, 2), hidden)
    run_case(inp, E, hidden, inter, sh_inter, m, k, cap, gen.ACT_SILU, tiled_ex, sh_tiled)


@pytest.mark.parametrize("m,E,k,cap", [(3, 8, 4, 4), (4, 8, 4, 5)])
def test_layer_union_past_experts(m, E, k, cap):
    # sub-batches whose union entries outnumber the experts, through the fused down
    hidden, inter, sh_inter = 512, 256, 384
    say("layer union past experts", m, E, k, cap)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4650 + m + E, shared_inter=sh_inter)
    rc, _, _, plan_o = oracle.moe_route(inp["logits"], k, cap)
    assert rc == 0 and plan_o[m + 2 + plan_o[0]] > E
    got, seed, ids, w = run_case(inp, E, hidden, inter, sh_inter, m, k, cap, gen.ACT_SILU, True, True)
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids, w, seed, inp["resid"])
    assert rel_l2_rows(got, want) <= TOL


@pytest.mark.parametrize("m,E,k", [(64, 8, 2), (96, 4, 1)])
def test_layer_prefill_sized(m, E, k):
    # 12 or more pairs per expert: the grouped prefill kernels for the routed
    # phases beside the shared expert's own launches
    hidden, inter, sh_inter, cap = 512, 256, 384, 32
    say("layer prefill sized", m, E, k)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4680 + m + E, shared_inter=sh_inter)
    got, seed, ids, w = run_case(inp, E, hidden, inter, sh_inter, m, k, cap, gen.ACT_SILU, True, True)
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids, w, seed, inp["resid"])
    assert rel_l2_rows(got, want) <= TOL


@pytest.mark.parametrize("tiled", [False, True])
def test_layer_without_shared_is_unseeded_routed(tiled):
    hidden, inter, E, m, k, cap = 512, 256, 16, 3, 4, 8
    say("layer no shared", tiled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4800)
    run_case(inp, E, hidden, inter, 0, m, k, cap, gen.ACT_SILU, tiled, tiled)


# ---------------------------------------------------------------------------
# ffnq_moe_layer_logits: route + layer in one call, bit for bit the two calls


def logits_call(ex, sh, E, hidden, inter, sh_inter, m, k, cap, act, x, gate, logits, resid0, scale=None):
    resid = resid0.clone()
    ids = torch.full((m, k), -9, dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.full((fq.plan_ints(m, k),), -9, dtype=torch.int32, device="cuda")
    fq.moe_layer_logits(ex, E, hidden, inter, m, k, act, sh, sh_inter, gate, x, logits, cap, ids, w, plan, resid,
                        expert_scale=scale)
    torch.cuda.synchronize()
    return host16(resid), ids.cpu().numpy(), w.cpu().numpy(), plan.cpu().numpy()


def route_then_layer(ex, sh, E, hidden, inter, sh_inter, m, k, cap, act, x, gate, logits, resid0, scale=None):
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    fq.moe_route(logits, m, E, k, cap, ids, w, plan, scale)
    got = one_call(ex, sh, E, hidden, inter, sh_inter, m, k, act, x, gate, ids, w, plan, resid0)
    return got, ids.cpu().numpy(), w.cpu().numpy(), plan.cpu().numpy()


@pytest.mark.parametrize("m,E,k,cap,sh_inter,tiled,scaled", [
    (1, 16, 4, 8, 384, True, False),      # routed inside the gate/up launch
    (3, 16, 4, 8, 384, True, False),      # several sub-batches
    (4, 32, 8, 32, 384, True, True),      # expert scale
    (2, 16, 4, 6, 0, True, False),        # no shared expert, a cap that splits
    (4, 16, 4, 8, 384, False, False),     # row-major: the router runs first
    (9, 16, 4, 8, 384, True, False),      # m > 4: the router runs first
])
def test_layer_logits_matches_route_then_layer(m, E, k, cap, sh_inter, tiled, scaled):
    hidden, inter = 512, 256
    say("layer logits small", m, E, k, cap, sh_inter, tiled, scaled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=4900 + m + E + k, shared_inter=sh_inter)
    ex_d, ex = mats(inp["experts"], tiled, E)
    sh = None
    if sh_inter:
        sh_d, sh = mats(inp["shared"], tiled)
    x, r0 = dev16(inp["x"]), dev16(inp["resid"])
    gate = dev16(inp["gate_vec"]) if sh_inter else None
    lg = dev(inp["logits"].astype(np.float32))
    scale = dev((0.5 + np.random.default_rng(m).random(E)).astype(np.float32)) if scaled else None
    a = logits_call(ex, sh, E, hidden, inter, sh_inter, m, k, cap, gen.ACT_SILU, x, gate, lg, r0, scale)
    b = route_then_layer(ex, sh, E, hidden, inter, sh_inter, m, k, cap, gen.ACT_SILU, x, gate, lg, r0, scale)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    rc, ids_o, w_o, plan_o = oracle.moe_route(inp["logits"], k, cap,
                                              None if scale is None else scale.cpu().numpy())
    assert rc == 0 and np.array_equal(a[1], ids_o) and np.array_equal(a[3], plan_o)


@pytest.mark.parametrize("c,m", [(3, 1), (3, 2), (3, 4), (4, 1), (4, 64)])
def test_layer_logits_workloads(c, m):
    cfg = gen.CONFIGS[c]
    say("layer logits workload", c, m)
    inp = gen.config_inputs(c, m)
    hidden, E, inter, k = cfg["hidden"], cfg["n_experts"], cfg["moe_inter"], cfg["top_k"]
    ex_d, ex = mats(inp["experts"], True, E)
    sh, gate = None, None
    if cfg["shared_inter"]:
        sh_d, sh = mats(inp["shared"], True)
        gate = dev16(inp["gate_vec"])
    x, r0, lg = dev16(inp["x"]), dev16(inp["resid"]), dev(inp["logits"].astype(np.float32))
    a = logits_call(ex, sh, E, hidden, inter, cfg["shared_inter"], m, k, cfg["cap"], cfg["act"], x, gate, lg, r0)
    b = route_then_layer(ex, sh, E, hidden, inter, cfg["shared_inter"], m, k, cfg["cap"], cfg["act"], x, gate, lg, r0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
