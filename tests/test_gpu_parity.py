"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Routes and plans must match bit for bit; bf16 outputs
must be within a per-row relative L2 error of 2e-3; in the integer-exact
regime the outputs must match bit for bit."""
import sys

import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from helpers import rel_l2_rows
from test_oracle_pins import integer_regime

pytestmark = pytest.mark.gpu
TOL = 2e-3
I8, I4 = gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host16(t):
    return t.cpu().numpy().view(np.uint16)


LAYOUTS = pytest.mark.parametrize("tiled", [False, True], ids=["rowmajor", "tiled"])


def mats_dev(f, tiled=False, n_experts=1):
    """Device copies of an FFN's matrices; tiled=True repacks them with ffnq_pack."""
    d = {n: fq.to_device(f[n]) for n in ("gate", "up", "down")}
    if tiled:
        d = {n: fq.pack(d[n], n_experts) for n in d}
    return d


def ffn_dev(f, tiled=False):
    d = mats_dev(f, tiled)
    return d, fq.ffn_struct(d)


def ulp_diag(got, want):
    g = gen.bf16_to_f32(got).astype(np.float64)
    w = gen.bf16_to_f32(want).astype(np.float64)
    rms = np.sqrt(np.mean(w * w, axis=-1, keepdims=True))
    ref = np.maximum(np.abs(w), rms)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(ref, 1e-30))) - 7)
    return float(np.max(np.abs(g - w) / ulp)), float(np.max(np.abs(g - w)))


def gpu_dense(inp, hidden, inter, act, tail, shared=False, aux=None, eps=1e-6, tiled=False):
    d, st = ffn_dev(inp["ffn"], tiled)
    x = dev16(inp["x"])
    m = inp["x"].shape[0]
    if shared:
        out = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
        fq.shared_expert(st, hidden, inter, m, act, tail, x, out, None if aux is None else dev16(aux), eps)
    else:
        out = dev16(inp["resid"]) if tail == gen.TAIL_RESIDUAL else torch.zeros((m, hidden), dtype=torch.int16,
                                                                                  device="cuda")
        fq.dense(st, hidden, inter, m, act, tail, x, out, None if aux is None else dev16(aux), eps)
    torch.cuda.synchronize()
    return host16(out)


def check(got, want, label):
    err = rel_l2_rows(got, want)
    ulp, mabs = ulp_diag(got, want)
    say(f"{label}: rel_l2 {err:.3e} max_ulp {ulp:.2f} max_abs {mabs:.3e}")
    assert err <= TOL, (label, err)
    assert ulp <= 2.0, (label, ulp)


# ---------------------------------------------------------------------------
# dense / shared expert, small shapes spanning several tiles and ragged token counts

DENSE_CASES = [(fg, fd, act, tail, m)
               for (fg, fd) in ((I8, I8), (I4, I4), (I8, I4), (I4, I8))
               for act in (gen.ACT_SILU, gen.ACT_GELU_TANH)
               for tail in (gen.TAIL_RESIDUAL, gen.TAIL_RMSNORM)
               for m in (1, 3, 17)]


@LAYOUTS
@pytest.mark.parametrize("fg,fd,act,tail,m", DENSE_CASES)
def test_dense_small(fg, fd, act, tail, m, tiled):
    hidden, inter = 512, 768
    say("dense_small", fg, fd, act, tail, m, "tiled" if tiled else "rowmajor")
    inp = gen.dense_inputs(hidden, inter, m, fg, seed=1000 + 10 * fg + fd + 100 * m, fmt_down=fd)
    aux = inp["norm_w"] if tail == gen.TAIL_RMSNORM else None
    want = oracle.dense(inp["ffn"], hidden, inter, act, tail, inp["x"],
                        inp["resid"] if tail == gen.TAIL_RESIDUAL else None, aux)
    got = gpu_dense(inp, hidden, inter, act, tail, aux=aux, tiled=tiled)
    check(got, want, f"dense fmt {fg}/{fd} act {act} tail {tail} m {m} tiled {tiled}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 2, 5, 8, 16, 33])
@pytest.mark.parametrize("tail", [gen.TAIL_NONE, gen.TAIL_RMSNORM, gen.TAIL_SIGMOID_GATE])
def test_shared_expert_small(tail, m, tiled):
    hidden, inter = 384, 640
    say("shared_small", tail, m, tiled)
    inp = gen.dense_inputs(hidden, inter, m, I8, seed=2000 + m + 7 * tail)
    aux = {gen.TAIL_NONE: None, gen.TAIL_RMSNORM: inp["norm_w"], gen.TAIL_SIGMOID_GATE: inp["gate_vec"]}[tail]
    want = oracle.shared_expert(inp["ffn"], hidden, inter, gen.ACT_GELU_TANH, tail, inp["x"], aux)
    got = gpu_dense(inp, hidden, inter, gen.ACT_GELU_TANH, tail, shared=True, aux=aux, tiled=tiled)
    check(got, want, f"shared tail {tail} m {m} tiled {tiled}")


@LAYOUTS
@pytest.mark.parametrize("fmt", [I8, I4])
@pytest.mark.parametrize("act", [gen.ACT_SILU, gen.ACT_GELU_TANH])
@pytest.mark.parametrize("m", [1, 4, 9])
def test_integer_regime_bit_exact(fmt, act, m, tiled):
    hidden, inter = 256, 384
    say("integer_regime", fmt, act, m, tiled)
    ffn, x, resid, h, rv = integer_regime(fmt, hidden, inter, m, 300 + fmt + m)
    want = oracle.dense(ffn, hidden, inter, act, gen.TAIL_RESIDUAL, x, resid)
    got = gpu_dense(dict(ffn=ffn, x=x, resid=resid), hidden, inter, act, gen.TAIL_RESIDUAL, tiled=tiled)
    assert np.array_equal(got, want)
    want = oracle.shared_expert(ffn, hidden, inter, act, gen.TAIL_NONE, x, None)
    got = gpu_dense(dict(ffn=ffn, x=x, resid=resid), hidden, inter, act, gen.TAIL_NONE, shared=True, tiled=tiled)
    assert np.array_equal(got, want)


@LAYOUTS
def test_zero_input_and_repeat_calls(tiled):
    hidden, inter = 512, 768
    inp = gen.dense_inputs(hidden, inter, 3, I4, seed=77)
    inp["x"] = np.zeros_like(inp["x"])
    got = gpu_dense(inp, hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, tiled=tiled)
    assert np.array_equal(got, inp["resid"])
    # the same call twice gives the same bits
    inp = gen.dense_inputs(hidden, inter, 3, I4, seed=78)
    a = gpu_dense(inp, hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, tiled=tiled)
    b = gpu_dense(inp, hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, tiled=tiled)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# router + plan


def gpu_route(logits, k, cap, scale=None):
    m, E = logits.shape
    lg = dev(logits.astype(np.float32))
    ids = torch.full((m, k), -9, dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.full((fq.plan_ints(m, k),), -9, dtype=torch.int32, device="cuda")
    fq.moe_route(lg, m, E, k, cap, ids, w, plan, None if scale is None else dev(scale.astype(np.float32)))
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), plan.cpu().numpy()


def check_route(logits, k, cap, scale=None, label=""):
    rc, ids_o, w_o, plan_o = oracle.moe_route(logits, k, cap, scale)
    assert rc == 0
    ids_g, w_g, plan_g = gpu_route(logits, k, cap, scale)
    say(f"route {label} m {logits.shape[0]} E {logits.shape[1]} k {k} cap {cap}")
    assert np.array_equal(ids_g, ids_o)
    assert np.array_equal(plan_g, plan_o)
    np.testing.assert_allclose(w_g, w_o, rtol=1e-6, atol=1e-30)


@pytest.mark.parametrize("m,E,k,cap", [(1, 8, 2, 32), (4, 128, 8, 32), (4, 128, 8, 12), (2, 128, 8, 16),
                                       (64, 8, 2, 32), (7, 16, 4, 5), (33, 64, 6, 7), (200, 40, 3, 9),
                                       (5, 1024, 32, 32), (3, 3, 3, 3),
                                       # one sub-batch over many pairs (parallel plan), and past the LDS id cache
                                       (300, 8, 2, 32), (1000, 16, 4, 32), (1100, 16, 4, 32), (64, 128, 8, 32)])
def test_route_random(m, E, k, cap):
    logits = gen.router_logits(gen.tensor_key(m * 1000 + E, k), m, E)
    check_route(logits, k, cap, label="random")


@pytest.mark.parametrize("m,hidden,E", [(1, 2048, 128), (4, 2048, 128), (64, 4096, 8), (3, 264, 17), (5, 4104, 1)])
def test_router_logits(m, hidden, E):
    # the router GEMV against the oracle: within fp32 reassociation of the exact dot product
    rng = np.random.default_rng(m * 7 + E)
    x = gen.bf16_bits(rng.standard_normal((m, hidden)))
    w = gen.bf16_bits(rng.standard_normal((E, hidden)) / np.sqrt(hidden))
    say(f"router_logits m {m} hidden {hidden} E {E}")
    lg = torch.empty((m, E), dtype=torch.float32, device="cuda")
    fq.router_logits(dev(x.view(np.int16)), dev(w.view(np.int16)), m, hidden, E, lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy().astype(np.float64)
    want = oracle.router_logits(x, w).astype(np.float64)
    # fp32 summation error bound: a chain of at most 8 * ceil(hidden / 512) + 6 roundings (a lane's terms,
    # 8 per 512 inputs, then the wave's 6-level tree), each at most 2^-24 of a running magnitude <= sum |w x|;
    # plus the oracle's one rounding of the exact value
    absdot = np.abs(gen.bf16_to_f32(x)).astype(np.float64) @ np.abs(gen.bf16_to_f32(w)).astype(np.float64).T
    chain = 8 * ((hidden + 511) // 512) + 6
    bound = chain * 2.0 ** -24 * absdot + 2.0 ** -24 * np.abs(want)
    assert np.all(np.abs(got - want) <= bound)


def test_router_logits_exact_selection_then_route():
    # a selection router gives the inputs themselves, bit for bit, and routing them matches the oracle
    rng = np.random.default_rng(11)
    m, hidden, E, k, cap = 4, 2048, 128, 8, 32
    x = gen.bf16_bits(rng.standard_normal((m, hidden)))
    pi = rng.permutation(hidden)[:E]
    w = np.zeros((E, hidden), np.uint16)
    w[np.arange(E), pi] = gen.bf16_bits(1.0)
    lg = torch.empty((m, E), dtype=torch.float32, device="cuda")
    fq.router_logits(dev(x.view(np.int16)), dev(w.view(np.int16)), m, hidden, E, lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    assert np.array_equal(got, oracle.router_logits(x, w))
    check_route(got, k, cap, label="selection router")


def test_route_ties_nan_inf_scale():
    rng = np.random.default_rng(5)
    lg = rng.integers(-2, 3, (16, 12)).astype(np.float32)          # many ties
    check_route(lg, 4, 8, label="ties")
    lg[::3, ::2] = np.nan
    lg[1, :] = -np.inf
    lg[2, 5] = np.inf
    lg[4, :] = np.nan
    lg[6, 3] = -0.0
    check_route(lg, 3, 6, label="nan/inf")
    scale = (0.5 + rng.random(12)).astype(np.float32)
    check_route(lg, 3, 6, scale, label="scale")


# ---------------------------------------------------------------------------
# routed half


def gpu_routed(ex_dev, ex_struct, E, hidden, inter, k, cap, inp, seed_bits, act=gen.ACT_SILU):
    m = inp["x"].shape[0]
    ids, w, plan = gpu_route(inp["logits"], k, cap)
    ids_t, w_t, plan_t = dev(ids), dev(w), dev(plan)
    resid = dev16(inp["resid"])
    fq.moe_routed_batched(ex_struct, E, hidden, inter, m, k, act, dev16(inp["x"]), ids_t, w_t, plan_t,
                          None if seed_bits is None else dev16(seed_bits), resid)
    torch.cuda.synchronize()
    return host16(resid), ids, w


@LAYOUTS
@pytest.mark.parametrize("m,k,cap,use_seed", [(1, 4, 8, True), (3, 4, 8, True), (8, 4, 8, True), (8, 4, 8, False),
                                              (20, 2, 16, True), (5, 6, 6, False)])
def test_routed_small(m, k, cap, use_seed, tiled):
    hidden, inter, E = 512, 256, 16
    say("routed_small", m, k, cap, use_seed, tiled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=3000 + m + 10 * k)
    seed_bits = gen.act_rows(gen.tensor_key(3100, m), m, hidden) if use_seed else None
    d = mats_dev(inp["experts"], tiled, E)
    got, ids, w = gpu_routed(d, fq.ffn_struct(d), E, hidden, inter, k, cap, inp, seed_bits)
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids, w, seed_bits,
                             inp["resid"])
    check(got, want, f"routed m {m} k {k} cap {cap} seed {use_seed}")


# ---------------------------------------------------------------------------
# full-size workloads (sampled where the oracle would be slow)


@LAYOUTS
@pytest.mark.parametrize("m", [1, 4])
def test_config0_dense_int8(m, tiled):
    c = gen.CONFIGS[0]
    say("config0", m, tiled)
    inp = gen.config_inputs(0, m)
    want = oracle.dense(inp["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], inp["x"], inp["resid"])
    got = gpu_dense(inp, c["hidden"], c["inter"], c["act"], c["tail"], tiled=tiled)
    check(got, want, f"config0 m {m} tiled {tiled}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 4])
def test_config1_llama_int4(m, tiled):
    c = gen.CONFIGS[1]
    say("config1", m, tiled)
    inp = gen.config_inputs(1, m)
    got = gpu_dense(inp, c["hidden"], c["inter"], c["act"], c["tail"], tiled=tiled)
    want = oracle.dense(inp["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], inp["x"], inp["resid"])
    check(got, want, f"config1 m {m}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 8])
def test_config2_gemma_shared(m, tiled):
    c = gen.CONFIGS[2]
    say("config2", m, tiled)
    inp = gen.config_inputs(2, m)
    got = gpu_dense(inp, c["hidden"], c["inter"], c["act"], c["tail"], shared=True, aux=inp["norm_w"], tiled=tiled)
    rows = list(range(m)) if m <= 2 else [0, m // 2, m - 1]
    want = oracle.shared_expert(inp["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], inp["x"][rows],
                                inp["norm_w"], c["eps"])
    check(got[rows], want, f"config2 m {m}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 2, 4])
def test_config3_qwen_moe(m, tiled):
    c = gen.CONFIGS[3]
    say("config3", m, tiled)
    inp = gen.config_inputs(3, m)
    hidden, E, inter, k = c["hidden"], c["n_experts"], c["moe_inter"], c["top_k"]
    sh_d, sh_st = ffn_dev(inp["shared"], tiled)
    seed = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
    fq.shared_expert(sh_st, hidden, c["shared_inter"], m, c["act"], gen.TAIL_SIGMOID_GATE, dev16(inp["x"]), seed,
                     dev16(inp["gate_vec"]))
    torch.cuda.synchronize()
    seed_bits = host16(seed)
    want_seed = oracle.shared_expert(inp["shared"], hidden, c["shared_inter"], c["act"], gen.TAIL_SIGMOID_GATE,
                                     inp["x"], inp["gate_vec"])
    check(seed_bits, want_seed, f"config3 shared m {m}")
    d = mats_dev(inp["experts"], tiled, E)
    got, ids, w = gpu_routed(d, fq.ffn_struct(d), E, hidden, inter, k, c["cap"], inp, seed_bits)
    # the routed half is checked on the GPU's own seed, so its error is the routed half's alone
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, c["act"], inp["x"], ids, w, seed_bits, inp["resid"])
    check(got, want, f"config3 routed m {m}")
    rc, ids_o, w_o, plan_o = oracle.moe_route(inp["logits"], k, c["cap"])
    assert np.array_equal(ids, ids_o)


@LAYOUTS
@pytest.mark.parametrize("m", [1, 64])
def test_config4_mixtral_moe(m, tiled):
    c = gen.CONFIGS[4]
    say("config4", m, tiled)
    inp = gen.config_inputs(4, m)
    hidden, E, inter, k = c["hidden"], c["n_experts"], c["moe_inter"], c["top_k"]
    d = mats_dev(inp["experts"], tiled, E)
    got, ids, w = gpu_routed(d, fq.ffn_struct(d), E, hidden, inter, k, c["cap"], inp, None)
    rows = list(range(m)) if m <= 2 else [0, 21, 42, 63]
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, c["act"], inp["x"][rows], ids[rows], w[rows], None,
                             inp["resid"][rows])
    check(got[rows], want, f"config4 m {m}")
    counts = np.bincount(ids.ravel(), minlength=E)
    say(f"config4 m {m} tokens per expert min {counts.min()} max {counts.max()}")
