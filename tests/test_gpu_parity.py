"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Routes and plans must match bit for bit; bf16 outputs
must be within a per-row relative L2 error of 2e-3; in the integer-exact
regime the outputs must match bit for bit."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from helpers import rel_l2_rows
from test_oracle_pins import integer_regime, rmsnorm_case, sigmoid_gate_case

pytestmark = pytest.mark.gpu
TOL = 2e-3
I8, I4 = gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


# The oracle computes each token on its own, so large cases run it on chunks of
# tokens in threads (ctypes releases the GIL during the call) and concatenate.
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_by_rows(fn, m, *row_args, **kw):
    """fn(*chunked row_args, **kw) over token chunks; row_args are [m][...] arrays (or None)."""
    nch = min(m, ORACLE_THREADS)
    bounds = [(m * i // nch, m * (i + 1) // nch) for i in range(nch)]
    def one(b):
        a, e = b
        return fn(*[None if r is None else r[a:e] for r in row_args], **kw)
    with ThreadPoolExecutor(nch) as ex:
        parts = list(ex.map(one, bounds))
    return np.concatenate(parts, axis=0)


_ORACLE_CACHE = {}


def cached(key, fn):
    """Oracle results shared by the row-major and tiled runs of a case."""
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = fn()
    return _ORACLE_CACHE[key]


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
    inp = gen.dense_inputs(hidden, inter, m, fg, seed=1000 + 10 * fg + fd + 100 * m, fmt_down=fd, row_scales=True)
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
    inp = gen.dense_inputs(hidden, inter, m, I8, seed=2000 + m + 7 * tail, row_scales=True)
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
@pytest.mark.parametrize("fmt", [I8, I4])
def test_sigmoid_gate_composed_bit_exact(fmt, tiled):
    # per-token logits 0, 100, -200 (from each token's own row of x) on the
    # integer-exact FFN: bf16(h/2), bf16(h) and +-0, bit for bit
    hidden, inter, m = 256, 384, 5
    say("sigmoid_composed", fmt, tiled)
    ffn, x, gv, want = sigmoid_gate_case(fmt, hidden, inter, m, 500 + fmt)
    assert np.array_equal(oracle.shared_expert(ffn, hidden, inter, gen.ACT_SILU, gen.TAIL_SIGMOID_GATE, x, gv), want)
    got = gpu_dense(dict(ffn=ffn, x=x), hidden, inter, gen.ACT_SILU, gen.TAIL_SIGMOID_GATE, shared=True, aux=gv,
                    tiled=tiled)
    assert np.array_equal(got, want)


@LAYOUTS
@pytest.mark.parametrize("fmt", [I8, I4])
@pytest.mark.parametrize("shared", [False, True], ids=["dense", "shared"])
def test_rmsnorm_composed_bit_exact(fmt, shared, tiled):
    # a constant-magnitude h per token: rmsnorm(h) * w = +-w with each token's
    # own sign pattern, bit for bit
    hidden, inter, m = 256, 384, 6
    say("rmsnorm_composed", fmt, shared, tiled)
    ffn, x, w, want = rmsnorm_case(fmt, hidden, inter, m, 600 + fmt)
    got = gpu_dense(dict(ffn=ffn, x=x), hidden, inter, gen.ACT_GELU_TANH, gen.TAIL_RMSNORM, shared=shared, aux=w,
                    tiled=tiled)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt,hidden,inter,m", [(I8, 1024, 1536, 2), (I8, 1024, 704, 9), (I4, 1024, 1152, 2),
                                                (I4, 2048, 1024, 9), (I4, 1024, 1536, 5), (I8, 2048, 704, 11)])
def test_dense_wide_gate_up(fmt, hidden, inter, m):
    # tiled dense calls with 2..11 rows take the gate/up shape with runs of two
    # tiles per workgroup (inter/16 is even whenever inter is a valid down K,
    # so every run has two tiles); INT8 K of 11 blocks, INT4 of 9 blocks
    say("dense_wide", fmt, hidden, inter, m)
    inp = gen.dense_inputs(hidden, inter, m, fmt, seed=5000 + hidden + inter + m, row_scales=True)
    want = oracle.dense(inp["ffn"], hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, inp["x"], inp["resid"])
    got = gpu_dense(inp, hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, tiled=True)
    check(got, want, f"dense wide fmt {fmt} {hidden}x{inter} m {m}")
    zero = dict(inp, resid=np.zeros_like(inp["resid"]))
    want0 = oracle.dense(inp["ffn"], hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, inp["x"], zero["resid"])
    check(gpu_dense(zero, hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, tiled=True), want0,
          f"dense wide (zero residual) fmt {fmt} {hidden}x{inter} m {m}")


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
                                       (300, 8, 2, 32), (1000, 16, 4, 32), (1100, 16, 4, 32), (64, 128, 8, 32),
                                       # one pair per thread: ids written by several waves, read by all threads
                                       (2, 16, 4, 32), (4, 16, 8, 32), (8, 16, 8, 32), (8, 64, 4, 32),
                                       (3, 128, 8, 32), (16, 8, 4, 32), (8, 128, 8, 32),
                                       # a thread per key (few experts per token), and past its weight bound
                                       (40, 12, 3, 6), (100, 32, 4, 32), (130, 31, 5, 9), (500, 8, 8, 32)])
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
    # the same cases over more tokens than one workgroup ranks in its small-batch path
    big = np.concatenate([lg, rng.integers(-2, 3, (48, 12)).astype(np.float32)])
    big[20::5, 1::3] = np.nan
    big[30, :] = np.inf
    big[31, 4] = -0.0
    check_route(big, 3, 6, label="nan/inf, 64 tokens")
    check_route(big, 4, 32, scale, label="scale, 64 tokens")


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


@LAYOUTS
@pytest.mark.parametrize("m,E,k,cap", [(3, 8, 4, 4), (4, 8, 4, 4), (8, 16, 8, 8)])
def test_routed_union_past_experts(m, E, k, cap, tiled):
    # a slot cap below the batch's union splits it into sub-batches whose
    # union entries, together, outnumber the experts: every entry must run
    hidden, inter = 512, 256
    say("routed union past experts", m, E, k, cap, tiled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=3200 + m + E + k)
    rc, _, _, plan_o = oracle.moe_route(inp["logits"], k, cap)
    assert rc == 0 and plan_o[m + 2 + plan_o[0]] > E   # the case this test is for
    seed_bits = gen.act_rows(gen.tensor_key(3201, m), m, hidden)
    d = mats_dev(inp["experts"], tiled, E)
    got, ids, w = gpu_routed(d, fq.ffn_struct(d), E, hidden, inter, k, cap, inp, seed_bits)
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids, w, seed_bits,
                             inp["resid"])
    check(got, want, f"routed union past experts m {m} E {E} k {k} cap {cap}")


# ---------------------------------------------------------------------------
# prefill-sized routed items (12 or more rows per expert), reduced width, every row


@LAYOUTS
@pytest.mark.parametrize("m,E,k,use_seed", [(64, 8, 2, True), (64, 4, 1, False), (96, 8, 2, False),
                                            (160, 4, 1, True)])   # entries past one pass of 32 pairs
def test_routed_prefill_sized(m, E, k, use_seed, tiled):
    hidden, inter, cap = 512, 1024, 32
    say("routed_prefill", m, E, k, use_seed, tiled)
    inp = gen.moe_inputs(hidden, E, inter, m, seed=3500 + m + E + k)
    seed_bits = gen.act_rows(gen.tensor_key(3600, m), m, hidden) if use_seed else None
    d = mats_dev(inp["experts"], tiled, E)
    for resid_kind in ("workload", "zero"):
        if resid_kind == "zero":
            inp = dict(inp, resid=np.zeros_like(inp["resid"]))
        got, ids, w = gpu_routed(d, fq.ffn_struct(d), E, hidden, inter, k, cap, inp, seed_bits)
        counts = np.bincount(ids.ravel(), minlength=E)
        assert counts.min() >= 12, counts
        want = oracle_by_rows(lambda xx, ii, ww, ss, rr: oracle.moe_routed(inp["experts"], E, hidden, inter,
                                                                          gen.ACT_SILU, xx, ii, ww, ss, rr),
                              m, inp["x"], ids, w, seed_bits, inp["resid"])
        check(got, want, f"routed prefill m {m} E {E} k {k} seed {use_seed} resid {resid_kind}")


# ---------------------------------------------------------------------------
# full-size workloads, every row, in the launch configuration bench.py times.
# "zero" residual variants make the output bf16(h) itself, so the tolerance
# applies to the FFN output undiluted by the residual stream; "row" scale
# variants of the INT8 workloads draw a scale per row.


def gpu_moe_layer(inp, c, m, tiled, resid):
    """ffnq_moe_route then ffnq_moe_layer (shared expert, if any, and routed half)."""
    hidden, E, inter, k = c["hidden"], c["n_experts"], c["moe_inter"], c["top_k"]
    ex = mats_dev(inp["experts"], tiled, E)
    sh_d, sh = ffn_dev(inp["shared"], tiled) if c["shared_inter"] else (None, None)   # sh_d keeps the tensors
    ids = torch.full((m, k), -9, dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.full((fq.plan_ints(m, k),), -9, dtype=torch.int32, device="cuda")
    fq.moe_route(dev(inp["logits"]), m, E, k, c["cap"], ids, w, plan)
    r = dev16(resid)
    fq.moe_layer(fq.ffn_struct(ex), E, hidden, inter, m, k, c["act"], sh, c["shared_inter"],
                 dev16(inp["gate_vec"]) if sh is not None else None, dev16(inp["x"]), ids, w, plan, r)
    torch.cuda.synchronize()
    return host16(r), ids.cpu().numpy(), w.cpu().numpy(), plan.cpu().numpy()


def oracle_moe_layer(inp, c, m, resid):
    """The oracle chain: route, gated shared expert (the seed), seeded routed half."""
    hidden, E, inter, k = c["hidden"], c["n_experts"], c["moe_inter"], c["top_k"]
    rc, ids, w, plan = oracle.moe_route(inp["logits"], k, c["cap"])
    assert rc == 0
    seed = None
    if c["shared_inter"]:
        seed = oracle_by_rows(lambda xx: oracle.shared_expert(inp["shared"], hidden, c["shared_inter"], c["act"],
                                                              gen.TAIL_SIGMOID_GATE, xx, inp["gate_vec"]),
                              m, inp["x"])
    out = oracle_by_rows(lambda xx, ii, ww, ss, rr: oracle.moe_routed(inp["experts"], E, hidden, inter, c["act"], xx,
                                                                     ii, ww, ss, rr),
                         m, inp["x"], ids, w, seed, resid)
    return ids, w, plan, seed, out


@LAYOUTS
@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("scales", ["workload", "row"])
def test_config0_dense_int8(m, scales, tiled):
    c = gen.CONFIGS[0]
    say("config0", m, scales, tiled)
    inp = gen.config_inputs(0, m, row_scales=scales == "row")
    want = oracle.dense(inp["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], inp["x"], inp["resid"])
    got = gpu_dense(inp, c["hidden"], c["inter"], c["act"], c["tail"], tiled=tiled)
    check(got, want, f"config0 m {m} scales {scales} tiled {tiled}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("resid_kind", ["workload", "zero"])
def test_config1_llama_int4(m, resid_kind, tiled):
    c = gen.CONFIGS[1]
    say("config1", m, resid_kind, tiled)
    inp = gen.config_inputs(1, m)
    if resid_kind == "zero":
        inp["resid"] = np.zeros_like(inp["resid"])
    got = gpu_dense(inp, c["hidden"], c["inter"], c["act"], c["tail"], tiled=tiled)
    want = cached(("c1", m, resid_kind), lambda: oracle_by_rows(
        lambda xx, rr: oracle.dense(inp["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], xx, rr),
        m, inp["x"], inp["resid"]))
    check(got, want, f"config1 m {m} resid {resid_kind}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 8])
@pytest.mark.parametrize("scales", ["workload", "row"])
def test_config2_gemma_shared(m, scales, tiled):
    c = gen.CONFIGS[2]
    say("config2", m, scales, tiled)
    inp = gen.config_inputs(2, m, row_scales=scales == "row")
    got = gpu_dense(inp, c["hidden"], c["inter"], c["act"], c["tail"], shared=True, aux=inp["norm_w"], tiled=tiled)
    want = cached(("c2", m, scales), lambda: oracle_by_rows(
        lambda xx: oracle.shared_expert(inp["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], xx, inp["norm_w"],
                                        c["eps"]), m, inp["x"]))
    check(got, want, f"config2 m {m} scales {scales}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 2, 4])
def test_config3_qwen_two_calls(m, tiled):
    # ffnq_shared_expert (sigmoid-gate tail) against the oracle, then
    # ffnq_moe_routed_batched on that seed against the oracle on the same seed
    c = gen.CONFIGS[3]
    say("config3 two calls", m, tiled)
    inp = gen.config_inputs(3, m)
    hidden, E, inter, k = c["hidden"], c["n_experts"], c["moe_inter"], c["top_k"]
    sh_d, sh_st = ffn_dev(inp["shared"], tiled)
    seed = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
    fq.shared_expert(sh_st, hidden, c["shared_inter"], m, c["act"], gen.TAIL_SIGMOID_GATE, dev16(inp["x"]), seed,
                     dev16(inp["gate_vec"]))
    torch.cuda.synchronize()
    seed_bits = host16(seed)
    want_seed = cached(("c3 seed", m), lambda: oracle.shared_expert(inp["shared"], hidden, c["shared_inter"], c["act"],
                                                                    gen.TAIL_SIGMOID_GATE, inp["x"], inp["gate_vec"]))
    check(seed_bits, want_seed, f"config3 shared m {m}")
    d = mats_dev(inp["experts"], tiled, E)
    got, ids, w = gpu_routed(d, fq.ffn_struct(d), E, hidden, inter, k, c["cap"], inp, seed_bits)
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, c["act"], inp["x"], ids, w, seed_bits, inp["resid"])
    check(got, want, f"config3 routed m {m}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 2, 4])
@pytest.mark.parametrize("resid_kind", ["workload", "zero"])
def test_config3_qwen_layer_end_to_end(m, resid_kind, tiled):
    # ffnq_moe_route + ffnq_moe_layer (the calls bench.py times) against the
    # oracle chain route -> gated shared expert -> seeded routed half, all on
    # the oracle's own routes, weights and seed
    c = gen.CONFIGS[3]
    say("config3 layer", m, resid_kind, tiled)
    inp = gen.config_inputs(3, m)
    if resid_kind == "zero":
        inp["resid"] = np.zeros_like(inp["resid"])
    ids_o, w_o, plan_o, _, want = cached(("c3 layer", m, resid_kind),
                                         lambda: oracle_moe_layer(inp, c, m, inp["resid"]))
    got, ids, w, plan = gpu_moe_layer(inp, c, m, tiled, inp["resid"])
    assert np.array_equal(ids, ids_o)
    assert np.array_equal(plan, plan_o)
    np.testing.assert_allclose(w, w_o, rtol=1e-6, atol=1e-30)
    check(got, want, f"config3 layer m {m} resid {resid_kind}")


@LAYOUTS
@pytest.mark.parametrize("m", [1, 64])
@pytest.mark.parametrize("resid_kind", ["workload", "zero"])
def test_config4_mixtral_moe(m, resid_kind, tiled):
    c = gen.CONFIGS[4]
    say("config4", m, resid_kind, tiled)
    inp = gen.config_inputs(4, m)
    if resid_kind == "zero":
        inp["resid"] = np.zeros_like(inp["resid"])
    ids_o, w_o, plan_o, _, want = cached(("c4", m, resid_kind), lambda: oracle_moe_layer(inp, c, m, inp["resid"]))
    got, ids, w, plan = gpu_moe_layer(inp, c, m, tiled, inp["resid"])
    assert np.array_equal(ids, ids_o)
    assert np.array_equal(plan, plan_o)
    np.testing.assert_allclose(w, w_o, rtol=1e-6, atol=1e-30)
    check(got, want, f"config4 m {m} resid {resid_kind}")
    counts = np.bincount(ids.ravel(), minlength=c["n_experts"])
    say(f"config4 m {m} tokens per expert min {counts.min()} max {counts.max()}")


@pytest.mark.parametrize("m", [1, 3])
def test_shared_expert_rmsnorm_row_past_lds(m):
    # hidden 8320 > 8192: the RMSNorm keeps no row in LDS and reads the
    # partials twice (the second pass re-sums them)
    hidden, inter = 8320, 256
    say("shared rmsnorm wide row", m)
    for fmt in (I8, I4):
        inp = gen.dense_inputs(hidden, inter, m, fmt, seed=2600 + m + fmt, row_scales=True)
        want = oracle.shared_expert(inp["ffn"], hidden, inter, gen.ACT_GELU_TANH, gen.TAIL_RMSNORM, inp["x"],
                                    inp["norm_w"])
        got = gpu_dense(inp, hidden, inter, gen.ACT_GELU_TANH, gen.TAIL_RMSNORM, shared=True, aux=inp["norm_w"],
                        tiled=True)
        check(got, want, f"shared rmsnorm wide row fmt {fmt} m {m}")
