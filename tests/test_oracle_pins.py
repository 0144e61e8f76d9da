"""Pins of the CPU oracle to things other than itself: hand-worked fixtures,
closed forms, invariants, brute force on tiny inputs and independent library
routines.  CPU only (no GPU marker)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from helpers import bf16_rne, bf16_val, f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# bf16 rounding


@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80), (-2.5, 0xC020), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2 ** -8, 0x3F80),              # tie -> even (1.0)
    (1.0 + 3 * 2 ** -8, 0x3F82),          # tie -> even (1 + 2^-6)
    (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),   # just above the tie -> up
    ((2 - 2 ** -7) * 2 ** 127, 0x7F7F),   # largest finite
    (2.0 ** 128, 0x7F80),                 # overflow -> inf
    (2.0 ** -133, 0x0001),                # smallest subnormal
    (2.0 ** -134, 0x0000),                # tie between 0 and 2^-133 -> even (0)
    (3 * 2.0 ** -134, 0x0002),            # tie between 1 and 2 subnormal units -> even (2)
    (2.0 ** -126, 0x0080),                # smallest normal
])
def test_bf16_round_textbook(v, bits):
    assert oracle.bf16_round(v) == bits


def test_bf16_round_matches_bit_rounding():
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 38, 4000),
                           rng.standard_normal(500) * 1e-39])
    for v in vals:
        assert oracle.bf16_round(float(v)) == bf16_rne(float(v)), v


def test_bf16_value_roundtrip():
    for b in [0x3F80, 0xC020, 0x0001, 0x7F7F, 0x0080, 0x4049]:
        assert oracle.bf16_round(oracle.bf16_value(b)) == b


# ---------------------------------------------------------------------------
# O1 dequantisation against the hand-worked fixture


def test_dequant_int4_hand():
    g = golden("dequant_hand.json")["int4"]
    k = g["k"]
    q = np.full((1, k // 2), g["byte_default"], np.uint8)
    for i, b in g["bytes_nondefault"].items():
        q[0, int(i)] = b
    mat = dict(fmt=gen.FMT_INT4_AFFINE_G64, n=1, k=k, q=q,
               s=gen.bf16_bits(np.array(g["s"])).reshape(1, -1), z=gen.bf16_bits(np.array(g["z"])).reshape(1, -1))
    w = oracle.dequant_matrix(mat)[0]
    for col, want in g["expect"].items():
        assert w[int(col)] == want, col


def test_dequant_int8_hand():
    g = golden("dequant_hand.json")["int8"]
    q = np.zeros((1, g["k"]), np.int8)
    q[0, :4] = g["q_head"]
    mat = dict(fmt=gen.FMT_INT8_ROW, n=1, k=g["k"], q=q, s=np.array([g["s"]], np.float32), z=None)
    w = oracle.dequant_matrix(mat)[0]
    assert list(w[:4]) == g["expect_head"]
    assert not np.any(w[4:])


def test_dequant_int8_rows_hand():
    # three rows with different scales: each row's weights carry its own scale
    g = golden("dequant_hand.json")["int8_rows"]
    n = len(g["s"])
    q = np.zeros((n, g["k"]), np.int8)
    q[:, :4] = g["q_head"]
    mat = dict(fmt=gen.FMT_INT8_ROW, n=n, k=g["k"], q=q, s=np.array(g["s"], np.float32), z=None)
    w = oracle.dequant_matrix(mat)
    for r in range(n):
        assert list(w[r, :4]) == g["expect_head"][r], r
        assert not np.any(w[r, 4:])


def test_dequant_int4_rows_hand():
    # two rows with the same codes and different scale/zero pairs
    g = golden("dequant_hand.json")["int4_rows"]
    k, n = g["k"], len(g["s"])
    q = np.full((n, k // 2), g["byte_default"], np.uint8)
    for i, b in g["bytes_nondefault"].items():
        q[:, int(i)] = b
    mat = dict(fmt=gen.FMT_INT4_AFFINE_G64, n=n, k=k, q=q, s=gen.bf16_bits(np.array(g["s"])),
               z=gen.bf16_bits(np.array(g["z"])))
    w = oracle.dequant_matrix(mat)
    for r in range(n):
        for col, want in g["expect"][r].items():
            assert w[r, int(col)] == want, (r, col)


def test_gemv_accumulates_beyond_fp32():
    # O2: the exact dot product 2^24 + 1 - 2^24 = 1 needs more than fp32's 24
    # bits while it is summed; the oracle sums in double and rounds once
    q = np.zeros((1, 64), np.int8)
    q[0, :3] = [64, 1, -64]
    mat = dict(fmt=gen.FMT_INT8_ROW, n=1, k=64, q=q, s=np.array([1.0], np.float32), z=None)
    x = np.zeros(64)
    x[:3] = [2.0 ** 18, 1.0, 2.0 ** 18]
    assert oracle.gemv(mat, x)[0] == 1.0


# ---------------------------------------------------------------------------
# O3 activations


def test_activation_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert oracle.silu(-1.0) == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    c = math.sqrt(2.0 / math.pi)
    assert oracle.gelu_tanh(1.0) == pytest.approx(0.5 * (1 + math.tanh(c * 1.044715)), rel=1e-15)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.gelu_tanh(-12.0)) < 1e-30


def test_activation_vs_torch():
    v = torch.linspace(-12, 12, 2001, dtype=torch.float64)
    silu = torch.nn.functional.silu(v)
    gelu = torch.nn.functional.gelu(v, approximate="tanh")
    for i in range(0, 2001, 7):
        x = float(v[i])
        assert oracle.silu(x) == pytest.approx(float(silu[i]), rel=1e-12, abs=1e-300)
        assert oracle.gelu_tanh(x) == pytest.approx(float(gelu[i]), rel=1e-12, abs=1e-15)


def test_act_gate_is_first_operand():
    # f(gate) * up: swapping the operands changes the value
    assert oracle.act(gen.ACT_SILU, 2.0, 3.0) == f32(3.0 * 2.0 / (1 + math.exp(-2.0)))
    assert oracle.act(gen.ACT_SILU, 2.0, 3.0) != oracle.act(gen.ACT_SILU, 3.0, 2.0)
    assert oracle.act(gen.ACT_SILU, 0.0, 5.0) == 0.0
    assert oracle.act(gen.ACT_GELU_TANH, 0.0, 5.0) == 0.0


# ---------------------------------------------------------------------------
# O4 tails


def test_rmsnorm_golden():
    for case in golden("rmsnorm_constant.json")["cases"]:
        if case["h"] == "const":
            h = np.full(case["n"], case["c"], np.float32)
            w = gen.bf16_bits(np.full(case["n"], case["w"]))
            out = oracle.rmsnorm_row(h, w, case["eps"])
            assert np.all(out == case["expect_bits"]), case
        else:
            h = np.array(case["h"], np.float32)
            w = gen.bf16_bits(np.full(h.shape[0], case["w"]))
            out = oracle.rmsnorm_row(h, w, case["eps"])
            assert list(out) == case["expect_bits"]


def test_rmsnorm_scale_invariance_and_zero():
    rng = np.random.default_rng(2)
    h = rng.standard_normal(256).astype(np.float32)
    w = gen.norm_weight(9, 256)
    a = oracle.rmsnorm_row(h, w, 0.0)
    b = oracle.rmsnorm_row(h * np.float32(4.0), w, 0.0)   # exact power-of-two scaling
    assert np.array_equal(a, b)
    z = oracle.rmsnorm_row(np.zeros(64, np.float32), gen.norm_weight(3, 64), 1e-6)
    assert np.all((z & 0x7FFF) == 0)


def test_residual_single_rounding():
    one = 0x3F80
    assert oracle.residual(one, 2.0 ** -8) == 0x3F80                 # tie -> even
    assert oracle.residual(one, 2.0 ** -8 + 2.0 ** -20) == 0x3F81    # above the tie
    assert oracle.residual(one, 3 * 2.0 ** -8) == 0x3F82             # tie -> even (up)
    assert oracle.residual(0xC000, 2.0) == 0x0000                    # -2 + 2 = +0
    # 1 + 2^-8 + 2^-30 is just above the tie, but an fp32 sum would drop the
    # 2^-30 and then round the tie to even: one rounding, from the exact sum
    assert oracle.residual(one, 2.0 ** -8 + 2.0 ** -30) == 0x3F81


def test_sigmoid_gate_closed_forms():
    # sigmoid(0) = 1/2 (P10): exact halving of the bf16 value
    rng = np.random.default_rng(3)
    for h in rng.standard_normal(200).astype(np.float32):
        want = bf16_rne(float(h) * 0.5)
        assert oracle.sigmoid_gate(float(h), 0.0) == want
    # sigmoid(ln 3) = 3/4
    v = oracle.sigmoid_gate(1.0, f32(math.log(3.0)))
    assert abs(bf16_val(v) - 0.75) <= 2 ** -9
    assert oracle.sigmoid_gate(2.0, 100.0) == 0x4000      # sigmoid -> 1
    assert oracle.sigmoid_gate(2.0, -200.0) == 0x0000     # sigmoid -> 0


def test_gate_logit_exact_integers():
    rng = np.random.default_rng(4)
    a = rng.integers(-8, 9, 2048)
    b = rng.integers(-8, 9, 2048)
    got = oracle.gate_logit(gen.bf16_bits(a), gen.bf16_bits(b))
    assert got == float(np.dot(a, b))


def test_router_logits_selection_hand_and_constant():
    # a selection router: row e of the weight is 1.0 at input pi(e), so logits[t][e] = x[t][pi(e)]
    # exactly (a transposed operand or a wrong row/column index fails)
    rng = np.random.default_rng(7)
    m, hidden, E = 3, 64, 16
    x = gen.bf16_bits(rng.standard_normal((m, hidden)))
    pi = rng.permutation(hidden)[:E]
    w = np.zeros((E, hidden), np.uint16)
    w[np.arange(E), pi] = gen.bf16_bits(1.0)
    got = oracle.router_logits(x, w)
    assert got.shape == (m, E)
    assert np.array_equal(got, gen.bf16_to_f32(x[:, pi]))
    # by hand: x = (1, 2, 3, 4, 0, ...), rows (1, 1, 1, 1, 0, ...) and (0.5, -1, 2, 0, ...) give 10 and 4.5
    x1 = np.zeros((1, 8), np.uint16)
    x1[0, :4] = gen.bf16_bits([1.0, 2.0, 3.0, 4.0])
    w1 = np.zeros((2, 8), np.uint16)
    w1[0, :4] = gen.bf16_bits([1.0, 1.0, 1.0, 1.0])
    w1[1, :3] = gen.bf16_bits([0.5, -1.0, 2.0])
    assert oracle.router_logits(x1, w1).tolist() == [[10.0, 4.5]]
    # constant rows against an all-ones token: hidden * 2^-e, exact
    hidden = 2048
    ones = np.full((1, hidden), gen.bf16_bits(1.0), np.uint16)
    wc = np.stack([np.full(hidden, gen.bf16_bits(2.0 ** -e), np.uint16) for e in range(6)])
    assert oracle.router_logits(ones, wc)[0].tolist() == [hidden * 2.0 ** -e for e in range(6)]


# ---------------------------------------------------------------------------
# O5 router


def _logits_from_fixture(vals):
    out = []
    for v in vals:
        out.append({"ln4": math.log(4.0), "ln2": math.log(2.0)}.get(v, v) if isinstance(v, str) else v)
    return np.array(out, np.float32)


def test_route_closed_form():
    g = golden("route_closed_form.json")
    lg = _logits_from_fixture(g["logits"])
    ids, w = oracle.topk_token(lg, g["top_k"])
    assert list(ids) == g["ids"]
    np.testing.assert_allclose(w, g["weights"], rtol=2e-7)
    ids, w = oracle.topk_token(lg, g["top_k"], np.array(g["scale"], np.float32))
    assert list(ids) == g["ids"]
    np.testing.assert_allclose(w, g["weights_scaled"], rtol=2e-7)


def _beats(l, a, b):
    va = -math.inf if math.isnan(l[a]) else l[a]
    vb = -math.inf if math.isnan(l[b]) else l[b]
    return va > vb or (va == vb and a < b)


@pytest.mark.parametrize("E", [1, 2, 3, 5, 8])
def test_topk_brute_force(E):
    rng = np.random.default_rng(E)
    cases = [rng.standard_normal(E).astype(np.float32) for _ in range(30)]
    cases += [rng.integers(-2, 3, E).astype(np.float32) for _ in range(30)]   # many ties
    nan_case = rng.standard_normal(E).astype(np.float32)
    nan_case[::2] = np.nan
    cases += [nan_case, np.full(E, -np.inf, np.float32)]
    for lg in cases:
        for k in range(1, E + 1):
            ids, w = oracle.topk_token(lg, k)
            assert len(set(ids.tolist())) == k
            for r in range(k):   # rank r is beaten by exactly r experts
                assert sum(_beats(lg, e, ids[r]) for e in range(E)) == r
            finite = np.where(np.isnan(lg), -np.inf, lg).astype(np.float64)
            if np.all(np.isfinite(finite)):
                best = max(sum(finite[list(c)]) for c in itertools.combinations(range(E), k))
                assert sum(finite[ids]) == best
                # renormalised full softmax (independent of the cancelled form)
                p = np.exp(finite - finite.max())
                p /= p.sum()
                sel = p[ids] / p[ids].sum()
                np.testing.assert_allclose(w, sel, rtol=1e-6)
                assert abs(float(np.sum(w.astype(np.float64))) - 1.0) < 1e-6


def test_route_degenerate_weights():
    ids, w = oracle.topk_token(np.full(4, -np.inf, np.float32), 3)
    assert list(ids) == [0, 1, 2]
    np.testing.assert_allclose(w, [1 / 3] * 3, rtol=1e-7)
    ids, w = oracle.topk_token(np.array([0.0, np.inf, 1.0], np.float32), 2)
    assert list(ids) == [1, 2] and list(w) == [1.0, 0.0]


# ---------------------------------------------------------------------------
# O7 union plan


def test_plan_golden():
    g = golden("plan_hand.json")
    rc, plan = oracle.moe_plan(np.array(g["ids"], np.int32), g["n_experts"], g["cap"])
    assert rc == 0
    f = oracle.plan_fields(plan, g["m"], g["top_k"])
    for key in ("n_sub", "sub_tok_begin", "sub_union_begin", "union_expert", "pair_slot", "slot_pair_begin",
                "slot_pairs"):
        got = f[key] if key == "n_sub" else list(f[key])
        assert got == g[key], key


def _check_plan_invariants(ids, E, cap, plan):
    m, k = ids.shape
    f = oracle.plan_fields(plan, m, k)
    S = f["n_sub"]
    stb, sub = f["sub_tok_begin"], f["sub_union_begin"]
    assert stb[0] == 0 and stb[S] == m and sub[0] == 0
    assert np.all(stb[S + 1:] == -1) and np.all(sub[S + 1:] == -1)
    U = sub[S]
    assert np.all(f["union_expert"][U:] == -1) and np.all(f["slot_pair_begin"][U + 1:] == -1)
    for b in range(S):
        t0, t1 = stb[b], stb[b + 1]
        assert t1 > t0
        # union in first-appearance pair order
        seen = []
        for p in range(t0 * k, t1 * k):
            if ids.flat[p] not in seen:
                seen.append(int(ids.flat[p]))
        assert list(f["union_expert"][sub[b]:sub[b + 1]]) == seen
        assert len(seen) <= cap
        if t1 < m:   # maximal: the next token would overflow
            nxt = set(seen) | set(ids[t1].tolist())
            assert len(nxt) > cap
        for p in range(t0 * k, t1 * k):
            assert f["union_expert"][sub[b] + f["pair_slot"][p]] == ids.flat[p]
    spb, sp = f["slot_pair_begin"], f["slot_pairs"]
    assert spb[0] == 0 and spb[U] == m * k
    assert sorted(sp.tolist()) == list(range(m * k))
    for g in range(U):
        grp = sp[spb[g]:spb[g + 1]]
        assert np.all(np.diff(grp) > 0)
        b = int(np.searchsorted(sub[:S + 1], g, side="right") - 1)
        for p in grp:
            assert sub[b] + f["pair_slot"][p] == g


def test_plan_brute_force():
    rng = np.random.default_rng(7)
    n = 0
    for m in range(1, 7):
        for E in range(1, 9):
            for k in range(1, min(E, 4) + 1):
                for cap in range(k, 9):
                    ids = np.array([rng.permutation(E)[:k] for _ in range(m)], np.int32)
                    rc, plan = oracle.moe_plan(ids, E, cap)
                    assert rc == 0
                    _check_plan_invariants(ids, E, cap, plan)
                    n += 1
    assert n > 500


def test_route_capacity_and_cap_limits():
    lg = gen.router_logits(1, 3, 16)
    rc, *_ = oracle.moe_route(lg, 4, 3)
    assert rc == oracle.ERR_CAPACITY
    rc, *_ = oracle.moe_route(lg, 4, 33)
    assert rc == oracle.ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# O8 seeded accumulation


def test_seeded_vs_posthoc_crafted():
    g = golden("seeded_vs_posthoc.json")
    got = oracle.seeded_sum(g["seed"], np.array(g["w"]), np.array(g["d"]))
    assert got == g["seeded"]
    post = np.float32(g["seed"]) + (np.float32(g["w"][0]) * np.float32(g["d"][0]) +
                                    np.float32(g["w"][1]) * np.float32(g["d"][1]))
    assert float(post) == g["posthoc"] and got != float(post)


def test_seeded_vs_posthoc_bound():
    rng = np.random.default_rng(8)
    for _ in range(500):
        k = int(rng.integers(1, 9))
        seed = float(np.float32(rng.standard_normal()))
        w = rng.random(k).astype(np.float32)
        d = rng.standard_normal(k).astype(np.float32)
        got = oracle.seeded_sum(seed, w, d)
        exact = seed + float(np.sum(w.astype(np.float64) * d.astype(np.float64)))
        bound = (k + 1) * 2.0 ** -24 * (abs(seed) + float(np.sum(np.abs(w.astype(np.float64) * d))))
        assert abs(got - exact) <= bound


# ---------------------------------------------------------------------------
# whole-FFN pins: permutation FFN (P1), zero input (P2), integer-exact regime (P11)


def _perm_ffn(fmt, hidden, inter, up_scale, rng):
    """gate/up select x[pi(n)] for n < hidden (extra rows zero); down = pi^-1.
    INT8: q in {0,1}, s = 1 (up: s = up_scale).  INT4: z = 8, codes in {8,9},
    s = 1 (up: s = up_scale)."""
    pi = rng.permutation(hidden)

    def mat(n, k, sel, scale):
        if fmt == gen.FMT_INT8_ROW:
            q = np.zeros((n, k), np.int8)
            for r, c in sel:
                q[r, c] = 1
            return dict(fmt=fmt, n=n, k=k, q=q, s=np.full(n, scale, np.float32), z=None)
        codes = np.full((n, k), 8, np.uint8)
        for r, c in sel:
            codes[r, c] = 9
        q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        return dict(fmt=fmt, n=n, k=k, q=q, s=gen.bf16_bits(np.full((n, k // 64), scale)),
                    z=gen.bf16_bits(np.full((n, k // 64), 8.0)))

    sel_gu = [(nn, pi[nn]) for nn in range(hidden)]
    inv = np.argsort(pi)
    sel_d = [(i, inv[i]) for i in range(hidden)]
    return dict(gate=mat(inter, hidden, sel_gu, 1.0), up=mat(inter, hidden, sel_gu, up_scale),
                down=mat(hidden, inter, sel_d, 1.0))


@pytest.mark.parametrize("fmt", [gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64])
@pytest.mark.parametrize("act", [gen.ACT_SILU, gen.ACT_GELU_TANH])
def test_permutation_ffn(fmt, act):
    rng = np.random.default_rng(10 + fmt + 3 * act)
    hidden, inter, m = 128, 192, 3
    ffn = _perm_ffn(fmt, hidden, inter, 2.0, rng)
    x = gen.act_rows(11, m, hidden)
    resid = gen.act_rows(12, m, hidden)
    out = oracle.dense(ffn, hidden, inter, act, gen.TAIL_RESIDUAL, x, resid)
    xv = torch.tensor(gen.bf16_to_f32(x).astype(np.float64))
    f = torch.nn.functional.silu(xv) if act == gen.ACT_SILU else torch.nn.functional.gelu(xv, approximate="tanh")
    a = (f * 2.0 * xv).numpy().astype(np.float32).astype(np.float64)    # act = fp32(f(g) * u), u = 2x
    rv = gen.bf16_to_f32(resid).astype(np.float64)
    want = np.vectorize(bf16_rne)(rv + a).astype(np.uint16)
    # the fp32 rounding of act may differ from torch's by an ulp only where f is not exact;
    # compare bits where the roundings agree and bound the rest
    diff = out != want
    assert diff.mean() < 0.01
    assert np.all(np.abs(gen.bf16_to_f32(out[diff]).astype(np.float64) - gen.bf16_to_f32(want[diff])) <=
                  np.abs(gen.bf16_to_f32(want[diff])) * 2 ** -7 + 1e-30)


def test_zero_input():
    ffn = gen.ffn(gen.FMT_INT4_AFFINE_G64, gen.FMT_INT4_AFFINE_G64, 128, 256, 21)
    x = np.zeros((2, 128), np.uint16)
    resid = gen.act_rows(22, 2, 128)
    out = oracle.dense(ffn, 128, 256, gen.ACT_SILU, gen.TAIL_RESIDUAL, x, resid)
    assert np.array_equal(out, resid)
    out = oracle.dense(ffn, 128, 256, gen.ACT_GELU_TANH, gen.TAIL_RMSNORM, x, None, gen.norm_weight(1, 128), 1e-6)
    assert np.all((out & 0x7FFF) == 0)


def integer_regime(fmt, hidden, inter, m, seed, free_col=False):
    """Inputs on which every partial sum is an exact dyadic number (P11).
    x in {-2..2} with x[:, :8] = 2; the gate's first eight columns carry a large
    weight so that g >= 24, where silu(g) == gelu(g) == g in fp32; g*u is a
    multiple of 1/4 below 2^13, so act is exact as a pair of bf16 halves (and
    the down projection's partial sums stay exact in fp32).  The
    scales are powers of two drawn per row (INT8) or per (row, group) (INT4):
    gate 2 or 4, up 1/4 or 1/2, down 2^-9, 2^-10 or 2^-11, so a kernel that
    applies another row's (or group's) scale loses bit-exactness.
    free_col: the last input column gets zero gate/up weights, so x[:, -1] may
    hold anything without changing h (the sigmoid-gate pin puts the logit there).
    Returns (ffn, x_bits, resid_bits, exact h [m][hidden], resid ints)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-2, 3, (m, hidden))
    x[:, :8] = 2
    sparse = lambda shape: rng.integers(-1, 2, shape) * (rng.random(shape) < 0.25)  # noqa: E731
    int8 = fmt == gen.FMT_INT8_ROW

    def scales(n, k, choices):
        return rng.choice(np.array(choices, np.float64), size=(n,) if int8 else (n, k // 64))

    def deq(q, s):   # the dequantised weights, exactly (float64)
        return q * (s[:, None] if int8 else np.repeat(s, 64, axis=1))

    def mk(q, s):
        n, k = q.shape
        if int8:
            return dict(fmt=fmt, n=n, k=k, q=q.astype(np.int8), s=s.astype(np.float32), z=None)
        codes = (q + 8).astype(np.uint8)
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        return dict(fmt=fmt, n=n, k=k, q=packed, s=gen.bf16_bits(s), z=gen.bf16_bits(np.full((n, k // 64), 8.0)))

    qg = sparse((inter, hidden))
    qg[:, :8] = 8 if int8 else 7
    qu = sparse((inter, hidden))
    qd = sparse((hidden, inter))
    if free_col:
        qg[:, -1] = 0
        qu[:, -1] = 0
    sg = scales(inter, hidden, [1.0, 2.0])
    su = scales(inter, hidden, [0.25, 0.5])
    sd = scales(hidden, inter, [2.0 ** -9, 2.0 ** -10, 2.0 ** -11])
    ffn = dict(gate=mk(qg, sg), up=mk(qu, su), down=mk(qd, sd))
    g = x @ deq(qg, sg).T
    u = x @ deq(qu, su).T
    assert np.all(g >= 24), "gate bias too small for this hidden"
    a = g * u
    assert np.all(np.abs(a) < 2 ** 13) and np.all(a * 4 == np.round(a * 4))
    h = a @ deq(qd, sd).T                     # exact in double: multiples of 2^-12, far below 2^53 of them
    resid = rng.integers(-64, 65, (m, hidden))
    return ffn, gen.bf16_bits(x), gen.bf16_bits(resid), h, resid


@pytest.mark.parametrize("fmt", [gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64])
@pytest.mark.parametrize("act", [gen.ACT_SILU, gen.ACT_GELU_TANH])
def test_integer_regime_exact(fmt, act):
    hidden, inter, m = 128, 192, 4
    ffn, x, resid, h, rv = integer_regime(fmt, hidden, inter, m, 30 + fmt)
    out = oracle.dense(ffn, hidden, inter, act, gen.TAIL_RESIDUAL, x, resid)
    want = np.vectorize(bf16_rne)(rv + h).astype(np.uint16)
    assert np.array_equal(out, want)
    out = oracle.shared_expert(ffn, hidden, inter, act, gen.TAIL_NONE, x, None)
    assert np.array_equal(out, np.vectorize(bf16_rne)(h).astype(np.uint16))


def half_bits(b):
    """bf16 bits of half a bf16 value (exact for normal values)."""
    return np.vectorize(lambda v: bf16_rne(bf16_val(int(v)) / 2.0))(b).astype(np.uint16)


@pytest.mark.parametrize("fmt", [gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64])
def test_shared_expert_zero_gate_halves(fmt):
    # P10 at m >= 2: a zero gate vector gives sigmoid(0) = 1/2 on every token,
    # so the gated branch is exactly half the ungated one
    hidden, inter, m = 256, 384, 5
    inp = gen.dense_inputs(hidden, inter, m, fmt, seed=90 + fmt, row_scales=True)
    none = oracle.shared_expert(inp["ffn"], hidden, inter, gen.ACT_GELU_TANH, gen.TAIL_NONE, inp["x"], None)
    gated = oracle.shared_expert(inp["ffn"], hidden, inter, gen.ACT_GELU_TANH, gen.TAIL_SIGMOID_GATE, inp["x"],
                                 np.zeros(hidden, np.uint16))
    assert np.array_equal(gated, half_bits(none))


SIG_LOGITS = (0.0, 100.0, -200.0)   # sigmoid: exactly 1/2, 1 and (to bf16) 0


def sigmoid_gate_case(fmt, hidden, inter, m, seed):
    """The integer-regime FFN with the last input column free; x[t][-1] holds
    token t's logit and the gate vector selects that column, so the logit of
    token t is exactly SIG_LOGITS[t % 3].  Returns (ffn, x, gate_vec, expected
    seed bits): bf16(h/2), bf16(h) and a signed zero."""
    ffn, x, _, h, _ = integer_regime(fmt, hidden, inter, m, seed, free_col=True)
    x = x.copy()
    lg = np.array([SIG_LOGITS[t % 3] for t in range(m)])
    x[:, -1] = gen.bf16_bits(lg)
    gv = np.zeros(hidden, np.uint16)
    gv[-1] = gen.bf16_bits(1.0)
    want = np.empty((m, hidden), np.uint16)
    for t in range(m):
        if lg[t] == 0.0:
            want[t] = [bf16_rne(v / 2.0) for v in h[t]]
        elif lg[t] > 0:
            want[t] = [bf16_rne(v) for v in h[t]]
        else:
            want[t] = np.where(h[t] < 0, 0x8000, 0x0000)
    return ffn, x, gv, want


@pytest.mark.parametrize("fmt", [gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64])
def test_sigmoid_gate_composed_per_token(fmt):
    # each token's logit comes from its own row of x (a logit read from another
    # token, or a bf16-rounded one, changes the result)
    ffn, x, gv, want = sigmoid_gate_case(fmt, 128, 192, 5, 95 + fmt)
    got = oracle.shared_expert(ffn, 128, 192, gen.ACT_SILU, gen.TAIL_SIGMOID_GATE, x, gv)
    assert np.array_equal(got, want)


RMS_G = (24.0, 32.0, 48.0, 64.0, 96.0, 128.0)


def rmsnorm_case(fmt, hidden, inter, m, seed):
    """A selection FFN whose h rows have constant magnitude, h_t[i] = +-G_t, so
    that rmsnorm(h_t) * w = +-w exactly (mean(h^2) = G_t^2, and eps = 1e-6
    moves G_t / sqrt(G_t^2 + eps) by under 1e-9, far below half a bf16 ulp).
    Gate row n selects input 0 (x_t[0] = G_t >= 24, where f(g) = g), up row
    n < hidden selects input 1 + n % (hidden - 1) (x = +-1 there; rows past
    hidden are zero), down row i selects act sigma(i) for a permutation sigma.
    Returns (ffn, x bits, norm weight bits, expected bits)."""
    rng = np.random.default_rng(seed)
    sigma = rng.permutation(hidden)

    def mat(n, k, sel):
        if fmt == gen.FMT_INT8_ROW:
            q = np.zeros((n, k), np.int8)
            for r, c in sel:
                q[r, c] = 1
            return dict(fmt=fmt, n=n, k=k, q=q, s=np.ones(n, np.float32), z=None)
        codes = np.full((n, k), 8, np.uint8)
        for r, c in sel:
            codes[r, c] = 9
        return dict(fmt=fmt, n=n, k=k, q=(codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8),
                    s=gen.bf16_bits(np.ones((n, k // 64))), z=gen.bf16_bits(np.full((n, k // 64), 8.0)))

    ffn = dict(gate=mat(inter, hidden, [(nn, 0) for nn in range(inter)]),
               up=mat(inter, hidden, [(nn, 1 + nn % (hidden - 1)) for nn in range(hidden)]),
               down=mat(hidden, inter, [(i, sigma[i]) for i in range(hidden)]))
    sgn = rng.choice([-1.0, 1.0], size=(m, hidden))
    x = sgn.copy()
    x[:, 0] = [RMS_G[t % len(RMS_G)] for t in range(m)]
    w = gen.norm_weight(seed + 1, hidden)
    neg = np.array([[x[t, 1 + sigma[i] % (hidden - 1)] < 0 for i in range(hidden)] for t in range(m)])
    want = np.where(neg, w | 0x8000, w).astype(np.uint16)
    return ffn, gen.bf16_bits(x), w, want


@pytest.mark.parametrize("fmt", [gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64])
def test_rmsnorm_composed_closed_form(fmt):
    # the RMSNorm tail of both the dense layer and the shared expert: +-w, with
    # each token's own sign pattern (a norm over another token's h, over inter
    # instead of hidden, or of a transposed FFN fails)
    hidden, inter, m = 128, 192, 4
    ffn, x, w, want = rmsnorm_case(fmt, hidden, inter, m, 70 + fmt)
    for act in (gen.ACT_SILU, gen.ACT_GELU_TANH):
        got = oracle.dense(ffn, hidden, inter, act, gen.TAIL_RMSNORM, x, None, w, 1e-6)
        assert np.array_equal(got, want)
        got = oracle.shared_expert(ffn, hidden, inter, act, gen.TAIL_RMSNORM, x, w, 1e-6)
        assert np.array_equal(got, want)


def test_batched_equals_per_token():
    ffn = gen.ffn(gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64, 128, 256, 41)
    x = gen.act_rows(42, 3, 128)
    resid = gen.act_rows(43, 3, 128)
    full = oracle.dense(ffn, 128, 256, gen.ACT_GELU_TANH, gen.TAIL_RESIDUAL, x, resid)
    for t in range(3):
        one = oracle.dense(ffn, 128, 256, gen.ACT_GELU_TANH, gen.TAIL_RESIDUAL, x[t:t + 1], resid[t:t + 1])
        assert np.array_equal(one[0], full[t])


# ---------------------------------------------------------------------------
# routed half


def test_moe_identical_experts_equals_dense():
    hidden, inter, E, k, m = 128, 128, 6, 3, 4
    one = gen.ffn(gen.FMT_INT4_AFFINE_G64, gen.FMT_INT4_AFFINE_G64, hidden, inter, 51)
    stack = {n: dict(one[n], q=np.stack([one[n]["q"]] * E), s=np.stack([one[n]["s"]] * E),
                     z=np.stack([one[n]["z"]] * E)) for n in one}
    x = gen.act_rows(52, m, hidden)
    resid = gen.act_rows(53, m, hidden)
    lg = gen.router_logits(54, m, E)
    rc, ids, w, _ = oracle.moe_route(lg, k, 8)
    assert rc == 0
    got = oracle.moe_routed(stack, E, hidden, inter, gen.ACT_SILU, x, ids, w, None, resid)
    want = oracle.dense(one, hidden, inter, gen.ACT_SILU, gen.TAIL_RESIDUAL, x, resid)
    d = np.abs(gen.bf16_to_f32(got).astype(np.float64) - gen.bf16_to_f32(want))
    assert np.all(d <= np.abs(gen.bf16_to_f32(want)) * 2 ** -7 + 1e-6)
    assert np.mean(got != want) < 0.02


def test_moe_labelled_experts_seeded():
    """Expert e's down matrix is (e+1) times a permutation, so the routed term
    of rank r is exactly (e_r+1)*act; pins expert strides, id lookup, weights
    and the seeded fp32 order."""
    hidden, inter, E, k, m = 128, 128, 5, 2, 3
    rng = np.random.default_rng(60)
    base = _perm_ffn(gen.FMT_INT4_AFFINE_G64, hidden, inter, 1.0, rng)
    stack = {}
    for n in ("gate", "up", "down"):
        mats = [dict(base[n]) for _ in range(E)]
        if n == "down":
            for e in range(E):
                mats[e]["s"] = gen.bf16_bits(np.full(base[n]["s"].shape, float(e + 1)))
        stack[n] = dict(base[n], q=np.stack([mm["q"] for mm in mats]), s=np.stack([mm["s"] for mm in mats]),
                        z=np.stack([mm["z"] for mm in mats]))
    x = gen.act_rows(61, m, hidden)
    resid = gen.act_rows(62, m, hidden)
    seed = gen.act_rows(63, m, hidden)
    ids = np.array([[3, 0], [1, 4], [4, 2]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [0.125, 0.875]], np.float32)
    got = oracle.moe_routed(stack, E, hidden, inter, gen.ACT_SILU, x, ids, w, seed, resid)
    xv = torch.tensor(gen.bf16_to_f32(x).astype(np.float64))
    a = (torch.nn.functional.silu(xv) * xv).numpy().astype(np.float32)   # act = fp32(silu(x) * x)
    want = np.empty_like(resid)
    for t in range(m):
        acc = gen.bf16_to_f32(seed[t]).copy()
        for r in range(k):
            d = (a[t] * np.float32(ids[t, r] + 1)).astype(np.float32)    # exact: small-int multiple
            acc = (acc + (np.float32(w[t, r]) * d).astype(np.float32)).astype(np.float32)
        want[t] = np.vectorize(bf16_rne)(gen.bf16_to_f32(resid[t]).astype(np.float64) + acc.astype(np.float64))
    diff = got != want
    assert diff.mean() < 0.01   # act's fp32 rounding may differ from torch's in the last ulp
    assert np.all(np.abs(gen.bf16_to_f32(got[diff]).astype(np.float64) - gen.bf16_to_f32(want[diff])) <=
                  np.abs(gen.bf16_to_f32(want[diff])) * 2 ** -7 + 1e-30)


# ---------------------------------------------------------------------------
# O9: the Gemma-style sandwich tail and the layer it ends


def _bits(rows):
    return gen.bf16_bits(np.array(rows, dtype=np.float64))


def test_sandwich_tail_hand():
    for case in golden("sandwich_hand.json")["cases"]:
        out = oracle.sandwich_tail(_bits(case["h1"]), _bits(case["r"]), _bits(case["w"]), case["eps"],
                                   _bits(case["resid"]))
        assert out.tolist() == case["expect_bits"], case["name"]


def test_sandwich_tail_invariants():
    rng = np.random.default_rng(81)
    m, n = 3, 96
    h1 = gen.bf16_bits(rng.standard_normal((m, n)))
    r = gen.bf16_bits(rng.standard_normal((m, n)))
    w = gen.norm_weight(82, n)
    resid = gen.act_rows(83, m, n)
    a = oracle.sandwich_tail(h1, r, w, 0.0, resid)
    # the join is a sum: the two rows commute
    assert np.array_equal(a, oracle.sandwich_tail(r, h1, w, 0.0, resid))
    # with eps = 0 the norm ignores a power-of-two scale of the joined row (bf16 doubling is exact)
    h2 = gen.bf16_bits(2.0 * gen.bf16_to_f32(h1).astype(np.float64))
    r2 = gen.bf16_bits(2.0 * gen.bf16_to_f32(r).astype(np.float64))
    assert np.array_equal(a, oracle.sandwich_tail(h2, r2, w, 0.0, resid))
    # an all-zero join adds +0 (eps > 0): the stream is unchanged
    z = np.zeros((m, n), np.uint16)
    assert np.array_equal(oracle.sandwich_tail(z, z, w, 1e-6, resid), resid)
    # rows are independent: one token at a time gives the same rows
    for t in range(m):
        one = oracle.sandwich_tail(h1[t:t + 1], r[t:t + 1], w, 0.0, resid[t:t + 1])
        assert np.array_equal(one[0], a[t])


@pytest.mark.parametrize("scale_kind", ["ones", "two"])
def test_sandwich_layer_identical_experts(scale_kind):
    """Routed experts that are all one FFN F: with route weights summing to 1 the
    unseeded routed sum is F(x_t) itself (to the fp32 rounding of the weighted
    sum), and with every expert scale 2 it is 2 F(x_t); so the layer is the
    sandwich tail of the shared branch's normed row and bf16(c F(x_t)), made
    here from oracle.shared_expert alone.  A routed sum seeded with the shared
    row, or a join that drops either row, fails this."""
    hidden, inter, sh_inter, E, k, m = 128, 128, 192, 6, 3, 4
    one = gen.ffn(gen.FMT_INT4_AFFINE_G64, gen.FMT_INT4_AFFINE_G64, hidden, inter, 71)
    stack = {n: dict(one[n], q=np.stack([one[n]["q"]] * E), s=np.stack([one[n]["s"]] * E),
                     z=np.stack([one[n]["z"]] * E)) for n in one}
    shared = gen.ffn(gen.FMT_INT8_ROW, gen.FMT_INT8_ROW, hidden, sh_inter, 72, row_scales=True)
    x = gen.act_rows(73, m, hidden)
    resid = gen.act_rows(74, m, hidden)
    lg = gen.router_logits(75, m, E)
    w1, wp = gen.norm_weight(76, hidden), gen.norm_weight(77, hidden)
    c = 1.0 if scale_kind == "ones" else 2.0
    scale = None if scale_kind == "ones" else np.full(E, c, np.float32)
    act, eps = gen.ACT_GELU_TANH, 1e-6
    rc, ids, w, plan, h1, r, out = oracle.moe_sandwich_layer(stack, E, hidden, inter, act, shared, sh_inter, w1, wp,
                                                             eps, x, lg, scale, k, 8, resid)
    assert rc == 0
    f = oracle.shared_expert(one, hidden, inter, act, gen.TAIL_NONE, x, None)       # bf16(F(x_t))
    rc_closed = gen.bf16_bits(c * gen.bf16_to_f32(f).astype(np.float64))             # exact: c is 1 or 2
    d = np.abs(gen.bf16_to_f32(r).astype(np.float64) - gen.bf16_to_f32(rc_closed))
    assert np.all(d <= np.abs(gen.bf16_to_f32(rc_closed)) * 2 ** -7 + 1e-30)
    assert np.mean(r != rc_closed) < 0.05
    h1_closed = oracle.shared_expert(shared, hidden, sh_inter, act, gen.TAIL_RMSNORM, x, w1, eps)
    assert np.array_equal(h1, h1_closed)
    want = oracle.sandwich_tail(h1_closed, rc_closed, wp, eps, resid)
    g = gen.bf16_to_f32(out).astype(np.float64)
    wv = gen.bf16_to_f32(want).astype(np.float64)
    assert np.all(np.abs(g - wv) <= np.abs(wv) * 2 ** -6 + 2 ** -10)
    assert np.mean(out != want) < 0.1
    # the shared row alone (routed term dropped) is far from the layer
    alone = oracle.sandwich_tail(h1_closed, np.zeros_like(h1_closed), wp, eps, resid)
    assert np.mean(alone != out) > 0.5
