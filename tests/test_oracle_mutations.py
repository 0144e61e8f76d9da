"""The oracle's pins have teeth: each case plants one plausible mistake in a
copy of oracle.c (on the CPU only), builds it, routes the oracle calls to that
build and checks that every pin named for it now fails.  The unmodified
oracle passes the same pins in test_oracle_pins.  CPU only."""
import os

import pytest

import gen
import oracle
import test_oracle_pins as P

I8, I4 = gen.FMT_INT8_ROW, gen.FMT_INT4_AFFINE_G64

# (name, [(text in oracle.c, replacement)], pins that must fail)
MUTATIONS = [
    ("int8 scale of row 0 for every row",
     [("return s[row] * qv;", "return s[0] * qv;")],
     [P.test_dequant_int8_rows_hand]),
    ("int4 scale/zero group without the row term",
     [("size_t g = (size_t)row * (w->k / 64) + col / 64;", "size_t g = col / 64;")],
     [P.test_dequant_int4_rows_hand]),
    ("int4 nibble order swapped",
     [("int code = (col & 1) ? (byte >> 4) : (byte & 0x0F);", "int code = (col & 1) ? (byte & 0x0F) : (byte >> 4);")],
     [P.test_dequant_int4_hand, P.test_dequant_int4_rows_hand]),
    ("int4 zero point with the wrong sign",
     [("float diff = (float)code - zp;", "float diff = zp - (float)code;")],
     [P.test_dequant_int4_hand]),
    ("dot product summed in fp32",
     [("        double acc = 0.0;\n        for (int k = 0; k < w->k; ++k) acc += (double)or_dequant(w, n, k) * x[k];",
       "        float acc = 0.0f;\n        for (int k = 0; k < w->k; ++k) acc += (float)((double)or_dequant(w, n, k) * x[k]);")],
     [P.test_gemv_accumulates_beyond_fp32]),
    ("up passed through the activation instead of gate",
     [("double f = (act == OR_ACT_SILU) ? or_silu((double)g) : or_gelu_tanh((double)g);\n    return (float)(f * (double)u);",
       "double f = (act == OR_ACT_SILU) ? or_silu((double)u) : or_gelu_tanh((double)u);\n    return (float)(f * (double)g);")],
     [P.test_act_gate_is_first_operand]),
    ("sigmoid-gate logit of token 0 for every token",
     [("float l = or_gate_logit(aux, xt, hidden);", "float l = or_gate_logit(aux, x, hidden);")],
     [lambda: P.test_sigmoid_gate_composed_per_token(I8), lambda: P.test_sigmoid_gate_composed_per_token(I4)]),
    ("sigmoid gate applied with the negated logit",
     [("double sg = 1.0 / (1.0 + exp(-(double)logit));", "double sg = 1.0 / (1.0 + exp((double)logit));")],
     [lambda: P.test_sigmoid_gate_composed_per_token(I8), P.test_sigmoid_gate_closed_forms]),
    ("rmsnorm mean over one element too many",
     [("double r = 1.0 / sqrt(ss / (double)n + (double)eps);",
       "double r = 1.0 / sqrt(ss / (double)(n + 1) + (double)eps);")],
     [lambda: P.test_rmsnorm_composed_closed_form(I8), lambda: P.test_rmsnorm_composed_closed_form(I4),
      P.test_rmsnorm_golden]),
    ("rmsnorm eps outside the square root",
     [("double r = 1.0 / sqrt(ss / (double)n + (double)eps);",
       "double r = 1.0 / (sqrt(ss / (double)n) + (double)eps);")],
     [P.test_rmsnorm_golden]),
    ("residual add rounded twice",
     [("return or_bf16_round(or_bf16_value(x) + (double)h);",
       "return or_bf16_round((float)(or_bf16_value(x) + (double)h));")],
     [P.test_residual_single_rounding]),
    ("router ties to the higher index",
     [("    return a < b;\n}", "    return a > b;\n}")],
     [lambda: P.test_topk_brute_force(5)]),
    ("route weights from the negated logit gap",
     [("ex[r] = (lr == l0) ? 1.0 : exp(lr - l0);", "ex[r] = (lr == l0) ? 1.0 : exp(l0 - lr);")],
     [P.test_route_closed_form]),
    ("plan closes a sub-batch one expert early",
     [("if (usize + fresh > cap) break;", "if (usize + fresh >= cap) break;")],
     [P.test_plan_brute_force, P.test_plan_golden]),
    ("phase 2 adds the seed after the ranks",
     [("    float acc = seed;\n    for (int r = 0; r < k; ++r) {\n        float prod = w[r] * d[r];\n"
       "        acc = acc + prod;\n    }\n    return acc;",
       "    float acc = 0.0f;\n    for (int r = 0; r < k; ++r) {\n        float prod = w[r] * d[r];\n"
       "        acc = acc + prod;\n    }\n    return acc + seed;")],
     [P.test_seeded_vs_posthoc_crafted]),
    ("expert stride of the int4 scales off by a factor of two",
     [("r.s = (const uint16_t*)w->s + (size_t)e * n * (k / 64);",
       "r.s = (const uint16_t*)w->s + (size_t)e * n * (k / 128);")],
     [P.test_moe_labelled_experts_seeded]),
    ("sandwich join drops the routed row",
     [("z[i] = or_bf16_value(ht[i]) + or_bf16_value(rt[i]);", "z[i] = or_bf16_value(ht[i]);")],
     [P.test_sandwich_tail_hand, P.test_sandwich_tail_invariants,
      lambda: P.test_sandwich_layer_identical_experts("ones")]),
    ("sandwich tail norm weight dropped",
     [("uint16_t nb = or_bf16_round(z[i] * inv * or_bf16_value(w[i]));", "uint16_t nb = or_bf16_round(z[i] * inv);")],
     [P.test_sandwich_tail_hand]),
    ("sandwich norm row added before its bf16 rounding",
     [("o[i] = or_bf16_round(or_bf16_value(o[i]) + or_bf16_value(nb));",
       "o[i] = or_bf16_round(or_bf16_value(o[i]) + z[i] * inv * or_bf16_value(w[i])); (void)nb;")],
     [P.test_sandwich_tail_hand]),
    ("sandwich eps outside the square root",
     [("double inv = 1.0 / sqrt(ss / (double)n + (double)eps);",
       "double inv = 1.0 / (sqrt(ss / (double)n) + (double)eps);")],
     [P.test_sandwich_tail_hand]),
]


@pytest.mark.parametrize("name,subs,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_its_pins(name, subs, pins, tmp_path):
    with open(oracle.SRC) as f:
        src = f.read()
    for old, new in subs:
        assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
        src = src.replace(old, new)
    path = os.path.join(tmp_path, "oracle_mut.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.compile_source(path, os.path.join(tmp_path, "liboracle_mut.so"))
    with oracle.using(lib):
        still_pass = []
        for pin in pins:
            try:
                pin()
            except AssertionError:
                continue
            still_pass.append(getattr(pin, "__name__", repr(pin)))
    assert not still_pass, f"{name}: pins still pass: {still_pass}"
