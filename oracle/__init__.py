"""TEST INFRASTRUCTURE ONLY: Python access to the CPU oracle in oracle.c.

The oracle is the plain, slow, single-threaded definition of the quantized
gated FFN and the MoE routed half that the HIP path is checked against.  Only
the tests, the smoke check and the benchmark's CPU-baseline leg may use it;
the library never does.  It shares no code with the HIP path: the only shared
code is the seeded input generator `gen`, which holds none of the method.

All arrays are host numpy arrays; bf16 values travel as uint16 bit patterns.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_CAPACITY = 0, -1, -2, -3
TAIL_NONE, TAIL_RESIDUAL, TAIL_RMSNORM, TAIL_SIGMOID_GATE = 0, 1, 2, 3   # oracle.h OR_TAIL_*


CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]


def compile_source(src: str, out: str, extra: tuple = ()) -> str:
    """gcc one oracle source file (oracle.c, or a test's variant of it) into a shared library."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", *CFLAGS, *extra, "-I", HERE, "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no FMA contraction, IEEE double)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < max(
            os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "oracle.h"))):
        compile_source(SRC, LIB)
    return LIB


class QMat(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("n", C.c_int32), ("k", C.c_int32),
                ("q", C.c_void_p), ("s", C.c_void_p), ("z", C.c_void_p)]


_lib = None


def _load(path: str):
    """Load an oracle build and declare its functions' signatures."""
    L = C.CDLL(path)
    vp, i32, f32 = C.c_void_p, C.c_int, C.c_float
    P = C.POINTER(QMat)
    sig = {
        "or_bf16_value": (C.c_double, [C.c_uint16]),
        "or_bf16_round": (C.c_uint16, [C.c_double]),
        "or_dequant": (f32, [P, i32, i32]),
        "or_dequant_matrix": (None, [P, vp]),
        "or_gemv": (None, [P, vp, vp]),
        "or_silu": (C.c_double, [C.c_double]),
        "or_gelu_tanh": (C.c_double, [C.c_double]),
        "or_act": (f32, [i32, f32, f32]),
        "or_residual": (C.c_uint16, [C.c_uint16, f32]),
        "or_rmsnorm_row": (None, [vp, vp, i32, f32, vp]),
        "or_gate_logit": (f32, [vp, vp, i32]),
        "or_sigmoid_gate": (C.c_uint16, [f32, f32]),
        "or_router_logits": (None, [vp, vp, i32, i32, i32, vp]),
        "or_dense": (i32, [P, P, P, i32, i32, i32, i32, i32, vp, vp, vp, f32]),
        "or_shared_expert": (i32, [P, P, P, i32, i32, i32, i32, i32, vp, vp, vp, f32]),
        "or_topk_token": (None, [vp, vp, i32, i32, vp, vp]),
        "or_moe_plan": (i32, [vp, i32, i32, i32, i32, vp]),
        "or_moe_route": (i32, [vp, vp, i32, i32, i32, i32, vp, vp, vp]),
        "or_seeded_sum": (f32, [f32, vp, vp, i32]),
        "or_moe_routed": (i32, [P, P, P, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
        "or_sandwich_tail": (None, [vp, vp, vp, i32, i32, f32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = _load(LIB)
    return _lib


@contextlib.contextmanager
def using(path: str):
    """Route every oracle call to another build of the oracle's source (a test
    plants a mistake in a copy of oracle.c this way and checks that a pin fails)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def qmat_struct(mat: dict, keep: list) -> QMat:
    """ctypes view of a gen-style matrix dict; arrays are kept alive in `keep`."""
    q = np.ascontiguousarray(mat["q"])
    s = np.ascontiguousarray(mat["s"])
    z = None if mat.get("z") is None else np.ascontiguousarray(mat["z"])
    keep += [q, s, z]
    return QMat(mat["fmt"], mat["n"], mat["k"], _p(q), _p(s), _p(z))


def plan_ints(m: int, k: int) -> int:
    return 1 + 2 * (m + 1) + 4 * m * k + 1


# ---------------------------------------------------------------------------
# steps


def bf16_round(v: float) -> int:
    return lib().or_bf16_round(float(v))


def bf16_value(b: int) -> float:
    return lib().or_bf16_value(int(b))


def dequant_matrix(mat: dict) -> np.ndarray:
    keep: list = []
    w = qmat_struct(mat, keep)
    out = np.empty((mat["n"], mat["k"]), dtype=np.float32)
    lib().or_dequant_matrix(C.byref(w), _p(out))
    return out


def gemv(mat: dict, x: np.ndarray) -> np.ndarray:
    keep: list = []
    w = qmat_struct(mat, keep)
    xd = _c(x, np.float64)
    y = np.empty(mat["n"], dtype=np.float32)
    lib().or_gemv(C.byref(w), _p(xd), _p(y))
    return y


def act(kind: int, g: float, u: float) -> float:
    return lib().or_act(kind, g, u)


def silu(v: float) -> float:
    return lib().or_silu(v)


def gelu_tanh(v: float) -> float:
    return lib().or_gelu_tanh(v)


def residual(x_bits: int, h: float) -> int:
    return lib().or_residual(int(x_bits), float(h))


def rmsnorm_row(h: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    h = _c(h, np.float32)
    w = _c(w_bits, np.uint16)
    out = np.empty(h.shape[0], dtype=np.uint16)
    lib().or_rmsnorm_row(_p(h), _p(w), h.shape[0], eps, _p(out))
    return out


def gate_logit(wg_bits: np.ndarray, x_bits: np.ndarray) -> float:
    wg = _c(wg_bits, np.uint16)
    x = _c(x_bits, np.uint16)
    return lib().or_gate_logit(_p(wg), _p(x), wg.shape[0])


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """logits [m][E] fp32 = x bf16 [m][hidden] times the router weight bf16 [E][hidden] (rows)."""
    x = _c(x_bits, np.uint16)
    w = _c(w_bits, np.uint16)
    m, hidden = x.shape
    E = w.shape[0]
    out = np.empty((m, E), dtype=np.float32)
    lib().or_router_logits(_p(x), _p(w), m, hidden, E, _p(out))
    return out


def sigmoid_gate(h: float, logit: float) -> int:
    return lib().or_sigmoid_gate(h, logit)


def seeded_sum(seed: float, w: np.ndarray, d: np.ndarray) -> float:
    w = _c(w, np.float32)
    d = _c(d, np.float32)
    return lib().or_seeded_sum(seed, _p(w), _p(d), w.shape[0])


# ---------------------------------------------------------------------------
# the four calls


def dense(ffn: dict, hidden: int, inter: int, act_kind: int, tail: int, x: np.ndarray,
          resid: np.ndarray | None, norm_w: np.ndarray | None = None, eps: float = 1e-6) -> np.ndarray:
    """Dense FFN half for x [m][hidden]; returns the bf16 output [m][hidden]."""
    keep: list = []
    g, u, d = (qmat_struct(ffn[n], keep) for n in ("gate", "up", "down"))
    x = _c(x, np.uint16)
    m = x.shape[0]
    out = np.array(resid, dtype=np.uint16, copy=True) if resid is not None else np.zeros((m, hidden), np.uint16)
    nw = _c(norm_w, np.uint16)
    rc = lib().or_dense(C.byref(g), C.byref(u), C.byref(d), hidden, inter, m, act_kind, tail, _p(x), _p(out),
                        _p(nw), eps)
    if rc != OK:
        raise ValueError(f"oracle dense: status {rc}")
    return out


def shared_expert(ffn: dict, hidden: int, inter: int, act_kind: int, tail: int, x: np.ndarray,
                  aux: np.ndarray | None, eps: float = 1e-6) -> np.ndarray:
    keep: list = []
    g, u, d = (qmat_struct(ffn[n], keep) for n in ("gate", "up", "down"))
    x = _c(x, np.uint16)
    m = x.shape[0]
    out = np.zeros((m, hidden), np.uint16)
    a = _c(aux, np.uint16)
    rc = lib().or_shared_expert(C.byref(g), C.byref(u), C.byref(d), hidden, inter, m, act_kind, tail, _p(x),
                                _p(out), _p(a), eps)
    if rc != OK:
        raise ValueError(f"oracle shared_expert: status {rc}")
    return out


def topk_token(logits: np.ndarray, k: int, scale: np.ndarray | None = None):
    lg = _c(logits, np.float32)
    sc = _c(scale, np.float32)
    ids = np.empty(k, np.int32)
    w = np.empty(k, np.float32)
    lib().or_topk_token(_p(lg), _p(sc), lg.shape[0], k, _p(ids), _p(w))
    return ids, w


def moe_plan(ids: np.ndarray, n_experts: int, cap: int):
    ids = _c(ids, np.int32)
    m, k = ids.shape
    plan = np.empty(plan_ints(m, k), np.int32)
    rc = lib().or_moe_plan(_p(ids), m, k, n_experts, cap, _p(plan))
    return rc, plan


def moe_route(logits: np.ndarray, k: int, cap: int, scale: np.ndarray | None = None):
    """Returns (status, ids [m][k], weights [m][k], plan)."""
    lg = _c(logits, np.float32)
    m, E = lg.shape
    sc = _c(scale, np.float32)
    ids = np.full((m, k), -1, np.int32)
    w = np.zeros((m, k), np.float32)
    plan = np.full(max(plan_ints(m, k), 1), -7, np.int32)
    rc = lib().or_moe_route(_p(lg), _p(sc), m, E, k, cap, _p(ids), _p(w), _p(plan))
    return rc, ids, w, plan


def moe_routed(experts: dict, n_experts: int, hidden: int, moe_inter: int, act_kind: int, x: np.ndarray,
               ids: np.ndarray, w: np.ndarray, seed: np.ndarray | None, resid: np.ndarray) -> np.ndarray:
    keep: list = []
    g, u, d = (qmat_struct(experts[n], keep) for n in ("gate", "up", "down"))
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    m, k = ids.shape
    sd = _c(seed, np.uint16)
    out = np.array(resid, dtype=np.uint16, copy=True)
    rc = lib().or_moe_routed(C.byref(g), C.byref(u), C.byref(d), n_experts, hidden, moe_inter, m, k, act_kind,
                             _p(x), _p(ids), _p(w), _p(sd), _p(out))
    if rc != OK:
        raise ValueError(f"oracle moe_routed: status {rc}")
    return out


def sandwich_tail(h1: np.ndarray, r: np.ndarray, w: np.ndarray, eps: float, resid: np.ndarray) -> np.ndarray:
    """The Gemma-style sandwich tail (or_sandwich_tail): resid + bf16(RMSNorm(h1 + r) * w), rounded to bf16."""
    h1 = _c(h1, np.uint16)
    r = _c(r, np.uint16)
    w = _c(w, np.uint16)
    m, n = h1.shape
    assert r.shape == (m, n) and w.shape == (n,)
    out = np.array(resid, dtype=np.uint16, copy=True)
    lib().or_sandwich_tail(_p(h1), _p(r), _p(w), m, n, eps, _p(out))
    return out


def moe_sandwich_layer(experts: dict, n_experts: int, hidden: int, moe_inter: int, act_kind: int, shared: dict,
                       shared_inter: int, shared_norm_w: np.ndarray, post_norm_w: np.ndarray, eps: float,
                       x: np.ndarray, logits: np.ndarray, scale: np.ndarray | None, k: int, cap: int,
                       resid: np.ndarray):
    """The Gemma-style routed layer ([qwen/moe_batch.rs] module doc, first bullet), step by step: router
    top-k with the per-expert scale and the plan; the shared branch with its own RMSNorm tail (h1, bf16);
    the routed half unseeded, its sum rounded to a bf16 row r (the routed call on a zero row); the
    sandwich tail.  Returns (status, ids, weights, plan, h1, r, resid_out)."""
    rc, ids, w, plan = moe_route(logits, k, cap, scale)
    if rc != OK:
        return rc, ids, w, plan, None, None, None
    h1 = shared_expert(shared, hidden, shared_inter, act_kind, TAIL_RMSNORM, x, shared_norm_w, eps)
    m = h1.shape[0]
    r = moe_routed(experts, n_experts, hidden, moe_inter, act_kind, x, ids, w, None, np.zeros((m, hidden), np.uint16))
    return rc, ids, w, plan, h1, r, sandwich_tail(h1, r, post_norm_w, eps, resid)


def plan_fields(plan: np.ndarray, m: int, k: int) -> dict:
    """Split a plan into its named arrays (views)."""
    o = 0
    out = {"n_sub": int(plan[0])}
    o = 1
    for name, size in (("sub_tok_begin", m + 1), ("sub_union_begin", m + 1), ("union_expert", m * k),
                       ("pair_slot", m * k), ("slot_pair_begin", m * k + 1), ("slot_pairs", m * k)):
        out[name] = plan[o:o + size]
        o += size
    return out
