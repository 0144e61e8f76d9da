"""Seeded synthetic inputs for the quantized gated FFN and the MoE routed half.

This module produces INPUTS only -- weights, activations, router logits -- as
host numpy arrays.  It computes no part of the method (no dequantisation, no
dot products, no activation, routing or plan) and is the only code that the
CPU oracle and the HIP path share.

Random numbers come from a counter-based SplitMix64 stream: element i of the
stream with key K is mix(K + (i + 1) * 0x9E3779B97F4A7C15), where mix is the
SplitMix64 output function (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014).  Each tensor gets its own key derived from
(config seed, tensor id), so any tensor can be regenerated on its own.
Uniforms use the top 53 bits; normals use the Box-Muller transform in double;
bf16 values are rounded from fp32 to nearest even.

Workload recipe (shapes and distributions of the pages' model families):
  INT8 per-row:     q ~ U{-127..127}, s = 1/(127*sqrt(K)) fp32 (the workloads' recipe);
                    row_scales=True draws s_n = U(0.5,1.5)/(127*sqrt(K)) per row instead,
                    so that a test sees which row's scale a kernel applies
  INT4 affine g64:  codes ~ U{0..15}, s = bf16(U(0.5,1.5)/(8*sqrt(K))), z = bf16(U(6,9))
  x, residual:      bf16(N(0,1)), token-major [M][hidden]
  RMSNorm weight:   bf16(U(0.8,1.2))
  router logits:    per token, E iid N(0,1) in double, sorted, + 2e-4*rank, scattered
                    back (keeps the iid order, makes every fp32 gap >= 1e-4)
  shared gate vec:  bf16(N(0,1)/sqrt(hidden))
"""
from __future__ import annotations

import math

import numpy as np

FMT_INT8_ROW = 1
FMT_INT4_AFFINE_G64 = 2
ACT_SILU = 1
ACT_GELU_TANH = 2
TAIL_NONE = 0
TAIL_RESIDUAL = 1
TAIL_RMSNORM = 2
TAIL_SIGMOID_GATE = 3

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def tensor_key(seed: int, tensor_id: int) -> int:
    """Key of one tensor's stream, from the config seed and a tensor id."""
    z = np.array([(seed * 0x100000001 + tensor_id * 0x10001 + 1) & ((1 << 64) - 1)], dtype=np.uint64)
    return int(_mix(z)[0])


def stream_u64(key: int, n: int) -> np.ndarray:
    """n uint64 draws of the counter-based stream with the given key."""
    out = np.empty(n, dtype=np.uint64)
    k = np.uint64(key)
    with np.errstate(over="ignore"):
        for a in range(0, n, _CHUNK):
            b = min(n, a + _CHUNK)
            i = np.arange(a + 1, b + 1, dtype=np.uint64)
            out[a:b] = _mix(k + i * _GOLDEN)
    return out


def uniform(key: int, n: int) -> np.ndarray:
    """n doubles, uniform on [0, 1)."""
    return (stream_u64(key, n) >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))


def normal(key: int, n: int) -> np.ndarray:
    """n standard normal doubles (Box-Muller on pairs of uniforms)."""
    m = (n + 1) // 2
    u = uniform(key, 2 * m)
    r = np.sqrt(-2.0 * np.log1p(-u[0::2]))
    t = 2.0 * math.pi * u[1::2]
    out = np.empty(2 * m)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out[:n]


def random_bytes(key: int, n: int) -> np.ndarray:
    """n uniform random bytes."""
    return stream_u64(key, (n + 7) // 8).view(np.uint8)[:n].copy()


def bf16_bits(a) -> np.ndarray:
    """Round values to bf16 (via fp32, ties to even); returns uint16 bit patterns."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# quantized matrices


def qmat(fmt: int, n: int, k: int, key: int, experts: int = 0, row_scales: bool = False) -> dict:
    """A random quantized matrix [n][k] (or a stack of `experts` of them).

    Returns {fmt, n, k, q, s, z} with numpy arrays laid out as the library's
    formats define (leading expert dimension when experts > 0).  INT8 row
    scales are the constant 1/(127*sqrt(k)) unless row_scales, which draws one
    per row from U(0.5,1.5)/(127*sqrt(k))."""
    e = max(1, experts)
    lead = (experts,) if experts else ()
    if fmt == FMT_INT8_ROW:
        assert k % 64 == 0
        cnt = e * n * k
        raw = stream_u64(tensor_key(key, 1), (cnt + 3) // 4).view(np.uint16)[:cnt]
        q = ((raw.astype(np.int32) % 255) - 127).astype(np.int8).reshape(lead + (n, k))
        if row_scales:
            s = ((0.5 + uniform(tensor_key(key, 2), e * n)) / (127.0 * math.sqrt(k))).astype(np.float32)
            s = s.reshape(lead + (n,))
        else:
            s = np.full(lead + (n,), 1.0 / (127.0 * math.sqrt(k)), dtype=np.float32)
        return dict(fmt=fmt, n=n, k=k, q=q, s=s, z=None)
    if fmt == FMT_INT4_AFFINE_G64:
        assert k % 64 == 0
        q = random_bytes(tensor_key(key, 1), e * n * k // 2).reshape(lead + (n, k // 2))
        g = e * n * (k // 64)
        s = bf16_bits((0.5 + uniform(tensor_key(key, 2), g)) / (8.0 * math.sqrt(k))).reshape(lead + (n, k // 64))
        z = bf16_bits(6.0 + 3.0 * uniform(tensor_key(key, 3), g)).reshape(lead + (n, k // 64))
        return dict(fmt=fmt, n=n, k=k, q=q, s=s, z=z)
    raise ValueError(f"unknown format {fmt}")


def ffn(fmt_gu: int, fmt_down: int, hidden: int, inter: int, key: int, experts: int = 0,
        row_scales: bool = False) -> dict:
    """gate/up [inter][hidden] and down [hidden][inter]."""
    return dict(
        gate=qmat(fmt_gu, inter, hidden, tensor_key(key, 11), experts, row_scales),
        up=qmat(fmt_gu, inter, hidden, tensor_key(key, 12), experts, row_scales),
        down=qmat(fmt_down, hidden, inter, tensor_key(key, 13), experts, row_scales),
    )


def act_rows(key: int, m: int, width: int) -> np.ndarray:
    """bf16(N(0,1)) activations [m][width] as uint16 bits."""
    return bf16_bits(normal(key, m * width)).reshape(m, width)


def norm_weight(key: int, width: int) -> np.ndarray:
    return bf16_bits(0.8 + 0.4 * uniform(key, width))


def gate_vector(key: int, width: int) -> np.ndarray:
    return bf16_bits(normal(key, width) / math.sqrt(width))


def router_logits(key: int, m: int, n_experts: int, gap: float = 2e-4) -> np.ndarray:
    """fp32 logits [m][E]: iid N(0,1) per token with adjacent gaps widened by `gap`."""
    raw = normal(key, m * n_experts).reshape(m, n_experts)
    out = np.empty((m, n_experts), dtype=np.float32)
    for t in range(m):
        order = np.argsort(raw[t], kind="stable")
        v = np.empty(n_experts)
        v[order] = raw[t][order] + gap * np.arange(n_experts)
        out[t] = v.astype(np.float32)
        srt = np.sort(out[t].astype(np.float64))
        assert n_experts < 2 or np.min(np.diff(srt)) >= 1e-4, "logit gap below 1e-4"
    return out


# ---------------------------------------------------------------------------
# the five workloads (shapes of the pages' model families)

CONFIGS = {
    0: dict(name="dense-int8-256x704", kind="dense", hidden=256, inter=704, fmt=FMT_INT8_ROW,
            act=ACT_SILU, tail=TAIL_RESIDUAL, ms=(1, 4)),
    1: dict(name="llama3-8b-ffn-int4", kind="dense", hidden=4096, inter=14336, fmt=FMT_INT4_AFFINE_G64,
            act=ACT_SILU, tail=TAIL_RESIDUAL, ms=(1, 4)),
    2: dict(name="gemma-shared-int8-rmsnorm", kind="shared", hidden=2816, inter=11264, fmt=FMT_INT8_ROW,
            act=ACT_GELU_TANH, tail=TAIL_RMSNORM, eps=1e-6, ms=(1, 4, 8)),
    3: dict(name="qwen3-moe-int4", kind="moe", hidden=2048, n_experts=128, moe_inter=768, top_k=8,
            shared_inter=5632, fmt=FMT_INT4_AFFINE_G64, act=ACT_SILU, cap=32, ms=(1, 2, 4)),
    4: dict(name="mixtral-8x7b-int4", kind="moe", hidden=4096, n_experts=8, moe_inter=14336, top_k=2,
            shared_inter=0, fmt=FMT_INT4_AFFINE_G64, act=ACT_SILU, cap=32, ms=(1, 64)),
    # the Gemma-style routed layer (sandwich tail): the shared branch is workload
    # 2's INT8 FFN with its RMSNorm; the routed experts' shape (128 experts, top 8,
    # 768 wide, INT4) is this generator's own choice -- the pages give none
    5: dict(name="gemma-style-moe-sandwich", kind="sandwich", hidden=2816, n_experts=128, moe_inter=768, top_k=8,
            shared_inter=11264, shared_fmt=FMT_INT8_ROW, fmt=FMT_INT4_AFFINE_G64, act=ACT_GELU_TANH, eps=1e-6,
            cap=32, ms=(1, 4)),
}


def dense_inputs(hidden: int, inter: int, m: int, fmt: int, seed: int, fmt_down: int | None = None,
                 row_scales: bool = False) -> dict:
    """Weights, x and residual of one dense FFN layer (row_scales: see qmat)."""
    return dict(
        ffn=ffn(fmt, fmt if fmt_down is None else fmt_down, hidden, inter, tensor_key(seed, 100),
                row_scales=row_scales),
        x=act_rows(tensor_key(seed, 101), m, hidden),
        resid=act_rows(tensor_key(seed, 102), m, hidden),
        norm_w=norm_weight(tensor_key(seed, 103), hidden),
        gate_vec=gate_vector(tensor_key(seed, 104), hidden),
    )


def moe_inputs(hidden: int, n_experts: int, moe_inter: int, m: int, seed: int,
               shared_inter: int = 0, fmt: int = FMT_INT4_AFFINE_G64) -> dict:
    """Stacked experts, optional shared expert, x, residual and router logits."""
    d = dict(
        experts=ffn(fmt, fmt, hidden, moe_inter, tensor_key(seed, 200), experts=n_experts),
        x=act_rows(tensor_key(seed, 201), m, hidden),
        resid=act_rows(tensor_key(seed, 202), m, hidden),
        logits=router_logits(tensor_key(seed, 203), m, n_experts),
    )
    if shared_inter:
        d["shared"] = ffn(fmt, fmt, hidden, shared_inter, tensor_key(seed, 204))
        d["gate_vec"] = gate_vector(tensor_key(seed, 205), hidden)
    return d


def sandwich_inputs(hidden: int, n_experts: int, moe_inter: int, m: int, seed: int, shared_inter: int,
                    shared_fmt: int = FMT_INT8_ROW, fmt: int = FMT_INT4_AFFINE_G64, row_scales: bool = False) -> dict:
    """The Gemma-style routed layer: moe_inputs' experts, x, residual and logits, a
    shared FFN, the two norm weights and a per-expert router scale U(0.5, 1.5)."""
    d = moe_inputs(hidden, n_experts, moe_inter, m, seed, 0, fmt)
    d["shared"] = ffn(shared_fmt, shared_fmt, hidden, shared_inter, tensor_key(seed, 204), row_scales=row_scales)
    d["shared_norm_w"] = norm_weight(tensor_key(seed, 206), hidden)
    d["post_norm_w"] = norm_weight(tensor_key(seed, 207), hidden)
    d["expert_scale"] = (0.5 + uniform(tensor_key(seed, 208), n_experts)).astype(np.float32)
    return d


def config_inputs(c: int, m: int, row_scales: bool = False) -> dict:
    """Inputs of workload c at m tokens; the seed of workload c is c.  row_scales
    replaces the INT8 workloads' constant row scale by per-row draws (qmat)."""
    cfg = CONFIGS[c]
    if cfg["kind"] in ("dense", "shared"):
        return dense_inputs(cfg["hidden"], cfg["inter"], m, cfg["fmt"], seed=c, row_scales=row_scales)
    if cfg["kind"] == "sandwich":
        return sandwich_inputs(cfg["hidden"], cfg["n_experts"], cfg["moe_inter"], m, seed=c,
                               shared_inter=cfg["shared_inter"], shared_fmt=cfg["shared_fmt"], fmt=cfg["fmt"],
                               row_scales=row_scales)
    return moe_inputs(cfg["hidden"], cfg["n_experts"], cfg["moe_inter"], m, seed=c,
                      shared_inter=cfg["shared_inter"], fmt=cfg["fmt"])


def expert_slice(mat: dict, e: int) -> dict:
    """Matrix e of a stacked expert tensor."""
    return dict(fmt=mat["fmt"], n=mat["n"], k=mat["k"], q=mat["q"][e], s=mat["s"][e],
                z=None if mat["z"] is None else mat["z"][e])
