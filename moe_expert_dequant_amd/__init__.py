"""Python binding of libffnq (quantized gated FFN + MoE routed half, gfx950).

A thin ctypes layer over the C ABI in include/ffnq.h: it marshals torch device
tensors into pointers and the current HIP stream, allocates workspaces with
torch, and raises on a non-OK status.  Every step of the computation runs in
the library's HIP kernels; there is no fallback path.  If libffnq.so has not
been built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from .build import LIB, build  # noqa: F401

FMT_INT8_ROW = 1
FMT_INT4_AFFINE_G64 = 2
FMT_INT8_ROW_TILED = 3
FMT_INT4_AFFINE_G64_TILED = 4
TILED = {FMT_INT8_ROW: FMT_INT8_ROW_TILED, FMT_INT4_AFFINE_G64: FMT_INT4_AFFINE_G64_TILED}
ACT_SILU = 1
ACT_GELU_TANH = 2
TAIL_NONE = 0
TAIL_RESIDUAL = 1
TAIL_RMSNORM = 2
TAIL_SIGMOID_GATE = 3

OK = 0
STATUS = {0: "OK", -1: "INVALID", -2: "UNSUPPORTED", -3: "CAPACITY", -4: "WORKSPACE", -5: "HIP"}
EXPORTS = ("ffnq_dense", "ffnq_dense_noalloc", "ffnq_shared_expert", "ffnq_router_logits", "ffnq_moe_route",
           "ffnq_moe_routed_batched",
           "ffnq_moe_layer", "ffnq_moe_layer_logits", "ffnq_moe_layer_sandwich", "ffnq_moe_routed_streamed",
           "ffnq_status_string", "ffnq_set_phase_events", "ffnq_stream_read", "ffnq_packed_bytes", "ffnq_pack")


def plan_ints(m: int, k: int) -> int:
    """int32 entries of a routing plan for m tokens at top-k (FFNQ_PLAN_INTS)."""
    return 1 + 2 * (m + 1) + 4 * m * k + 1


class FfnqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status})")
        self.status = status


class QMat(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("n", C.c_int32), ("k", C.c_int32),
                ("q", C.c_void_p), ("s", C.c_void_p), ("z", C.c_void_p)]


class Ffn(C.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat)]


class SlotCacheC(C.Structure):
    _fields_ = [("slots", C.c_void_p), ("slots_bytes", C.c_size_t), ("n_slots", C.c_int32),
                ("expert", C.c_void_p), ("last_use", C.c_void_p), ("clock", C.c_uint64), ("copied", C.c_uint64)]


_lib = None


def lib():
    """The loaded libffnq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"libffnq.so is not built ({LIB}); run __graft_entry__.build()")
        L = C.CDLL(LIB)
        vp, i32, f32, sz = C.c_void_p, C.c_int, C.c_float, C.POINTER(C.c_size_t)
        FP = C.POINTER(Ffn)
        L.ffnq_dense.argtypes = [FP, i32, i32, i32, i32, i32, vp, vp, vp, f32, vp, sz, vp]
        L.ffnq_shared_expert.argtypes = [FP, i32, i32, i32, i32, i32, vp, vp, vp, f32, vp, sz, vp]
        L.ffnq_dense_noalloc.argtypes = [FP, i32, i32, i32, i32, i32, vp, vp, vp, f32, vp]
        L.ffnq_router_logits.argtypes = [vp, vp, i32, i32, i32, vp, vp]
        L.ffnq_moe_route.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, C.c_size_t, vp]
        L.ffnq_moe_routed_batched.argtypes = [FP, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ffnq_moe_layer.argtypes = [FP, i32, i32, i32, i32, i32, i32, FP, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.ffnq_moe_layer_logits.argtypes = [FP, i32, i32, i32, i32, i32, i32, FP, i32, vp, vp, vp, vp, i32, vp, vp, vp,
                                            C.c_size_t, vp, vp, sz, vp]
        L.ffnq_moe_layer_sandwich.argtypes = [FP, i32, i32, i32, i32, i32, i32, FP, i32, vp, vp, f32, vp, vp, vp,
                                              i32, vp, vp, vp, C.c_size_t, vp, vp, sz, vp]
        L.ffnq_moe_routed_streamed.argtypes = [FP, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                               C.POINTER(SlotCacheC), vp, vp, sz, vp]
        for f in ("ffnq_dense", "ffnq_dense_noalloc", "ffnq_shared_expert", "ffnq_router_logits", "ffnq_moe_route",
                  "ffnq_moe_routed_batched",
                  "ffnq_moe_layer", "ffnq_moe_layer_logits", "ffnq_moe_layer_sandwich", "ffnq_moe_routed_streamed"):
            getattr(L, f).restype = C.c_int
        L.ffnq_status_string.argtypes = [C.c_int]
        L.ffnq_status_string.restype = C.c_char_p
        L.ffnq_set_phase_events.argtypes = [vp]
        L.ffnq_set_phase_events.restype = C.c_int
        L.ffnq_stream_read.argtypes = [vp, C.c_size_t, vp, vp]
        L.ffnq_stream_read.restype = C.c_int
        L.ffnq_packed_bytes.argtypes = [i32, i32, i32]
        L.ffnq_packed_bytes.restype = C.c_size_t
        L.ffnq_pack.argtypes = [C.POINTER(QMat), i32, vp, C.c_size_t, vp]
        L.ffnq_pack.restype = C.c_int
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def qmat(fmt: int, n: int, k: int, q, s, z=None) -> QMat:
    return QMat(fmt, n, k, _ptr(q), _ptr(s), _ptr(z))


def ffn_struct(mats: dict) -> Ffn:
    """mats: {gate, up, down} -> dict(fmt, n, k, q, s, z) with torch device tensors (or pointers)."""
    return Ffn(*(qmat(mats[n]["fmt"], mats[n]["n"], mats[n]["k"], mats[n]["q"], mats[n]["s"], mats[n].get("z"))
                 for n in ("gate", "up", "down")))


def _check(fn: str, rc: int):
    if rc != OK:
        raise FfnqError(fn, rc)


class PhaseEvents:
    """Four torch timing events that the library attaches to its kernel
    launches (ffnq_set_phase_events): start/stop of the gate/up kernel and
    start/stop of the down kernel.

    Use as a context manager around one call; afterwards (once the stream is
    synchronised) durations() gives (gate/up, down) kernel times in ms."""

    def __init__(self, stream=None):
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in self.ev:   # torch creates the underlying hipEvent_t on first record
            e.record(self.stream)
        self.arr = (C.c_void_p * 4)(*[e.cuda_event for e in self.ev])

    def __enter__(self):
        _check("ffnq_set_phase_events", lib().ffnq_set_phase_events(C.cast(self.arr, C.c_void_p)))
        return self

    def __exit__(self, *exc):
        lib().ffnq_set_phase_events(None)
        return False

    def durations(self):
        e = self.ev
        return e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3])


class Workspace:
    """A reusable device workspace that grows on demand (torch allocation)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf, self.buf.numel()


def _ws(fn, args, ws: Workspace | None):
    size = C.c_size_t(0)
    rc = fn(*args, None, C.byref(size), None)
    _check(fn.__name__, rc)
    ws = ws or Workspace()
    buf, n = ws.get(size.value)
    return buf, C.c_size_t(n)


def dense(ffn: Ffn, hidden: int, inter: int, m: int, act: int, tail: int, x, out, norm_w=None,
          eps: float = 1e-6, ws: Workspace | None = None, stream=None):
    """ffnq_dense: out is the residual stream (RESIDUAL, in/out) or the norm output (RMSNORM)."""
    L = lib()
    args = (C.byref(ffn), hidden, inter, m, act, tail, _ptr(x), _ptr(out), _ptr(norm_w), eps)
    buf, n = _ws(L.ffnq_dense, args, ws)
    _check("ffnq_dense", L.ffnq_dense(*args, _ptr(buf), C.byref(n), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 8 << 20   # FFNQ_NOALLOC_SCRATCH_BYTES


def dense_noalloc(ffn: Ffn, hidden: int, inter: int, m: int, act: int, tail: int, x, out, norm_w=None,
                  eps: float = 1e-6, stream=None):
    """ffnq_dense_noalloc: ffnq_dense on the library's own per-GPU scratch array (no workspace argument)."""
    _check("ffnq_dense_noalloc", lib().ffnq_dense_noalloc(C.byref(ffn), hidden, inter, m, act, tail, _ptr(x),
                                                          _ptr(out), _ptr(norm_w), eps, _stream(stream)))


def shared_expert(ffn: Ffn, hidden: int, inter: int, m: int, act: int, tail: int, x, h_out, aux=None,
                  eps: float = 1e-6, ws: Workspace | None = None, stream=None):
    L = lib()
    args = (C.byref(ffn), hidden, inter, m, act, tail, _ptr(x), _ptr(h_out), _ptr(aux), eps)
    buf, n = _ws(L.ffnq_shared_expert, args, ws)
    _check("ffnq_shared_expert", L.ffnq_shared_expert(*args, _ptr(buf), C.byref(n), _stream(stream)))


def router_logits(x, w, m: int, hidden: int, n_experts: int, logits, stream=None):
    """ffnq_router_logits: logits [m][E] fp32 = x bf16 [m][hidden] times the router weight bf16 [E][hidden]."""
    L = lib()
    _check("ffnq_router_logits", L.ffnq_router_logits(_ptr(x), _ptr(w), m, hidden, n_experts, _ptr(logits),
                                                      _stream(stream)))


def moe_route(logits, m: int, n_experts: int, top_k: int, slot_cap: int, topk_ids, topk_w, plan,
              expert_scale=None, stream=None):
    L = lib()
    nbytes = plan.numel() * plan.element_size() if hasattr(plan, "numel") else 0
    _check("ffnq_moe_route", L.ffnq_moe_route(_ptr(logits), _ptr(expert_scale), m, n_experts, top_k, slot_cap,
                                              _ptr(topk_ids), _ptr(topk_w), _ptr(plan), nbytes, _stream(stream)))


def moe_routed_batched(experts: Ffn, n_experts: int, hidden: int, moe_inter: int, m: int, top_k: int, act: int,
                       x, topk_ids, topk_w, plan, seed, resid, ws: Workspace | None = None, stream=None):
    L = lib()
    args = (C.byref(experts), n_experts, hidden, moe_inter, m, top_k, act, _ptr(x), _ptr(topk_ids), _ptr(topk_w),
            _ptr(plan), _ptr(seed), _ptr(resid))
    buf, n = _ws(L.ffnq_moe_routed_batched, args, ws)
    _check("ffnq_moe_routed_batched", L.ffnq_moe_routed_batched(*args, _ptr(buf), C.byref(n), _stream(stream)))


def moe_layer(experts: Ffn, n_experts: int, hidden: int, moe_inter: int, m: int, top_k: int, act: int,
              shared: Ffn | None, shared_inter: int, shared_gate, x, topk_ids, topk_w, plan, resid,
              ws: Workspace | None = None, stream=None):
    """ffnq_moe_layer: the gated shared expert (or none) and the routed half in one call."""
    L = lib()
    args = (C.byref(experts), n_experts, hidden, moe_inter, m, top_k, act,
            None if shared is None else C.byref(shared), shared_inter, _ptr(shared_gate), _ptr(x), _ptr(topk_ids),
            _ptr(topk_w), _ptr(plan), _ptr(resid))
    buf, n = _ws(L.ffnq_moe_layer, args, ws)
    _check("ffnq_moe_layer", L.ffnq_moe_layer(*args, _ptr(buf), C.byref(n), _stream(stream)))


def moe_layer_logits(experts: Ffn, n_experts: int, hidden: int, moe_inter: int, m: int, top_k: int, act: int,
                     shared: Ffn | None, shared_inter: int, shared_gate, x, logits, slot_cap: int, topk_ids, topk_w,
                     plan, resid, expert_scale=None, ws: Workspace | None = None, stream=None):
    """ffnq_moe_layer_logits: route the batch (writing topk_ids, topk_w, plan) and run the layer in one call."""
    L = lib()
    nbytes = plan.numel() * plan.element_size()
    args = (C.byref(experts), n_experts, hidden, moe_inter, m, top_k, act,
            None if shared is None else C.byref(shared), shared_inter, _ptr(shared_gate), _ptr(x), _ptr(logits),
            _ptr(expert_scale), slot_cap, _ptr(topk_ids), _ptr(topk_w), _ptr(plan), nbytes, _ptr(resid))
    buf, n = _ws(L.ffnq_moe_layer_logits, args, ws)
    _check("ffnq_moe_layer_logits", L.ffnq_moe_layer_logits(*args, _ptr(buf), C.byref(n), _stream(stream)))


def moe_layer_sandwich(experts: Ffn, n_experts: int, hidden: int, moe_inter: int, m: int, top_k: int, act: int,
                       shared: Ffn, shared_inter: int, shared_norm_w, post_norm_w, eps: float, x, logits,
                       slot_cap: int, topk_ids, topk_w, plan, resid, expert_scale=None, ws: Workspace | None = None,
                       stream=None):
    """ffnq_moe_layer_sandwich: the Gemma-style routed layer (route with the per-expert scale, the shared branch
    with its RMSNorm tail, the unseeded routed sum, the sandwich tail) in one call."""
    L = lib()
    nbytes = plan.numel() * plan.element_size()
    args = (C.byref(experts), n_experts, hidden, moe_inter, m, top_k, act, C.byref(shared), shared_inter,
            _ptr(shared_norm_w), _ptr(post_norm_w), eps, _ptr(x), _ptr(logits), _ptr(expert_scale), slot_cap,
            _ptr(topk_ids), _ptr(topk_w), _ptr(plan), nbytes, _ptr(resid))
    buf, n = _ws(L.ffnq_moe_layer_sandwich, args, ws)
    _check("ffnq_moe_layer_sandwich", L.ffnq_moe_layer_sandwich(*args, _ptr(buf), C.byref(n), _stream(stream)))


class SlotCache:
    """A device slot cache for routed experts streamed from host memory (ffnq_slot_cache): n_slots slots sized
    for one tiled INT4 expert of (hidden, moe_inter) each, with the host-side slot table kept between calls."""

    def __init__(self, n_slots: int, hidden: int, moe_inter: int, device="cuda"):
        import numpy as np
        gb = packed_bytes(FMT_INT4_AFFINE_G64_TILED, moe_inter, hidden)
        db = packed_bytes(FMT_INT4_AFFINE_G64_TILED, hidden, moe_inter)
        self.slots = torch.empty(n_slots * (2 * gb + db), dtype=torch.uint8, device=device)
        self.expert = np.full(n_slots, -1, np.int32)
        self.last_use = np.zeros(n_slots, np.uint64)
        self.c = SlotCacheC(self.slots.data_ptr(), self.slots.numel(), n_slots, self.expert.ctypes.data,
                            self.last_use.ctypes.data, 0, 0)

    @property
    def copied(self) -> int:
        return int(self.c.copied)


def host_experts(packed: dict) -> tuple:
    """Pinned host copies of tiled, packed expert tensors (as fq.pack returns them) and their Ffn struct."""
    h = {n: dict(packed[n], q=packed[n]["q"].cpu().pin_memory()) for n in ("gate", "up", "down")}
    return h, ffn_struct(h)


def moe_routed_streamed(host_ffn: Ffn, n_experts: int, hidden: int, moe_inter: int, m: int, top_k: int, act: int,
                        x, topk_ids, topk_w, plan, seed, resid, cache: SlotCache, ws: Workspace | None = None,
                        stream=None):
    """ffnq_moe_routed_streamed: the routed half with the experts in (pinned) host memory, each sub-batch's
    union copied into the cache's slots first."""
    L = lib()
    staging = torch.empty(plan_ints(m, top_k) + m * top_k, dtype=torch.int32).pin_memory()
    args = (C.byref(host_ffn), n_experts, hidden, moe_inter, m, top_k, act, _ptr(x), _ptr(topk_ids), _ptr(topk_w),
            _ptr(plan), _ptr(seed), _ptr(resid), C.byref(cache.c), staging.data_ptr())
    buf, n = _ws(L.ffnq_moe_routed_streamed, args, ws)
    _check("ffnq_moe_routed_streamed", L.ffnq_moe_routed_streamed(*args, _ptr(buf), C.byref(n), _stream(stream)))


def workspace_bytes(kind: str, *args) -> int:
    """Workspace query (ws == NULL) for 'dense', 'shared' or 'routed' with the call's leading arguments."""
    L = lib()
    fn = {"dense": L.ffnq_dense, "shared": L.ffnq_shared_expert, "routed": L.ffnq_moe_routed_batched,
          "layer": L.ffnq_moe_layer}[kind]
    size = C.c_size_t(0)
    _check(fn.__name__, fn(*args, None, C.byref(size), None))
    return size.value


def to_device(mat: dict, device="cuda") -> dict:
    """numpy matrix dict (fmt, n, k, q, s, z) -> the same with torch device tensors."""
    def t(a):
        if a is None:
            return None
        import numpy as np
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device)
        return torch.from_numpy(a).to(device)
    return dict(fmt=mat["fmt"], n=mat["n"], k=mat["k"], q=t(mat["q"]), s=t(mat["s"]), z=t(mat.get("z")))


def stream_read(buf, sink, stream=None) -> None:
    """ffnq_stream_read: a plain streaming read of the whole of `buf` (a CUDA
    tensor, 16-byte aligned, a multiple of 16 bytes), for measuring the read
    rate the GPU reaches; `sink` is a CUDA int32 tensor of at least one element."""
    _check("ffnq_stream_read", lib().ffnq_stream_read(C.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                                      C.c_void_p(sink.data_ptr()), C.c_void_p(_stream(stream))))


def packed_bytes(fmt: int, n: int, k: int) -> int:
    """Bytes of one n x k matrix (one expert) in the tiled form of `fmt` (0 if unsupported)."""
    return int(lib().ffnq_packed_bytes(fmt, n, k))


def pack(mat: dict, n_experts: int = 1, stream=None) -> dict:
    """Repack a row-major device matrix dict (fmt, n, k, q, s, z; n_experts
    stacked) into the tiled format the GPU streams fastest (ffnq_pack).
    Returns the tiled matrix dict (q = packed buffer, s = z = None)."""
    fmt, n, k = mat["fmt"], mat["n"], mat["k"]
    eb = packed_bytes(fmt, n, k)
    if eb == 0:
        raise FfnqError("ffnq_packed_bytes", -2)
    dst = torch.empty(eb * n_experts, dtype=torch.uint8, device=mat["q"].device)
    src = qmat(fmt, n, k, mat["q"], mat["s"], mat.get("z"))
    _check("ffnq_pack", lib().ffnq_pack(C.byref(src), n_experts, dst.data_ptr(), dst.numel(), _stream(stream)))
    return dict(fmt=TILED[fmt], n=n, k=k, q=dst, s=None, z=None)
