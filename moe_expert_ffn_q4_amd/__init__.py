"""Python binding of libtq (block-quantized decode GEMV and top-k MoE expert FFN on gfx950).

Argument marshalling only: every call forwards device pointers, sizes and the current HIP stream
to the C ABI declared in ``include/tq.h``; all computation happens in the library's kernels.
PyTorch supplies device memory and streams. The library must be built
(``python -m moe_expert_ffn_q4_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

Q4_K, Q6_K, Q8_0, Q5_K, Q4_0 = 1, 2, 3, 4, 5
TYPES = {"q4_k": Q4_K, "q6_k": Q6_K, "q8_0": Q8_0, "q5_k": Q5_K, "q4_0": Q4_0}
F32, BF16 = 0, 1
PATH_AUTO, PATH_F32, PATH_BF16_MFMA = 0, 1, 2
MOE_ROUTE, MOE_EXPERTS, MOE_COMBINE, MOE_ALL = 1, 2, 4, 7
STATUS = {0: "TQ_OK", 1: "TQ_EINVAL", 2: "TQ_ESHAPE", 3: "TQ_EALIGN", 4: "TQ_ENOSPC",
          5: "TQ_EUNSUPPORTED", 6: "TQ_EDEVICE"}


class TQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """The loaded libtq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtq.so not found at {LIB_PATH}; build it with "
                               "`python -m moe_expert_ffn_q4_amd.build`")
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


_vp, _i64, _int = C.c_void_p, C.c_int64, C.c_int


class Expert(C.Structure):
    _fields_ = [("gate", _vp), ("up", _vp), ("down", _vp)]


class MoeDesc(C.Structure):
    _fields_ = [("type", _int), ("hidden", _i64), ("ffn", _i64), ("n_experts", _i64),
                ("top_k", _i64), ("router_w", _vp), ("experts", _vp), ("experts_host", _vp),
                ("shared", Expert), ("renormalize", _int), ("experts_on_host", _int),
                ("copy_stream", _vp), ("path", _int), ("expert_cache", _vp)]


class ExpertCacheStats(C.Structure):
    _fields_ = [("calls", _i64), ("hits", _i64), ("misses", _i64), ("fallbacks", _i64),
                ("prefetched", _i64), ("prefetch_hits", _i64), ("bytes_copied", _i64)]


class ChainOp(C.Structure):
    _fields_ = [("nparts", _int), ("swiglu", _int), ("w", _vp * 4), ("n", _i64 * 4),
                ("y", _vp * 4), ("k", _i64), ("x", _vp)]


class MoeRouting(C.Structure):
    _fields_ = [("topk_ids", _vp), ("topk_w", _vp), ("logits", _vp), ("counts", _vp),
                ("offsets", _vp), ("pairs", _vp)]


def _declare(L: C.CDLL) -> None:
    L.tq_block_weights.argtypes = [_int]
    L.tq_block_weights.restype = _i64
    L.tq_block_bytes.argtypes = [_int]
    L.tq_block_bytes.restype = _i64
    L.tq_row_bytes.argtypes = [_int, _i64]
    L.tq_row_bytes.restype = _i64
    L.tq_last_error.argtypes = []
    L.tq_last_error.restype = C.c_char_p
    L.tq_dequant.argtypes = [_int, _vp, _i64, _i64, _int, _vp, _vp]
    L.tq_dequant.restype = _int
    L.tq_gemv_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
    L.tq_gemv_workspace_bytes.restype = C.c_size_t
    L.tq_gemv.argtypes = [_int, _vp, _i64, _i64, _vp, _i64, _vp, _vp, C.c_size_t, _vp]
    L.tq_gemv.restype = _int
    L.tq_gemv_noalloc.argtypes = [_int, _vp, _i64, _i64, _vp, _i64, _vp, _vp]
    L.tq_gemv_noalloc.restype = _int
    L.tq_swiglu.argtypes = [_vp, _vp, _i64, _vp, _vp]
    L.tq_swiglu.restype = _int
    L.tq_gemv_multi_workspace_bytes.argtypes = [_int, _int, C.POINTER(_i64), _i64, _i64]
    L.tq_gemv_multi_workspace_bytes.restype = C.c_size_t
    L.tq_gemv_multi.argtypes = [_int, _int, C.POINTER(_vp), C.POINTER(_i64), C.POINTER(_vp), _i64,
                                _vp, _i64, _vp, C.c_size_t, _vp]
    L.tq_gemv_multi.restype = _int
    L.tq_gemv_swiglu_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
    L.tq_gemv_swiglu_workspace_bytes.restype = C.c_size_t
    L.tq_gemv_swiglu.argtypes = [_int, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp, C.c_size_t, _vp]
    L.tq_gemv_swiglu.restype = _int
    L.tq_chain_plan_bytes.argtypes = [_int]
    L.tq_chain_plan_bytes.restype = C.c_size_t
    L.tq_chain_prepare.argtypes = [_int, C.POINTER(ChainOp), _int, _vp, C.c_size_t]
    L.tq_chain_prepare.restype = _int
    L.tq_chain_run.argtypes = [_vp, _vp]
    L.tq_chain_run.restype = _int
    L.tq_chain_status.argtypes = [_vp, _vp]
    L.tq_chain_status.restype = _int
    if hasattr(L, "tq_moe_ffn"):
        L.tq_moe_workspace_bytes.argtypes = [C.POINTER(MoeDesc), _i64]
        L.tq_moe_workspace_bytes.restype = C.c_size_t
        L.tq_moe_ffn.argtypes = [C.POINTER(MoeDesc), _vp, _i64, _vp, _vp, C.c_size_t,
                                 C.POINTER(MoeRouting), _vp]
        L.tq_moe_ffn.restype = _int
        L.tq_moe_ffn_stages.argtypes = [C.POINTER(MoeDesc), _vp, _i64, _vp, _vp, C.c_size_t,
                                        C.POINTER(MoeRouting), _int, _vp]
        L.tq_moe_ffn_stages.restype = _int
        L.tq_tuning_set.argtypes = [_int, _int]
        L.tq_tuning_set.restype = _int
        L.tq_tuning_get.argtypes = [_int]
        L.tq_tuning_get.restype = _int
        L.tq_expert_cache_slot_bytes.argtypes = [C.POINTER(MoeDesc)]
        L.tq_expert_cache_slot_bytes.restype = C.c_size_t
        L.tq_expert_cache_state_bytes.argtypes = [C.POINTER(MoeDesc), _i64]
        L.tq_expert_cache_state_bytes.restype = C.c_size_t
        L.tq_expert_cache_init.argtypes = [_vp, C.c_size_t, C.POINTER(MoeDesc), _i64, _i64, _vp,
                                           C.c_size_t]
        L.tq_expert_cache_init.restype = _int
        L.tq_expert_cache_stats_get.argtypes = [_vp, C.POINTER(ExpertCacheStats)]
        L.tq_expert_cache_stats_get.restype = _int
        L.tq_expert_cache_destroy.argtypes = [_vp]
        L.tq_expert_cache_destroy.restype = _int


def _check(rc: int) -> None:
    if rc != 0:
        raise TQError(rc, lib().tq_last_error().decode())


def _type(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def row_bytes(t, k: int) -> int:
    return int(lib().tq_row_bytes(_type(t), k))


def dequant(t, w: torch.Tensor, n: int, k: int, out_dtype: str = "f32", out=None, stream=None):
    """Dense [n][k] weights: fp32 values, or bf16 bit patterns as int16 ('bf16')."""
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32 if out_dtype == "f32" else torch.int16,
                          device=w.device)
    _check(lib().tq_dequant(_type(t), _ptr(w), n, k, F32 if out_dtype == "f32" else BF16,
                            _ptr(out), _stream(stream)))
    return out


_workspaces: dict = {}


def workspace(nbytes: int, device=None, purpose: str = "gemv") -> torch.Tensor:
    """A device scratch buffer of at least nbytes, reused across calls on one stream. The
    library takes workspaces with any contents; one buffer per (device, purpose) keeps calls
    that the caller runs on different streams from sharing one."""
    dev = torch.device(device if device is not None else "cuda")
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    key = (dev.type, dev.index, purpose)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = buf
    return buf


def gemv_workspace_bytes(t, n: int, k: int, batch: int) -> int:
    return int(lib().tq_gemv_workspace_bytes(_type(t), n, k, batch))


def gemv(t, w: torch.Tensor, n: int, k: int, x: torch.Tensor, out=None, ws=None, stream=None):
    """y[b][r] = sum_c W[r][c] x[b][c] for x of shape [batch, k] (or [k]); fp32.

    ws: workspace tensor (default: the shared per-device buffer); pass False for none.
    """
    x2 = x.reshape(-1, k)
    batch = x2.shape[0]
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(gemv_workspace_bytes(t, n, k, batch), x.device)
    wsp, wsn = (None, 0) if ws is False else (ws.data_ptr(), ws.numel() * ws.element_size())
    _check(lib().tq_gemv(_type(t), _ptr(w), n, k, _ptr(x2), batch, _ptr(out), wsp, wsn,
                         _stream(stream)))
    return out


GEMV_NOALLOC_MAX_BYTES = 16 << 20  # TQ_GEMV_NOALLOC_MAX_BYTES


def gemv_noalloc(t, w: torch.Tensor, n: int, k: int, x: torch.Tensor, out: torch.Tensor,
                 stream=None):
    """tq_gemv_noalloc: y = W x into the preallocated out [batch, n], with the library's own
    per-device scratch instead of a workspace (nothing is allocated)."""
    x2 = x.reshape(-1, k)
    _check(lib().tq_gemv_noalloc(_type(t), _ptr(w), n, k, _ptr(x2), x2.shape[0], _ptr(out),
                                 _stream(stream)))
    return out


def gemv_multi(t, ws_: list, ns: list, k: int, x: torch.Tensor, outs=None, ws=None, stream=None):
    """[W_p x for each p] in one call (matrices ws_[p] of ns[p] rows sharing x [batch, k])."""
    x2 = x.reshape(-1, k)
    batch, P = x2.shape[0], len(ns)
    if outs is None:
        outs = [torch.empty((batch, n), dtype=torch.float32, device=x.device) for n in ns]
    narr = (_i64 * P)(*ns)
    if ws is None:
        ws = workspace(int(lib().tq_gemv_multi_workspace_bytes(_type(t), P, narr, k, batch)),
                       x.device)
    _check(lib().tq_gemv_multi(_type(t), P, (_vp * P)(*[w.data_ptr() for w in ws_]), narr,
                               (_vp * P)(*[o.data_ptr() for o in outs]), k, x2.data_ptr(), batch,
                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))
    return outs


def gemv_swiglu(t, w_gate: torch.Tensor, w_up: torch.Tensor, n: int, k: int, x: torch.Tensor,
                out=None, ws=None, stream=None):
    """h = silu(W_gate x) * (W_up x), fp32 [batch, n]."""
    x2 = x.reshape(-1, k)
    batch = x2.shape[0]
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    if ws is None:
        need = int(lib().tq_gemv_swiglu_workspace_bytes(_type(t), n, k, batch))
        ws = workspace(need, x.device, "swiglu")
    _check(lib().tq_gemv_swiglu(_type(t), w_gate.data_ptr(), w_up.data_ptr(), n, k, x2.data_ptr(),
                                batch, out.data_ptr(), ws.data_ptr(),
                                ws.numel() * ws.element_size(), _stream(stream)))
    return out


def swiglu(g: torch.Tensor, u: torch.Tensor, out=None, stream=None):
    if out is None:
        out = torch.empty_like(g)
    _check(lib().tq_swiglu(_ptr(g), _ptr(u), g.numel(), _ptr(out), _stream(stream)))
    return out


class Chain:
    """A prepared chain of batch-1 Q4_K products (tq_chain_prepare / tq_chain_run), run as one
    persistent launch. ops: list of dicts with keys w (list of uint8 blobs), n (list of rows),
    y (list of fp32 output tensors), k, x (fp32 input tensor), and optionally swiglu=True (w =
    [gate, up], y = [h]). Op i reads its x only after op i-1 has stored all of its outputs. The
    tensors are kept alive here."""

    def __init__(self, t, ops: list, device=None):
        self.keep = []
        arr = (ChainOp * len(ops))()
        for i, op in enumerate(ops):
            c = arr[i]
            sw = bool(op.get("swiglu", False))
            c.nparts = len(op["w"])
            c.swiglu = int(sw)
            for p, w in enumerate(op["w"]):
                c.w[p] = w.data_ptr()
                c.n[p] = int(op["n"][p])
            for p, y in enumerate(op["y"]):
                c.y[p] = y.data_ptr()
            c.k = int(op["k"])
            c.x = op["x"].data_ptr()
            self.keep += list(op["w"]) + list(op["y"]) + [op["x"]]
        self.ops = arr
        nbytes = int(lib().tq_chain_plan_bytes(len(ops)))
        if nbytes == 0:
            raise ValueError(f"chain of {len(ops)} ops is out of range")
        dev = device if device is not None else ops[0]["x"].device
        self.plan = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _check(lib().tq_chain_prepare(_type(t), arr, len(ops), self.plan.data_ptr(), nbytes))

    def run(self, stream=None):
        _check(lib().tq_chain_run(self.plan.data_ptr(), _stream(stream)))

    def status(self, stream=None) -> int:
        """0 (TQ_OK) or TQ_EDEVICE if a run gave up a wait since the last call (the reason is in
        last_error())."""
        rc = int(lib().tq_chain_status(self.plan.data_ptr(), _stream(stream)))
        self.last_error = lib().tq_last_error().decode() if rc else ""
        return rc


class MoeLayer:
    """MoE layer for tq_moe_ffn: router weights, the expert blobs and an optional shared expert.
    Blobs are torch uint8 tensors (kept alive here). Routed experts on the device (a device
    table of blob pointers), or, when they are CPU tensors, in pinned host memory (the
    host-resident variant: the selected experts are copied per call on `copy_stream`, a
    torch.cuda.Stream, or on the call's stream when None). The shared expert is always on the
    device."""

    def __init__(self, t, hidden: int, ffn: int, router_w: torch.Tensor, experts, shared=None,
                 top_k: int = 2, renormalize: bool = True, path: int = PATH_AUTO,
                 copy_stream=None):
        self.blobs = [b for e in experts for b in e] + (list(shared) if shared else [])
        self.router_w = router_w
        E = len(experts)
        on_host = experts[0][0].device.type == "cpu"
        if on_host and not all(b.is_pinned() for e in experts for b in e):
            raise ValueError("host-resident expert blobs must be pinned (pin_memory=True)")
        self.copy_stream = copy_stream
        if on_host:
            self.host_table = (Expert * E)(*[Expert(*[b.data_ptr() for b in e]) for e in experts])
            self.table = None
        else:
            table = torch.tensor([[b.data_ptr() for b in e] for e in experts], dtype=torch.int64)
            self.table = table.to(router_w.device)
        self.desc = MoeDesc()
        self.desc.type = _type(t)
        self.desc.hidden, self.desc.ffn = hidden, ffn
        self.desc.n_experts, self.desc.top_k = E, top_k
        self.desc.router_w = router_w.data_ptr()
        self.desc.experts = None if on_host else self.table.data_ptr()
        self.desc.experts_host = C.addressof(self.host_table) if on_host else None
        if shared:
            self.desc.shared = Expert(*[b.data_ptr() for b in shared])
        self.desc.renormalize = int(renormalize)
        self.desc.experts_on_host = int(on_host)
        self.desc.copy_stream = copy_stream.cuda_stream if copy_stream is not None else None
        self.desc.path = path

    def attach_cache(self, slots: int, prefetch: int = 0) -> "ExpertCache":
        """A residency cache of `slots` device slots (host-resident experts only), used by every
        later call of this layer; returns it (its stats() count hits, misses, prefetches)."""
        self.cache = ExpertCache(self, slots, prefetch)
        self.desc.expert_cache = self.cache.state_ptr
        return self.cache

    def detach_cache(self) -> None:
        self.desc.expert_cache = None
        if getattr(self, "cache", None) is not None:
            self.cache.close()
            self.cache = None

    def workspace_bytes(self, tokens: int) -> int:
        """Bytes of workspace tq_moe_ffn needs (0 when the descriptor is invalid)."""
        return int(lib().tq_moe_workspace_bytes(C.byref(self.desc), tokens))

    def __call__(self, x: torch.Tensor, out=None, ws=None, routing: dict | None = None,
                 stream=None, stages: int = MOE_ALL):
        """y = MoE(x) for x [T, hidden] fp32. routing: dict of preallocated device tensors
        (topk_ids, topk_w, logits, counts, offsets, pairs) to receive the routing. stages: a
        subset of MOE_ROUTE | MOE_EXPERTS | MOE_COMBINE (tq_moe_ffn_stages); the same ws must
        then be passed to the calls that run the later stages."""
        T = x.shape[0]
        if out is None and stages & MOE_COMBINE:
            out = torch.empty_like(x)
        if ws is None:
            need = self.workspace_bytes(T)
            ws = workspace(need, x.device, "moe") if need else None
        r = None
        if routing is not None:
            r = MoeRouting(*[(routing[f].data_ptr() if routing.get(f) is not None else None)
                             for f, _ in MoeRouting._fields_])
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        rr = C.byref(r) if r is not None else None
        if stages == MOE_ALL:
            _check(lib().tq_moe_ffn(C.byref(self.desc), x.data_ptr(), T, out.data_ptr(),
                                    _ptr(ws), nbytes, rr, _stream(stream)))
        else:
            _check(lib().tq_moe_ffn_stages(C.byref(self.desc), x.data_ptr(), T, _ptr(out),
                                           _ptr(ws), nbytes, rr, stages, _stream(stream)))
        return out


class ExpertCache:
    """The device slots and host state of a residency cache (tq_expert_cache_init) for one
    host-resident MoE layer. Keeps its memory alive; close() releases the state's events."""

    def __init__(self, layer: MoeLayer, slots: int, prefetch: int = 0):
        L = lib()
        nstate = int(L.tq_expert_cache_state_bytes(C.byref(layer.desc), slots))
        nslot = int(L.tq_expert_cache_slot_bytes(C.byref(layer.desc)))
        if not nstate or not nslot:
            raise TQError(1, "invalid layer descriptor or slot count for an expert cache")
        self._state = (C.c_char * (nstate + 64))()  # host memory, 64-byte aligned below
        base = C.addressof(self._state)
        self.state_ptr = (base + 63) & ~63
        self.slots = torch.empty(slots * nslot, dtype=torch.uint8, device=layer.router_w.device)
        _check(L.tq_expert_cache_init(self.state_ptr, nstate, C.byref(layer.desc), slots, prefetch,
                                      self.slots.data_ptr(), self.slots.numel()))
        self.open = True

    def stats(self) -> dict:
        s = ExpertCacheStats()
        _check(lib().tq_expert_cache_stats_get(self.state_ptr, C.byref(s)))
        return {f: getattr(s, f) for f, _ in ExpertCacheStats._fields_}

    def close(self) -> None:
        if self.open:
            torch.cuda.synchronize()
            _check(lib().tq_expert_cache_destroy(self.state_ptr))
            self.open = False


# Tuning knobs (TQ_KNOB_* of tq.h), for tests and tuning sweeps: the defaults are the production
# choices; an override changes which kernel or launch shape a call takes.
KNOBS = {
    "gemv_target_wg": 0,
    "gemv_max_waves": 1,
    "gemv_klane": 2,
    "kl_groups": 3,
    "kl_rows": 4,
    "kl_target_waves": 5,
    "gemm_f32m": 6,
    "f32m_upk": 7,
    "gemv_i8": 8,
    "i8_upk": 9,
    "moe_qmm": 10,
    "qmm_nt": 11,
    "moe_nt": 12,
    "router_kl": 13,
    "router_steps": 14,
    "router_mf": 15,
    "group1": 16,
    "combine4": 17,
    "fuse_combine": 18,
    "gemv_qmm": 19,
    "qmm_upk": 20,
    "qmm_inline": 21,
    "qmm_inline_upk": 22,
    "qmm_inline_nr": 23,
    "gemv_mf": 24,
    "mf_wgs": 25,
    "mf_kb": 26,
    "mf_deep": 27,
    "moe_mf": 28,
    "moe_route1": 29,
    "f32m_t4": 30,
    "mf_ksplit": 31,
}


def set_knob(name: str, value: int) -> None:
    """Override a tuning knob process-wide (value < 0: back to the default)."""
    _check(lib().tq_tuning_set(KNOBS[name], int(value)))


def get_knob(name: str) -> int:
    """The knob's override, or -1 while its default is in effect."""
    return int(lib().tq_tuning_get(KNOBS[name]))


class knobs:
    """Context manager: knobs(gemv_i8=2, kl_rows=2) sets overrides and restores the previous
    values on exit."""

    def __init__(self, **values):
        self.values = values

    def __enter__(self):
        self.old = {k: get_knob(k) for k in self.values}
        for k, v in self.values.items():
            set_knob(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.old.items():
            set_knob(k, v)
        return False
