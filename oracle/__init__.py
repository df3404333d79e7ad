"""ctypes wrapper of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. It shares no code with the GPU library and never
touches a GPU: every argument is a host numpy array.

The C functions behind each wrapper, and the passages of the pages they follow, are documented
in ``tq_oracle.h`` / ``tq_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

Q4_K, Q6_K, Q8_0, Q5_K, Q4_0 = 1, 2, 3, 4, 5
TYPES = {"q4_k": Q4_K, "q6_k": Q6_K, "q8_0": Q8_0, "q5_k": Q5_K, "q4_0": Q4_0}

_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_p = C.c_void_p
_i64 = C.c_int64


def _declare(L: C.CDLL) -> None:
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = C.c_int
    L.orc_set_num_threads.argtypes = [C.c_int]
    L.orc_set_num_threads.restype = None
    L.orc_block_weights.argtypes = [C.c_int]
    L.orc_block_weights.restype = _i64
    L.orc_block_bytes.argtypes = [C.c_int]
    L.orc_block_bytes.restype = _i64
    L.orc_half_to_double.argtypes = [C.c_uint16]
    L.orc_half_to_double.restype = C.c_double
    L.orc_block_weight.argtypes = [C.c_int, _p, C.c_int]
    L.orc_block_weight.restype = C.c_double
    L.orc_block_fields.argtypes = [C.c_int, _p, _p, _p, _p, _p, _p]
    L.orc_block_fields.restype = C.c_int
    for name in ("orc_dequant_f64", "orc_dequant_f32", "orc_dequant_bf16"):
        getattr(L, name).argtypes = [C.c_int, _p, _i64, _i64, _p]
        getattr(L, name).restype = C.c_int
    L.orc_f32_to_bf16.argtypes = [C.c_float]
    L.orc_f32_to_bf16.restype = C.c_uint16
    for name in ("orc_gemv", "orc_gemv_f64x"):
        getattr(L, name).argtypes = [C.c_int, _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p]
        getattr(L, name).restype = C.c_int
    L.orc_swiglu_f32.argtypes = [_p, _p, _i64, _p]
    L.orc_swiglu_f64.argtypes = [_p, _p, _i64, _p]
    L.orc_router_logits.argtypes = [_p, _i64, _p, _i64, _i64, _p]
    for name in ("orc_topk_f32", "orc_topk_f64"):
        getattr(L, name).argtypes = [_p, _i64, _i64, _i64, C.c_int, _p, _p]
        getattr(L, name).restype = C.c_int
    L.orc_group.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p]
    L.orc_group.restype = C.c_int
    L.orc_moe.argtypes = [C.c_int, _i64, _i64, _p, _i64, _p, _p, _i64, _i64, _p, _p, _p, _i64,
                          _p, _p]
    L.orc_moe.restype = C.c_int
    L.orc_moe_bf16.argtypes = L.orc_moe.argtypes
    L.orc_moe_bf16.restype = C.c_int
    L.orc_moe_grouped.argtypes = L.orc_moe.argtypes
    L.orc_moe_grouped.restype = C.c_int
    L.orc_requant.argtypes = [C.c_int, _p, _p, _i64, _i64, _p]
    L.orc_requant.restype = C.c_int
    L.orc_quantize.argtypes = [C.c_int, _p, _i64, _i64, _p]
    L.orc_quantize.restype = C.c_int


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _type(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on."""
    lib().orc_set_num_threads(int(n))


def block_weights(t) -> int:
    return int(lib().orc_block_weights(_type(t)))


def block_bytes(t) -> int:
    return int(lib().orc_block_bytes(_type(t)))


def row_bytes(t, k: int) -> int:
    return k // block_weights(t) * block_bytes(t)


def half_to_double(h: int) -> float:
    return float(lib().orc_half_to_double(int(h)))


def block_fields(t, block: np.ndarray) -> dict:
    t = _type(t)
    block = np.ascontiguousarray(block, dtype=np.uint8)
    d = C.c_double()
    dmin = C.c_double()
    sc = np.zeros(16, np.int32)
    m = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    _check(lib().orc_block_fields(t, _ptr(block), C.byref(d), C.byref(dmin), _ptr(sc), _ptr(m),
                                  _ptr(q)), "block_fields")
    out = {"d": d.value}
    if t in (Q4_K, Q5_K):
        out.update(dmin=dmin.value, sc=sc[:8].copy(), m=m.copy(), q=q.copy())
    elif t == Q6_K:
        out.update(sc=sc.copy(), q=q.copy())
    else:
        out.update(q=q[:32].copy())
    return out


def dequant(t, w: np.ndarray, n: int, k: int, out: str = "f32") -> np.ndarray:
    """Dequantized [n][k]: 'f64' exact values, 'f32' one RNE rounding, 'bf16' uint16 patterns."""
    t = _type(t)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    assert w.size == n * row_bytes(t, k), "blob size does not match n x k"
    if out == "f64":
        y = np.empty((n, k), np.float64)
        _check(lib().orc_dequant_f64(t, _ptr(w), n, k, _ptr(y)), "dequant")
    elif out == "f32":
        y = np.empty((n, k), np.float32)
        _check(lib().orc_dequant_f32(t, _ptr(w), n, k, _ptr(y)), "dequant")
    elif out == "bf16":
        y = np.empty((n, k), np.uint16)
        _check(lib().orc_dequant_bf16(t, _ptr(w), n, k, _ptr(y)), "dequant")
    else:
        raise ValueError(out)
    return y


def f32_to_bf16(f: float) -> int:
    return int(lib().orc_f32_to_bf16(float(f)))


def gemv(t, w: np.ndarray, n: int, k: int, x: np.ndarray, rows=None):
    """(y, mag): y[b][r] = sum_k w[row_r][k] x[b][k] in fp64 and the sum of |products|.

    x is [batch][k] (fp32 or fp64); rows selects a subset of output rows (all when None).
    """
    t = _type(t)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    assert w.size == n * row_bytes(t, k), "blob size does not match n x k"
    x = np.asarray(x)
    x2 = x.reshape(-1, k)
    batch = x2.shape[0]
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = n if rows_a is None else rows_a.size
    y = np.empty((batch, nr), np.float64)
    mag = np.empty((batch, nr), np.float64)
    if x2.dtype == np.float64:
        x2 = np.ascontiguousarray(x2)
        rc = lib().orc_gemv_f64x(t, _ptr(w), n, k, _ptr(x2), batch, _ptr(rows_a),
                                 0 if rows_a is None else nr, _ptr(y), _ptr(mag))
    else:
        x2 = np.ascontiguousarray(x2, dtype=np.float32)
        rc = lib().orc_gemv(t, _ptr(w), n, k, _ptr(x2), batch, _ptr(rows_a),
                            0 if rows_a is None else nr, _ptr(y), _ptr(mag))
    _check(rc, "gemv")
    return y, mag


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.asarray(g)
    u = np.asarray(u)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.float64)
    if g.dtype == np.float64 or u.dtype == np.float64:
        g64 = np.ascontiguousarray(g, np.float64)
        u64 = np.ascontiguousarray(u, np.float64)
        lib().orc_swiglu_f64(_ptr(g64), _ptr(u64), g.size, _ptr(h))
    else:
        g32 = np.ascontiguousarray(g, np.float32)
        u32 = np.ascontiguousarray(u, np.float32)
        lib().orc_swiglu_f32(_ptr(g32), _ptr(u32), g.size, _ptr(h))
    return h


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    wr = np.ascontiguousarray(wr, np.float32)
    E, H = wr.shape
    x2 = x.reshape(-1, H)
    T = x2.shape[0]
    out = np.empty((T, E), np.float64)
    lib().orc_router_logits(_ptr(x2), T, _ptr(wr), E, H, _ptr(out))
    return out


def topk(logits: np.ndarray, k: int, renormalize: bool = True):
    """(ids int32 [T][k], weights fp64 [T][k]) from a logits tensor [T][E] (fp32 or fp64)."""
    lg = np.asarray(logits)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    wts = np.empty((T, k), np.float64)
    if lg.dtype == np.float64:
        lg = np.ascontiguousarray(lg)
        rc = lib().orc_topk_f64(_ptr(lg), T, E, k, int(renormalize), _ptr(ids), _ptr(wts))
    else:
        lg = np.ascontiguousarray(lg, np.float32)
        rc = lib().orc_topk_f32(_ptr(lg), T, E, k, int(renormalize), _ptr(ids), _ptr(wts))
    _check(rc, "topk")
    return ids, wts


def group(ids: np.ndarray, n_experts: int):
    """(counts [E], offsets [E+1], pairs [T*k]) int32 from ids [T][k]."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(n_experts, np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    pairs = np.empty(T * k, np.int32)
    _check(lib().orc_group(_ptr(ids), T, k, n_experts, _ptr(counts), _ptr(offsets), _ptr(pairs)),
           "group")
    return counts, offsets, pairs


class _Expert(C.Structure):
    _fields_ = [("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p)]


def moe(t, hidden: int, ffn: int, experts, shared, x: np.ndarray, ids: np.ndarray,
        weights: np.ndarray, tokens=None, bf16: bool = False, grouped: bool = True):
    """(y, mag) of the MoE FFN for a given routing, fp64 [n_tok][hidden].

    experts: list of (gate, up, down) uint8 blobs; shared: one such tuple or None.
    bf16: x, the weights and h rounded to bf16 first (orc_moe_bf16).
    grouped (fp32 operands only): orc_moe_grouped, the same bits as orc_moe (token by token)
    with the tokens of one expert taken together, which is what makes whole large layers
    affordable.
    """
    t = _type(t)
    keep = []

    def mk(e):
        arrs = [np.ascontiguousarray(a, dtype=np.uint8) for a in e]
        keep.extend(arrs)
        return _Expert(*[a.ctypes.data for a in arrs])

    arr = (_Expert * len(experts))(*[mk(e) for e in experts])
    sh = C.byref(mk(shared)) if shared is not None else None
    x = np.ascontiguousarray(x, np.float32).reshape(-1, hidden)
    T = x.shape[0]
    ids = np.ascontiguousarray(ids, np.int32)
    weights = np.ascontiguousarray(weights, np.float64)
    k = ids.shape[1]
    tok = None if tokens is None else np.ascontiguousarray(tokens, np.int64)
    nt = T if tok is None else tok.size
    y = np.empty((nt, hidden), np.float64)
    mag = np.empty((nt, hidden), np.float64)
    fn = lib().orc_moe_bf16 if bf16 else lib().orc_moe_grouped if grouped else lib().orc_moe
    rc = fn(t, hidden, ffn, arr, len(experts), sh, _ptr(x), T, k, _ptr(ids),
                       _ptr(weights), _ptr(tok), 0 if tok is None else nt, _ptr(y), _ptr(mag))
    _check(rc, "moe")
    return y, mag


def requant(t, blob: np.ndarray, w: np.ndarray, n: int, k: int) -> np.ndarray:
    t = _type(t)
    blob = np.ascontiguousarray(blob, np.uint8)
    w = np.ascontiguousarray(w, np.float64).reshape(n, k)
    out = np.empty_like(blob)
    _check(lib().orc_requant(t, _ptr(blob), _ptr(w), n, k, _ptr(out)), "requant")
    return out


def quantize(t, w: np.ndarray) -> np.ndarray:
    t = _type(t)
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    out = np.empty(n * row_bytes(t, k), np.uint8)
    _check(lib().orc_quantize(t, _ptr(w), n, k, _ptr(out)), "quantize")
    return out
