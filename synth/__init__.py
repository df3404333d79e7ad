"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random inputs only; it holds none of the method's arithmetic (no decoding,
no products, no routing). Blobs are built from uniform random bytes, which gives independent
uniform fields for every packed quant, scale and min of the three block formats, and the fp16
scale fields are overwritten with draws of the stated distributions rounded to fp16 (numpy's
float64 -> float16 conversion rounds to nearest even). Only the byte offsets of the fp16 fields
are format knowledge here:

  Q4_K (144 B / 256 weights): d at byte 0, dmin at byte 2.
  Q6_K (210 B / 256 weights): d at byte 208.
  Q8_0 (34 B / 32 weights):   d at byte 0; the int8 quants are drawn from U{-127..127}.
  Q5_K (176 B / 256 weights): d at byte 0, dmin at byte 2 (5-bit quants ~ U{0..31}).
  Q4_0 (18 B / 32 weights):   d at byte 0 (4-bit quants ~ U{0..15}).

Default distributions follow the workload descriptions: d ~ U(1e-3, 1e-2), dmin ~ U(0, 5e-3),
6-bit scales and mins ~ U{0..63}, 4-bit quants ~ U{0..15}, Q6_K int8 scales ~ U{-128..127} and
6-bit quants ~ U{0..63}, activations ~ N(0, 1) (drawn in fp64, rounded to fp32), router weights
~ N(0, 1/hidden) so that router logits are ~ N(0, 1).

Every generator is keyed by (seed, tag...), so each tensor is reproducible on its own.
"""
from __future__ import annotations

import hashlib

import numpy as np

Q4_K, Q6_K, Q8_0, Q5_K, Q4_0 = "q4_k", "q6_k", "q8_0", "q5_k", "q4_0"
BLOCK_WEIGHTS = {Q4_K: 256, Q6_K: 256, Q8_0: 32, Q5_K: 256, Q4_0: 32}
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, Q8_0: 34, Q5_K: 176, Q4_0: 18}
DEFAULT_SEED = 42


def row_bytes(t: str, k: int) -> int:
    return k // BLOCK_WEIGHTS[t] * BLOCK_BYTES[t]


def rng(seed: int, *tags) -> np.random.Generator:
    """A PCG64 stream keyed by the base seed and a stable hash of the tags."""
    h = hashlib.sha256(repr(tags).encode()).digest()
    words = [int.from_bytes(h[i:i + 4], "little") for i in range(0, 16, 4)]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed & 0xFFFFFFFF,
                                                                       *words])))


def _fp16_field(g: np.random.Generator, count: int, lo: float, hi: float,
                value: float | None) -> np.ndarray:
    if value is not None:
        v = np.full(count, value, np.float64)
    else:
        v = g.uniform(lo, hi, count)
    return v.astype(np.float16).view(np.uint8).reshape(count, 2)


def blob(t: str, g: np.random.Generator, n: int, k: int, *, d_range=(1e-3, 1e-2),
         dmin_range=(0.0, 5e-3), d_value: float | None = None,
         dmin_value: float | None = None, q8_range=(-127, 127)) -> np.ndarray:
    """A weight blob [n rows][k] of format t, as a flat uint8 array of n * row_bytes(t, k)."""
    bw, bb = BLOCK_WEIGHTS[t], BLOCK_BYTES[t]
    if k % bw:
        raise ValueError(f"k={k} is not a multiple of {bw}")
    nblk = n * (k // bw)
    raw = np.frombuffer(g.bytes(nblk * bb), np.uint8).copy().reshape(nblk, bb)
    if t in (Q4_K, Q5_K):
        raw[:, 0:2] = _fp16_field(g, nblk, *d_range, d_value)
        raw[:, 2:4] = _fp16_field(g, nblk, *dmin_range, dmin_value)
    elif t == Q4_0:
        raw[:, 0:2] = _fp16_field(g, nblk, *d_range, d_value)
    elif t == Q6_K:
        raw[:, 208:210] = _fp16_field(g, nblk, *d_range, d_value)
    elif t == Q8_0:
        raw[:, 0:2] = _fp16_field(g, nblk, *d_range, d_value)
        lo, hi = q8_range
        raw[:, 2:34] = g.integers(lo, hi + 1, (nblk, 32), dtype=np.int8).view(np.uint8)
    else:
        raise ValueError(t)
    return raw.reshape(-1)


def normal_f32(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape) * scale).astype(np.float32)


def ternary_f32(g: np.random.Generator, shape) -> np.ndarray:
    """Values in {-1, 0, 1}: with lattice weights every partial sum is exact in fp32."""
    return g.integers(-1, 2, shape).astype(np.float32)


def router_weights(g: np.random.Generator, n_experts: int, hidden: int) -> np.ndarray:
    return normal_f32(g, (n_experts, hidden), 1.0 / np.sqrt(hidden))


def zipf_router(g: np.random.Generator, n_experts: int, hidden: int, s: float = 1.0,
                spread: float = 0.5):
    """(router weights [E][H], offset v [H]) for routing traces with Zipf-like expert popularity.
    Activations are drawn as x = z + v with z ~ N(0, 1): the logit of expert e is then about
    N(0, 2) + b_e with b_e = spread * log(1 / rank_e^s), the ranks 1..E in a random order, so the
    experts are chosen with a popularity that falls off with their rank."""
    base = router_weights(g, n_experts, hidden).astype(np.float64)
    v = g.choice(np.array([-1.0, 1.0]), hidden)  # |v|^2 = hidden
    ranks = g.permutation(n_experts).astype(np.float64) + 1.0
    b = -spread * s * np.log(ranks)
    w = base + np.outer(b, v) / hidden
    return w.astype(np.float32), v.astype(np.float32)


# ---------------------------------------------------------------------------------------------
# Workload shapes (the five configurations; sizes only).
# ---------------------------------------------------------------------------------------------

LLAMA8B = dict(name="llama3-8b", hidden=4096, kv=1024, ffn=14336, layers=32)
LLAMA70B = dict(name="llama3-70b", hidden=8192, kv=1024, ffn=28672, layers=1)
MIXTRAL = dict(name="mixtral-8x7b", hidden=4096, ffn=14336, n_experts=8, top_k=2, shared=False)
DEEPSEEK = dict(name="deepseek-v3", hidden=7168, ffn=2048, n_experts=256, top_k=8, shared=True)


def dense_projections(shape: dict):
    """(name, n_out, k_in) of the seven projections of one dense decoder layer."""
    h, kv, f = shape["hidden"], shape["kv"], shape["ffn"]
    return [("q", h, h), ("k", kv, h), ("v", kv, h), ("o", h, h), ("gate", f, h), ("up", f, h),
            ("down", h, f)]


def moe_layer(shape: dict, t: str, seed: int = DEFAULT_SEED, tag: str = "moe") -> dict:
    """Host-side weights of one MoE layer: router [E][H] fp32 and (gate, up, down) blobs."""
    H, F, E = shape["hidden"], shape["ffn"], shape["n_experts"]
    wr = router_weights(rng(seed, tag, "router"), E, H)
    experts = []
    for e in range(E):
        experts.append(tuple(blob(t, rng(seed, tag, "expert", e, name), n, k)
                             for name, n, k in (("gate", F, H), ("up", F, H), ("down", H, F))))
    shared = None
    if shape.get("shared"):
        shared = tuple(blob(t, rng(seed, tag, "shared", name), n, k)
                       for name, n, k in (("gate", F, H), ("up", F, H), ("down", H, F)))
    return dict(router=wr, experts=experts, shared=shared)
