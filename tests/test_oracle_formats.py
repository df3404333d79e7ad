"""Pins of the oracle's block decoding (CPU only).

What pins what:
  * fp16 -> fp64: all 65,536 bit patterns against numpy's own float16 conversion.
  * Layouts: hand-built blocks with hand-derived values (tests/golden/kquant_blocks.txt) and two
    byte-pattern blocks whose values follow in closed form from the construction (below).
  * Rounding: fp32 output equals the single nearest-even rounding of the exact value; bf16 output
    against torch's float32 -> bfloat16 conversion.
  * Round trips: re-deriving the quants of a random blob from its own decoded values and scale
    fields gives the blob back; the from-scratch quantizer stays within one grid step.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.golden_io import load_blocks


def test_half_to_double_exhaustive():
    L = oracle.lib()
    pats = np.arange(65536, dtype=np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([L.orc_half_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("fx", load_blocks(), ids=lambda f: f["name"])
def test_golden_block(fx):
    t = fx["type"]
    k = synth.BLOCK_WEIGHTS[t]
    w64 = oracle.dequant(t, fx["block"], 1, k, out="f64")[0]
    w32 = oracle.dequant(t, fx["block"], 1, k, out="f32")[0]
    exp = fx["expect"]
    assert np.array_equal(w64, exp), (w64, exp)
    assert np.array_equal(w32.astype(np.float64), exp)
    assert np.array_equal(np.signbit(w32), np.signbit(exp)), "sign of zero"
    for i in (0, k // 3, k - 1):
        assert oracle.lib().orc_block_weight(oracle.TYPES[t], fx["block"].ctypes.data, i) == exp[i]


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_0"])
def test_row_decode_equals_per_weight_definition(t):
    """Rows are decoded a block at a time; every value equals orc_block_weight's, bit for bit."""
    n, k = 3, 1024
    blob = synth.blob(t, synth.rng(41, "rowdec", t), n, k)
    w64 = oracle.dequant(t, blob, n, k, out="f64")
    bw, bb = synth.BLOCK_WEIGHTS[t], synth.BLOCK_BYTES[t]
    L, tt = oracle.lib(), oracle.TYPES[t]
    rows = blob.reshape(n, -1)
    for r in range(n):
        for c in range(k):
            blk = np.ascontiguousarray(rows[r, (c // bw) * bb:(c // bw + 1) * bb])
            assert L.orc_block_weight(tt, blk.ctypes.data, c % bw) == w64[r, c], (r, c)


def test_q4k_fields_of_scale_fixture():
    fx = {f["name"]: f for f in load_blocks()}["q4k_scales_q15"]
    fl = oracle.block_fields("q4_k", fx["block"])
    assert fl["d"] == 0.5 and fl["dmin"] == 0.25
    assert list(fl["sc"]) == [1, 2, 3, 4, 17, 33, 49, 63]
    assert list(fl["m"]) == [0, 5, 10, 15, 20, 40, 60, 63]
    assert set(fl["q"]) == {15}


def test_q4k_quant_order_pattern():
    """d = 1, dmin = 0, all sc = 1, m = 0; quant byte b = (b & 15) | (15 - b // 8) << 4.

    With c = i // 64 and r = i % 64, weight i reads the low nibble of byte 32c + r when r < 32,
    which is r % 16, and the high nibble of byte 32c + r - 32 otherwise, which is
    15 - 4c - (r - 32) // 8.  Region offsets and within-region order both show up.
    """
    blk = np.zeros(144, np.uint8)
    blk[0:2] = [0x00, 0x3C]
    blk[4:16] = [1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1]
    b = np.arange(128)
    blk[16:] = (b & 15) | ((15 - b // 8) << 4)
    i = np.arange(256)
    c, r = i // 64, i % 64
    exp = np.where(r < 32, r % 16, 15 - 4 * c - (r - 32) // 8).astype(np.float64)
    got = oracle.dequant("q4_k", blk, 1, 256, out="f64")[0]
    assert np.array_equal(got, exp)


def test_q6k_nibble_pattern():
    """d = 1, all scales 1, qh = 0 (high bits 0); ql byte b = (b % 16) | (15 - b % 16) << 4.

    For 32-weight group g of a half, l = i % 32: groups 0, 1 take low nibbles -> q = l % 16,
    groups 2, 3 take high nibbles -> q = 15 - l % 16; w = q - 32.
    """
    blk = np.zeros(210, np.uint8)
    b = np.arange(128)
    blk[0:128] = (b % 16) | ((15 - b % 16) << 4)
    blk[192:208] = 1
    blk[208:210] = [0x00, 0x3C]
    i = np.arange(256)
    g, l = (i % 128) // 32, i % 32
    exp = np.where(g < 2, l % 16, 15 - l % 16).astype(np.float64) - 32
    got = oracle.dequant("q6_k", blk, 1, 256, out="f64")[0]
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_0"])
def test_f32_is_one_rounding_of_exact(t):
    g = synth.rng(7, "f32-rounding", t)
    n, k = 6, 512
    w = synth.blob(t, g, n, k)
    w64 = oracle.dequant(t, w, n, k, out="f64")
    w32 = oracle.dequant(t, w, n, k, out="f32")
    assert np.array_equal(w64.astype(np.float32), w32)
    if t not in ("q4_k", "q5_k"):
        # d*sc*(q-32), d*q and d*(q-8) carry at most 23 significant bits: exact in fp32
        assert np.array_equal(w32.astype(np.float64), w64)


def test_bf16_matches_torch_rne():
    g = synth.rng(3, "bf16")
    vals = np.concatenate([
        g.standard_normal(4096).astype(np.float32),
        # exact ties between two bf16 neighbours: low 16 bits 0x8000, both parities
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000, 0x00018000],
                 np.uint32).view(np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(v) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_0"])
def test_requant_round_trip(t):
    """Quants re-derived from a blob's own decoded values and scale fields equal the blob's."""
    g = synth.rng(11, "requant", t)
    n, k = 8, 1024
    w = synth.blob(t, g, n, k)
    vals = oracle.dequant(t, w, n, k, out="f64")
    back = oracle.requant(t, w, vals, n, k)
    bb, bw = synth.BLOCK_BYTES[t], synth.BLOCK_WEIGHTS[t]
    wb, bk = w.reshape(-1, bb), back.reshape(-1, bb)
    for blk in range(wb.shape[0]):
        f0 = oracle.block_fields(t, wb[blk])
        f1 = oracle.block_fields(t, bk[blk])
        if t in ("q4_k", "q5_k"):
            assert np.array_equal(wb[blk, :16], bk[blk, :16])
            live = np.repeat(f0["sc"] != 0, 32) & (f0["d"] != 0)
        elif t == "q6_k":
            assert np.array_equal(wb[blk, 192:], bk[blk, 192:])
            live = np.repeat(f0["sc"] != 0, 16) & (f0["d"] != 0)
        else:
            assert np.array_equal(wb[blk, :2], bk[blk, :2])
            live = np.full(bw, f0["d"] != 0)
        assert np.array_equal(f0["q"][live], f1["q"][live])
    # fp32-rounded values round-trip as well (half a grid step is far above fp32 rounding)
    vals32 = oracle.dequant(t, w, n, k, out="f32").astype(np.float64)
    back32 = oracle.requant(t, w, vals32, n, k)
    assert np.array_equal(back32, back)


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_0"])
def test_quantizer_error_within_one_step(t):
    g = synth.rng(5, "quantize", t)
    n, k = 16, 512
    data = synth.normal_f32(g, (n, k))
    blob = oracle.quantize(t, data)
    back = oracle.dequant(t, blob, n, k, out="f64")
    err = np.abs(back - data.astype(np.float64))
    bb, bw = synth.BLOCK_BYTES[t], synth.BLOCK_WEIGHTS[t]
    steps = np.empty((n * k // bw, bw))
    for blk, raw in enumerate(blob.reshape(-1, bb)):
        f = oracle.block_fields(t, raw)
        if t in ("q4_k", "q5_k"):
            steps[blk] = np.repeat(f["d"] * f["sc"], 32)
        elif t == "q6_k":
            steps[blk] = np.repeat(f["d"] * np.abs(f["sc"]), 16)
        else:
            steps[blk] = f["d"]
    steps = steps.reshape(n, k)
    assert np.all(err <= steps * 1.0 + 1e-12), float(np.max(err / np.maximum(steps, 1e-30)))
    # most weights land within half a step
    assert np.mean(err <= 0.5 * steps + 1e-12) > 0.97


def test_synth_is_deterministic_and_in_range():
    a = synth.blob("q4_k", synth.rng(1, "x"), 4, 512)
    b = synth.blob("q4_k", synth.rng(1, "x"), 4, 512)
    c = synth.blob("q4_k", synth.rng(2, "x"), 4, 512)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    blk = a.reshape(-1, 144)
    d = blk[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    dmin = blk[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    assert np.all((d >= 9.99e-4) & (d <= 1.0001e-2)) and np.all((dmin >= 0) & (dmin <= 5.01e-3))
    q8 = synth.blob("q8_0", synth.rng(1, "y"), 64, 1024).reshape(-1, 34)[:, 2:].view(np.int8)
    assert q8.min() >= -127 and q8.max() <= 127
    for t, bb, fields in (("q5_k", 176, (0, 2)), ("q4_0", 18, (0,))):
        blk = synth.blob(t, synth.rng(1, "z", t), 8, 512).reshape(-1, bb)
        d = blk[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
        assert np.all((d >= 9.99e-4) & (d <= 1.0001e-2))
        if 2 in fields:
            dmin = blk[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
            assert np.all((dmin >= 0) & (dmin <= 5.01e-3))
