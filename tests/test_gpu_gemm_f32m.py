"""GPU parity of the Q6_K / Q8_0 products of 2..16 tokens on the fp32 matrix cores.

Weights are dequantized once per block into exact fp32 operands (Q8_0: d * q; Q6_K: sc * (q - 32)
with d applied to the block's sum), the tokens' fp32 activations are the other operand, and the
matrix cores form and add the products in fp32, so the bar is that of every fp32-accumulated
product: 1e-3 * sum|w x| + 1e-5 per element against the fp64 oracle. Shapes cover ragged row
counts (not a multiple of the 128-row workgroup or the 16-row tile), k in one slice and in up to
eight slices, batches 2..16, and both block alignments of Q6_K (odd blocks start two bytes past a
dword). The k slices are a function of k alone, so one-launch multi and SwiGLU calls equal single
GEMVs bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_product_close, dev, host

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


@pytest.fixture(autouse=True)
def every_batch(knobs):
    """Every batch of 2..16 on the matrix-core path (by default Q6_K takes it from 2 tokens on the
    4-token form, from 4 without it)."""
    knobs("gemm_f32m", 2)


def _case(*a):
    print("case:", *a, flush=True)


@pytest.mark.parametrize("t", ["q6_k", "q8_0"])
@pytest.mark.parametrize("n,k", [(1, 512), (31, 1024), (100, 4096), (129, 3584), (257, 2048),
                                 (64, 14336), (97, 16384), (300, 8192)])
@pytest.mark.parametrize("batch", [2, 5, 16])
def test_f32m_random(t, n, k, batch):
    _case("f32m", t, n, k, batch)
    g = synth.rng(701, "f32m", t, n, k, batch)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (batch, k))
    y = host(tq.gemv(t, dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv(t, w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"f32m {t} {n}x{k} b{batch}")
    assert worst < 0.05, worst  # fp32 level, far inside the bar


@pytest.mark.parametrize("t", ["q6_k", "q8_0"])
@pytest.mark.parametrize("batch", [3, 4, 7, 8, 9, 13, 15])
def test_f32m_every_batch(t, batch):
    n, k = 77, 2560 if t == "q8_0" else 3072
    _case("f32m-batch", t, batch)
    g = synth.rng(702, "f32m-batch", t, batch)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (batch, k))
    y = host(tq.gemv(t, dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv(t, w, n, k, x)
    assert assert_product_close(y, ref, mag, what=f"f32m {t} b{batch}") < 0.05


@pytest.mark.parametrize("t,k", [("q6_k", 3072), ("q8_0", 4096), ("q6_k", 14336)])
def test_f32m_multi_and_swiglu_match_single_gemvs(t, k):
    """q|k|v in one launch and gate|up with the SwiGLU in one launch give bitwise the results of
    single GEMVs (and of tq_swiglu on them)."""
    _case("f32m-multi", t, k)
    batch = 4
    g = synth.rng(703, "f32m-multi", t, k)
    ns = [256, 96, 144]
    ws = [synth.blob(t, g, n, k) for n in ns]
    x = dev(synth.normal_f32(g, (batch, k)))
    outs = tq.gemv_multi(t, [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv(t, dev(w), n, k, x)))
    F = 200
    wg, wu = synth.blob(t, g, F, k), synth.blob(t, g, F, k)
    h = host(tq.gemv_swiglu(t, dev(wg), dev(wu), F, k, x))
    gg = tq.gemv(t, dev(wg), F, k, x)
    uu = tq.gemv(t, dev(wu), F, k, x)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))
    ref, mag = oracle.gemv(t, wg, F, k, host(x))
    assert_product_close(host(gg), ref, mag, what="gate")


@pytest.mark.parametrize("batch", [3, 6])
def test_f32m_workspace_any_contents_and_repeatable(batch):
    """Sliced k: a workspace of random bytes gives the bits of a zeroed one, and repeated calls
    on the same workspace give the same bits (batch 3: the 4-token form)."""
    t, n, k = "q6_k", 300, 16384
    g = synth.rng(704, "f32m-ws")
    w, x = dev(synth.blob(t, g, n, k)), dev(synth.normal_f32(g, (batch, k)))
    nbytes = max(tq.gemv_workspace_bytes(t, n, k, batch), 256)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    y1 = host(tq.gemv(t, w, n, k, x, ws=ws))
    ws.copy_(torch.from_numpy(g.integers(0, 256, nbytes, dtype=np.uint8)).to("cuda:0"))
    for i in range(5):
        assert np.array_equal(y1, host(tq.gemv(t, w, n, k, x, ws=ws))), f"call {i}"


@pytest.mark.parametrize("t", ["q6_k", "q8_0"])
@pytest.mark.parametrize("batch", [2, 8])
def test_f32m_agrees_with_fp32_gemv(knobs, t, batch):
    """The matrix-core path and the fp32 vector GEMV differ by fp32 rounding only."""
    n, k = 200, 4096
    g = synth.rng(705, "f32m-vs", t)
    w, x = dev(synth.blob(t, g, n, k)), dev(synth.normal_f32(g, (batch, k)))
    a = host(tq.gemv(t, w, n, k, x))
    knobs("gemm_f32m", 0)
    b = host(tq.gemv(t, w, n, k, x))
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-6


@pytest.mark.parametrize("t", ["q6_k", "q8_0"])
@pytest.mark.parametrize("batch", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(77, 3072), (300, 16384)])
def test_f32m_four_token_form_agrees_with_padded_form(knobs, t, batch, n, k):
    """Up to 4 tokens the 4x4x1 form (quarters of k summed at the end) and the 16-token form
    (TQ_KNOB_F32M_T4 = 0) differ by fp32 rounding only; both within the oracle's bar."""
    _case("f32m-t4", t, batch, n, k)
    g = synth.rng(706, "f32m-t4", t, batch, n, k)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (batch, k))
    a = host(tq.gemv(t, dev(w), n, k, dev(x)))
    knobs("f32m_t4", 0)
    b = host(tq.gemv(t, dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv(t, w, n, k, x)
    assert assert_product_close(a, ref, mag, what="4-token form") < 0.05
    assert assert_product_close(b, ref, mag, what="16-token form") < 0.05
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-6
