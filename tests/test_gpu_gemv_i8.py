"""GPU parity of the batch-1 Q4_K GEMV on the int8 matrix cores (activation digits + MFMA).

The kernel runs by default from k = 16384 on; TQ_KNOB_GEMV_I8 = 2 sends every Q4_K batch-1 shape to it,
which these tests use to cover small and ragged shapes. Bars as for every fp32-accumulated
product (1e-3 * sum|w x| + 1e-5 against the fp64 oracle), bitwise on the integer lattice (the
activation digits of integer-valued blocks are exact and every partial sum is an integer below
2^24), and bitwise agreement between the one-launch multi / SwiGLU calls and single GEMVs.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import blobs
from tests.gpu_util import assert_product_close, dev, host

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


@pytest.fixture
def i8(knobs):
    knobs("gemv_i8", 2)


def _case(*a):
    print("case:", *a, flush=True)


@pytest.mark.parametrize("n,k", [(1, 256), (31, 512), (33, 1024), (100, 4096), (257, 3072),
                                 (64, 14336), (96, 28672)])
def test_i8_gemv_random(i8, n, k):
    _case("i8", n, k)
    g = synth.rng(501, "i8", n, k)
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (1, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"i8 {n}x{k}")
    assert worst < 0.05, worst  # fp32 level, far inside the bar


def test_i8_gemv_default_threshold(knobs):
    """Without the override, and with the fp16 matrix-core kernel limited to unsliced rows
    (TQ_KNOB_GEMV_MF = 1), the kernel takes k > 16384 (and agrees with the oracle there)."""
    knobs("gemv_mf", 1)
    n, k = 40, 20480
    g = synth.rng(502, "i8-default")
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (1, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert_product_close(y, ref, mag, what="i8 default")


@pytest.mark.parametrize("n,k", [(64, 4096), (50, 16384)])
def test_i8_gemv_lattice_bitwise(i8, n, k):
    """Scales 2^-8, x in {-1, 0, 1}: each block's digits are the integers themselves, every sum
    is exact, so the result must equal the oracle's bit for bit."""
    g = synth.rng(503, "i8-lattice", n, k)
    w = synth.blob("q4_k", g, n, k, d_value=2.0 ** -8, dmin_value=2.0 ** -8)
    x = synth.ternary_f32(g, (1, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, _ = oracle.gemv("q4_k", w, n, k, x)
    assert np.array_equal(y.astype(np.float64), ref)


def test_i8_gemv_identity_recovers_x_blocks(i8):
    """W = I: y = x exactly for blocks whose values need few significant bits (digits exact),
    and within fp32 rounding for N(0,1) blocks."""
    n = 1024
    w = blobs.identity(n)
    g = synth.rng(504, "i8-identity")
    x = synth.normal_f32(g, (1, n))
    x[0, :256] = np.round(x[0, :256] * 64) / 64  # 6 fractional bits
    y = host(tq.gemv("q4_k", dev(w), n, n, dev(x)))
    assert np.array_equal(y[0, :256], x[0, :256])
    assert np.allclose(y[0], x[0], rtol=1e-6, atol=1e-6)


def test_i8_gemv_blocks_of_any_scale(i8):
    """Each 256-value block has its own power-of-two scale: blocks of magnitude 1e-30, 1e30, zero
    blocks and a block with one outlier all keep fp32 accuracy."""
    n, k = 64, 2048
    g = synth.rng(505, "i8-scale")
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (1, k))
    x[0, 0:256] *= np.float32(1e-30)
    x[0, 256:512] *= np.float32(1e30)
    x[0, 512:768] = 0.0
    x[0, 800] = np.float32(5e4)
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what="i8 scales")
    assert worst < 0.05, worst


def test_i8_multi_and_swiglu_match_single_gemvs(i8):
    """One-launch q/k/v and gate/up (SwiGLU) give bitwise the single-GEMV results: the kernel's
    summation order depends on k only."""
    k = 2048
    g = synth.rng(506, "i8-multi")
    ns = [512, 96, 96]
    ws = [synth.blob("q4_k", g, n, k) for n in ns]
    x = dev(synth.normal_f32(g, (1, k)))
    outs = tq.gemv_multi("q4_k", [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv("q4_k", dev(w), n, k, x)))
    F = 320
    wg, wu = synth.blob("q4_k", g, F, k), synth.blob("q4_k", g, F, k)
    h = host(tq.gemv_swiglu("q4_k", dev(wg), dev(wu), F, k, x))
    gg = tq.gemv("q4_k", dev(wg), F, k, x)
    uu = tq.gemv("q4_k", dev(wu), F, k, x)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))


def test_i8_agrees_with_lanes_along_k(knobs):
    """The int8 and the lanes-along-k kernels both meet the bar and differ by fp32 rounding."""
    n, k = 128, 8192
    g = synth.rng(507, "i8-vs-kl")
    w, x = dev(synth.blob("q4_k", g, n, k)), dev(synth.normal_f32(g, (1, k)))
    knobs("gemv_i8", 2)
    a = host(tq.gemv("q4_k", w, n, k, x))
    knobs("gemv_i8", 0)
    knobs("gemv_mf", 0)  # the lanes-along-k kernel, not the fp16 matrix-core one
    b = host(tq.gemv("q4_k", w, n, k, x))
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-6
