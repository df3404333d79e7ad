"""Batch-1 Q4_K GEMV on the fp16 matrix cores (k_gemv_mf) against the oracle.

The kernel takes whole 16-row tiles and all of k per workgroup (wave w: blocks w KB .. w KB + KB - 1,
KB = 1, 2 or 4 by k), so the cases cover one block per row, a last wave with fewer blocks than
the others, 16-wave workgroups, row counts that leave a partial last tile, several tiles per
workgroup (the tile order is strided over the grid), parts of a multi launch that change inside a
tile, SwiGLU pairs, and activation blocks whose scales span the fp32 range. A row's sum does not
depend on the launch, so launches of other shapes and tilings must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_product_close, dev, host

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


def _case(*a):
    print("case:", *a, flush=True)


# (n, k): k = 256 / 768 / 2048 one block per wave; 2304 / 4096 / 4352 / 8192 two (4352: 17 blocks,
# the last wave one); 8448 / 14336 / 15104 four (8448: 33 blocks, the last wave one; 15104: 59
# blocks, 15 waves, the most LDS).
SHAPES = [(1, 256), (37, 768), (300, 2048), (15, 2304), (4096, 4096), (17, 4352), (1000, 8192),
          (33, 8448), (4096, 14336), (250, 15104)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_mf_against_oracle(knobs, n, k):
    _case("mf", n, k)
    knobs("gemv_mf", 1)
    g = synth.rng(130, "mf", n, k)
    w, x = synth.blob("q4_k", g, n, k), synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    y = host(tq.gemv("q4_k", wd, n, k, xd))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"mf {n}x{k}")
    assert worst < 0.05, worst
    assert np.array_equal(y, host(tq.gemv("q4_k", wd, n, k, xd))), "not deterministic"
    # the lanes-along-k kernel (fp32 FMAs on the vector units) is within the same bar, and the two
    # differ by the activations' last bits: x enters the matrix cores with 22 significant bits
    # (relative error up to 2^-22 per product), which the cancellation inside Q4_K weights
    # (d sc q against dmin m) can raise a few times against |y|
    knobs("gemv_mf", 0)
    y0 = host(tq.gemv("q4_k", wd, n, k, xd))
    assert_product_close(y0, ref, mag, what=f"kl {n}x{k}")
    assert np.linalg.norm(y - y0) <= 2e-5 * np.linalg.norm(y0) + 1e-30


@pytest.mark.parametrize("n,k", [(300, 4096), (1000, 2048), (4099, 4096), (200, 14336)])
@pytest.mark.parametrize("wgs", [1, 3, 7, 64])
def test_mf_tiles_per_workgroup_bitwise(knobs, n, k, wgs):
    """A launch aimed at `wgs` workgroups gives each several tiles (the LDS keeps as many as fit);
    every row's sum is formed the same way, so the result equals the default launch bit for bit."""
    _case("mf tiles", n, k, wgs)
    g = synth.rng(131, "mf-tiles", n, k)
    w, x = synth.blob("q4_k", g, n, k), synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    a = host(tq.gemv("q4_k", wd, n, k, xd))
    knobs("mf_wgs", wgs)
    b = host(tq.gemv("q4_k", wd, n, k, xd))
    assert np.array_equal(a, b)
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert_product_close(b, ref, mag, what=f"mf {n}x{k} wgs {wgs}")


@pytest.mark.parametrize("kb", [1, 2, 4])
def test_mf_blocks_per_wave(knobs, kb):
    """The blocks per wave change the k partition (and so the rounding of the waves' sums): each
    setting stays within the bar."""
    n, k = 203, 4096
    _case("mf kb", kb)
    g = synth.rng(132, "mf-kb")
    w, x = synth.blob("q4_k", g, n, k), synth.normal_f32(g, (1, k))
    knobs("mf_kb", kb)
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert_product_close(y, ref, mag, what=f"mf kb {kb}")


def test_mf_multi_and_swiglu_bitwise():
    """One launch over three matrices whose boundaries fall inside 16-row tiles, and a gate|up
    launch with SwiGLU (an odd row count), equal the single products bit for bit."""
    _case("mf multi swiglu")
    k = 4096
    g = synth.rng(133, "mf-multi")
    ns = [100, 37, 250]
    ws = [synth.blob("q4_k", g, n, k) for n in ns]
    x = dev(synth.normal_f32(g, (1, k)))
    outs = tq.gemv_multi("q4_k", [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv("q4_k", dev(w), n, k, x)))
    F = 301
    wg, wu = synth.blob("q4_k", g, F, k), synth.blob("q4_k", g, F, k)
    h = host(tq.gemv_swiglu("q4_k", dev(wg), dev(wu), F, k, x))
    gg = tq.gemv("q4_k", dev(wg), F, k, x)
    uu = tq.gemv("q4_k", dev(wu), F, k, x)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))


def test_mf_activation_scales():
    """Sub-blocks of x at 1e-30, 1e-38 (fp32 subnormal range), zero and 1e20, one sub-block with a
    single large value among tiny ones, and weight blocks with the largest and subnormal fp16 d:
    every output within the bar (the power-of-two scale per sub-block keeps x's significant bits)."""
    n, k = 160, 4096
    _case("mf scales")
    g = synth.rng(134, "mf-scales")
    w = synth.blob("q4_k", g, n, k)
    blk = w.reshape(-1, 144)
    blk[0::5, 0:2] = np.frombuffer(np.float16(65504.0).tobytes(), np.uint8)
    blk[1::7, 0:2] = np.frombuffer(np.float16(2.0 ** -20).tobytes(), np.uint8)
    x = synth.normal_f32(g, (1, k))
    x[0, 0:256] *= np.float32(1e-30)
    x[0, 256:288] *= np.float32(1e-38)
    x[0, 512:768] = 0.0
    x[0, 768:1024] *= np.float32(1e20)
    x[0, 1024:1056] *= np.float32(1e-6)
    x[0, 1030] = np.float32(3e4)
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert_product_close(y, ref, mag, what="mf activation scales")


def test_mf_graph_replay():
    """The kernel captured into a HIP graph (no workspace, no counters) replays to the eager bits."""
    _case("mf graph")
    n, k = 1000, 4096
    g = synth.rng(135, "mf-graph")
    w, x = synth.blob("q4_k", g, n, k), synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tq.gemv("q4_k", wd, n, k, xd, out=y)
        torch.cuda.synchronize()
        eager = host(y).copy()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            tq.gemv("q4_k", wd, n, k, xd, out=y)
        for _ in range(5):
            y.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(y), eager)
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert_product_close(eager, ref, mag, what="mf graph")


# ---- Q6_K ----------------------------------------------------------------------------------------
# k a multiple of 512 up to 8192: k = 512 one wave of two blocks; 3072 (12 blocks, 6 waves); 4096
# (8 waves of 2); 4608 (18 blocks: 4 a wave, the last wave 2); 8192 (8 waves of 4). Odd blocks sit
# two bytes off a dword.
SHAPES6 = [(1, 512), (37, 3072), (300, 4096), (17, 4608), (1000, 8192), (4099, 8192)]


@pytest.mark.parametrize("n,k", SHAPES6)
def test_mf_q6_k_against_oracle(knobs, n, k):
    _case("mf q6_k", n, k)
    g = synth.rng(140, "mf6", n, k)
    w, x = synth.blob("q6_k", g, n, k), synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    y = host(tq.gemv("q6_k", wd, n, k, xd))
    ref, mag = oracle.gemv("q6_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"mf q6_k {n}x{k}")
    assert worst < 0.05, worst
    assert np.array_equal(y, host(tq.gemv("q6_k", wd, n, k, xd))), "not deterministic"
    knobs("gemv_mf", 0)  # the lane-per-row fp32 kernel
    y0 = host(tq.gemv("q6_k", wd, n, k, xd))
    assert_product_close(y0, ref, mag, what=f"k_gemv q6_k {n}x{k}")
    assert np.linalg.norm(y - y0) <= 2e-5 * np.linalg.norm(y0) + 1e-30


@pytest.mark.parametrize("wgs", [1, 5, 64])
def test_mf_q6_k_tiles_per_workgroup_bitwise(knobs, wgs):
    n, k = 1001, 8192
    _case("mf q6_k tiles", wgs)
    g = synth.rng(141, "mf6-tiles")
    w, x = synth.blob("q6_k", g, n, k), synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    a = host(tq.gemv("q6_k", wd, n, k, xd))
    knobs("mf_wgs", wgs)
    assert np.array_equal(a, host(tq.gemv("q6_k", wd, n, k, xd)))


def test_mf_q6_k_multi_and_swiglu_bitwise():
    """Q6_K one-token multi and gate|up + SwiGLU launches (now one launch each) equal the single
    products bit for bit."""
    _case("mf q6_k multi swiglu")
    k = 4096
    g = synth.rng(142, "mf6-multi")
    ns = [100, 37, 250]
    ws = [synth.blob("q6_k", g, n, k) for n in ns]
    x = dev(synth.normal_f32(g, (1, k)))
    outs = tq.gemv_multi("q6_k", [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv("q6_k", dev(w), n, k, x)))
    F = 301
    wg, wu = synth.blob("q6_k", g, F, k), synth.blob("q6_k", g, F, k)
    h = host(tq.gemv_swiglu("q6_k", dev(wg), dev(wu), F, k, x))
    gg = tq.gemv("q6_k", dev(wg), F, k, x)
    uu = tq.gemv("q6_k", dev(wu), F, k, x)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))


def test_mf_q6_k_extremes():
    """Scales -128 and 127, quants 0 and 63 (q - 32 at both ends), d at the largest and subnormal
    fp16, and activation sub-blocks at 1e-30, zero and 1e20: every output within the bar."""
    n, k = 96, 4096
    _case("mf q6_k extremes")
    g = synth.rng(143, "mf6-ext")
    w = synth.blob("q6_k", g, n, k)
    blk = w.reshape(-1, 210)
    blk[0::3, 192:208] = np.uint8(0x80)  # -128
    blk[1::3, 192:208] = np.uint8(0x7F)  # 127
    blk[2::5, 0:192] = np.uint8(0xFF)    # q = 63
    blk[3::5, 0:192] = np.uint8(0x00)    # q = 0
    blk[0::7, 208:210] = np.frombuffer(np.float16(65504.0).tobytes(), np.uint8)
    blk[1::11, 208:210] = np.frombuffer(np.float16(2.0 ** -20).tobytes(), np.uint8)
    x = synth.normal_f32(g, (1, k))
    x[0, 0:256] *= np.float32(1e-30)
    x[0, 512:528] = 0.0
    x[0, 768:1024] *= np.float32(1e20)
    y = host(tq.gemv("q6_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q6_k", w, n, k, x)
    assert_product_close(y, ref, mag, what="mf q6_k extremes")


# Longer Q6_K rows in k slices (equal slices of an even number of blocks, at most 32): k = 9216
# (2 x 18), 11264 (2 x 22), 16384 (2 x 32), 28672 (4 x 28, the 70B-shaped down projection).
SLICED6 = [(37, 9216), (300, 11264), (17, 16384), (1000, 28672)]


@pytest.mark.parametrize("n,k", SLICED6)
def test_mf_q6_k_k_slices(knobs, n, k):
    """The slices' sums meet through the workspace (arrival counters, the last slice adds them in
    slice order): within the bar, deterministic, and the same with a workspace full of random
    bytes; without a workspace the lane-per-row kernel runs instead."""
    _case("mf q6_k slices", n, k)
    g = synth.rng(144, "mf6-slices", n, k)
    w, x = synth.blob("q6_k", g, n, k), synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    nbytes = tq.gemv_workspace_bytes("q6_k", n, k, 1)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    y = host(tq.gemv("q6_k", wd, n, k, xd, ws=ws))
    ref, mag = oracle.gemv("q6_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"mf q6_k slices {n}x{k}")
    assert worst < 0.05, worst
    ws.copy_(torch.from_numpy(g.integers(0, 256, nbytes, dtype=np.uint8)).to(ws.device))
    assert np.array_equal(y, host(tq.gemv("q6_k", wd, n, k, xd, ws=ws)))
    y0 = host(tq.gemv("q6_k", wd, n, k, xd, ws=False))
    assert_product_close(y0, ref, mag, what=f"no workspace {n}x{k}")
    knobs("gemv_mf", 0)
    y1 = host(tq.gemv("q6_k", wd, n, k, xd, ws=ws))
    assert np.linalg.norm(y - y1) <= 2e-5 * np.linalg.norm(y1) + 1e-30


@pytest.mark.parametrize("n,k", [(300, 16384), (1000, 28672)])
def test_mf_q4_k_k_slices(knobs, n, k):
    """Q4_K rows from k = 16384 in k slices (TQ_KNOB_GEMV_MF = 2, the default; 1 sends them to
    the int8 kernel): within the bar and within 2e-5 of the int8 kernel."""
    _case("mf q4_k slices", n, k)
    g = synth.rng(145, "mf4-slices", n, k)
    w, x = synth.blob("q4_k", g, n, k), synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    knobs("gemv_mf", 2)
    ws = torch.zeros(tq.gemv_workspace_bytes("q4_k", n, k, 1), dtype=torch.uint8, device="cuda:0")
    y = host(tq.gemv("q4_k", wd, n, k, xd, ws=ws))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"mf q4_k slices {n}x{k}")
    assert worst < 0.05, worst
    knobs("gemv_mf", 1)
    ws2 = torch.zeros(tq.gemv_workspace_bytes("q4_k", n, k, 1), dtype=torch.uint8, device="cuda:0")
    y8 = host(tq.gemv("q4_k", wd, n, k, xd, ws=ws2))
    assert np.linalg.norm(y - y8) <= 2e-5 * np.linalg.norm(y8) + 1e-30
