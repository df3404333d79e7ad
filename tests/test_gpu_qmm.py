"""GPU parity of the fp32-accurate fp16 matrix-core expert kernels (Q4_K MoE steps of 2 or more
tokens per call take them by default on the fp32 path).

Bars, as for every fp32-accumulated product: routing and grouping bitwise, y within
1e-3 * sum|products| + 1e-5 of the fp64 oracle. On top of that, the kernels are checked to be at
fp32 level -- far inside that bound -- and against the grouped fp32 GEMV they replace.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev, host
from tests.test_gpu_moe import _case, _layer_to_device, _run, check_moe

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


def _tile_env(knobs, nt):
    knobs("qmm_nt", nt)
    knobs("moe_qmm", -1)


# Few experts and top-1 or top-2, so that per-expert counts land on both sides of the chunk
# sizes (16 and 32 positions) and chunks split into near-equal parts.
BOUNDARY = [
    (dict(hidden=512, ffn=768, n_experts=2, shared=False), 1, [2, 15, 16, 17, 31, 32, 33, 40, 70]),
    (dict(hidden=768, ffn=512, n_experts=4, shared=True), 2, [3, 16, 33, 64, 97]),
]


@pytest.mark.parametrize("nt", [1, 2])
@pytest.mark.parametrize("shape,k,Ts", BOUNDARY, ids=["E2k1", "E4k2-shared"])
def test_qmm_chunk_boundaries(knobs, nt, shape, k, Ts):
    _tile_env(knobs, nt)
    layer = synth.moe_layer(shape, "q4_k", seed=401, tag=f"qmm-{shape['n_experts']}")
    moe = None
    for T in Ts:
        _case("qmm-boundary", nt, shape, k, T)
        x = synth.normal_f32(synth.rng(401, "x", T, nt), (T, shape["hidden"]))
        moe, y, (worst, l2) = check_moe("q4_k", shape, layer, x, k, moe=moe)
        # fp32 level: the largest error stays far below the 1e-3 bound
        assert worst < 0.05, f"T={T}: worst error / bound {worst}"
        y2, _ = _run(moe, x, shape["n_experts"], k)
        assert np.array_equal(y, y2), "not deterministic"


def test_qmm_agrees_with_grouped_gemv(knobs):
    """The matrix-core kernels and the grouped fp32 GEMV both meet the bar; their difference is
    fp32 rounding order only (relative L2 difference at the 1e-6 level)."""
    shape, k, T = dict(hidden=1024, ffn=1536, n_experts=8, shared=True), 2, 48
    layer = synth.moe_layer(shape, "q4_k", seed=402, tag="qmm-vs-gemv")
    x = synth.normal_f32(synth.rng(402, "x"), (T, shape["hidden"]))
    _tile_env(knobs, 2)
    _, y_q, (wq, lq) = check_moe("q4_k", shape, layer, x, k)
    knobs("moe_qmm", 0)
    _, y_g, (wg, lg) = check_moe("q4_k", shape, layer, x, k)
    print(f"qmm worst {wq:.3g} l2 {lq:.3g}; grouped GEMV worst {wg:.3g} l2 {lg:.3g}")
    d = float(np.linalg.norm(y_q - y_g) / np.linalg.norm(y_g))
    assert d < 1e-5, d
    assert wq < 0.05 and lq < 1e-5


def test_qmm_rows_of_any_scale(knobs):
    """Each activation row is rescaled by its own power of two: rows of magnitude 1e-12 and 1e12,
    an all-zero row and a row with one huge element keep fp32 accuracy."""
    _tile_env(knobs, 1)
    shape, k, T = dict(hidden=512, ffn=512, n_experts=4, shared=True), 2, 12
    layer = synth.moe_layer(shape, "q4_k", seed=403, tag="qmm-scale")
    x = synth.normal_f32(synth.rng(403, "x"), (T, shape["hidden"]))
    x[1] *= np.float32(1e-12)
    x[2] *= np.float32(1e12)
    x[3] = 0.0
    x[4, 7] = np.float32(3e4)
    x[5] *= np.float32(2.0 ** -100)
    _case("qmm-scale", T)
    _, y, (worst, _) = check_moe("q4_k", shape, layer, x, k)
    assert worst < 0.05, worst
    assert np.all(np.isfinite(y))


def test_qmm_workspace_sizes_differ_by_tile(knobs):
    """The chunk table grows when chunks hold 16 rather than 32 positions (fp32 path forced: at
    100 routed tokens per expert the automatic choice is the bf16 prefill path)."""
    shape = dict(hidden=512, ffn=512, n_experts=4, shared=False)
    layer = synth.moe_layer(shape, "q4_k", seed=404, tag="qmm-ws")
    _tile_env(knobs, 1)
    moe = _layer_to_device("q4_k", shape, layer, 2, path=tq.PATH_F32)
    w1 = moe.workspace_bytes(200)
    _tile_env(knobs, 2)
    w2 = moe.workspace_bytes(200)
    assert w1 > w2 > 0
    y = host(moe(dev(synth.normal_f32(synth.rng(404, "x"), (200, 512)))))
    assert np.all(np.isfinite(y))


# ---- dense products of 2..32 tokens (tq_gemv / tq_gemv_multi / tq_gemv_swiglu) -------------------

import oracle  # noqa: E402
from tests.gpu_util import assert_product_close  # noqa: E402


@pytest.mark.parametrize("n,k,batch", [(300, 4096, 2), (128, 1024, 4), (1000, 2048, 8), (64, 14336, 8),
                                       (257, 512, 16), (96, 3072, 17), (130, 4096, 32)])
def test_qmm_dense_gemv(n, k, batch):
    _case("qmm-dense", n, k, batch)
    g = synth.rng(410, "dense", n, k, batch)
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (batch, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"dense {n}x{k} b{batch}")
    assert worst < 0.05, worst
    y2 = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    assert np.array_equal(y, y2), "not deterministic"


def test_qmm_dense_multi_and_swiglu_bitwise():
    """The fused q/k/v launch and the fused gate/up + SwiGLU launch give bitwise the single-GEMV
    results (k slices of a fixed size, added in order)."""
    k, batch = 4096, 8
    g = synth.rng(411, "dense-multi")
    ns = [512, 128, 128]
    ws = [synth.blob("q4_k", g, n, k) for n in ns]
    x = dev(synth.normal_f32(g, (batch, k)))
    outs = tq.gemv_multi("q4_k", [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv("q4_k", dev(w), n, k, x)))
    F = 448
    wg, wu = synth.blob("q4_k", g, F, k), synth.blob("q4_k", g, F, k)
    h = host(tq.gemv_swiglu("q4_k", dev(wg), dev(wu), F, k, x))
    gg = tq.gemv("q4_k", dev(wg), F, k, x)
    uu = tq.gemv("q4_k", dev(wu), F, k, x)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))


def test_qmm_dense_agrees_with_fp32_gemv(knobs):
    """Matrix-core path vs the fp32 multi-token GEMV (TQ_KNOB_GEMV_QMM = 0): fp32 rounding apart."""
    n, k, batch = 512, 8192, 8
    g = synth.rng(412, "dense-vs")
    w, x = dev(synth.blob("q4_k", g, n, k)), dev(synth.normal_f32(g, (batch, k)))
    a = host(tq.gemv("q4_k", w, n, k, x))
    knobs("gemv_qmm", 0)
    b = host(tq.gemv("q4_k", w, n, k, x))
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-6


def test_qmm_dense_without_workspace():
    """No workspace: the fp32 GEMV runs (still within the bar)."""
    n, k, batch = 200, 2048, 4
    g = synth.rng(413, "dense-nows")
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (batch, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x), ws=False))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert_product_close(y, ref, mag, what="dense no-ws")


# ---- the in-kernel split (2..16 tokens): every launch shape -----------------------------------

INLINE_SHAPES = [(300, 4096, 2), (1000, 2048, 8), (64, 14336, 8), (257, 512, 16), (130, 4608, 9),
                 (70, 768, 5), (129, 1280, 3)]


@pytest.mark.parametrize("upk,nr", [(2, 1), (2, 2), (4, 1), (4, 2)])
@pytest.mark.parametrize("n,k,batch", INLINE_SHAPES)
def test_qmm_dense_inline_launch_shapes(knobs, upk, nr, n, k, batch):
    """Slices of 2 or 4 blocks (a ragged last slice where the block count is not a multiple),
    one or two 16-row weight tiles per wave, 8 or 16 token rows per block, ragged row tiles; every
    output against the oracle, at fp32 level, and repeatable bitwise."""
    knobs("qmm_inline_upk", upk)
    knobs("qmm_inline_nr", nr)
    _case("qmm-inline", upk, nr, n, k, batch)
    g = synth.rng(415, "inline", n, k, batch)
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (batch, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"inline {n}x{k} b{batch} upk{upk} nr{nr}")
    assert worst < 0.05, worst
    y2 = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    assert np.array_equal(y, y2), "not deterministic"


@pytest.mark.parametrize("upk", [2, 4])
@pytest.mark.parametrize("F,k,batch", [(448, 4096, 8), (200, 1536, 13), (64, 2304, 2)])
def test_qmm_dense_inline_swiglu_and_multi(knobs, upk, F, k, batch):
    """gate|up + SwiGLU and a three-matrix launch against the single products of the same
    slices, bitwise; the single products against the oracle."""
    knobs("qmm_inline_upk", upk)
    _case("qmm-inline-fused", upk, F, k, batch)
    g = synth.rng(416, "inline-fused", F, k, batch)
    wg, wu = synth.blob("q4_k", g, F, k), synth.blob("q4_k", g, F, k)
    xh = synth.normal_f32(g, (batch, k))
    x = dev(xh)
    gg = tq.gemv("q4_k", dev(wg), F, k, x)
    uu = tq.gemv("q4_k", dev(wu), F, k, x)
    ref, mag = oracle.gemv("q4_k", wg, F, k, xh)
    assert assert_product_close(host(gg), ref, mag, what="gate") < 0.05
    h = host(tq.gemv_swiglu("q4_k", dev(wg), dev(wu), F, k, x))
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))
    ns = [F, 96, 33]
    ws = [wg, synth.blob("q4_k", g, 96, k), synth.blob("q4_k", g, 33, k)]
    outs = tq.gemv_multi("q4_k", [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv("q4_k", dev(w), n, k, x)))


def test_qmm_dense_inline_blocks_of_any_scale():
    """Each (token, 256-value block) gets its own power of two: blocks of magnitude 1e-12 and
    1e12 in one row, an all-zero block, one huge element, a row at 2^-100 and one at 1e30 keep
    fp32 accuracy."""
    n, k, batch = 256, 2048, 7
    g = synth.rng(417, "inline-scale")
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (batch, k))
    x[0, :256] *= np.float32(1e-12)
    x[0, 256:512] *= np.float32(1e12)
    x[1, 512:768] = 0.0
    x[2, 1000] = np.float32(3e4)
    x[3] *= np.float32(2.0 ** -100)
    x[4] *= np.float32(1e30)
    x[5, 1792:] *= np.float32(1e-30)
    _case("qmm-inline-scale")
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what="inline any-scale")
    assert worst < 0.05, worst
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("n,k,batch", [(1000, 4096, 8), (96, 3072, 12)])
def test_qmm_dense_inline_agrees_with_split_launch(knobs, n, k, batch):
    """The in-kernel split against the separate split launch (per-row scale): fp32 rounding apart."""
    g = synth.rng(418, "inline-vs-split", n, k, batch)
    w, x = dev(synth.blob("q4_k", g, n, k)), dev(synth.normal_f32(g, (batch, k)))
    a = host(tq.gemv("q4_k", w, n, k, x))
    knobs("qmm_inline", 0)
    b = host(tq.gemv("q4_k", w, n, k, x))
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-6
