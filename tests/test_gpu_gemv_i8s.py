"""GPU parity of the streaming batch-1 Q4_K GEMV on the int8 matrix cores (k <= 16384).

Each workgroup makes the activation digits for all of k in LDS, each wave streams one 32-row tile
over one k part with several blocks of loads in flight, and the parts of a tile are added in part
order inside the workgroup. The launch shape (waves per workgroup, blocks in flight, k parts) is
forced through TQ_KNOB_I8S_NW / TQ_KNOB_I8S_D / TQ_KNOB_I8S_KS to cover every compiled form, including parts
left empty when k has fewer blocks than parts. Bars: 1e-3 * sum|w x| + 1e-5 per element against
the fp64 oracle; bitwise on the integer lattice (every digit and partial sum exact); bitwise
agreement of the one-launch multi and SwiGLU calls with single GEMVs (the k parts depend on k
only, so a row's sum is formed the same way in every call).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import blobs
from tests.gpu_util import assert_product_close, dev, host

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")

CONFIGS = [None, ("4", "2", "1"), ("4", "6", "2"), ("8", "2", "8"), ("16", "2", "16"),
           ("8", "6", "4"), ("8", "4", "2")]


def _case(*a):
    print("case:", *a, flush=True)


def _config(knobs, cfg):
    knobs("gemv_i8s", 1)
    if cfg is not None:
        nw, d, ks = cfg
        knobs("i8s_nw", int(nw))
        knobs("i8s_d", int(d))
        knobs("i8s_ks", int(ks))


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "default" if c is None else "-".join(c))
@pytest.mark.parametrize("n,k", [(1, 256), (31, 512), (33, 1024), (100, 4096), (257, 3072),
                                 (64, 14336), (97, 16384), (1000, 2304)])
def test_i8s_gemv_random(knobs, cfg, n, k):
    _case("i8s", cfg, n, k)
    _config(knobs, cfg)
    g = synth.rng(601, "i8s", n, k)
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (1, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"i8s {cfg} {n}x{k}")
    assert worst < 0.05, worst  # fp32 level, far inside the bar


@pytest.mark.parametrize("cfg", [None, ("4", "2", "1"), ("16", "2", "16")],
                         ids=lambda c: "default" if c is None else "-".join(c))
@pytest.mark.parametrize("n,k", [(64, 4096), (50, 16384), (33, 768)])
def test_i8s_gemv_lattice_bitwise(knobs, cfg, n, k):
    """Scales 2^-8, x in {-1, 0, 1}: the digits are the integers themselves and every partial sum
    is exact, so the result equals the oracle's bit for bit."""
    _case("i8s-lattice", cfg, n, k)
    _config(knobs, cfg)
    g = synth.rng(602, "i8s-lattice", n, k)
    w = synth.blob("q4_k", g, n, k, d_value=2.0 ** -8, dmin_value=2.0 ** -8)
    x = synth.ternary_f32(g, (1, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, _ = oracle.gemv("q4_k", w, n, k, x)
    assert np.array_equal(y.astype(np.float64), ref)


def test_i8s_identity_and_blocks_of_any_scale(knobs):
    """W = I gives x back (exactly for blocks with few significant bits); blocks of x scaled by
    1e-30 and 1e30, a zero block and an outlier keep fp32 accuracy (per-block power-of-two
    digit scales)."""
    _config(knobs, None)
    n = 1024
    g = synth.rng(603, "i8s-identity")
    x = synth.normal_f32(g, (1, n))
    x[0, :256] = np.round(x[0, :256] * 64) / 64
    y = host(tq.gemv("q4_k", dev(blobs.identity(n)), n, n, dev(x)))
    assert np.array_equal(y[0, :256], x[0, :256])
    assert np.allclose(y[0], x[0], rtol=1e-6, atol=1e-6)
    n, k = 96, 2048
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (1, k))
    x[0, 0:256] *= np.float32(1e-30)
    x[0, 256:512] *= np.float32(1e30)
    x[0, 512:768] = 0.0
    x[0, 800] = np.float32(5e4)
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert assert_product_close(y, ref, mag, what="i8s scales") < 0.05


@pytest.mark.parametrize("k", [2048, 4096, 14336])
def test_i8s_multi_and_swiglu_match_single_gemvs(knobs, k):
    """q|k|v in one launch and gate|up with the SwiGLU in one launch give bitwise the results of
    single GEMVs (and of tq_swiglu on them): the k parts are chosen from k alone."""
    _case("i8s-multi", k)
    _config(knobs, None)
    g = synth.rng(604, "i8s-multi", k)
    ns = [512, 96, 160]
    ws = [synth.blob("q4_k", g, n, k) for n in ns]
    x = dev(synth.normal_f32(g, (1, k)))
    outs = tq.gemv_multi("q4_k", [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv("q4_k", dev(w), n, k, x)))
    F = 336
    wg, wu = synth.blob("q4_k", g, F, k), synth.blob("q4_k", g, F, k)
    h = host(tq.gemv_swiglu("q4_k", dev(wg), dev(wu), F, k, x))
    gg = tq.gemv("q4_k", dev(wg), F, k, x)
    uu = tq.gemv("q4_k", dev(wu), F, k, x)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))


@pytest.mark.parametrize("name,n,k", [("o", 4096, 4096), ("gate", 14336, 4096),
                                      ("down", 4096, 14336)])
def test_i8s_llama8b_shapes_all_rows(knobs, name, n, k):
    """The 8B-shaped projections at full size, every output row against the oracle."""
    _case("i8s-8b", name, n, k)
    _config(knobs, None)
    g = synth.rng(605, "i8s-8b", name)
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (1, k))
    y = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert assert_product_close(y, ref, mag, what=f"i8s {name}") < 0.05


def test_i8s_agrees_with_other_kernels(knobs):
    """The streaming kernel, the k-sliced int8 kernel and the lanes-along-k kernel all meet the
    bar on the same inputs and differ by fp32 rounding only."""
    n, k = 200, 8192
    g = synth.rng(606, "i8s-vs")
    w, x = dev(synth.blob("q4_k", g, n, k)), dev(synth.normal_f32(g, (1, k)))
    _config(knobs, None)
    a = host(tq.gemv("q4_k", w, n, k, x))
    knobs("gemv_i8s", 0)
    knobs("gemv_i8", 2)
    b = host(tq.gemv("q4_k", w, n, k, x))
    knobs("gemv_i8", 0)
    c = host(tq.gemv("q4_k", w, n, k, x))
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-6
    assert np.linalg.norm(a - c) / np.linalg.norm(c) < 1e-6
