"""Pins of the oracle's products, SwiGLU, routing, grouping and MoE combine (CPU only).

Each oracle function is checked against something other than itself:
  * GEMV: dense fp64 matmul (numpy) of the dequantized matrix on tiny shapes; x = e_j picks a
    column exactly; x = 1 over blocks with constant scale/min has the closed form
    sum_blocks (d*sc*sum(q) - 256*dmin*m), where sum(q) is the sum of all nibbles of the block.
  * SwiGLU: scipy's logistic function; limits at 0 and +-infinity.
  * Router logits: numpy matmul.
  * Top-k: a full stable sort per token; equal logits; k = E is the dense softmax (scipy).
  * Grouping: numpy stable argsort, plus the permutation / ordering invariants.
  * MoE: a dense numpy FFN per expert; expert relabelling; the shared expert as an additive term.
"""
import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth


def _dense(t, w, n, k):
    return oracle.dequant(t, w, n, k, out="f64")


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_0"])
@pytest.mark.parametrize("n,k,b", [(1, 256, 1), (3, 512, 2), (2, 256, 3)])
def test_gemv_brute_force(t, n, k, b):
    g = synth.rng(21, "gemv-bf", t, n, k, b)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (b, k))
    y, mag = oracle.gemv(t, w, n, k, x)
    dense = _dense(t, w, n, k)
    ref = x.astype(np.float64) @ dense.T
    refmag = np.abs(x.astype(np.float64)) @ np.abs(dense).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mag, refmag, rtol=1e-12)


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_0"])
def test_gemv_unit_vector_picks_column(t):
    g = synth.rng(22, "gemv-ej", t)
    n, k = 5, 512
    w = synth.blob(t, g, n, k)
    dense = _dense(t, w, n, k)
    for j in (0, 1, 255, 256, 511):
        x = np.zeros((1, k), np.float32)
        x[0, j] = 1.0
        y, _ = oracle.gemv(t, w, n, k, x)
        assert np.array_equal(y[0], dense[:, j])


def test_gemv_row_subset_matches_full():
    g = synth.rng(23, "rows")
    n, k = 9, 768
    w = synth.blob("q4_k", g, n, k)
    x = synth.normal_f32(g, (2, k))
    y, mag = oracle.gemv("q4_k", w, n, k, x)
    rows = [8, 0, 3]
    ys, ms = oracle.gemv("q4_k", w, n, k, x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(ms, mag[:, rows])


def test_q4k_gemv_closed_form_constant_scales():
    """x = 1 and every sub-block of a block sharing (sc, m): y = sum_b d*sc*sum(q) - 256*dmin*m."""
    g = synth.rng(24, "closed-form")
    n, k = 4, 1024
    w = synth.blob("q4_k", g, n, k).reshape(-1, 144)
    scs = g.integers(0, 64, w.shape[0])
    ms = g.integers(0, 64, w.shape[0])
    for i, (s, m) in enumerate(zip(scs, ms)):
        # six-bit packing of a constant (sc, m): low bits in bytes 0..7, high bits in 6..7
        w[i, 4:8] = (s & 63) | ((s >> 4) << 6)
        w[i, 8:12] = (m & 63) | ((m >> 4) << 6)
        w[i, 12:16] = (s & 15) | ((m & 15) << 4)
    x = np.ones((1, k), np.float32)
    y, _ = oracle.gemv("q4_k", w.reshape(-1), n, k, x)
    d = w[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    dmin = w[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    qsum = (w[:, 16:] & 15).sum(1) + (w[:, 16:] >> 4).sum(1)
    per_block = d * scs * qsum - 256.0 * dmin * ms
    ref = per_block.reshape(n, k // 256).sum(1)
    np.testing.assert_allclose(y[0], ref, rtol=1e-13, atol=1e-13)


def test_swiglu_against_logistic():
    g = synth.rng(25, "swiglu")
    a = synth.normal_f32(g, 4096, 4.0)
    b = synth.normal_f32(g, 4096)
    h = oracle.swiglu(a, b)
    ref = a.astype(np.float64) * expit(a.astype(np.float64)) * b.astype(np.float64)
    np.testing.assert_allclose(h, ref, rtol=1e-14, atol=1e-300)
    lim = oracle.swiglu(np.array([0.0, 800.0, -800.0, 1.0]), np.array([3.0, 2.0, 5.0, 1.0]))
    assert lim[0] == 0.0 and lim[1] == 1600.0 and lim[2] == 0.0
    assert abs(lim[3] - 0.7310585786300049) < 1e-16  # 1 / (1 + e^-1)


def test_router_logits_matmul():
    g = synth.rng(26, "router")
    T, E, H = 5, 8, 512
    x = synth.normal_f32(g, (T, H))
    wr = synth.router_weights(g, E, H)
    lg = oracle.router_logits(x, wr)
    np.testing.assert_allclose(lg, x.astype(np.float64) @ wr.astype(np.float64).T, rtol=1e-12,
                               atol=1e-13)


def _topk_sort(lg, k):
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))  # value desc, index asc
        ids[t] = order[:k]
    return ids


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (5, 5), (1, 1)])
def test_topk_brute_force(E, k):
    g = synth.rng(27, "topk", E, k)
    T = 64
    lg = synth.normal_f32(g, (T, E))
    lg[3, :] = 0.5  # every logit equal
    if E >= 4:
        lg[4, 1] = lg[4, 3] = lg[4].max() + 1  # a tie at the top
    ids, w = oracle.topk(lg, k)
    assert np.array_equal(ids, _topk_sort(lg, k))
    assert np.array_equal(ids[3], np.arange(k))
    np.testing.assert_allclose(w[3], np.full(k, 1.0 / k), rtol=1e-15)
    l64 = lg.astype(np.float64)
    sel = np.take_along_axis(l64, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, softmax(sel, axis=1), rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    _, wfull = oracle.topk(lg, k, renormalize=False)
    np.testing.assert_allclose(wfull, np.take_along_axis(softmax(l64, axis=1),
                                                         ids.astype(np.int64), 1), rtol=1e-13)
    if k == E:
        np.testing.assert_allclose(np.take_along_axis(w, np.argsort(ids, 1), 1),
                                   softmax(l64, axis=1), rtol=1e-13)


def test_topk_fp64_and_fp32_entry_points_agree_on_fp32_values():
    g = synth.rng(28, "topk64")
    lg = synth.normal_f32(g, (32, 16))
    a = oracle.topk(lg, 4)
    b = oracle.topk(lg.astype(np.float64), 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (64, 8, 2), (256, 256, 8), (7, 4, 4)])
def test_group_against_stable_sort(T, E, k):
    g = synth.rng(29, "group", T, E, k)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, pairs = oracle.group(ids, E)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(pairs, np.argsort(flat, kind="stable"))
    assert np.array_equal(np.sort(pairs), np.arange(T * k))
    for e in range(E):
        seg = pairs[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg // k) > 0)


def test_group_all_tokens_on_one_expert_and_empty_experts():
    ids = np.zeros((9, 1), np.int32) + 2
    counts, offsets, pairs = oracle.group(ids, 4)
    assert list(counts) == [0, 0, 9, 0] and list(offsets) == [0, 0, 0, 9, 9]
    assert np.array_equal(pairs, np.arange(9))


def _dense_ffn(t, ex, H, F, x64):
    gate = _dense(t, ex[0], F, H)
    up = _dense(t, ex[1], F, H)
    down = _dense(t, ex[2], H, F)
    gg, uu = gate @ x64, up @ x64
    h = gg * expit(gg) * uu
    return down @ h, np.abs(down) @ np.abs(h)


@pytest.mark.parametrize("t", ["q4_k", "q8_0", "q5_k", "q4_0"])
def test_moe_against_dense_numpy(t):
    H, F, E, k, T = 256, 512, 4, 2, 3
    shape = dict(hidden=H, ffn=F, n_experts=E, shared=True)
    layer = synth.moe_layer(shape, t, seed=31, tag="tiny")
    x = synth.normal_f32(synth.rng(31, "x"), (T, H))
    lg = oracle.router_logits(x, layer["router"])
    ids, wts = oracle.topk(lg.astype(np.float32), k)
    y, mag = oracle.moe(t, H, F, layer["experts"], layer["shared"], x, ids, wts)
    for tt in range(T):
        x64 = x[tt].astype(np.float64)
        ref = np.zeros(H)
        refm = np.zeros(H)
        for j in range(k):
            o, om = _dense_ffn(t, layer["experts"][ids[tt, j]], H, F, x64)
            ref += wts[tt, j] * o
            refm += wts[tt, j] * om
        o, om = _dense_ffn(t, layer["shared"], H, F, x64)
        ref += o
        refm += om
        np.testing.assert_allclose(y[tt], ref, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(mag[tt], refm, rtol=1e-10)
    # token subset, and the shared expert as a separable additive term
    ys, _ = oracle.moe(t, H, F, layer["experts"], layer["shared"], x, ids, wts, tokens=[2, 0])
    assert np.array_equal(ys, y[[2, 0]])
    yn, _ = oracle.moe(t, H, F, layer["experts"], None, x, ids, wts)
    o, _ = _dense_ffn(t, layer["shared"], H, F, x[1].astype(np.float64))
    np.testing.assert_allclose(y[1] - yn[1], o, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("t,shape,k,T", [
    ("q4_k", dict(hidden=256, ffn=512, n_experts=5, shared=True), 2, 7),
    ("q6_k", dict(hidden=512, ffn=256, n_experts=3, shared=False), 3, 4),
    ("q8_0", dict(hidden=256, ffn=256, n_experts=8, shared=True), 4, 9),
])
def test_moe_grouped_equals_token_by_token(t, shape, k, T):
    """The expert-grouped MoE gives the token-by-token MoE's bits: all tokens, a token subset in
    any order (with repeats), and empty experts."""
    layer = synth.moe_layer(shape, t, seed=33, tag=f"grouped-{t}")
    H, F = shape["hidden"], shape["ffn"]
    x = synth.normal_f32(synth.rng(33, "x", t), (T, H))
    ids, wts = oracle.topk(oracle.router_logits(x, layer["router"]).astype(np.float32), k)
    for toks in (None, [T - 1, 0, 2, 0]):
        yg, mg = oracle.moe(t, H, F, layer["experts"], layer["shared"], x, ids, wts, tokens=toks)
        yt, mt = oracle.moe(t, H, F, layer["experts"], layer["shared"], x, ids, wts, tokens=toks,
                            grouped=False)
        assert np.array_equal(yg, yt) and np.array_equal(mg, mt)
    ids0 = np.zeros_like(ids) + np.arange(k, dtype=np.int32)  # experts k.. stay empty
    yg, _ = oracle.moe(t, H, F, layer["experts"], layer["shared"], x, ids0, wts)
    yt, _ = oracle.moe(t, H, F, layer["experts"], layer["shared"], x, ids0, wts, grouped=False)
    assert np.array_equal(yg, yt)


def test_moe_relabelling_experts_leaves_output_unchanged():
    H, F, E, k, T = 256, 256, 4, 2, 4
    layer = synth.moe_layer(dict(hidden=H, ffn=F, n_experts=E), "q4_k", seed=32, tag="perm")
    x = synth.normal_f32(synth.rng(32, "x"), (T, H))
    ids, wts = oracle.topk(oracle.router_logits(x, layer["router"]).astype(np.float32), k)
    y, _ = oracle.moe("q4_k", H, F, layer["experts"], None, x, ids, wts)
    perm = np.array([2, 0, 3, 1])  # new index of old expert e is perm[e]
    experts2 = [None] * E
    for e in range(E):
        experts2[perm[e]] = layer["experts"][e]
    y2, _ = oracle.moe("q4_k", H, F, experts2, None, x, perm[ids].astype(np.int32), wts)
    assert np.array_equal(y, y2)


# ---- the bf16-operand MoE (arithmetic of the matrix-core path) -------------------------------

def _bf16(a):
    """Round to fp32, then to bf16 (nearest even), widened back to fp64 -- torch's conversion."""
    import torch

    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_identity_blob_is_identity():
    from tests import blobs

    for n in (256, 512):
        assert np.array_equal(oracle.dequant("q4_k", blobs.identity(n), n, n), np.eye(n))


def test_moe_bf16_unit_vectors_reduce_to_elementwise_rounding():
    """E = 1, k = 1, down = identity, x_t = s_t e_{c_t}: every product has a single term, so
    y_t[i] = bf16(silu(g) u) with g = bf16(w_gate[i][c]) bf16(s), u likewise."""
    from tests import blobs

    H = F = 256
    g = synth.rng(40, "unit")
    gate, up = synth.blob("q4_k", g, F, H), synth.blob("q4_k", g, F, H)
    T = 6
    cols = np.array([0, 1, 63, 64, 200, 255])
    s = np.array([1.2345678, -3.1415927, 0.1, 7.77, -0.333, 1e-3], np.float32)
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), cols] = s
    ids, wts = np.zeros((T, 1), np.int32), np.ones((T, 1))
    experts = [(gate, up, blobs.identity(H))]
    y, _ = oracle.moe("q4_k", H, F, experts, None, x, ids, wts, bf16=True)
    wg = oracle.dequant("q4_k", gate, F, H)
    wu = oracle.dequant("q4_k", up, F, H)
    for t in range(T):
        gg = _bf16(wg[:, cols[t]]) * _bf16(s[t])
        uu = _bf16(wu[:, cols[t]]) * _bf16(s[t])
        ref = _bf16(gg * expit(gg) * uu)
        assert np.array_equal(y[t], ref), t
    yx, _ = oracle.moe("q4_k", H, F, experts, None, x, ids, wts)
    assert not np.array_equal(y, yx)


def test_moe_bf16_lattice_only_h_is_rounded():
    """Weights 0..15 and x in {-1, 0, 1} are exact in bf16, so the bf16 MoE differs from the fp64
    one only by the rounding of h: |diff| <= (2^-9 + 2^-24) * mag, and it is not zero."""
    from tests import blobs

    H, F, E, k, T = 256, 512, 3, 2, 5
    g = synth.rng(41, "lattice")
    experts = [(blobs.lattice(g, F, H), blobs.lattice(g, F, H), blobs.lattice(g, H, F))
               for _ in range(E)]
    shared = (blobs.lattice(g, F, H), blobs.lattice(g, F, H), blobs.lattice(g, H, F))
    x = synth.ternary_f32(synth.rng(41, "x"), (T, H))
    ids = np.array([[0, 1], [2, 0], [1, 2], [0, 2], [1, 0]], np.int32)
    wts = np.full((T, k), 0.5)
    y, mag = oracle.moe("q4_k", H, F, experts, shared, x, ids, wts)
    yb, magb = oracle.moe("q4_k", H, F, experts, shared, x, ids, wts, bf16=True)
    diff = np.abs(yb - y)
    assert np.all(diff <= (2.0**-9 + 2.0**-24) * mag)
    assert diff.max() > 0
    np.testing.assert_allclose(magb, mag, rtol=2.0**-8)
