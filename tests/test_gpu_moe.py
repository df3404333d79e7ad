"""GPU parity of tq_moe_ffn (router, top-k, grouping, grouped expert FFN, combine) vs the oracle.

Contract checked here:
  * router logits within 1e-3 * sum|x w| + 1e-5 of the oracle's fp64 logits;
  * selection: the oracle's top-k re-run on the GPU's fp32 logits gives the same ids, bitwise;
    weights within 1e-5 * w + 1e-7; with the oracle's own fp64 logits only near ties may differ;
  * grouping (counts, offsets, pairs) bitwise equal to the oracle's grouping of the GPU ids;
  * y within 1e-3 * sum|products| + 1e-5 of the oracle MoE evaluated with that routing;
  * bitwise determinism across calls.
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


def _layer_to_device(t, shape, layer, top_k, renormalize=True, path=0):
    experts = [tuple(dev(b) for b in e) for e in layer["experts"]]
    shared = tuple(dev(b) for b in layer["shared"]) if layer["shared"] is not None else None
    moe = tq.MoeLayer(t, shape["hidden"], shape["ffn"], dev(layer["router"]), experts, shared,
                      top_k=top_k, renormalize=renormalize, path=path)
    return moe


def _run(moe, x, E, k):
    T = x.shape[0]
    r = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device="cuda:0"),
             topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda:0"),
             logits=torch.empty((T, E), dtype=torch.float32, device="cuda:0"),
             counts=torch.empty(E, dtype=torch.int32, device="cuda:0"),
             offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda:0"),
             pairs=torch.empty(T * k, dtype=torch.int32, device="cuda:0"))
    y = moe(dev(x), routing=r)
    return host(y), {f: host(v) for f, v in r.items()}


def check_moe(t, shape, layer, x, k, tokens=None, renormalize=True, moe=None, rel=1e-3, path=0,
              bf16=False):
    """Routing bitwise, y within rel * mag + 1e-5 of the oracle (its bf16-operand variant when
    bf16 is set); returns (layer, y, stats) where stats = (largest err / bound, relative L2 error
    of the checked rows)."""
    E = len(layer["experts"])
    moe = moe or _layer_to_device(t, shape, layer, k, renormalize, path)
    y, r = _run(moe, x, E, k)
    T = x.shape[0]
    # logits
    ref_lg = oracle.router_logits(x, layer["router"])
    mag_lg = np.abs(x.astype(np.float64)) @ np.abs(layer["router"].astype(np.float64)).T
    assert_product_close(r["logits"], ref_lg, mag_lg, what="router logits")
    # selection on the GPU's fp32 logits: bitwise
    ids, wts = oracle.topk(r["logits"], k, renormalize)
    assert np.array_equal(r["topk_ids"], ids), "top-k ids"
    assert np.all(np.abs(r["topk_w"] - wts) <= 1e-5 * wts + 1e-7), "routing weights"
    # selection on the oracle's own logits: differences only at near ties
    own, _ = oracle.topk(ref_lg, k, renormalize)
    diff = np.any(np.sort(own, 1) != np.sort(ids, 1), axis=1)
    if diff.any() and k < E:
        srt = np.sort(ref_lg, 1)[:, ::-1]
        gap = srt[:, k - 1] - srt[:, k]
        scale = np.max(mag_lg, axis=1)
        assert np.all(gap[diff] < 1e-4 * scale[diff]), "selection differs beyond a near tie"
    # grouping: bitwise
    counts, offsets, pairs = oracle.group(ids, E)
    assert np.array_equal(r["counts"], counts) and np.array_equal(r["offsets"], offsets)
    assert np.array_equal(r["pairs"], pairs)
    # output, with the GPU's routing and oracle weights from the GPU's logits
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    ref, mag = oracle.moe(t, shape["hidden"], shape["ffn"], layer["experts"], layer["shared"], x,
                          ids, wts, tokens=toks, bf16=bf16)
    worst = assert_product_close(y[toks], ref, mag, rel=rel, what=f"moe {t} T={T}")
    l2 = float(np.linalg.norm(y[toks] - ref) / max(np.linalg.norm(ref), 1e-30))
    return moe, y, (worst, l2)


SMALL = [
    ("q4_k", dict(hidden=512, ffn=1024, n_experts=8, shared=False), 2, [1, 5, 64, 130]),
    ("q4_k", dict(hidden=768, ffn=512, n_experts=16, shared=True), 4, [1, 33]),
    ("q8_0", dict(hidden=512, ffn=768, n_experts=6, shared=True), 2, [3, 70]),
    ("q6_k", dict(hidden=1024, ffn=512, n_experts=5, shared=False), 3, [2, 65]),
    ("q5_k", dict(hidden=512, ffn=768, n_experts=6, shared=True), 2, [1, 3, 40]),
    ("q4_0", dict(hidden=768, ffn=512, n_experts=8, shared=False), 2, [1, 5, 33]),
]


@pytest.mark.parametrize("t,shape,k,Ts", SMALL, ids=lambda v: str(v)[:24])
def test_moe_small_shapes(t, shape, k, Ts):
    layer = synth.moe_layer(shape, t, seed=201, tag=f"small-{t}")
    moe = None
    for T in Ts:
        _case("moe-small", t, shape, k, T)
        x = synth.normal_f32(synth.rng(201, "x", t, T), (T, shape["hidden"]))
        moe, y, _ = check_moe(t, shape, layer, x, k, moe=moe)
        y2, _ = _run(moe, x, shape["n_experts"], k)
        assert np.array_equal(y, y2), "not deterministic"


def test_moe_not_renormalized():
    t, shape, k = "q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=False), 2
    layer = synth.moe_layer(shape, t, seed=202, tag="norenorm")
    x = synth.normal_f32(synth.rng(202, "x"), (9, 512))
    check_moe(t, shape, layer, x, k, renormalize=False)


def test_moe_equal_logits_all_tokens_on_first_experts():
    """A zero router: every logit ties, so every token picks experts 0..k-1 with weight 1/k."""
    t, shape, k = "q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=True), 2
    layer = synth.moe_layer(shape, t, seed=203, tag="ties")
    layer["router"] = np.zeros_like(layer["router"])
    x = synth.normal_f32(synth.rng(203, "x"), (70, 512))
    moe, _, _ = check_moe(t, shape, layer, x, k)
    _, r = _run(moe, x, 8, k)
    assert np.all(r["topk_ids"] == np.arange(k)) and np.allclose(r["topk_w"], 0.5)
    assert list(r["counts"]) == [70, 70, 0, 0, 0, 0, 0, 0]


def test_moe_single_expert_equals_dense_ffn():
    """E = 1, k = 1: the layer is one SwiGLU FFN; compare with tq_gemv + tq_swiglu + tq_gemv."""
    t, shape = "q4_k", dict(hidden=512, ffn=1024, n_experts=1, shared=False)
    layer = synth.moe_layer(shape, t, seed=204, tag="one")
    x = synth.normal_f32(synth.rng(204, "x"), (5, 512))
    _, y, _ = check_moe(t, shape, layer, x, 1)
    g, u, d = (dev(b) for b in layer["experts"][0])
    xd = dev(x)
    hg = tq.gemv(t, g, 1024, 512, xd)
    hu = tq.gemv(t, u, 1024, 512, xd)
    yd = host(tq.gemv(t, d, 512, 1024, tq.swiglu(hg, hu)))
    ref, mag = oracle.moe(t, 512, 1024, layer["experts"], None, x, np.zeros((5, 1), np.int32),
                          np.ones((5, 1)))
    assert_product_close(yd, ref, mag, what="chained dense")
    assert_product_close(y, ref, mag, what="moe E=1")


def test_moe_top_k_equals_n_experts():
    t, shape = "q4_k", dict(hidden=512, ffn=512, n_experts=4, shared=False)
    layer = synth.moe_layer(shape, t, seed=205, tag="dense-mix")
    x = synth.normal_f32(synth.rng(205, "x"), (17, 512))
    check_moe(t, shape, layer, x, 4)


def test_moe_rejects_bad_arguments():
    t, shape = "q4_k", dict(hidden=512, ffn=512, n_experts=4, shared=False)
    layer = synth.moe_layer(shape, t, seed=206, tag="bad")
    moe = _layer_to_device(t, shape, layer, 2)
    x = dev(synth.normal_f32(synth.rng(206, "x"), (3, 512)))
    small = torch.empty(256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(tq.TQError) as e:
        moe(x, ws=small)
    assert e.value.status == 4
    moe.desc.top_k = 5
    with pytest.raises(tq.TQError) as e:
        moe(x)
    assert e.value.status == 2


NAN_CASES = [(dict(hidden=512, ffn=512, n_experts=8, shared=True), 2, T) for T in (1, 5)] + \
            [(dict(hidden=256, ffn=256, n_experts=256, shared=False), 8, T) for T in (1, 9)]


@pytest.mark.parametrize("shape,k,T", NAN_CASES, ids=lambda v: str(v)[:24])
def test_moe_nan_activation_routes_in_range(shape, k, T):
    """A NaN in one token's activations makes all its logits NaN. NaN ranks below every number,
    so that token takes experts 0..k-1 (ties go to the lower id), its weights and output row are
    NaN, and every other token's routing and output are those of the oracle."""
    t, E = "q4_k", shape["n_experts"]
    _case("moe nan activation", E, k, T)
    layer = synth.moe_layer(shape, t, seed=230, tag=f"nan-{E}")
    x = synth.normal_f32(synth.rng(230, "x", E, T), (T, shape["hidden"]))
    bad = T // 2
    x[bad, 7] = np.nan
    moe = _layer_to_device(t, shape, layer, k)
    y, r = _run(moe, x, E, k)
    ids = r["topk_ids"]
    assert np.all((ids >= 0) & (ids < E)), "expert id out of range"
    assert np.array_equal(ids[bad], np.arange(k)), "NaN token's experts"
    assert np.all(np.isnan(r["topk_w"][bad])) and np.all(np.isnan(y[bad]))
    counts, offsets, pairs = oracle.group(ids, E)
    assert np.array_equal(r["counts"], counts) and np.array_equal(r["offsets"], offsets)
    assert np.array_equal(r["pairs"], pairs)
    ok = np.array([i for i in range(T) if i != bad], dtype=np.int64)
    if ok.size:
        ref_ids, ref_w = oracle.topk(r["logits"][ok], k)
        assert np.array_equal(ids[ok], ref_ids)
        assert np.all(np.abs(r["topk_w"][ok] - ref_w) <= 1e-5 * ref_w + 1e-7)
        wts = np.zeros((T, k))
        wts[ok] = ref_w
        ref, mag = oracle.moe(t, shape["hidden"], shape["ffn"], layer["experts"], layer["shared"],
                              x, ids, wts, tokens=ok)
        assert_product_close(y[ok], ref, mag, what="tokens without NaN")


def test_moe_nan_router_row_never_chosen():
    """One expert's router row is NaN: its logit is NaN for every token and ranks below every
    number, so it is never chosen; the routing and output equal the oracle's with that logit
    taken as -inf."""
    t, shape, k, E, T = "q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=True), 2, 8, 40
    layer = synth.moe_layer(shape, t, seed=231, tag="nan-row")
    layer["router"][3, 100] = np.nan
    x = synth.normal_f32(synth.rng(231, "x"), (T, 512))
    moe = _layer_to_device(t, shape, layer, k)
    y, r = _run(moe, x, E, k)
    assert np.all(np.isnan(r["logits"][:, 3]))
    lg = np.where(np.isnan(r["logits"]), -np.inf, r["logits"]).astype(np.float32)
    ref_ids, ref_w = oracle.topk(lg, k)
    assert not np.any(ref_ids == 3)
    assert np.array_equal(r["topk_ids"], ref_ids)
    assert np.all(np.abs(r["topk_w"] - ref_w) <= 1e-5 * ref_w + 1e-7)
    ref, mag = oracle.moe(t, 512, 512, layer["experts"], layer["shared"], x, ref_ids, ref_w)
    assert_product_close(y, ref, mag, what="moe with a NaN router row")


# ---- full-size layers, sampled tokens --------------------------------------------------------


@pytest.fixture(scope="module")
def mixtral():
    return synth.moe_layer(synth.MIXTRAL, "q4_k", tag="mixtral")


@pytest.mark.parametrize("T", [1, 16, 64])
def test_moe_mixtral_shape_every_token(mixtral, T):
    """Full-size Mixtral-shaped layer: every output element of every token against the oracle
    (its expert-grouped form, which decodes each expert once for all its tokens)."""
    _case("mixtral", T)
    x = synth.normal_f32(synth.rng(synth.DEFAULT_SEED, "mixtral-x", T), (T, 4096))
    check_moe("q4_k", synth.MIXTRAL, mixtral, x, 2)


@pytest.fixture(scope="module")
def deepseek():
    return synth.moe_layer(synth.DEEPSEEK, "q4_k", tag="deepseek")


@pytest.mark.parametrize("T", [1, 256])
def test_moe_deepseek_shape_every_token(deepseek, T):
    """Full-size DeepSeek-shaped layer (256 routed experts + shared): every output element of
    every token against the oracle."""
    _case("deepseek", T)
    x = synth.normal_f32(synth.rng(synth.DEFAULT_SEED, "deepseek-x", T), (T, 7168))
    check_moe("q4_k", synth.DEEPSEEK, deepseek, x, 8)


@pytest.mark.parametrize("path", [0, 2], ids=["auto-f32", "bf16-mfma"])
def test_moe_stages_equal_one_call(path):
    """tq_moe_ffn_stages: route, experts and combine as three calls on one workspace give the
    one-call result bitwise."""
    t, shape, k, T = "q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=True), 2, 300
    layer = synth.moe_layer(shape, t, seed=207, tag="stages")
    moe = _layer_to_device(t, shape, layer, k, path=path)
    x = dev(synth.normal_f32(synth.rng(207, "x"), (T, 512)))
    y_all = host(moe(x))
    ws = torch.zeros(moe.workspace_bytes(T), dtype=torch.uint8, device="cuda:0")
    moe(x, ws=ws, stages=tq.MOE_ROUTE)
    moe(x, ws=ws, stages=tq.MOE_EXPERTS)
    y = torch.full_like(x, float("nan"))
    moe(x, out=y, ws=ws, stages=tq.MOE_COMBINE)
    assert np.array_equal(host(y), y_all)
    moe(x, out=y, ws=ws, stages=tq.MOE_ROUTE | tq.MOE_EXPERTS)
    y2 = moe(x, ws=ws, stages=tq.MOE_COMBINE)
    assert np.array_equal(host(y2), y_all)


def test_moe_grouping_many_tokens_many_experts():
    """T = 8192 tokens, E = 256, k = 8: 65536 pairs through the grouping kernel (its LDS tables
    exceed 64 KB here), routing checked bitwise, output on sampled tokens (fp32 path)."""
    shape = dict(hidden=256, ffn=256, n_experts=256, shared=True)
    layer = synth.moe_layer(shape, "q4_k", seed=208, tag="many")
    x = synth.normal_f32(synth.rng(208, "x"), (8192, 256))
    check_moe("q4_k", shape, layer, x, 8, tokens=[0, 4095, 8191], path=tq.PATH_F32)


def test_moe_one_token_lane_groups_bitwise(knobs):
    """One-token Q4_K steps with k <= 2048 per product (hidden 2048: gate/up in 2 lane groups per
    wave; ffn 1024: down in 4) give bitwise the whole-wave results (TQ_KNOB_KL_GROUPS = 1)."""
    t, shape, k = "q4_k", dict(hidden=2048, ffn=1024, n_experts=8, shared=True), 2
    layer = synth.moe_layer(shape, t, seed=215, tag="kl-groups")
    x = synth.normal_f32(synth.rng(215, "x"), (1, shape["hidden"]))
    _case("moe-kl-groups", shape, k)
    knobs("moe_mf", 0)  # the lanes-along-k kernel
    moe, y, _ = check_moe(t, shape, layer, x, k)
    knobs("kl_groups", 1)
    y1, _ = _run(moe, x, shape["n_experts"], k)
    assert np.array_equal(y, y1)


@pytest.mark.parametrize("shape,k", [(dict(hidden=768, ffn=512, n_experts=16, shared=True), 4),
                                     (dict(hidden=512, ffn=1024, n_experts=8, shared=False), 2),
                                     (dict(hidden=1024, ffn=512, n_experts=300, shared=True), 8)])
def test_moe_one_token_grouping_in_topk_equals_group_kernel(knobs, shape, k):
    """For one token the top-k wave writes the grouping itself; it must equal the grouping
    kernel's (TQ_KNOB_GROUP1 = 0) bit for bit, and so must the layer output."""
    _case("group1", shape, k)
    t = "q4_k"
    layer = synth.moe_layer(shape, t, seed=231, tag="group1")
    x = synth.normal_f32(synth.rng(231, "x", shape["n_experts"]), (1, shape["hidden"]))
    moe = _layer_to_device(t, shape, layer, k)
    E = shape["n_experts"]
    y1, r1 = _run(moe, x, E, k)
    knobs("group1", 0)
    y0, r0 = _run(moe, x, E, k)
    for f in ("topk_ids", "counts", "offsets", "pairs"):
        assert np.array_equal(r1[f], r0[f]), f
    assert np.array_equal(y1, y0)
    knobs("group1", -1)
    check_moe(t, shape, layer, x, k, moe=moe)


def test_moe_router_weights_not_16_byte_aligned():
    """Router weights must be 16-byte aligned (the decode-sized router reads them 16 bytes at a
    time): tq_moe_ffn rejects others with TQ_EINVAL before launching anything."""
    t, shape, k = "q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=False), 2
    layer = synth.moe_layer(shape, t, seed=232, tag="misaligned")
    E, H = shape["n_experts"], shape["hidden"]
    buf = torch.zeros(E * H + 1, dtype=torch.float32, device="cuda:0")
    buf[1:] = dev(layer["router"]).reshape(-1)
    router = buf[1:].view(E, H)  # 4 bytes past a 256-byte boundary
    assert router.data_ptr() % 16 == 4
    experts = [tuple(dev(b) for b in e) for e in layer["experts"]]
    moe = tq.MoeLayer(t, H, shape["ffn"], router, experts, None, top_k=k)
    x = dev(synth.normal_f32(synth.rng(232, "x"), (3, H)))
    y = torch.full((3, H), 7.0, device="cuda:0")
    with pytest.raises(tq.TQError) as err:
        moe(x, out=y)
    assert "router_w" in str(err.value)
    assert bool(torch.all(y == 7.0))  # nothing was launched


@pytest.mark.parametrize("mf", ["1", "0"], ids=["matrix-cores", "vector"])
def test_moe_router_many_tokens_ragged_tiles(knobs, mf):
    """T = 130 tokens and E = 300 experts: neither fills whole 64 x 64 tiles of the matrix-core
    router (rows clamped on load, not stored); its logits and the vector router's both meet the
    oracle's bar, and routing and grouping follow bitwise."""
    knobs("router_mf", int(mf))
    t, shape, k = "q4_k", dict(hidden=1024, ffn=256, n_experts=300, shared=True), 8
    _case("router-ragged", mf, shape, k)
    layer = synth.moe_layer(shape, t, seed=233, tag="router-ragged")
    x = synth.normal_f32(synth.rng(233, "x"), (130, shape["hidden"]))
    check_moe(t, shape, layer, x, k, tokens=[0, 63, 64, 127, 128, 129])


def test_moe_router_hidden_slices_not_whole_blocks():
    """T = 8192, E = 320, hidden 1280: the matrix-core router runs 640 tiles in 4 hidden slices
    of 320 values (20 steps of 16, not whole 256-value blocks)."""
    t, shape, k = "q4_k", dict(hidden=1280, ffn=256, n_experts=320, shared=False), 2
    _case("router-slices", shape, k)
    layer = synth.moe_layer(shape, t, seed=234, tag="router-slices")
    x = synth.normal_f32(synth.rng(234, "x"), (8192, shape["hidden"]))
    check_moe(t, shape, layer, x, k, tokens=[0, 4097, 8191], path=tq.PATH_F32)


@pytest.mark.parametrize("T,path", [(1, 0), (33, 0), (33, 1), (300, 2)],
                         ids=["T1", "T33-auto", "T33-f32", "T300-bf16"])
def test_moe_combine_column_runs_bitwise(knobs, T, path):
    """The combine with a workgroup per token and 16-byte column runs gives bitwise the
    element-wise combine's output (TQ_KNOB_COMBINE4 = 0); an output 4 bytes off 16-byte alignment takes
    the element-wise combine and gives the same bits."""
    t, shape, k = "q4_k", dict(hidden=768, ffn=512, n_experts=16, shared=True), 4
    _case("combine4", T, path)
    layer = synth.moe_layer(shape, t, seed=235, tag="combine4")
    x = synth.normal_f32(synth.rng(235, "x", T), (T, shape["hidden"]))
    moe = _layer_to_device(t, shape, layer, k, path=path)
    xd = dev(x)
    y4 = host(moe(xd))
    knobs("combine4", 0)
    y1 = host(moe(xd))
    knobs("combine4", -1)
    assert np.array_equal(y4, y1)
    buf = torch.empty(T * shape["hidden"] + 1, dtype=torch.float32, device="cuda:0")
    out = buf[1:].view(T, shape["hidden"])
    assert out.data_ptr() % 16 == 4
    moe(xd, out=out)
    assert np.array_equal(host(out), y4)
    if path != 2:  # the bf16 path's parity is covered by the prefill tests
        check_moe(t, shape, layer, x, k, moe=moe, tokens=[0, T - 1])


@pytest.mark.parametrize("shape,k", [(dict(hidden=768, ffn=512, n_experts=16, shared=True), 4),
                                     (dict(hidden=2048, ffn=1024, n_experts=8, shared=False), 2),
                                     (dict(hidden=1024, ffn=512, n_experts=300, shared=True), 8)])
def test_moe_one_token_combine_in_down_launch_bitwise(knobs, shape, k):
    """One token, every stage in one call: the last down workgroup of each row range adds the
    slots (counters cleared by the gate/up launch of the same call). Bitwise equal to the separate
    combine (TQ_KNOB_FUSE_COMBINE = 0) and to a call split into stages, on three calls in a row with
    different tokens, and within the oracle's bar."""
    t = "q4_k"
    _case("fused-combine", shape, k)
    layer = synth.moe_layer(shape, t, seed=236, tag="fused-combine")
    moe = _layer_to_device(t, shape, layer, k)
    E = shape["n_experts"]
    ws = torch.empty(moe.workspace_bytes(1), dtype=torch.uint8, device="cuda:0")
    for i in range(3):
        x = synth.normal_f32(synth.rng(236, "x", i), (1, shape["hidden"]))
        xd = dev(x)
        y_f = host(moe(xd, ws=ws))
        knobs("fuse_combine", 0)
        y_s = host(moe(xd, ws=ws))
        knobs("fuse_combine", -1)
        assert np.array_equal(y_f, y_s), f"call {i}"
        y_st = torch.full_like(xd, float("nan"))
        moe(xd, out=y_st, ws=ws, stages=tq.MOE_ROUTE)
        moe(xd, out=y_st, ws=ws, stages=tq.MOE_EXPERTS | tq.MOE_COMBINE)
        assert np.array_equal(host(y_st), y_f), f"stages, call {i}"
        if i == 2:
            check_moe(t, shape, layer, x, k, moe=moe)
