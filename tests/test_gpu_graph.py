"""Calls captured into a HIP graph and replayed, against the eager call and the oracle.

A replay runs the recorded launches with the arguments they were captured with, so anything a
kernel expects to find in the workspace must hold on every replay, not just the first. Each test
captures a sequence of calls, replays it a dozen times with eager work in between (other calls on
the same workspace, the workspace overwritten with random bytes, the outputs reset to NaN, a
synchronization), checks every replay bitwise against the eager run, and checks the last replay
against the oracle element by element.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_product_close, assert_swiglu_close, dev, host
from tests.test_gpu_moe import check_moe

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")

REPLAYS = 12


def _case(*a):
    print("case:", *a, flush=True)


def _replays(run, outs, between):
    """Eager run, capture, then REPLAYS replays with `between()` (eager work) before each; every
    replay's outputs must equal the eager run's bits. Returns the last replay's outputs."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
        torch.cuda.synchronize()
        eager = [host(o).copy() for o in outs]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            run()
        got = None
        for r in range(REPLAYS):
            for o in outs:
                o.fill_(float("nan"))
            between(r)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = [host(o).copy() for o in outs]
            for i, (a, b) in enumerate(zip(eager, got)):
                assert np.array_equal(a, b), f"replay {r}: output {i} differs from the eager run"
    return got


def _scramble(ws, g):
    ws.copy_(torch.from_numpy(g.integers(0, 256, ws.numel(), dtype=np.uint8)).to(ws.device))


@pytest.mark.parametrize("batch", [1, 8])
def test_graph_llama8b_layer(batch):
    """One Llama-3-8B-shaped layer as the decode step runs it (q|k|v sharing x, o, gate|up with the
    SwiGLU fused, down reading h), all four calls on one workspace. Batch 1 takes the lanes-along-k
    kernel, batch 8 the k-sliced fp16 matrix-core kernel."""
    _case("graph llama8b layer", batch)
    shape = synth.LLAMA8B
    H, KV, F = shape["hidden"], shape["kv"], shape["ffn"]
    wh = {name: synth.blob("q4_k", synth.rng(71, "graph8b", name), n, k)
          for name, n, k in synth.dense_projections(shape)}
    w = {name: dev(b) for name, b in wh.items()}
    g = synth.rng(71, "graph8b-x", batch)
    xh, ah = synth.normal_f32(g, (batch, H)), synth.normal_f32(g, (batch, H))
    x, a = dev(xh), dev(ah)
    out = {name: torch.empty((batch, n), dtype=torch.float32, device="cuda:0")
           for name, n in (("q", H), ("k", KV), ("v", KV), ("o", H), ("h", F), ("down", H))}
    need = max(tq.gemv_workspace_bytes("q4_k", n, k, batch) for _, n, k in synth.dense_projections(shape))
    need = max(need, int(tq.lib().tq_gemv_swiglu_workspace_bytes(tq.Q4_K, F, H, batch)))
    ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device="cuda:0")
    other_w = dev(synth.blob("q4_k", g, 700, H))
    other_y = torch.empty((batch, 700), dtype=torch.float32, device="cuda:0")

    def run():
        tq.gemv_multi("q4_k", [w["q"], w["k"], w["v"]], [H, KV, KV], H, x,
                      outs=[out["q"], out["k"], out["v"]], ws=ws)
        tq.gemv("q4_k", w["o"], H, H, a, out=out["o"], ws=ws)
        tq.gemv_swiglu("q4_k", w["gate"], w["up"], F, H, x, out=out["h"], ws=ws)
        tq.gemv("q4_k", w["down"], H, F, out["h"], out=out["down"], ws=ws)

    def between(r):
        if r % 2:
            _scramble(ws, g)
        else:
            tq.gemv("q4_k", other_w, 700, H, x, out=other_y, ws=ws)

    names = ("q", "k", "v", "o", "h", "down")
    got = dict(zip(names, _replays(run, [out[n] for n in names], between)))
    rows = {name: n for name, n, _ in synth.dense_projections(shape)}
    for name in ("q", "k", "v", "o"):
        src = ah if name == "o" else xh
        ref, mag = oracle.gemv("q4_k", wh[name], rows[name], H, src)
        assert_product_close(got[name], ref, mag, what=f"{name} (last replay)")
    gref, gm = oracle.gemv("q4_k", wh["gate"], F, H, xh)
    uref, um = oracle.gemv("q4_k", wh["up"], F, H, xh)
    assert_swiglu_close(got["h"], gref, gm, uref, um, what="gate|up + SwiGLU (last replay)")
    ref, mag = oracle.gemv("q4_k", wh["down"], H, F, got["h"])
    assert_product_close(got["down"], ref, mag, what="down (last replay)")


K_SPLIT = [("q4_k", 600, 16384, 1),   # fp16 matrix cores (Q4_K), k slices
           ("q4_k", 900, 4096, 8),    # fp16 matrix cores, k slices
           ("q8_0", 500, 8192, 4),    # fp32 matrix cores, k slices
           ("q8_0", 700, 8192, 1),    # int8 matrix cores (Q8_0), k slices
           ("q6_k", 400, 8192, 1),    # fp16 matrix cores (Q6_K)
           ("q6_k", 300, 16384, 1),   # fp16 matrix cores (Q6_K), two k slices
           ("q6_k", 200, 4096, 3),    # fp32 matrix cores, 4-token form, k slices
           ("q4_0", 200, 8192, 3)]    # lane-per-row GEMV, 3 tokens, k split


def test_graph_k_split_kernels_share_a_workspace():
    """Every kernel that adds k slices through completion counters, captured as one graph of one
    call each on one workspace; the workspace is overwritten with random bytes before every replay."""
    _case("graph k-split kernels")
    g = synth.rng(72, "graph-split")
    cases = []
    need = 0
    for t, n, k, b in K_SPLIT:
        wb = synth.blob(t, g, n, k)
        xb = synth.normal_f32(g, (b, k))
        cases.append((t, n, k, b, wb, xb, dev(wb), dev(xb),
                      torch.empty((b, n), dtype=torch.float32, device="cuda:0")))
        need = max(need, tq.gemv_workspace_bytes(t, n, k, b))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")

    def run():
        for t, n, k, b, _, _, wd, xd, y in cases:
            tq.gemv(t, wd, n, k, xd, out=y, ws=ws)

    got = _replays(run, [c[-1] for c in cases], lambda r: _scramble(ws, g))
    for (t, n, k, b, wb, xb, *_), y in zip(cases, got):
        ref, mag = oracle.gemv(t, wb, n, k, xb)
        assert_product_close(y, ref, mag, what=f"{t} {n}x{k} b{b} (last replay)")


@pytest.mark.parametrize("name,shape,T", [("deepseek", synth.DEEPSEEK, 1),
                                          ("mixtral", synth.MIXTRAL, 16)])
def test_graph_moe_layer(name, shape, T):
    """A full-size MoE layer call (routing, grouping, expert FFNs, combine; the shared expert
    for DeepSeek) with its routing outputs, captured and replayed; between replays the same
    workspace serves an eager call on other activations. Routing bitwise and y against the
    oracle on the last replay."""
    _case("graph moe", name, T)
    k, E, Hd = shape["top_k"], shape["n_experts"], shape["hidden"]
    layer = synth.moe_layer(shape, "q4_k", tag=name)
    experts = [tuple(dev(b) for b in e) for e in layer["experts"]]
    shared = tuple(dev(b) for b in layer["shared"]) if layer["shared"] is not None else None
    moe = tq.MoeLayer("q4_k", Hd, shape["ffn"], dev(layer["router"]), experts, shared, top_k=k,
                      path=tq.PATH_F32)
    xh = synth.normal_f32(synth.rng(73, "graph-moe", name, T), (T, Hd))
    x = dev(xh)
    x2 = dev(synth.normal_f32(synth.rng(73, "graph-moe-2", name, T), (T, Hd)))
    y = torch.empty_like(x)
    y2 = torch.empty_like(x)
    ws = torch.zeros(moe.workspace_bytes(T), dtype=torch.uint8, device="cuda:0")
    r = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device="cuda:0"),
             topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda:0"),
             logits=torch.empty((T, E), dtype=torch.float32, device="cuda:0"),
             counts=torch.empty(E, dtype=torch.int32, device="cuda:0"),
             offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda:0"),
             pairs=torch.empty(T * k, dtype=torch.int32, device="cuda:0"))

    def run():
        moe(x, out=y, ws=ws, routing=r)

    def between(_):
        moe(x2, out=y2, ws=ws)

    outs = [y] + [r[f] for f in ("logits", "topk_w")]
    for f in ("topk_ids", "counts", "offsets", "pairs"):
        r[f].fill_(-1)
    got = _replays(run, outs, between)
    ids = host(r["topk_ids"])
    # the last replay against the oracle: routing from its logits, y every element
    ref_ids, ref_w = oracle.topk(got[1], k, True)
    assert np.array_equal(ids, ref_ids)
    assert np.all(np.abs(got[2] - ref_w) <= 1e-5 * ref_w + 1e-7)
    counts, offsets, pairs = oracle.group(ids, E)
    assert np.array_equal(host(r["counts"]), counts) and np.array_equal(host(r["offsets"]), offsets)
    assert np.array_equal(host(r["pairs"]), pairs)
    ref, mag = oracle.moe("q4_k", Hd, shape["ffn"], layer["experts"], layer["shared"], xh, ids,
                          ref_w)
    assert_product_close(got[0], ref, mag, what=f"{name} T={T} (last replay)")
    # and the eager path on the same inputs agrees with the oracle too (routing bitwise)
    check_moe("q4_k", shape, layer, xh, k, moe=moe)
