"""GPU parity of the persistent decode chain (tq_chain_prepare / tq_chain_run).

Every output row of every op of a chain is checked against the oracle on the input the GPU
actually read: |err| <= 1e-3 * sum|w x| + 1e-5 for products, and for a fused SwiGLU op the same
bar carried through silu(g) * u (|d silu / dz| <= 1.1). Chains where an op's input is the previous
op's output check that the device-side dependency waits order the work: the outputs start as NaN,
so an op that read its input too early would not match. Runs are bitwise repeatable.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_product_close, assert_swiglu_close, dev, host

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="the persistent chain is switched off (tq_chain_run returns "
                            "TQ_EUNSUPPORTED): a run of its timing workload left the GPU hung; "
                            "its device-side waits need every workgroup resident at once, which a "
                            "plain launch does not guarantee"),
]

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


def _case(*a):
    print("case:", *a, flush=True)


def _nan(n):
    return torch.full((n,), float("nan"), dtype=torch.float32, device="cuda:0")


def _blob(tag, n, k):
    return synth.blob("q4_k", synth.rng(61, "chain", tag, n, k), n, k)


def _check_chain(ops, blobs):
    """ops: the dicts given to tq.Chain; blobs: the host blobs of each op's matrices."""
    for i, (op, bl) in enumerate(zip(ops, blobs)):
        x = host(op["x"]).reshape(1, -1)
        k = op["k"]
        if op.get("swiglu"):
            n = op["n"][0]
            g, mg = oracle.gemv("q4_k", bl[0], n, k, x)
            u, mu = oracle.gemv("q4_k", bl[1], n, k, x)
            h = host(op["y"][0]).reshape(1, -1)
            assert_swiglu_close(h, g, mg, u, mu, what=f"op {i} swiglu")
        else:
            for p, (n, b) in enumerate(zip(op["n"], bl)):
                got = host(op["y"][p]).reshape(1, -1)
                ref, mag = oracle.gemv("q4_k", b, n, k, x)
                assert_product_close(got, ref, mag, what=f"op {i} part {p}")


def _dependent_chain():
    """k from one block (fewer blocks than multiplying waves) to 64 (the largest), ragged row
    counts, multi-matrix and SwiGLU ops, where ops 1-3 read the previous op's output."""
    ops, blobs = [], []
    x0 = dev(synth.normal_f32(synth.rng(61, "x0"), (1024,)))
    b = [_blob("a", 256, 1024), _blob("b", 130, 1024)]
    y0 = [_nan(256), _nan(130)]
    ops.append(dict(w=[dev(a) for a in b], n=[256, 130], y=y0, k=1024, x=x0))
    blobs.append(b)
    b = [_blob("c", 512, 256)]
    y1 = [_nan(512)]
    ops.append(dict(w=[dev(b[0])], n=[512], y=y1, k=256, x=y0[0]))            # x = op 0's output
    blobs.append(b)
    b = [_blob("g", 768, 512), _blob("u", 768, 512)]
    h = _nan(768)
    ops.append(dict(w=[dev(a) for a in b], n=[768, 768], y=[h], k=512, x=y1[0], swiglu=True))
    blobs.append(b)
    b = [_blob("d", 301, 768)]
    ops.append(dict(w=[dev(b[0])], n=[301], y=[_nan(301)], k=768, x=h))     # x = the SwiGLU output
    blobs.append(b)
    for tag, n, k in (("e", 100, 4608), ("f", 70, 8192), ("h", 37, 14336), ("i", 9, 16384)):
        b = [_blob(tag, n, k)]
        ops.append(dict(w=[dev(b[0])], n=[n], y=[_nan(n)], k=k,
                        x=dev(synth.normal_f32(synth.rng(61, "x", tag), (k,)))))
        blobs.append(b)
    b = [_blob("p", 40, 4096), _blob("q", 3, 4096), _blob("r", 17, 4096), _blob("s", 64, 4096)]
    ops.append(dict(w=[dev(a) for a in b], n=[40, 3, 17, 64], y=[_nan(n) for n in (40, 3, 17, 64)],
                    k=4096, x=dev(synth.normal_f32(synth.rng(61, "x4"), (4096,)))))
    blobs.append(b)
    return ops, blobs


def test_chain_dependent_ops():
    _case("chain dependent ops")
    ops, blobs = _dependent_chain()
    ch = tq.Chain("q4_k", ops)
    ch.run()
    assert ch.status() == 0, ch.last_error
    _check_chain(ops, blobs)


def test_chain_repeat_bitwise():
    """Fifty runs of one chain give the same bits (outputs reset to NaN between runs)."""
    _case("chain repeat")
    ops, _ = _dependent_chain()
    ch = tq.Chain("q4_k", ops)
    ch.run()
    first = [host(y).copy() for op in ops for y in op["y"]]
    for r in range(50):
        for op in ops:
            for y in op["y"]:
                y.fill_(float("nan"))
        ch.run()
        got = [host(y) for op in ops for y in op["y"]]
        for a, b in zip(first, got):
            assert np.array_equal(a, b), f"run {r + 1} differs"
    assert ch.status() == 0, ch.last_error


def _layer_ops(layer, bufs, H=4096, F=14336):
    """The four ops of one Llama-3-8B-shaped layer: q|k|v (x), o (a), gate|up + SwiGLU (x), down (h)."""
    w, x, a = layer
    return [
        dict(w=[w["q"], w["k"], w["v"]], n=[H, 1024, 1024], y=[bufs["q"], bufs["k"], bufs["v"]], k=H, x=x),
        dict(w=[w["o"]], n=[H], y=[bufs["o"]], k=H, x=a),
        dict(w=[w["gate"], w["up"]], n=[F, F], y=[bufs["h"]], k=H, x=x, swiglu=True),
        dict(w=[w["down"]], n=[H], y=[bufs["down"]], k=F, x=bufs["h"]),
    ]


def test_chain_llama8b_two_layers_every_row():
    """Two Llama-3-8B-shaped layers (eight ops, the second layer waiting on the first's down
    projection), every output row of every op against the oracle. The second layer's outputs are
    checked; the first layer's are overwritten."""
    _case("chain llama8b 2 layers")
    shape = synth.LLAMA8B
    layers, hosts = [], []
    for li in range(2):
        wh = {name: synth.blob("q4_k", synth.rng(62, "8b", li, name), n, k)
              for name, n, k in synth.dense_projections(shape)}
        g = synth.rng(62, "8b-x", li)
        x = dev(synth.normal_f32(g, (4096,)))
        a = dev(synth.normal_f32(g, (4096,)))
        layers.append(({k_: dev(v) for k_, v in wh.items()}, x, a))
        hosts.append(wh)
    bufs = {name: _nan(n) for name, n in (("q", 4096), ("k", 1024), ("v", 1024), ("o", 4096),
                                          ("h", 14336), ("down", 4096))}
    ops = _layer_ops(layers[0], bufs) + _layer_ops(layers[1], bufs)
    ch = tq.Chain("q4_k", ops)
    ch.run()
    assert ch.status() == 0, ch.last_error
    wh = hosts[1]
    blobs = [[wh["q"], wh["k"], wh["v"]], [wh["o"]], [wh["gate"], wh["up"]], [wh["down"]]]
    _check_chain(ops[4:], blobs)


def test_chain_graph_replay():
    """The run (counter reset + persistent kernel) captured into a HIP graph and replayed ten
    times, with eager work and synchronisations in between: every replay equals the eager run."""
    _case("chain graph replay")
    ops, _ = _dependent_chain()
    ch = tq.Chain("q4_k", ops)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ch.run()
        torch.cuda.synchronize()
        ref = [host(y).copy() for op in ops for y in op["y"]]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            ch.run()
        for r in range(10):
            for op in ops:
                for y in op["y"]:
                    y.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = [host(y) for op in ops for y in op["y"]]
            for a, b in zip(ref, got):
                assert np.array_equal(a, b), f"replay {r} differs"
    assert ch.status() == 0, ch.last_error
