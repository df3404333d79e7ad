"""Host-resident routed experts (pinned host memory, copied per call) against the device-resident
layer and the oracle: the same routing and bitwise the same output as the device-resident layer,
and the output within the product bar of the oracle (the bf16-operand oracle on the matrix-core
path), on the fp32 and the matrix-core paths, with and without a separate copy stream. Each layer
is called again with other activations, which route to other experts, so the staging area is
reused with different contents."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev, host
from tests.test_gpu_moe import _run, check_moe

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


def _case(*a):
    print("case:", *a, flush=True)


def _layers(t, shape, layer, k, path, copy_stream):
    router = dev(layer["router"])
    shared = tuple(dev(b) for b in layer["shared"]) if layer["shared"] is not None else None
    on_dev = tq.MoeLayer(t, shape["hidden"], shape["ffn"], router,
                         [tuple(dev(b) for b in e) for e in layer["experts"]], shared, top_k=k,
                         path=path)
    pinned = [tuple(torch.from_numpy(b).pin_memory() for b in e) for e in layer["experts"]]
    on_host = tq.MoeLayer(t, shape["hidden"], shape["ffn"], router, pinned, shared, top_k=k,
                          path=path, copy_stream=copy_stream)
    return on_dev, on_host


CASES = [
    ("q4_k", dict(hidden=512, ffn=512, n_experts=16, shared=True), 4, [1, 5, 40], tq.PATH_F32),
    ("q8_0", dict(hidden=512, ffn=768, n_experts=6, shared=False), 2, [3, 17], tq.PATH_F32),
    ("q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=True), 2, [300], tq.PATH_BF16_MFMA),
]


@pytest.mark.parametrize("side_stream", [True, False], ids=["copy-stream", "same-stream"])
@pytest.mark.parametrize("t,shape,k,Ts,path", CASES, ids=lambda v: str(v)[:20])
def test_host_resident_matches_device_resident(t, shape, k, Ts, path, side_stream):
    layer = synth.moe_layer(shape, t, seed=401, tag="host")
    cs = torch.cuda.Stream() if side_stream else None
    on_dev, on_host = _layers(t, shape, layer, k, path, cs)
    bf16 = path == tq.PATH_BF16_MFMA
    for T in Ts:
        for rep in range(2):
            _case("host-resident", t, shape, k, T, path, side_stream, rep)
            x = synth.normal_f32(synth.rng(401, "x", T, rep), (T, shape["hidden"]))
            yd, rd = _run(on_dev, x, shape["n_experts"], k)
            yh, rh = _run(on_host, x, shape["n_experts"], k)
            for f in rd:
                assert np.array_equal(rd[f], rh[f]), f
            assert np.array_equal(yd, yh)
            check_moe(t, shape, layer, x, k, moe=on_host, bf16=bf16,
                      rel=1e-3 + 2.0**-8 if bf16 else 1e-3)


def test_host_resident_deepseek_shape_one_token():
    _case("host-resident deepseek", 1)
    layer = synth.moe_layer(synth.DEEPSEEK, "q4_k", tag="deepseek")
    on_dev, on_host = _layers("q4_k", synth.DEEPSEEK, layer, 8, tq.PATH_AUTO, torch.cuda.Stream())
    for rep in range(2):
        x = synth.normal_f32(synth.rng(synth.DEFAULT_SEED, "deepseek-x", 1, rep), (1, 7168))
        yd, _ = _run(on_dev, x, 256, 8)
        yh, _ = _run(on_host, x, 256, 8)
        assert np.array_equal(yd, yh)
        check_moe("q4_k", synth.DEEPSEEK, layer, x, 8, moe=on_host)


def test_host_resident_rejects_unpinned_blobs():
    shape = dict(hidden=256, ffn=256, n_experts=2, shared=False)
    layer = synth.moe_layer(shape, "q4_k", seed=402, tag="unpinned")
    with pytest.raises(ValueError):
        tq.MoeLayer("q4_k", 256, 256, dev(layer["router"]),
                    [tuple(torch.from_numpy(b) for b in e) for e in layer["experts"]], top_k=1)
