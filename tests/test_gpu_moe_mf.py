"""One-token Q4_K MoE steps on the fp16 matrix-core kernel (k_moe_mf): every active expert's
gate|up (SwiGLU fused) and down products, the combine fused into the down launch.

Checked here, on layers whose gate/up and down products take one, two and four blocks a wave:
  * y within the oracle's bar (routing bitwise), as in the other MoE tests;
  * the lanes-along-k kernel (TQ_KNOB_MOE_MF = 0) within the same bar, and not bitwise equal (so the
    knob really switches kernels);
  * bitwise the same y whatever the launch shape (workgroups aimed for, tiles in flight) and with
    the combine as its own launch, on calls in a row with different tokens;
  * the top-k selection made inside the gate/up launch (one call running every stage): routing
    outputs (ids, weights, logits, grouping) and y bitwise those of the top-k kernel's launch
    (TQ_KNOB_MOE_ROUTE1 = 0), for 8 to 256 experts, with and without a shared expert.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev, host
from tests.test_gpu_moe import _layer_to_device, _run, check_moe

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")

SHAPES = [
    (dict(hidden=512, ffn=1024, n_experts=8, shared=False), 2),     # k 512 and 1024: 1 block a wave
    (dict(hidden=2048, ffn=1536, n_experts=16, shared=True), 4),    # k 2048 and 1536
    (dict(hidden=7168, ffn=2048, n_experts=24, shared=True), 8),    # DeepSeek's expert shape
    (dict(hidden=1024, ffn=14336, n_experts=4, shared=False), 2),   # down k 14336: 4 blocks a wave
]


def _case(*a):
    print("case:", *a, flush=True)


@pytest.mark.parametrize("shape,k", SHAPES, ids=lambda v: str(v)[:32])
def test_moe_mf_one_token(knobs, shape, k):
    t = "q4_k"
    _case("moe-mf", shape, k)
    layer = synth.moe_layer(shape, t, seed=241, tag="moe-mf")
    moe = _layer_to_device(t, shape, layer, k)
    ws = torch.empty(moe.workspace_bytes(1), dtype=torch.uint8, device="cuda:0")
    for i in range(2):
        x = synth.normal_f32(synth.rng(241, "x", i), (1, shape["hidden"]))
        xd = dev(x)
        _, y, _ = check_moe(t, shape, layer, x, k, moe=moe)
        assert np.array_equal(host(moe(xd, ws=ws)), y), f"call {i}: workspace given"
        for name, v in (("mf_wgs", 16), ("mf_wgs", 1024), ("mf_deep", 0), ("mf_deep", 2),
                        ("fuse_combine", 0)):
            knobs(name, v)
            got = host(moe(xd, ws=ws))
            knobs(name, -1)
            assert np.array_equal(got, y), f"call {i}: {name} = {v}"
        knobs("moe_mf", 0)
        _, y_kl, _ = check_moe(t, shape, layer, x, k, moe=moe)
        knobs("moe_mf", -1)
        if shape["hidden"] >= 2048:
            assert not np.array_equal(y_kl, y), "the knob did not switch kernels"


ROUTE1 = [
    (dict(hidden=512, ffn=512, n_experts=8, shared=True), 2),
    (dict(hidden=768, ffn=512, n_experts=64, shared=False), 6),
    (dict(hidden=1024, ffn=512, n_experts=65, shared=True), 4),
    (dict(hidden=2048, ffn=1024, n_experts=256, shared=True), 8),
    (dict(hidden=512, ffn=256, n_experts=200, shared=False), 1),
]


@pytest.mark.parametrize("shape,k", ROUTE1, ids=lambda v: str(v)[:32])
def test_moe_mf_selection_in_gate_up_launch(knobs, shape, k):
    t, E = "q4_k", shape["n_experts"]
    _case("moe-mf route1", shape, k)
    layer = synth.moe_layer(shape, t, seed=242, tag="route1")
    moe = _layer_to_device(t, shape, layer, k)
    for i in range(3):
        x = synth.normal_f32(synth.rng(242, "x", E, i), (1, shape["hidden"]))
        if i == 2:
            x[0, :] = 0.0  # every logit equal: ties to the lower ids
        y, r = _run(moe, x, E, k)
        knobs("moe_route1", 0)
        y0, r0 = _run(moe, x, E, k)
        knobs("moe_route1", -1)
        for f in r:
            assert np.array_equal(r[f], r0[f]), f"call {i}: routing output {f}"
        assert np.array_equal(y, y0), f"call {i}: y"
        if i == 2:
            assert np.array_equal(r["topk_ids"][0], np.arange(k))
        else:
            check_moe(t, shape, layer, x, k, moe=moe)
