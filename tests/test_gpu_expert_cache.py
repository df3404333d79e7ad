"""GPU parity of the expert residency cache of the host-resident MoE variant.

A sequence of calls with activations x = z + v from a router whose routing favours some experts
(synth.zipf_router), so that experts recur between calls: every call's routing and output must be
bitwise those of the device-resident layer (and so of the oracle within the product bar, checked
on some calls), whatever the cache held, evicted or prefetched. The cache's counters must account
for every routed expert and every byte copied.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_product_close, dev, host
from tests.test_gpu_moe import _run

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


def _case(*a):
    print("case:", *a, flush=True)


def _layers(t, shape, k, path, seed):
    E, H = shape["n_experts"], shape["hidden"]
    layer = synth.moe_layer(shape, t, seed=seed, tag="cache")
    wr, v = synth.zipf_router(synth.rng(seed, "zipf"), E, H)
    layer["router"] = wr
    router = dev(wr)
    shared = tuple(dev(b) for b in layer["shared"]) if layer["shared"] is not None else None
    on_dev = tq.MoeLayer(t, H, shape["ffn"], router, [tuple(dev(b) for b in e) for e in layer["experts"]],
                         shared, top_k=k, path=path)
    pinned = [tuple(torch.from_numpy(b).pin_memory() for b in e) for e in layer["experts"]]
    on_host = tq.MoeLayer(t, H, shape["ffn"], router, pinned, shared, top_k=k, path=path,
                          copy_stream=torch.cuda.Stream())
    return layer, v, on_dev, on_host


CASES = [
    # (type, shape, top_k, tokens per call, path, slots, prefetch)
    ("q4_k", dict(hidden=512, ffn=512, n_experts=16, shared=True), 2, 1, tq.PATH_F32, 6, 2),
    ("q4_k", dict(hidden=512, ffn=768, n_experts=16, shared=False), 2, 3, tq.PATH_F32, 8, 0),
    ("q8_0", dict(hidden=512, ffn=512, n_experts=12, shared=True), 3, 2, tq.PATH_F32, 5, 3),
    ("q4_k", dict(hidden=512, ffn=512, n_experts=16, shared=True), 2, 5, tq.PATH_F32, 1, 0),
    ("q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=True), 2, 40, tq.PATH_F32, 6, 2),
    ("q4_k", dict(hidden=512, ffn=512, n_experts=8, shared=True), 2, 300, tq.PATH_BF16_MFMA, 8, 0),
]


@pytest.mark.parametrize("t,shape,k,T,path,slots,prefetch", CASES, ids=lambda v: str(v)[:20])
def test_cache_calls_equal_device_resident(t, shape, k, T, path, slots, prefetch):
    _case("expert cache", t, shape, k, T, path, slots, prefetch)
    E, H = shape["n_experts"], shape["hidden"]
    layer, v, on_dev, on_host = _layers(t, shape, k, path, seed=501)
    cache = on_host.attach_cache(slots, prefetch)
    g = synth.rng(501, "calls", t, T)
    routed = 0
    for call in range(14):
        x = synth.normal_f32(g, (T, H)) + v
        yd, rd = _run(on_dev, x, E, k)
        yh, rh = _run(on_host, x, E, k)
        for f in rd:
            assert np.array_equal(rd[f], rh[f]), (call, f)
        assert np.array_equal(yd, yh), f"call {call}: output differs from the device-resident layer"
        routed += int((rd["counts"] > 0).sum())
        if call in (0, 13):
            ids, wts = oracle.topk(rh["logits"], k)
            bf16 = path == tq.PATH_BF16_MFMA
            ref, mag = oracle.moe(t, H, shape["ffn"], layer["experts"], layer["shared"], x, ids, wts,
                                  bf16=bf16)
            assert_product_close(yh, ref, mag, rel=1e-3 + 2.0 ** -8 if bf16 else 1e-3,
                                 what=f"call {call} vs oracle")
    st = cache.stats()
    print("  stats:", st, flush=True)
    nbytes = int(tq.lib().tq_expert_cache_slot_bytes(on_host.desc))
    expert_bytes = sum(b.size for b in layer["experts"][0])
    assert st["calls"] == 14
    assert st["hits"] + st["misses"] + st["fallbacks"] == routed
    assert st["bytes_copied"] == (st["misses"] + st["fallbacks"] + st["prefetched"]) * expert_bytes
    assert nbytes >= expert_bytes and nbytes % 256 == 0
    assert st["prefetch_hits"] <= st["prefetched"]
    if slots >= 2 * k:
        assert st["hits"] > 0
    if prefetch == 0:
        assert st["prefetched"] == 0
    if slots == 1 and T * k > 1:
        assert st["fallbacks"] > 0
    on_host.detach_cache()
    # the same layer without the cache gives the same bits again
    x = synth.normal_f32(g, (T, H)) + v
    yd, _ = _run(on_dev, x, E, k)
    yh, _ = _run(on_host, x, E, k)
    assert np.array_equal(yd, yh)


def test_cache_rejects_other_layer_and_device_resident_use():
    shape = dict(hidden=512, ffn=512, n_experts=8, shared=False)
    _, _, on_dev, on_host = _layers("q4_k", shape, 2, tq.PATH_F32, seed=502)
    cache = on_host.attach_cache(4)
    other = dict(hidden=768, ffn=512, n_experts=8, shared=False)
    _, _, _, other_host = _layers("q4_k", other, 2, tq.PATH_F32, seed=503)
    other_host.desc.expert_cache = cache.state_ptr
    x = dev(synth.normal_f32(synth.rng(502, "x"), (2, 768)))
    with pytest.raises(tq.TQError) as e:
        other_host(x)
    assert e.value.status == 1
    on_dev.desc.expert_cache = cache.state_ptr
    with pytest.raises(tq.TQError) as e:
        on_dev(dev(synth.normal_f32(synth.rng(502, "x2"), (2, 512))))
    assert e.value.status == 1
    on_dev.desc.expert_cache = None
    on_host.detach_cache()
