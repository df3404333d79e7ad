"""GPU parity of tq_gemv_noalloc (the entry point for callers that cannot allocate) with tq_gemv.

tq_gemv_noalloc runs tq_gemv's kernels on a scratch array the library holds on each device. Its
output must be bitwise that of tq_gemv given a workspace of tq_gemv_workspace_bytes: here for
shapes that take each k-split path (which use the scratch) and one that needs none, on two calls
in a row, the second with a smaller input (the scratch then holds the first call's leftovers).
Both outputs are also held to the product bar against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_product_close, dev, host

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")

# (type, (n, k, batch) of the first call, (n, k, batch) of the second, smaller call)
CASES = [
    ("q4_k", (600, 16384, 1), (300, 16384, 1)),   # fp16 matrix cores (Q4_K), k slices
    ("q4_k", (1000, 4096, 16), (200, 2048, 8)),   # fp16 matrix cores, k slices
    ("q8_0", (700, 8192, 8), (100, 4096, 4)),     # fp32 matrix cores, k slices
    ("q6_k", (500, 8192, 1), (130, 4096, 1)),     # lane-per-row GEMV, k split
    ("q6_k", (300, 8192, 3), (64, 8192, 2)),      # lane-per-row GEMV, 3 and 2 tokens
    ("q4_k", (4096, 4096, 1), (1024, 4096, 1)),   # lanes-along-k kernel: no scratch at all
]


def _one(t, n, k, batch, tag):
    print("case: noalloc", t, n, k, batch, tag, flush=True)
    g = synth.rng(901, "noalloc", t, n, k, batch, tag)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (batch, k))
    wd, xd = dev(w), dev(x)
    need = tq.gemv_workspace_bytes(t, n, k, batch)
    assert need <= tq.GEMV_NOALLOC_MAX_BYTES
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda:0")
    ref = host(tq.gemv(t, wd, n, k, xd, ws=ws))
    out = torch.full((batch, n), float("nan"), dtype=torch.float32, device="cuda:0")
    got = host(tq.gemv_noalloc(t, wd, n, k, xd, out))
    assert np.array_equal(got, ref), f"{t} {n}x{k} batch {batch}: differs from tq_gemv"
    oref, mag = oracle.gemv(t, w, n, k, x)
    assert_product_close(got, oref, mag, what=f"noalloc {t} {n}x{k} b{batch}")
    return need


@pytest.mark.parametrize("t,first,second", CASES, ids=lambda v: str(v))
def test_noalloc_equals_gemv_two_calls(t, first, second):
    need1 = _one(t, *first, "first")
    need2 = _one(t, *second, "second")
    assert need2 <= need1


def test_noalloc_rejects_oversized_workspace():
    """A shape whose workspace exceeds the scratch is refused before anything is enqueued."""
    t, n, k, batch = "q4_k", 128256, 4096, 32
    assert tq.gemv_workspace_bytes(t, n, k, batch) > tq.GEMV_NOALLOC_MAX_BYTES
    w = torch.empty(n * 2304, dtype=torch.uint8, device="cuda:0")
    x = torch.zeros((batch, k), dtype=torch.float32, device="cuda:0")
    out = torch.full((batch, n), 7.0, dtype=torch.float32, device="cuda:0")
    with pytest.raises(tq.TQError) as e:
        tq.gemv_noalloc(t, w, n, k, x, out)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
