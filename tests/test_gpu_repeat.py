"""Bitwise repeatability of the matrix-core kernels whose LDS pipelines wait on hand-counted load
counts (the fp16 few-token kernels for dense and MoE products, the bf16 prefill kernel), and of the
int8 GEMV: fifty calls, each compared with the first call's bits, stopping at the first mismatch.
A wait that let a barrier pass before its tile had landed would show up as a call whose result
differs from the others."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev, host
from tests.test_gpu_moe import _layer_to_device

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")

CALLS = 50


def _case(*a):
    print("case:", *a, flush=True)


def _repeat(call, out):
    first = host(call()).copy()
    assert np.isfinite(first).all()
    for i in range(1, CALLS):
        out.fill_(float("nan"))
        got = host(call())
        if not np.array_equal(got, first):
            bad = int((got != first).sum())
            raise AssertionError(f"call {i}: {bad} of {got.size} elements differ from call 0")


@pytest.mark.parametrize("n,k,batch", [(1000, 4096, 8), (4096, 14336, 16), (640, 2048, 32)])
def test_repeat_qmm_dense(n, k, batch):
    """k_qmm_dense (Q4_K, 2..32 tokens, k slices added by the last workgroup)."""
    _case("repeat qmm_dense", n, k, batch)
    g = synth.rng(81, "rep-dense", n, k, batch)
    w = dev(synth.blob("q4_k", g, n, k))
    x = dev(synth.normal_f32(g, (batch, k)))
    y = torch.empty((batch, n), dtype=torch.float32, device="cuda:0")
    ws = torch.zeros(max(tq.gemv_workspace_bytes("q4_k", n, k, batch), 256), dtype=torch.uint8,
                     device="cuda:0")
    _repeat(lambda: tq.gemv("q4_k", w, n, k, x, out=y, ws=ws), y)


@pytest.mark.parametrize("t,n,k,mf", [("q4_k", 3000, 16384, 1), ("q8_0", 3000, 8192, 2),
                                       ("q4_k", 3000, 16384, 2)])
def test_repeat_gemv_i8(knobs, t, n, k, mf):
    """k_gemv_i8 (Q4_K from k = 16384 under TQ_KNOB_GEMV_MF = 1, Q8_0: one token) and, with the
    knob at its default 2, the k-sliced fp16 matrix-core kernel on the same Q4_K rows."""
    _case("repeat gemv_i8", t, n, k, mf)
    knobs("gemv_mf", mf)
    g = synth.rng(82, "rep-i8", t)
    w = dev(synth.blob(t, g, n, k))
    x = dev(synth.normal_f32(g, (1, k)))
    y = torch.empty((1, n), dtype=torch.float32, device="cuda:0")
    ws = torch.zeros(tq.gemv_workspace_bytes(t, n, k, 1), dtype=torch.uint8, device="cuda:0")
    _repeat(lambda: tq.gemv(t, w, n, k, x, out=y, ws=ws), y)


@pytest.mark.parametrize("path,T", [(tq.PATH_F32, 16), (tq.PATH_F32, 64),
                                    (tq.PATH_BF16_MFMA, 300), (tq.PATH_BF16_MFMA, 1100)])
def test_repeat_moe_matrix_cores(path, T):
    """k_qmm (fp32-accurate fp16 matrix cores, few tokens per expert) and k_prefill (bf16 matrix
    cores), through whole MoE layer calls."""
    shape = dict(hidden=1024, ffn=1536, n_experts=8, shared=True)
    _case("repeat moe", path, T)
    layer = synth.moe_layer(shape, "q4_k", seed=83, tag="repeat")
    moe = _layer_to_device("q4_k", shape, layer, 2, path=path)
    x = dev(synth.normal_f32(synth.rng(83, "x", T), (T, shape["hidden"])))
    y = torch.empty_like(x)
    ws = torch.zeros(moe.workspace_bytes(T), dtype=torch.uint8, device="cuda:0")
    _repeat(lambda: moe(x, out=y, ws=ws), y)
