"""GPU parity of the bf16 matrix-core expert path of tq_moe_ffn (prompt-sized batches).

Routing (logits, top-k, grouping) is checked exactly as on the fp32 path. y is checked against
the oracle with the GPU's routing, element by element:
  * the oracle's bf16-operand MoE (x, weights and h rounded to bf16, fp64 sums), the exact
    arithmetic of the path: within (1e-3 + 2^-8) * sum|products| + 1e-5. 1e-3 is the
    fp32-accumulation rule; 2^-8 covers h values that sit on a bf16 rounding tie, which the GPU
    (rounding its fp32 h) and the oracle (rounding its fp64 h) may resolve to neighbouring bf16
    values -- one bf16 ulp of a term is at most 2^-8 of its magnitude. On top of that at most
    one element in 1000 may exceed 1e-3 * sum|products| + 1e-5, and the relative L2 error must
    stay below 2e-5;
  * the exact fp64 MoE: at the DeepSeek-shaped 4096-token prefill (67 tokens spread over the
    whole batch, so over every expert's chunks) within 2e-2 * sum|products| + 1e-5 per element;
    on the small shapes, where a gate or up sum that cancels can turn the bf16 roundings of x
    and of the weights into a larger relative change of h, the relative L2 error of y within
    2e-2 (the per-element figure is printed).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_product_close, dev, host
from tests.test_gpu_moe import _layer_to_device, _run, check_moe

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")

REL = 2e-2
TIE = 2.0**-8


def _check_bf16(y, ref, mag, what):
    worst = assert_product_close(y, ref, mag, rel=1e-3 + TIE, what=what)
    over = np.abs(y - ref) > 1e-3 * mag + 1e-5
    assert over.mean() <= 1e-3, f"{what}: {int(over.sum())} elements beyond 1e-3 * mag"
    l2 = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-30))
    assert l2 < 2e-5, f"{what}: relative L2 {l2:.2e}"
    return worst, int(over.sum()), l2


def _check_vs_bf16_oracle(moe, shape, layer, x, k, tokens=None):
    """Routing as on the fp32 path (check_moe at a tolerance that admits the bf16 ties), then the
    bf16-operand oracle checks of _check_bf16; returns y."""
    _, y, _ = check_moe("q4_k", shape, layer, x, k, moe=moe, bf16=True, rel=1e-3 + TIE,
                        tokens=tokens)
    _, r = _run(moe, x, shape["n_experts"], k)
    ids, wts = oracle.topk(r["logits"], k, True)
    toks = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    ref, mag = oracle.moe("q4_k", shape["hidden"], shape["ffn"], layer["experts"],
                          layer["shared"], x, ids, wts, tokens=toks, bf16=True)
    worst, over, l2 = _check_bf16(y[toks], ref, mag, f"T={x.shape[0]} vs bf16 oracle")
    print(f"  vs bf16 oracle: worst err/bound {worst:.3f}, {over} elements beyond 1e-3 * mag, "
          f"rel L2 {l2:.2e}", flush=True)
    return y


def _report_fp64(shape, layer, x, k, y, moe, tokens=None):
    """Relative L2 error against the exact fp64 oracle within 2e-2; the largest |err| / mag
    is printed."""
    E = shape["n_experts"]
    _, r = _run(moe, x, E, k)
    ids, wts = oracle.topk(r["logits"], k, True)
    toks = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    ref, mag = oracle.moe("q4_k", shape["hidden"], shape["ffn"], layer["experts"],
                          layer["shared"], x, ids, wts, tokens=toks)
    e = np.abs(y[toks] - ref)
    l2 = float(np.linalg.norm(y[toks] - ref) / np.linalg.norm(ref))
    print(f"  vs fp64 oracle: max err/mag {np.max(e / (mag + 1e-30)):.2e}, rel L2 {l2:.2e}",
          flush=True)
    assert l2 <= REL, f"relative L2 {l2:.2e} against the fp64 oracle"


def _case(*a):
    print("case:", *a, flush=True)


SMALL = [
    # ~75 tokens per expert, one chunk each; the shared expert's 300 rows split into 2 chunks
    (dict(hidden=512, ffn=512, n_experts=8, shared=True), 2, [300, 1, 33]),
    # ~250 tokens per expert: every expert split into 2 chunks
    (dict(hidden=768, ffn=1024, n_experts=4, shared=False), 2, [500]),
    # few tokens per expert, some experts empty; k = 3
    (dict(hidden=256, ffn=256, n_experts=16, shared=True), 3, [37, 170]),
]


@pytest.mark.parametrize("shape,k,Ts", SMALL, ids=lambda v: str(v)[:30])
def test_prefill_small_shapes(shape, k, Ts):
    layer = synth.moe_layer(shape, "q4_k", seed=301, tag="prefill-small")
    moe = _layer_to_device("q4_k", shape, layer, k, path=tq.PATH_BF16_MFMA)
    for T in Ts:
        _case("prefill-small", shape, k, T)
        x = synth.normal_f32(synth.rng(301, "x", T), (T, shape["hidden"]))
        y = _check_vs_bf16_oracle(moe, shape, layer, x, k)
        _report_fp64(shape, layer, x, k, y, moe)
        y2, _ = _run(moe, x, shape["n_experts"], k)
        assert np.array_equal(y, y2), "not deterministic"


def test_prefill_auto_takes_matrix_cores_for_large_batches():
    """AUTO: 64+ routed tokens per expert on average -> matrix-core path (bitwise equal to the
    forced one); fewer -> fp32 path (bitwise equal to the forced fp32 one)."""
    shape = dict(hidden=512, ffn=512, n_experts=8, shared=True)
    layer = synth.moe_layer(shape, "q4_k", seed=302, tag="auto")
    layers = {p: _layer_to_device("q4_k", shape, layer, 2, path=p)
              for p in (tq.PATH_AUTO, tq.PATH_F32, tq.PATH_BF16_MFMA)}
    for T, expect in ((256, tq.PATH_BF16_MFMA), (255, tq.PATH_F32)):
        x = synth.normal_f32(synth.rng(302, "x", T), (T, 512))
        ys = {p: _run(m, x, 8, 2)[0] for p, m in layers.items()}
        assert np.array_equal(ys[tq.PATH_AUTO], ys[expect]), f"T={T}"
        assert not np.array_equal(ys[tq.PATH_F32], ys[tq.PATH_BF16_MFMA])


def test_prefill_all_tokens_on_two_experts():
    """Zero router: every token on experts 0 and 1 (400 rows each, 3 chunks), the rest empty."""
    shape = dict(hidden=512, ffn=768, n_experts=8, shared=True)
    layer = synth.moe_layer(shape, "q4_k", seed=303, tag="ties")
    layer["router"] = np.zeros_like(layer["router"])
    x = synth.normal_f32(synth.rng(303, "x"), (400, 512))
    moe = _layer_to_device("q4_k", shape, layer, 2, path=tq.PATH_BF16_MFMA)
    _check_vs_bf16_oracle(moe, shape, layer, x, 2)


def test_prefill_lattice_gate_up_exact():
    """d = 1, dmin = 0, every scale 1, x in {-1, 0, 1}: weights 0..15 and every partial sum are
    exact in bf16 / fp32, so with E = 1, k = 1 and a unit down matrix the layer output is
    silu(g) * u rounded to bf16, with g and u exact integers."""
    H = F = 256
    shape = dict(hidden=H, ffn=F, n_experts=1, shared=False)
    layer = synth.moe_layer(shape, "q4_k", seed=304, tag="lattice")
    g, u = (synth.blob("q4_k", synth.rng(304, m), F, H, d_value=1.0, dmin_value=0.0)
            for m in ("g", "u"))
    for b in (g, u):  # every 6-bit scale 1, every min 0
        blocks = b.reshape(-1, 144)
        blocks[:, 4:12] = np.array([1, 1, 1, 1, 0, 0, 0, 0], np.uint8)
        blocks[:, 12:16] = np.array([1, 1, 1, 1], np.uint8)
    # down = identity: row i has weight 1 at column i (q = 1 there, 0 elsewhere)
    down = np.zeros((H, 144), np.uint8)
    down[:, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    down[:, 4:8], down[:, 12:16] = 1, 1
    for i in range(H):
        c, r = divmod(i, 64)
        byte = 16 + 32 * c + (r % 32)
        down[i, byte] = 1 if r < 32 else 0x10
    layer["experts"] = [(g, u, down.reshape(-1))]
    x = synth.ternary_f32(synth.rng(304, "x"), (200, H))
    moe = _layer_to_device("q4_k", shape, layer, 1, path=tq.PATH_BF16_MFMA)
    y, _ = _run(moe, x, 1, 1)
    wg = oracle.dequant("q4_k", g, F, H).astype(np.float64)
    wu = oracle.dequant("q4_k", u, F, H).astype(np.float64)
    assert set(np.unique(wg)) <= set(range(16)) and np.array_equal(
        oracle.dequant("q4_k", layer["experts"][0][2], H, F), np.eye(H, dtype=np.float32))
    gv = x.astype(np.float64) @ wg.T
    uv = x.astype(np.float64) @ wu.T
    # the GPU's h: fp32 silu(g) * u rounded to bf16; compare to within that rounding only
    h = (gv * uv / (1.0 + np.exp(-gv))).astype(np.float32)
    bound = np.abs(h) * 2.0**-8 + 1e-6
    assert np.all(np.abs(y - h) <= bound)


@pytest.fixture(scope="module")
def deepseek():
    return synth.moe_layer(synth.DEEPSEEK, "q4_k", tag="deepseek")


def test_prefill_deepseek_4096_sampled_tokens(deepseek):
    """Routing of all 4096 tokens bitwise; y of 67 tokens spread over the batch (the first two,
    64 evenly spaced, the last: about 540 routed pairs over the experts' chunks) against the fp64
    oracle per element; 8 of them against the bf16-operand oracle."""
    T = 4096
    _case("deepseek prefill", T)
    x = synth.normal_f32(synth.rng(synth.DEFAULT_SEED, "deepseek-x", T), (T, 7168))
    toks = sorted(set([0, 1] + list(range(31, T, 64)) + [T - 1]))
    assert len(toks) >= 64
    moe, y, (worst, l2) = check_moe("q4_k", synth.DEEPSEEK, deepseek, x, 8, tokens=toks, rel=REL,
                                    path=tq.PATH_BF16_MFMA)
    print(f"  vs fp64 oracle ({len(toks)} tokens): worst err/bound {worst:.3f}, rel L2 {l2:.2e}",
          flush=True)
    # some of them against the bf16-operand oracle
    toks = toks[::9]
    _, r = _run(moe, x, 256, 8)
    ids, wts = oracle.topk(r["logits"], 8, True)
    ref, mag = oracle.moe("q4_k", 7168, 2048, deepseek["experts"], deepseek["shared"], x, ids,
                          wts, tokens=toks, bf16=True)
    worst, over, l2 = _check_bf16(y[toks], ref, mag, "deepseek prefill vs bf16 oracle")
    print(f"  vs bf16 oracle: worst err/bound {worst:.3f}, {over} beyond 1e-3 * mag, "
          f"rel L2 {l2:.2e}", flush=True)


def test_prefill_rejects_other_block_types():
    shape = dict(hidden=512, ffn=512, n_experts=4, shared=False)
    layer = synth.moe_layer(shape, "q8_0", seed=305, tag="q8")
    moe = _layer_to_device("q8_0", shape, layer, 2, path=tq.PATH_BF16_MFMA)
    x = dev(synth.normal_f32(synth.rng(305, "x"), (3, 512)))
    with pytest.raises(tq.TQError) as e:
        moe(x)
    assert e.value.status == 5
