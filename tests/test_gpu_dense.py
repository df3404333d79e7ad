"""GPU parity of tq_dequant, tq_gemv and tq_swiglu against the CPU oracle.

Bars: dequantized weights and all-integer-lattice products bitwise; other products within
|err| <= 1e-3 * sum|w x| + 1e-5 per output; SwiGLU on identical inputs within 1e-5 |h| + 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.golden_io import load_blocks
from tests.gpu_util import assert_product_close, dev, host

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("moe_expert_ffn_q4_amd")


def _print_case(*a):
    print("case:", *a, flush=True)


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0", "q5_k", "q4_0"])
@pytest.mark.parametrize("n,k", [(1, 256), (67, 1024), (130, 4608), (3, 768)])
def test_dequant_bitwise(t, n, k):
    _print_case("dequant", t, n, k)
    g = synth.rng(101, "dq", t, n, k)
    w = synth.blob(t, g, n, k)
    wd = dev(w)
    f32 = host(tq.dequant(t, wd, n, k, "f32"))
    assert np.array_equal(f32.view(np.uint32), oracle.dequant(t, w, n, k, "f32").view(np.uint32))
    bf = host(tq.dequant(t, wd, n, k, "bf16")).view(np.uint16)
    assert np.array_equal(bf, oracle.dequant(t, w, n, k, "bf16"))


def test_dequant_golden_blocks_bitwise():
    for fx in load_blocks():
        t, blk = fx["type"], fx["block"]
        k = synth.BLOCK_WEIGHTS[t]
        _print_case("golden", fx["name"])
        got = host(tq.dequant(t, dev(blk), 1, k, "f32"))[0]
        assert np.array_equal(got.astype(np.float64), fx["expect"]), fx["name"]
        assert np.array_equal(np.signbit(got), np.signbit(fx["expect"])), fx["name"]


# shapes span several 64-row groups with a ragged last group, several waves along k with an
# uneven split, and (q6_k k=768, q8_0 k=96/800) the shapes whose rows are not dword aligned
GEMV_CASES = [
    ("q4_k", 200, 2304), ("q4_k", 64, 256), ("q4_k", 1, 4096), ("q4_k", 333, 9216),
    ("q6_k", 150, 3072), ("q6_k", 70, 768), ("q6_k", 64, 512),
    ("q8_0", 190, 2560), ("q8_0", 65, 96), ("q8_0", 33, 800),
    ("q5_k", 150, 2304), ("q5_k", 64, 256), ("q5_k", 70, 5120),
    ("q4_0", 190, 2560), ("q4_0", 65, 96), ("q4_0", 33, 800),
]


@pytest.mark.parametrize("t,n,k", GEMV_CASES)
@pytest.mark.parametrize("batch", [1, 2, 3, 8, 9, 16])
def test_gemv_parity(t, n, k, batch):
    _print_case("gemv", t, n, k, batch)
    g = synth.rng(102, "gemv", t, n, k, batch)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (batch, k))
    y = host(tq.gemv(t, dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv(t, w, n, k, x)
    assert_product_close(y, ref, mag, what=f"{t} {n}x{k} b{batch}")


@pytest.mark.parametrize("t,n,k", [("q4_k", 300, 4096), ("q6_k", 200, 3584 * 2), ("q8_0", 129, 2048),
                                   ("q6_k", 64, 1280), ("q8_0", 64, 352), ("q5_k", 150, 4096),
                                   ("q4_0", 129, 2048), ("q4_0", 64, 352)])
@pytest.mark.parametrize("batch", [1, 5, 8])
def test_gemv_integer_lattice_bitwise(t, n, k, batch):
    """Scales 2^-8 and x in {-1,0,1}: every partial sum is exact in fp32, so any summation order
    gives the exact result and the GPU must match the oracle bit for bit."""
    _print_case("lattice", t, n, k, batch)
    g = synth.rng(103, "lattice", t, n, k)
    kw = (dict(d_value=2.0 ** -8, dmin_value=2.0 ** -8) if t in ("q4_k", "q5_k")
          else dict(d_value=2.0 ** -8))
    w = synth.blob(t, g, n, k, **kw)
    if t == "q6_k":  # keep |sc*(q-32)| <= 256 so sums stay below 2^16 in units of 2^-8
        blk = w.reshape(-1, 210)
        blk[:, 192:208] = (blk[:, 192:208].view(np.int8) // 16).view(np.uint8)
    x = synth.ternary_f32(g, (batch, k))
    y = host(tq.gemv(t, dev(w), n, k, dev(x)))
    ref, _ = oracle.gemv(t, w, n, k, x)
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("t,n,k", [("q4_k", 200, 4096), ("q6_k", 130, 3072), ("q8_0", 70, 2048),
                                   ("q5_k", 130, 4096), ("q4_0", 70, 2048)])
@pytest.mark.parametrize("batch", [1, 7])
def test_gemv_without_workspace(t, n, k, batch):
    """No workspace: every row group in one workgroup; and an explicit workspace."""
    _print_case("no-ws", t, n, k, batch)
    g = synth.rng(107, "nows", t, n, k, batch)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (batch, k))
    wd, xd = dev(w), dev(x)
    y0 = host(tq.gemv(t, wd, n, k, xd, ws=False))
    ref, mag = oracle.gemv(t, w, n, k, x)
    assert_product_close(y0, ref, mag, what="no workspace")
    nbytes = tq.gemv_workspace_bytes(t, n, k, batch)
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda:0")
    y1 = host(tq.gemv(t, wd, n, k, xd, ws=ws))
    assert_product_close(y1, ref, mag, what="own workspace")


@pytest.mark.parametrize("t,n,k,batch", [("q4_k", 300, 16384, 1), ("q4_k", 200, 4096, 8),
                                         ("q8_0", 200, 8192, 4), ("q6_k", 300, 4096, 1),
                                         ("q6_k", 100, 8192, 3)])
def test_gemv_workspace_any_contents(t, n, k, batch):
    """The k-split paths (int8 matrix cores, fp16 and fp32 matrix cores, the lane-per-row split)
    take a workspace with any contents: all-ones bytes, random bytes, or what a call of another
    shape left give bitwise the result of a zeroed workspace, call after call."""
    _print_case("ws-contents", t, n, k, batch)
    g = synth.rng(108, "wsany", t, n, k, batch)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (batch, k))
    wd, xd = dev(w), dev(x)
    nbytes = max(tq.gemv_workspace_bytes(t, n, k, batch), 256)
    assert nbytes > 65536, "shape must take a k-split path"
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    ref = host(tq.gemv(t, wd, n, k, xd, ws=ws))
    oref, mag = oracle.gemv(t, w, n, k, x)
    assert_product_close(ref, oref, mag, what="zeroed workspace")
    ws.fill_(255)
    assert np.array_equal(host(tq.gemv(t, wd, n, k, xd, ws=ws)), ref), "all-ones workspace"
    ws.copy_(torch.from_numpy(g.integers(0, 256, nbytes, dtype=np.uint8)).to("cuda:0"))
    for i in range(3):
        assert np.array_equal(host(tq.gemv(t, wd, n, k, xd, ws=ws)), ref), f"random bytes, call {i}"
    w2 = dev(synth.blob(t, g, 2 * n + 7, k))
    tq.gemv(t, w2, 2 * n + 7, k, dev(synth.normal_f32(g, (batch, k))), ws=ws)
    assert np.array_equal(host(tq.gemv(t, wd, n, k, xd, ws=ws)), ref), "after another shape"


def test_gemv_unit_vector_picks_dequantized_column():
    t, n, k = "q4_k", 130, 1024
    g = synth.rng(104, "ej")
    w = synth.blob(t, g, n, k)
    x = np.zeros((3, k), np.float32)
    x[0, 0] = x[1, 511] = x[2, 1023] = 1.0
    y = host(tq.gemv(t, dev(w), n, k, dev(x)))
    dense = oracle.dequant(t, w, n, k, "f32")
    assert np.array_equal(y[0], dense[:, 0]) and np.array_equal(y[1], dense[:, 511])
    assert np.array_equal(y[2], dense[:, 1023])


def test_gemv_deterministic_across_interleaved_shapes():
    """Same inputs give the same bits, also when other shapes use the shared workspace between."""
    t, n, k = "q4_k", 4096, 4096
    g = synth.rng(105, "det")
    wd, xd = dev(synth.blob(t, g, n, k)), dev(synth.normal_f32(g, (8, k)))
    n2, k2 = 28672, 8192
    w2, x2 = dev(synth.blob("q6_k", g, n2, k2)), dev(synth.normal_f32(g, (3, k2)))
    a = host(tq.gemv(t, wd, n, k, xd[:1]))
    c = host(tq.gemv(t, wd, n, k, xd))
    e = host(tq.gemv("q6_k", w2, n2, k2, x2))
    b = host(tq.gemv(t, wd, n, k, xd[:1]))
    f = host(tq.gemv("q6_k", w2, n2, k2, x2))
    d = host(tq.gemv(t, wd, n, k, xd))
    assert np.array_equal(a, b) and np.array_equal(c, d) and np.array_equal(e, f)


def test_gemv_full_4096x4096_all_rows():
    """The 4096 x 4096 batch-1 Q4_K case, every output row against the oracle."""
    t, n, k = "q4_k", 4096, 4096
    g = synth.rng(synth.DEFAULT_SEED, "c1")
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(g, (1, k))
    y = host(tq.gemv(t, dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv(t, w, n, k, x)
    assert_product_close(y, ref, mag, what="4096x4096")


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q8_0"])
@pytest.mark.parametrize("name,n,k", [("gate", 28672, 8192), ("down", 8192, 28672), ("k", 1024, 8192)])
@pytest.mark.parametrize("batch", [1, 4, 16])
def test_gemv_70b_shapes_sampled_rows(t, name, n, k, batch):
    """Full 70B-layer projection shapes, sampled output rows checked one by one."""
    _print_case("70b", t, name, batch)
    g = synth.rng(synth.DEFAULT_SEED, "70b", t, name)
    w = synth.blob(t, g, n, k)
    x = synth.normal_f32(synth.rng(synth.DEFAULT_SEED, "70b-x", batch), (batch, k))
    y = host(tq.gemv(t, dev(w), n, k, dev(x)))
    rows = np.unique(np.concatenate([[0, 63, 64, n - 1], g.integers(0, n, 60)]))
    ref, mag = oracle.gemv(t, w, n, k, x, rows=rows)
    assert_product_close(y[:, rows], ref, mag, what=f"{t} {name} b{batch}")


def test_swiglu_on_identical_inputs():
    g = synth.rng(106, "swiglu")
    a = synth.normal_f32(g, 100003, 3.0)
    b = synth.normal_f32(g, 100003)
    a[:4] = [0.0, -100.0, 100.0, -800.0]
    h = host(tq.swiglu(dev(a), dev(b)))
    ref = oracle.swiglu(a, b)
    err = np.abs(h.astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * np.abs(ref) + 1e-5)


@pytest.mark.parametrize("t,ns,k,batch", [
    ("q4_k", [4096, 1024, 1024], 4096, 1),   # q, k, v of the 8B shape: one launch
    ("q4_k", [37, 5, 100, 3], 1024, 1),      # parts straddle the kernel's row groups
    ("q4_k", [300, 77], 2048, 3),            # batch > 1: one launch per part
    ("q6_k", [130, 64], 3072, 1),
    ("q8_0", [70, 33], 2048, 2),
])
def test_gemv_multi_equals_separate_gemvs(t, ns, k, batch):
    _print_case("gemv_multi", t, ns, k, batch)
    blobs = [synth.blob(t, synth.rng(51, t, i, n, k), n, k) for i, n in enumerate(ns)]
    x = dev(synth.normal_f32(synth.rng(51, "x", k, batch), (batch, k)))
    ws_ = [dev(b) for b in blobs]
    outs = tq.gemv_multi(t, ws_, ns, k, x)
    for w, n, o, b in zip(ws_, ns, outs, blobs):
        ref = host(tq.gemv(t, w, n, k, x))
        assert np.array_equal(host(o), ref)
    # one part against the oracle as well
    y, mag = oracle.gemv(t, blobs[0], ns[0], k, host(x))
    assert_product_close(host(outs[0]), y, mag, what="gemv_multi part 0")


@pytest.mark.parametrize("t,n,k,batch", [("q4_k", 14336, 4096, 1), ("q4_k", 1001, 2048, 1),
                                         ("q4_k", 500, 4096, 2), ("q8_0", 300, 2048, 1)])
def test_gemv_swiglu_equals_gemv_gemv_swiglu(t, n, k, batch):
    _print_case("gemv_swiglu", t, n, k, batch)
    g = dev(synth.blob(t, synth.rng(52, "g", n, k), n, k))
    u = dev(synth.blob(t, synth.rng(52, "u", n, k), n, k))
    x = dev(synth.normal_f32(synth.rng(52, "x", k, batch), (batch, k)))
    h = host(tq.gemv_swiglu(t, g, u, n, k, x))
    ref = host(tq.swiglu(tq.gemv(t, g, n, k, x), tq.gemv(t, u, n, k, x)))
    assert np.array_equal(h, ref)


@pytest.mark.parametrize("n,k", [(37, 256), (130, 768), (64, 1024), (301, 1280), (130, 2048)])
def test_gemv_lane_groups_bitwise(knobs, n, k):
    """Batch-1 Q4_K rows of k <= 2048 are split over 2 or 4 lane groups per wave; each row's lane
    partials are added in the same tree as with whole-wave rows (whose extra lanes add exact
    zeros), so the results are bitwise those of TQ_KNOB_KL_GROUPS = 1, and within the bar."""
    _print_case("kl-groups", n, k)
    knobs("gemv_mf", 0)  # the lanes-along-k kernel (batch-1 Q4_K goes to the matrix cores by default)
    g = synth.rng(120, "kl-groups", n, k)
    w, x = synth.blob("q4_k", g, n, k), synth.normal_f32(g, (1, k))
    a = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q4_k", w, n, k, x)
    assert_product_close(a, ref, mag, what=f"kl groups {n}x{k}")
    knobs("kl_groups", 1)
    b = host(tq.gemv("q4_k", dev(w), n, k, dev(x)))
    assert np.array_equal(a, b)
    knobs("kl_groups", -1)
    F = n + (n & 1)
    wg, wu = synth.blob("q4_k", g, F, k), synth.blob("q4_k", g, F, k)
    xd = dev(x)
    h = host(tq.gemv_swiglu("q4_k", dev(wg), dev(wu), F, k, xd))
    gg, uu = tq.gemv("q4_k", dev(wg), F, k, xd), tq.gemv("q4_k", dev(wu), F, k, xd)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))


# ---- Q8_0 at batch 1 on the int8 matrix cores -----------------------------------------------------

@pytest.mark.parametrize("n,k", [(1000, 8192), (64, 256), (333, 28672), (77, 512), (130, 2304),
                                 (4096, 1024)])
def test_q8_0_int8_matrix_cores(knobs, n, k):
    """One token of Q8_0 on the int8 matrix cores (8 blocks of 34 bytes per 256-weight unit, the
    even blocks realigned in registers): one slice (k = 256, 512, 1024), several with a ragged
    last slice (k = 2304, 28672); every output against the oracle at fp32 level, and against
    the lane-per-row fp32 kernel (TQ_KNOB_GEMV_I8 = 0)."""
    _print_case("q8_0 int8", n, k)
    g = synth.rng(109, "q8i8", n, k)
    w = synth.blob("q8_0", g, n, k)
    x = synth.normal_f32(g, (1, k))
    wd, xd = dev(w), dev(x)
    y = host(tq.gemv("q8_0", wd, n, k, xd))
    ref, mag = oracle.gemv("q8_0", w, n, k, x)
    worst = assert_product_close(y, ref, mag, what=f"q8_0 {n}x{k}")
    assert worst < 0.05, worst
    assert np.array_equal(y, host(tq.gemv("q8_0", wd, n, k, xd))), "not deterministic"
    knobs("gemv_i8", 0)
    y0 = host(tq.gemv("q8_0", wd, n, k, xd))
    assert np.linalg.norm(y - y0) / np.linalg.norm(y0) < 1e-6


def test_q8_0_int8_extremes():
    """Quants at -128 and 127 in every block, fp16 scales at their largest and in the subnormal
    range, and activation blocks of 1e-30, 1e20 and zero: the digit sums stay exact and the fold
    stays within the bar."""
    n, k = 96, 2048
    _print_case("q8_0 int8 extremes")
    g = synth.rng(110, "q8i8-ext")
    w = synth.blob("q8_0", g, n, k)
    blk = w.reshape(-1, 34)
    blk[0::3, 2:] = np.uint8(0x80)  # -128
    blk[1::3, 2:] = np.uint8(0x7F)  # 127
    blk[0::5, 0:2] = np.frombuffer(np.float16(65504.0).tobytes(), np.uint8)
    blk[1::7, 0:2] = np.frombuffer(np.float16(2.0 ** -20).tobytes(), np.uint8)
    x = synth.normal_f32(g, (1, k))
    x[0, :256] *= np.float32(1e-30)
    x[0, 256:512] = 0.0
    x[0, 512:768] *= np.float32(1e20)
    y = host(tq.gemv("q8_0", dev(w), n, k, dev(x)))
    ref, mag = oracle.gemv("q8_0", w, n, k, x)
    assert_product_close(y, ref, mag, what="q8_0 extremes")


def test_q8_0_int8_multi_and_swiglu_bitwise():
    """Q8_0 one-token multi and gate|up + SwiGLU launches on the int8 matrix cores give bitwise
    the single products (k slices set by k alone)."""
    k = 4096
    g = synth.rng(111, "q8i8-multi")
    ns = [512, 128, 96]
    ws = [synth.blob("q8_0", g, n, k) for n in ns]
    x = dev(synth.normal_f32(g, (1, k)))
    outs = tq.gemv_multi("q8_0", [dev(w) for w in ws], ns, k, x)
    for w, n, o in zip(ws, ns, outs):
        assert np.array_equal(host(o), host(tq.gemv("q8_0", dev(w), n, k, x)))
    F = 320
    wg, wu = synth.blob("q8_0", g, F, k), synth.blob("q8_0", g, F, k)
    h = host(tq.gemv_swiglu("q8_0", dev(wg), dev(wu), F, k, x))
    gg = tq.gemv("q8_0", dev(wg), F, k, x)
    uu = tq.gemv("q8_0", dev(wu), F, k, x)
    assert np.array_equal(h, host(tq.swiglu(gg, uu)))
