"""The C ABI on the host (no GPU needed): symbols, size helpers, and argument checks.

Every call here fails validation, which happens before any HIP call, so nothing is launched.
"""
import os
import re

import pytest

import moe_expert_ffn_q4_amd as tq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "tq.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(tq_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"tq_dequant", "tq_gemv", "tq_gemv_workspace_bytes", "tq_swiglu", "tq_last_error"} <= set(names)
    L = tq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_size_helpers():
    L = tq.lib()
    assert [L.tq_block_weights(t) for t in (1, 2, 3, 4, 5)] == [256, 256, 32, 256, 32]
    assert [L.tq_block_bytes(t) for t in (1, 2, 3, 4, 5)] == [144, 210, 34, 176, 18]
    assert L.tq_row_bytes(4, 4096) == 2816 and L.tq_row_bytes(5, 96) == 54
    assert L.tq_block_weights(9) == 0
    assert L.tq_row_bytes(1, 4096) == 2304 and L.tq_row_bytes(2, 8192) == 6720
    assert L.tq_row_bytes(3, 28672) == 30464 and L.tq_row_bytes(3, 33) == -1


@pytest.mark.parametrize("args,code", [
    ((7, 16, 4, 256, 16, 1, 16), 1),      # unknown type
    ((1, 0, 4, 256, 16, 1, 16), 1),       # null w
    ((1, 16, 4, 256, 0, 1, 16), 1),       # null x
    ((1, 16, 4, 100, 16, 1, 16), 2),      # k not a block multiple
    ((3, 16, 4, 16, 16, 1, 16), 2),       # k below the block size
    ((1, 16, 0, 256, 16, 1, 16), 2),      # n = 0
    ((1, 16, 4, 256, 16, 0, 16), 2),      # batch = 0
    ((1, 16, 4, 256, 16, 5000, 16), 2),   # batch too large
    ((1, 8, 4, 256, 16, 1, 16), 3),       # w not 16-byte aligned
    ((1, 16, 4, 256, 18, 1, 16), 3),      # x not 4-byte aligned
])
def test_gemv_rejects(args, code):
    L = tq.lib()
    t, w, n, k, x, b, y = args
    assert L.tq_gemv(t, w or None, n, k, x or None, b, y or None, None, 0, None) == code
    assert L.tq_last_error()


@pytest.mark.parametrize("args,code", [
    ((7, 16, 4, 256, 16, 1, 16), 1),          # unknown type
    ((1, 16, 4, 256, 16, 1, 0), 1),           # null y
    ((1, 16, 4, 100, 16, 1, 16), 2),          # k not a block multiple
    ((1, 16, 4, 256, 16, 5000, 16), 2),       # batch too large
    ((1, 8, 4, 256, 16, 1, 16), 3),           # w not 16-byte aligned
    ((1, 16, 4, 256, 16, 1, 18), 3),          # y not 4-byte aligned
    ((1, 16, 128256, 4096, 16, 32, 16), 4),   # its workspace would exceed the scratch
])
def test_gemv_noalloc_rejects(args, code):
    L = tq.lib()
    t, w, n, k, x, b, y = args
    assert L.tq_gemv_noalloc(t, w or None, n, k, x or None, b, y or None, None) == code
    assert L.tq_last_error()
    if code == 4:
        assert L.tq_gemv_workspace_bytes(t, n, k, b) > tq.GEMV_NOALLOC_MAX_BYTES


def test_gemv_noalloc_max_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define TQ_GEMV_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == tq.GEMV_NOALLOC_MAX_BYTES


def test_gemv_rejects_misaligned_workspace():
    L = tq.lib()
    assert L.tq_gemv(1, 16, 4, 256, 16, 1, 16, 128, 4096, None) == 3


def test_dequant_and_swiglu_reject():
    L = tq.lib()
    assert L.tq_dequant(1, 16, 4, 100, 0, 16, None) == 2
    assert L.tq_dequant(1, 16, 4, 256, 7, 16, None) == 1
    assert L.tq_dequant(1, 8, 4, 256, 0, 16, None) == 3
    assert L.tq_dequant(1, None, 0, 256, 0, None, None) == 0  # empty: nothing to do
    assert L.tq_swiglu(16, 16, -1, 16, None) == 2
    assert L.tq_swiglu(None, 16, 4, 16, None) == 1
    assert L.tq_swiglu(16, 16, 0, 16, None) == 0


def _moe_desc(t=1, hidden=7168, ffn=2048, E=256, k=8, path=0):
    d = tq.MoeDesc()
    d.type, d.hidden, d.ffn, d.n_experts, d.top_k = t, hidden, ffn, E, k
    d.router_w = 0x10000  # never dereferenced: every call below fails validation first
    d.experts = 0x20000
    d.path = path
    return d


def test_moe_workspace_sizes_follow_the_path():
    import ctypes as C

    L = tq.lib()
    f32 = L.tq_moe_workspace_bytes(C.byref(_moe_desc(path=tq.PATH_F32)), 4096)
    mf = L.tq_moe_workspace_bytes(C.byref(_moe_desc(path=tq.PATH_BF16_MFMA)), 4096)
    auto = L.tq_moe_workspace_bytes(C.byref(_moe_desc(path=tq.PATH_AUTO)), 4096)
    P = 4096 * 8
    assert mf == auto  # 128 routed tokens per expert: AUTO takes the matrix cores
    assert mf >= P * 7168 * 4 + P * 2048 * 2 + 4096 * 7168 * 2 and f32 >= P * 2048 * 4
    assert L.tq_moe_workspace_bytes(C.byref(_moe_desc(t=2, path=tq.PATH_BF16_MFMA)), 4096) == 0


def test_moe_stages_and_path_rejected_before_any_launch():
    import ctypes as C

    L = tq.lib()
    d = _moe_desc(hidden=512, ffn=512, E=8, k=2)
    for stages in (0, 8, -1):
        assert L.tq_moe_ffn_stages(C.byref(d), 0x30000, 4, 0x40000, 0x50000, 1 << 30, None,
                                   stages, None) == 1
    assert L.tq_moe_ffn_stages(C.byref(d), 0x30000, 4, 0x40000, 0x50000, 256, None,
                               tq.MOE_ALL, None) == 4  # workspace too small
    d6 = _moe_desc(t=2, hidden=512, ffn=512, E=8, k=2, path=tq.PATH_BF16_MFMA)
    assert L.tq_moe_ffn(C.byref(d6), 0x30000, 4, 0x40000, 0x50000, 1 << 30, None, None) == 5
    assert "Q4_K" in L.tq_last_error().decode()


def test_moe_host_resident_rejects_null_host_blob():
    import ctypes as C

    L = tq.lib()
    d = _moe_desc(hidden=512, ffn=512, E=2, k=1)
    table = (tq.Expert * 2)(tq.Expert(0x100000, 0x200000, 0x300000), tq.Expert(0x400000, None, 0x500000))
    d.experts = None
    d.experts_host = C.addressof(table)
    d.experts_on_host = 1
    assert L.tq_moe_ffn(C.byref(d), 0x30000, 4, 0x40000, 0x50000, 1 << 34, None, None) == 1
    assert "experts_host" in L.tq_last_error().decode()


def _chain_op(**kw):
    op = tq.ChainOp()
    op.nparts, op.swiglu, op.k = kw.get("nparts", 1), kw.get("swiglu", 0), kw.get("k", 4096)
    for p in range(4):
        op.w[p] = kw.get("w", 4096)
        op.n[p] = kw.get("n", 64)
        op.y[p] = kw.get("y", 4096)
    op.x = kw.get("x", 4096)
    return op


@pytest.mark.parametrize("kw,code", [
    (dict(k=100), 2),             # k not a multiple of 256
    (dict(k=16640), 2),           # k beyond 16384
    (dict(nparts=0), 1),          # no matrix
    (dict(nparts=5), 1),          # too many matrices
    (dict(swiglu=2), 1),          # swiglu flag not 0/1
    (dict(swiglu=1, nparts=3), 1),
    (dict(x=0), 1),               # null x
    (dict(x=4100), 3),            # x not 16-byte aligned
    (dict(w=4104), 3),            # w not 16-byte aligned
    (dict(n=0), 2),               # no rows
])
def test_chain_prepare_rejects(kw, code):
    """Every op is checked before anything touches the device."""
    L = tq.lib()
    ops = (tq.ChainOp * 2)(_chain_op(), _chain_op(**kw))
    nbytes = L.tq_chain_plan_bytes(2)
    assert nbytes > 0
    assert L.tq_chain_prepare(1, ops, 2, 4096, nbytes) == code
    assert L.tq_last_error()


def test_chain_prepare_and_run_argument_checks():
    L = tq.lib()
    ops = (tq.ChainOp * 1)(_chain_op())
    assert L.tq_chain_plan_bytes(0) == 0 and L.tq_chain_plan_bytes(5000) == 0
    assert L.tq_chain_prepare(2, ops, 1, 4096, 1 << 20) == 5     # Q6_K: unsupported
    assert L.tq_chain_prepare(9, ops, 1, 4096, 1 << 20) == 1     # unknown type
    assert L.tq_chain_prepare(1, ops, 1, 4096, 16) == 4          # plan too small
    assert L.tq_chain_prepare(1, ops, 1, 4100, 1 << 20) == 3     # plan not 256-byte aligned
    assert L.tq_chain_run(None, None) == 1
    assert L.tq_chain_run(4100, None) == 3
    # the persistent chain is switched off in this build: refused before any launch
    assert L.tq_chain_run(4096, None) == 5
    assert "switched off" in L.tq_last_error().decode()


def test_tuning_knobs_match_header_and_round_trip():
    src = open(HEADER).read()
    declared = {m.group(1).lower(): int(m.group(2))
                for m in re.finditer(r"TQ_KNOB_([A-Z0-9_]+) = (\d+)", src)}
    count = declared.pop("count")
    assert declared == tq.KNOBS and count == len(tq.KNOBS)
    L = tq.lib()
    for name, i in tq.KNOBS.items():
        assert L.tq_tuning_get(i) == -1, name
    assert L.tq_tuning_set(tq.KNOBS["gemv_i8"], 2) == 0 and L.tq_tuning_get(tq.KNOBS["gemv_i8"]) == 2
    assert L.tq_tuning_set(tq.KNOBS["gemv_i8"], 0) == 0 and L.tq_tuning_get(tq.KNOBS["gemv_i8"]) == 0
    assert L.tq_tuning_set(tq.KNOBS["gemv_i8"], -1) == 0 and L.tq_tuning_get(tq.KNOBS["gemv_i8"]) == -1
    assert L.tq_tuning_set(count, 1) == 1 and L.tq_tuning_set(-1, 1) == 1
    assert L.tq_tuning_get(count) == -1
    with tq.knobs(moe_nt=4, kl_rows=8):
        assert tq.get_knob("moe_nt") == 4 and tq.get_knob("kl_rows") == 8
    assert tq.get_knob("moe_nt") == -1 and tq.get_knob("kl_rows") == -1


def test_library_reads_no_environment():
    """Kernel selection is set through the tuning knobs only: no source of the library reads the
    environment."""
    import glob

    root = os.path.join(os.path.dirname(HEADER), "..", "moe_expert_ffn_q4_amd", "csrc")
    for path in glob.glob(os.path.join(root, "**", "*.*"), recursive=True):
        if path.endswith((".hip", ".h", ".cpp")):
            assert "getenv" not in open(path).read(), path
