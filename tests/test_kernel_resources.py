"""The hot kernels as compiled for gfx950: no scratch memory, and the occupancy they were tuned
at. Scratch use has twice crept in unnoticed (a pointer map built inside a kernel and indexed at
run time, a HIP float4 array of prefetched values); each time it put a full wait on the memory
pipeline into the inner loop. The figures are the compiler's kernel-resource-usage remarks,
recorded by the build (or compiled here when no build has recorded them)."""
import re

import pytest

from moe_expert_ffn_q4_amd import build

# (pattern on the mangled name, least occupancy in waves per SIMD)
HOT = [
    (r"k_gemv_mfILi1ELi\d+ELi\d+ELi[01]E", 4),  # batch-1 Q4_K GEMV, fp16 matrix cores
    (r"k_gemv_mfILi1ELi\d+ELi\d+ELi2E", 3),     # the same, two tiles in flight
    (r"k_gemv_mfILi2E", 2),                      # batch-1 Q6_K GEMV (8-wave workgroups)
    (r"k_gemv_klILi4E", 2),          # batch-1 Q4_K GEMV, lanes along k
    (r"k_moe_klILi4E", 2),           # one-token MoE experts
    (r"k_moe_mfILi1ELi\d+ELi\d+ELi[01]E", 4),   # one-token MoE experts, fp16 matrix cores
    (r"k_moe_mfILi1ELi\d+ELi\d+ELi2E", 3),      # the same, two tiles in flight
    (r"k_gemv_i8ILi1E", 4),          # batch-1 Q4_K GEMV, int8 matrix cores, sliced k
    (r"k_gemv_i8ILi3E", 3),          # batch-1 Q8_0 GEMV, int8 matrix cores, sliced k
    (r"k_gemm_f32m_q8", 4),          # Q8_0 batches, fp32 matrix cores
    (r"k_gemm_f32m_q6", 2),          # Q6_K batches
    (r"k_qmm_denseI", 1),            # dense few-token Q4_K products, fp16 matrix cores
    (r"k_qmm_dense2I", 2),           # the same with the activations split in the kernel
    (r"k_qmmILb", 1),                # MoE few-token products
    (r"k_prefillI", 1),              # prompt-sized MoE products, bf16 matrix cores
    (r"k_gemvILi[123]ELi[1248]E", 1),  # fp32 lane-per-row GEMV
    (r"k_router|k_topk|k_group|k_moe_combine|k_moe_swiglu|k_split_rows|k_dequant", 1),
]


@pytest.fixture(scope="module")
def resources():
    return build.kernel_resources()


def test_remarks_parsed(resources):
    assert len(resources) >= 20, sorted(resources)
    some = next(iter(resources.values()))
    assert {"vgprs", "scratch", "occupancy"} <= set(some), some


@pytest.mark.parametrize("pattern,occ", HOT, ids=[p for p, _ in HOT])
def test_hot_kernels_use_no_scratch(resources, pattern, occ):
    hits = {k: v for k, v in resources.items() if re.search(pattern, k)}
    assert hits, f"no kernel matches {pattern}"
    for name, r in hits.items():
        assert r["scratch"] == 0, f"{name}: {r['scratch']} bytes of scratch per lane"
        assert r["occupancy"] >= occ, f"{name}: occupancy {r['occupancy']} < {occ}"


# (pattern, largest LDS bytes per workgroup): the lanes-along-k kernels keep only their reduction
# table in LDS. The one-token MoE kernel once carried 20 KB more: the compiler had turned the
# pick between the gate and up pointers into a per-lane table in LDS, sized for the 512-thread
# bound and read back before every pass's loads.
# The fp16 matrix-core GEMV kernels plan their dynamic LDS below 64 KB less these static bytes.
SMALL_LDS = [(r"k_gemv_klILi", 1024), (r"k_moe_klILi", 1024), (r"k_router_mf|k_router_kl", 0),
             (r"k_gemv_mfI", 64), (r"k_moe_mfI", 1152)]


@pytest.mark.parametrize("pattern,most", SMALL_LDS, ids=[p for p, _ in SMALL_LDS])
def test_lanes_along_k_kernels_keep_lds_small(resources, pattern, most):
    hits = {k: v for k, v in resources.items() if re.search(pattern, k)}
    assert hits, f"no kernel matches {pattern}"
    for name, r in hits.items():
        assert r["lds"] <= most, f"{name}: {r['lds']} bytes of LDS"
