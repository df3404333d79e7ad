"""Build libtq.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m moe_expert_ffn_q4_amd.build [-v]
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
OBJ = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 ops stay off: plain v_fma_f32 / v_add_f32 everywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


RESOURCES = os.path.join(OBJ, "kernel_resources.json")
REMARKS = "-Rpass-analysis=kernel-resource-usage"


def parse_resource_remarks(text: str) -> dict:
    """Per-kernel register, scratch, occupancy and LDS figures from the compiler's
    kernel-resource-usage remarks: {mangled name: {field: int}}."""
    import re

    out, cur = {}, None
    fields = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
              "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].strip()
        body = re.sub(r"\s*\[-Rpass-analysis=kernel-resource-usage\]$", "", body)
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
            continue
        if cur is None or ":" not in body:
            continue
        key, val = body.rsplit(":", 1)
        key = key.strip()
        if key in fields and val.strip().lstrip("-").isdigit():
            out[cur][fields[key]] = int(val)
    return out


def _compile(src: str, verbose: bool) -> tuple:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, REMARKS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj, parse_resource_remarks(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [o for o, _ in results]
    resources = {}
    for _, r in results:
        resources.update(r)
    import json

    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_read_ref(verbose)
    return LIB


READ_REF = os.path.join(HERE, "libtq_readref.so")


def build_read_ref(verbose: bool = False) -> str:
    """libtq_readref.so: the plain streaming-read kernel the benchmark compares the GEMV with."""
    src = os.path.join(CSRC, "ref", "tq_read_ref.hip")
    tmp = READ_REF + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, READ_REF)
    return READ_REF


def kernel_resources() -> dict:
    """The per-kernel figures recorded by the last build (compiling the sources, without linking,
    when no build has recorded them or a source is newer than the record)."""
    import json

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
    if os.path.exists(RESOURCES) and all(os.path.getmtime(RESOURCES) >= os.path.getmtime(p)
                                         for p in srcs):
        with open(RESOURCES) as f:
            return json.load(f)
    os.makedirs(OBJ, exist_ok=True)

    def one(src):
        cmd = [HIPCC, *FLAGS, REMARKS, "--offload-device-only", "-c", src, "-o", os.devnull]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return parse_resource_remarks(r.stderr)

    hips = [p for p in srcs if p.endswith(".hip")]
    out = {}
    with ThreadPoolExecutor(max_workers=min(8, len(hips))) as ex:
        for r in ex.map(one, hips):
            out.update(r)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
