"""Benchmark: decode throughput of block-quantized projections on one MI355X.

Default workload: a Llama-3-8B-shaped decode step over 32 layers of Q4_K projections at batch 1
(per layer q 4096->4096, k/v 4096->1024, o 4096->4096, gate/up 4096->14336, SwiGLU,
down 14336->4096), seeded synthetic weights and N(0,1) activations resident in HBM.
One step = every projection of every layer plus the SwiGLU, through the C ABI: per layer four
launches (q|k|v sharing x, o, gate|up with the SwiGLU fused, down).

Prints one JSON line: tokens/s for the whole step, the roofline of the dominant kernel (the
Q4_K GEMV; achieved = algorithmic bytes / its average launch time measured with HIP events on
the launch stream), and the CPU oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X
# Sources of the batch-1 Q4_K GEMV; the committed counter summary records their hash, and its
# HBM traffic is reported only while the kernel is unchanged since the counters were taken.
GEMV_SOURCES = ("moe_expert_ffn_q4_amd/csrc/tq_gemv_mf.hip", "moe_expert_ffn_q4_amd/csrc/tq_gemv_mf.h",
                "moe_expert_ffn_q4_amd/csrc/tq_dense.hip", "moe_expert_ffn_q4_amd/csrc/tq_gemv_core.h",
                "moe_expert_ffn_q4_amd/csrc/tq_device.h")
GEMV_COUNTERS = "profiles/k_gemv_mf_llama8b_b1_hbm_counters.txt"
# The same for the few-token products of the batch-8 step (tq::k_qmm_dense2).
QMM_SOURCES = ("moe_expert_ffn_q4_amd/csrc/tq_qmm.hip", "moe_expert_ffn_q4_amd/csrc/tq_qmm.h",
               "moe_expert_ffn_q4_amd/csrc/tq_gemv_core.h", "moe_expert_ffn_q4_amd/csrc/tq_mfma.h",
               "moe_expert_ffn_q4_amd/csrc/tq_device.h")
B8_COUNTERS = "profiles/k_qmm_dense2_llama8b_b8_hbm_counters.txt"
C1_COUNTERS = "profiles/k_gemv_mf_c1_4096x4096_hbm_counters.txt"
METRIC = "Q4_K GEMV HBM GB/s (% of peak); decode tokens/s for 8B-shaped and MoE layers"


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--batch", type=int, default=1, help="tokens per decode step (1 or 8)")
    p.add_argument("--workload", default="llama8b",
                   choices=["llama8b", "c1", "llama70b", "mixtral", "deepseek", "deepseek-prefill",
                            "deepseek-host"],
                   help="llama8b: 32-layer dense decode step (default); c1: one 4096x4096 Q4_K "
                        "GEMV at batch 1 over 64 distinct weight copies, next to a plain read of "
                        "the same bytes; mixtral / deepseek: one "
                        "MoE layer at --batch tokens; deepseek-prefill: one DeepSeek-shaped MoE "
                        "layer over --tokens (default 4096) on the bf16 matrix-core path; "
                        "deepseek-host: the DeepSeek decode layer at --batch tokens with the routed "
                        "experts in pinned host memory, copied per step; llama70b: one "
                        "Llama-3-70B-shaped layer in each of Q4_K, Q6_K and Q8_0 at batch 1, 4 "
                        "and 16")
    p.add_argument("--tokens", type=int, default=4096, help="tokens of the prefill workload")
    p.add_argument("--cache-slots", type=int, nargs="*", default=None,
                   help="deepseek-host: also sweep an expert residency cache of these slot "
                        "counts over a Zipf-skewed routing trace (0 = no cache)")
    p.add_argument("--prefetch", type=int, nargs="*", default=[0, 4],
                   help="deepseek-host cache sweep: experts prefetched per call (each value is "
                        "swept with every slot count)")
    p.add_argument("--seed", type=int, default=42)
    p.add_argument("--knob", action="append", default=[], metavar="NAME=VALUE",
                   help="override a library tuning knob (tq.KNOBS) for a tuning run; the "
                        "defaults are the production choices")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (the known-size reference for the "
                        "FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--kernel-summary", nargs="+", metavar="CSV",
                   help="no GPU: print the kernel statistics of a rocprofv3 kernel-stats CSV and "
                        "the per-kernel averages of any counter-collection CSVs that follow")
    p.add_argument("--summarize", nargs=3, metavar=("KERNEL_STATS", "FETCH_CSV", "WRITE_CSV"),
                   help="no GPU: print a text summary of a rocprofv3 kernel-stats CSV and two "
                        "counter-collection CSVs (FETCH_SIZE, WRITE_SIZE) of the llama8b batch-1 "
                        "step (or of --workload c1), with per-launch HBM traffic of the Q4_K "
                        "GEMV")
    return p.parse_args()


def source_hash(paths=GEMV_SOURCES):
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def timed_replays(torch, graph, stream, steps):
    """The timed region: `steps` replays of `graph` back to back on `stream`, bracketed by device
    synchronizations, with a HIP event recorded on that stream before each replay and after the
    last. Returns (wall-clock seconds of the region, per-replay milliseconds from the events)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i].record(stream)
        graph.replay()
    evs[steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]


def trial_stats(ms, per=1):
    """Median and 10th / 90th percentiles of per-replay times (divided by `per` launches)."""
    import numpy as np

    a = np.asarray(ms, np.float64) / per
    return {"trials": int(a.size), "median_ms": round(float(np.median(a)), 5),
            "p10_ms": round(float(np.percentile(a, 10)), 5),
            "p90_ms": round(float(np.percentile(a, 90)), 5)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def oracle_repeat(fn, budget_s, max_reps):
    """Calls fn() until about budget_s of wall time or max_reps calls; (calls, seconds)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s or reps >= max_reps:
            return reps, elapsed


def single_thread(fn, budget_s, max_reps):
    """oracle_repeat with the oracle's loops on one thread (the default restored after)."""
    import oracle

    n = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        return oracle_repeat(fn, budget_s, max_reps)
    finally:
        oracle.set_num_threads(n)


def check_against(got, ref, mag):
    """Every element of a GPU result against the oracle's: the worst |err| / (1e-3 mag + 1e-5)."""
    import numpy as np

    err = np.abs(np.asarray(got, np.float64) - ref)
    worst = float(np.max(err / (1e-3 * mag + 1e-5))) if err.size else 0.0
    return {"elements": int(err.size), "max_err_over_bound": float(f"{worst:.3g}"),
            "pass": bool(worst <= 1.0)}


def llama8b_bytes_per_launch(synth, batch=1):
    """Algorithmic bytes of the average GEMV launch of the dense step's GEMV pass: per layer the
    launches q|k|v, o, gate|up and down, each reading its weight blobs once plus fp32 x and y."""
    shapes = {name: (n, k) for name, n, k in synth.dense_projections(synth.LLAMA8B)}
    launches = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    tot = 0
    for names in launches:
        k = shapes[names[0]][1]
        rows = sum(shapes[m][0] for m in names)
        tot += rows * (k // 256) * 144 + 4 * batch * (rows + k)
    return tot / len(launches)


def summarize(kt_csv, fetch_csv, write_csv, workload="llama8b", batch=1):
    """Text summary of the profiler's CSVs for the GEMV of the llama8b step at this batch (or of
    the c1 workload). FETCH_SIZE and WRITE_SIZE are scaled by what they read for the 1 GiB copy
    (--calibrate-copy)."""
    import csv
    from collections import defaultdict

    import synth

    lines = []
    lines.append("# per-kernel statistics (rocprofv3 --kernel-trace --stats)")
    lines.append(f"{'kernel':<64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}")
    for r in csv.DictReader(open(kt_csv)):
        lines.append(f"{r['Name'][:64]:<64s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:9.3f} "
                     f"{float(r['MinNs'])/1e3:8.3f} {float(r['MaxNs'])/1e3:8.3f} "
                     f"{float(r['Percentage']):6.2f}")

    def load(p):
        d = defaultdict(list)
        for r in csv.DictReader(open(p)):
            key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]))
            d[key].append(float(r["Counter_Value"]))
        return d

    fetch, write = load(fetch_csv), load(write_csv)
    copy = [k for k in fetch if "copyBuffer" in k[0] and sum(fetch[k]) / len(fetch[k]) > 1e5]
    if len(copy) != 1:
        raise SystemExit("expected exactly one 1 GiB copy launch (run the bench with "
                         "--calibrate-copy)")
    gib_kib = float(1 << 20)
    f_factor = gib_kib / fetch[copy[0]][0]
    w_factor = gib_kib / write[copy[0]][0]
    lines.append("")
    lines.append("# HBM counters (rocprofv3 --pmc, one counter per run), KiB per dispatch")
    lines.append(f"1 GiB copy: FETCH_SIZE {fetch[copy[0]][0]:.1f} KiB -> factor {f_factor:.4f}; "
                 f"WRITE_SIZE {write[copy[0]][0]:.1f} KiB -> factor {w_factor:.4f}")
    lines.append(f"{'kernel':<40s} {'grid':>8s} {'wg':>4s} {'n':>6s} {'FETCH_KiB':>11s} "
                 f"{'WRITE_KiB':>10s} {'bytes/launch (scaled)':>22s}")
    tot_bytes, tot_n = 0.0, 0
    kern = b1_kernel() if batch == 1 else "k_qmm_dense"
    for key in sorted(fetch, key=lambda k: -sum(fetch[k])):
        if kern not in key[0]:
            continue
        fv, wv = fetch[key], write.get(key, [0.0])
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        b = (fk * f_factor + wk * w_factor) * 1024
        tot_bytes += b * len(fv)
        tot_n += len(fv)
        lines.append(f"{key[0][:40]:<40s} {key[1]:8d} {key[2]:4d} {len(fv):6d} {fk:11.1f} "
                     f"{wk:10.1f} {b:22.0f}")
    algo = C1_BYTES_PER_LAUNCH if workload == "c1" else llama8b_bytes_per_launch(synth, batch)
    traffic = tot_bytes / tot_n
    lines.append("")
    lines.append(f"algorithmic_bytes_per_launch: {algo:.0f}")
    lines.append(f"traffic_bytes_per_launch: {traffic:.0f}")
    lines.append(f"traffic_over_algorithmic: {traffic / algo:.4f}")
    lines.append(f"kernel_source_sha256: {source_hash(GEMV_SOURCES if batch == 1 else QMM_SOURCES)}")
    return "\n".join(lines)


def kernel_summary(stats_csv, *counter_csvs):
    """Kernel statistics table plus per-(kernel, grid) averages of the collected counters."""
    import csv
    from collections import defaultdict

    lines = [f"{'kernel':<72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in csv.DictReader(open(stats_csv)):
        lines.append(f"{r['Name'][:72]:<72s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.3f} "
                     f"{float(r['MinNs'])/1e3:9.3f} {float(r['MaxNs'])/1e3:9.3f} "
                     f"{float(r['Percentage']):6.2f}")
    for path in counter_csvs:
        agg = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"][:60], int(r["Grid_Size"]), int(r["Workgroup_Size"]))
            agg[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        lines.append("")
        lines.append(f"# counters per dispatch (mean over dispatches) from {os.path.basename(os.path.dirname(path))}")
        for key in sorted(agg, key=lambda k: -max(sum(v) for v in agg[k].values())):
            vals = " ".join(f"{c}={sum(v) / len(v):.4g}" for c, v in sorted(agg[key].items()))
            n = max(len(v) for v in agg[key].values())
            lines.append(f"{key[0]:<60s} grid={key[1]} wg={key[2]} n={n} {vals}")
    return "\n".join(lines)


def recorded_traffic(summary=GEMV_COUNTERS, sources=GEMV_SOURCES):
    """HBM bytes per GEMV launch from a committed counter summary, or None when the kernel's
    sources have changed since the counters were taken (or there is no summary)."""
    path = os.path.join(ROOT, summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != source_hash(sources):
        return None
    return float(fields["traffic_bytes_per_launch"])


def build_dense_model(tq, synth, torch, batch, seed):
    shape = synth.LLAMA8B
    layers = []
    for layer in range(shape["layers"]):
        projs = {}
        for name, n, k in synth.dense_projections(shape):
            w = synth.blob("q4_k", synth.rng(seed, "8b", layer, name), n, k)
            projs[name] = (torch.from_numpy(w).to("cuda"), n, k)
        g = synth.rng(seed, "8b-act", layer, batch)
        x = torch.from_numpy(synth.normal_f32(g, (batch, shape["hidden"]))).to("cuda")
        a = torch.from_numpy(synth.normal_f32(g, (batch, shape["hidden"]))).to("cuda")
        layers.append((projs, x, a))
    return layers


def b1_kernel(tq=None):
    """The kernel of batch-1 Q4_K products with k < 16384 under the current knobs (the fp16
    matrix-core kernel unless switched off; the int8 one only when its knob is 2)."""
    if tq is None:
        import moe_expert_ffn_q4_amd as tq
    if tq.get_knob("gemv_i8") == 2:
        return "k_gemv_i8"
    return "k_gemv_kl" if tq.get_knob("gemv_mf") == 0 else "k_gemv_mf"


def gemv_kernel_name(tq, batch):
    """The kernel that tq_gemv runs for the 8B shapes (k = 4096 and 14336) at this batch, given
    its workspace."""
    if batch == 1:
        return f"tq_gemv Q4_K batch 1 (tq::{b1_kernel(tq)})"
    if batch <= 16 and tq.get_knob("gemv_qmm") != 0 and tq.get_knob("qmm_inline") != 0:
        return f"tq_gemv Q4_K batch {batch} (tq::k_qmm_dense2, activations split in the kernel)"
    if batch <= 32 and tq.get_knob("gemv_qmm") != 0:
        return f"tq_gemv Q4_K batch {batch} (tq::k_qmm_dense, after tq::k_split_rows)"
    return f"tq_gemv Q4_K batch {batch} (tq::k_gemv)"


def make_step(tq, torch, layers, batch, events=None, gemv_only=False):
    """One decode step through the C ABI. Per layer: q, k and v (input x) in one tq_gemv_multi
    launch, o (input: the attention stand-in a), gate and up (input x) with the SwiGLU between
    them in one tq_gemv_swiglu launch, down (input: the SwiGLU output). gemv_only: the same
    products without the SwiGLU (gate and up as a two-matrix tq_gemv_multi), for timing the
    GEMV kernel alone."""
    import ctypes as C

    H = 4096
    F = 14336
    dev = "cuda"
    bufs = dict(q=torch.empty(batch, H, device=dev), k=torch.empty(batch, 1024, device=dev),
                v=torch.empty(batch, 1024, device=dev), o=torch.empty(batch, H, device=dev),
                gate=torch.empty(batch, F, device=dev), up=torch.empty(batch, F, device=dev),
                h=torch.empty(batch, F, device=dev), down=torch.empty(batch, H, device=dev))
    L = tq.lib()
    shapes = ((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336))
    ws_bytes = max([tq.gemv_workspace_bytes("q4_k", n, k, batch) for n, k in shapes] +
                   [int(L.tq_gemv_swiglu_workspace_bytes(tq.Q4_K, F, H, batch)),
                    tq.gemv_workspace_bytes("q4_k", F, H, batch)])
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def check(rc):
        if rc:
            raise tq.TQError(rc, L.tq_last_error().decode())

    def nbytes(names, projs):
        return sum(projs[m][0].numel() for m in names)

    def multi(names, projs, x):
        P = len(names)
        w = (C.c_void_p * P)(*[projs[m][0].data_ptr() for m in names])
        n = (C.c_int64 * P)(*[projs[m][1] for m in names])
        y = (C.c_void_p * P)(*[bufs[m].data_ptr() for m in names])
        k = projs[names[0]][2]
        stream = torch.cuda.current_stream().cuda_stream
        check(L.tq_gemv_multi(tq.Q4_K, P, w, n, y, k, x.data_ptr(), batch, ws.data_ptr(),
                              ws.numel(), stream))
        if events is not None:  # algorithmic bytes of this launch
            events.append(nbytes(names, projs) + 4 * batch * (sum(projs[m][1] for m in names) + k))

    def swiglu(projs, x):
        stream = torch.cuda.current_stream().cuda_stream
        check(L.tq_gemv_swiglu(tq.Q4_K, projs["gate"][0].data_ptr(), projs["up"][0].data_ptr(), F,
                               H, x.data_ptr(), batch, bufs["h"].data_ptr(), ws.data_ptr(),
                               ws.numel(), stream))

    def step():
        for projs, x, a in layers:
            multi(("q", "k", "v"), projs, x)
            multi(("o",), projs, a)
            if gemv_only:
                multi(("gate", "up"), projs, x)
            else:
                swiglu(projs, x)
            multi(("down",), projs, bufs["h"])

    return step


def cpu_baseline(synth, batch, seed, budget_s, tq, torch):
    """The oracle (as it is) on a bounded sample of the same step: whole layers (layer 0's seven
    Q4_K projections at the bench's batch), on all the host's threads until about budget_s,
    then on one thread for about a third of that, each scaled to a 32-layer step. The outputs of
    the all-core run are checked element by element against the GPU's for the same inputs."""
    import oracle

    shape = synth.LLAMA8B
    projs = []
    for name, n, k in synth.dense_projections(shape):
        w = synth.blob("q4_k", synth.rng(seed, "8b", 0, name), n, k)
        x = synth.normal_f32(synth.rng(seed, "cpu-x", name, batch), (batch, k))
        projs.append((w, n, k, x))
    refs = []

    def layer():
        refs[:] = [oracle.gemv("q4_k", w, n, k, x) for w, n, k, x in projs]

    layers, elapsed = oracle_repeat(layer, budget_s, 100 * shape["layers"])
    cores = oracle.num_threads()
    # the same products on the GPU, every element against the oracle's
    checks = []
    for (w, n, k, x), (ref, mag) in zip(projs, refs):
        y = tq.gemv("q4_k", torch.from_numpy(w).cuda(), n, k, torch.from_numpy(x).cuda())
        checks.append(check_against(y.cpu().numpy(), ref, mag))
    one = lambda: [oracle.gemv("q4_k", w, n, k, x) for w, n, k, x in projs[:4]]
    reps1, el1 = single_thread(one, budget_s / 3, 10000)
    frac4 = sum(w.size for w, *_ in projs[:4]) / sum(w.size for w, *_ in projs)
    step1 = el1 / reps1 / frac4 * shape["layers"]
    step_s = elapsed / layers * shape["layers"]
    return {"value": round(batch / step_s, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{layers} full layers (7 Q4_K projections each, batch {batch}) in "
                      f"{elapsed:.1f} s on {cores} threads, scaled to a 32-layer step",
            "single_thread": {"value": round(batch / step1, 5), "unit": "tokens/s",
                              "sample": f"{reps1} x (q, k, v, o) in {el1:.1f} s on 1 thread, "
                                        f"scaled by blob bytes to a 32-layer step"},
            "checked_vs_gpu": {"elements": sum(c["elements"] for c in checks),
                               "max_err_over_bound": max(c["max_err_over_bound"] for c in checks),
                               "pass": all(c["pass"] for c in checks),
                               "what": "layer 0's 7 projections, every output element, the "
                                       "all-core oracle's result against tq_gemv's"}}


def c1_cpu_baseline(w, x, y_gpu, n, k, budget_s):
    """The oracle on the same 4096x4096 GEMV: all threads, then one thread; GB/s of blob bytes
    processed. The all-core result is checked element by element against the GPU's."""
    import oracle

    out = {}

    def gemv():
        out["ref"] = oracle.gemv("q4_k", w, n, k, x)

    reps, el = oracle_repeat(gemv, budget_s, 100000)
    cores = oracle.num_threads()
    ref, mag = out["ref"]
    reps1, el1 = single_thread(lambda: oracle.gemv("q4_k", w, n, k, x), budget_s / 3, 10000)
    return {"value": round(w.size * reps / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{reps} GEMVs of the same 4096x4096 Q4_K blob in {el:.1f} s on {cores} "
                      f"threads",
            "single_thread": {"value": round(w.size * reps1 / el1 / 1e9, 5), "unit": "GB/s",
                              "sample": f"{reps1} GEMVs in {el1:.1f} s on 1 thread"},
            "checked_vs_gpu": dict(check_against(y_gpu, ref, mag),
                                   what="every output row of the GEMV")}


def moe_cpu_baseline(synth, shape, layer, x, y_gpu, ids_gpu, budget_s):
    """The oracle (as it is) on a bounded sample of the same layer: routing of the tokens and
    their MoE output, on all the host's threads one token at a time until about budget_s, then
    on one thread for about a third of that. The all-core outputs are checked element by
    element against the GPU's y for the tokens whose oracle routing picked the same experts."""
    import numpy as np

    import oracle

    k = shape["top_k"]
    H, F = shape["hidden"], shape["ffn"]
    T = x.shape[0]
    res = []
    n = [0]

    def token():  # the T tokens in turn (again from the first when T are done within the budget)
        t = n[0] % T
        xt = x[t:t + 1]
        ids, wts = oracle.topk(oracle.router_logits(xt, layer["router"]), k)
        y, mag = oracle.moe("q4_k", H, F, layer["experts"], layer["shared"], xt, ids, wts,
                            grouped=False)
        if n[0] < T:
            res.append((ids, y, mag))
        n[0] += 1

    done, elapsed = oracle_repeat(token, budget_s, 1 << 30)
    cores = oracle.num_threads()
    checks, skipped = [], 0
    for t, (ids, y, mag) in enumerate(res):
        if np.array_equal(np.sort(ids[0]), np.sort(ids_gpu[t])):
            checks.append(check_against(y_gpu[t:t + 1], y, mag))
        else:  # a near tie the two evaluations of the logits resolved differently
            skipped += 1
    checks = checks or [{"elements": 0, "max_err_over_bound": 0.0, "pass": False}]
    n1 = [0]

    def token1():
        xt = x[n1[0] % x.shape[0]:n1[0] % x.shape[0] + 1]
        ids, wts = oracle.topk(oracle.router_logits(xt, layer["router"]), k)
        oracle.moe("q4_k", H, F, layer["experts"], layer["shared"], xt, ids, wts, grouped=False)
        n1[0] += 1

    done1, el1 = single_thread(token1, budget_s / 3, 1 << 30)
    return {"value": round(done / elapsed, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} token evaluations of the same layer (its {T} tokens in turn; "
                      f"routing + fp64 MoE output, one token at a time) in {elapsed:.1f} s on "
                      f"{cores} threads",
            "single_thread": {"value": round(done1 / el1, 5), "unit": "tokens/s",
                              "sample": f"{done1} tokens in {el1:.1f} s on 1 thread"},
            "checked_vs_gpu": {"elements": sum(c["elements"] for c in checks),
                               "max_err_over_bound": max(c["max_err_over_bound"] for c in checks),
                               "pass": all(c["pass"] for c in checks),
                               "tokens_skipped_on_near_ties": skipped,
                               "what": f"y of the {len(res)} sampled tokens, every element, the "
                                       f"all-core oracle's (its own routing) against the GPU's"}}


def moe_bench(args, torch, tq, synth):
    """One MoE layer (Mixtral- or DeepSeek-shaped, Q4_K experts), graph-captured: decode batches
    on the fp32 GEMV path, or the 4096-token prefill on the bf16 matrix-core path.

    Roofline of the expert products (the stage that holds the dominant kernels), replayed alone
    as a graph between two events on its stream: decode -> HBM bytes (blobs of the experts the
    routing selected plus the shared expert, each read once, and the activations); prefill ->
    FFN flops (2 * 3 * hidden * ffn per routed pair and per token for the shared expert)."""
    import numpy as np

    prefill = args.workload == "deepseek-prefill"
    shape = synth.MIXTRAL if args.workload == "mixtral" else synth.DEEPSEEK
    k = shape["top_k"]
    T = args.tokens if prefill else args.batch
    tag = "deepseek" if prefill else args.workload
    layer = synth.moe_layer(shape, "q4_k", seed=args.seed, tag=tag)
    experts = [tuple(torch.from_numpy(b).cuda() for b in e) for e in layer["experts"]]
    shared = tuple(torch.from_numpy(b).cuda() for b in layer["shared"]) if layer["shared"] else None
    path = tq.PATH_BF16_MFMA if prefill else tq.PATH_F32
    moe = tq.MoeLayer("q4_k", shape["hidden"], shape["ffn"], torch.from_numpy(layer["router"]).cuda(),
                      experts, shared, top_k=k, path=path)
    xh = synth.normal_f32(synth.rng(args.seed, "bench-x", T), (T, shape["hidden"]))
    x = torch.from_numpy(xh).cuda()
    y = torch.empty_like(x)
    ws = torch.empty(moe.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    E = shape["n_experts"]
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    ids_gpu = torch.empty((T, k), dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        moe(x, out=y, ws=ws, routing=dict(counts=counts, topk_ids=ids_gpu))
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            moe(x, out=y, ws=ws)
        for _ in range(args.warmup):
            graph.replay()
        elapsed, per_step = timed_replays(torch, graph, stream, args.steps)
        # the expert-product stage alone (routing already in the workspace)
        egraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(egraph, stream=stream):
            moe(x, ws=ws, stages=tq.MOE_EXPERTS)
        egraph.replay()
        reps = max(3, args.steps)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            egraph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
    stage_s = ev0.elapsed_time(ev1) / 1000 / reps
    c = counts.cpu().numpy()
    H, F = shape["hidden"], shape["ffn"]
    eb = sum(b.numel() for b in experts[0])
    active = int((c > 0).sum()) + (1 if shared else 0)
    ms = elapsed * 1000 / args.steps
    if prefill:
        rows = T * k + (T if shared else 0)
        flops = 2 * 3 * H * F * rows
        achieved = flops / stage_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "tq_moe_ffn expert stage: k_prefill gate/up+SwiGLU and down "
                          "(with x->bf16 and the chunk table)",
                "avg_launch_us": round(stage_s * 1e6, 1)}
        dtype = "q4_k weights, bf16 MFMA operands, fp32 accumulation"
    else:
        stage_bytes = active * eb + 4 * T * H * 2
        achieved = stage_bytes / stage_s / 1e9
        if T > 1 and tq.get_knob("moe_qmm") != 0:
            kern = ("tq_moe_ffn expert stage: k_qmm gate/up+SwiGLU and down on the fp16 matrix "
                    "cores, fp32-accurate (with the row splits and the chunk table)")
        elif T == 1 and tq.get_knob("moe_mf") != 0:
            kern = ("tq_moe_ffn expert stage: k_moe_mf gate/up+SwiGLU and down on the fp16 matrix "
                    "cores (combine in the down launch)")
        elif T == 1:
            kern = "tq_moe_ffn expert stage: k_moe_kl gate/up+SwiGLU and down"
        else:
            kern = "tq_moe_ffn expert stage: k_moe_gemv gate/up, SwiGLU, down"
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": kern, "avg_launch_us": round(stage_s * 1e6, 1)}
        dtype = "q4_k weights, f32 activations and accumulation"
    out = {
        "metric": METRIC, "value": round(T * args.steps / elapsed, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded random Q4_K experts, N(0,1) activations and router)",
        "config": {"workload": f"{tag}-shaped MoE layer{' prefill' if prefill else ''}, top-{k} "
                               f"of {E}{' + shared expert' if shared else ''}, {T} tokens",
                   "global_batch": T, "seq_len": T if prefill else 1,
                   "parallelism": "none (1 GPU)"},
        "active_experts": active,
        "step_ms": trial_stats(per_step),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = moe_cpu_baseline(synth, shape, layer, xh, y.cpu().numpy(),
                                               ids_gpu.cpu().numpy(), args.cpu_seconds)
    return out


C1_COPIES = 64
C1_BYTES_PER_LAUNCH = 4096 * 16 * 144 + 4 * (4096 + 4096)  # blob + fp32 x and y


def c1_bench(args, torch, tq, synth):
    """One 4096x4096 Q4_K GEMV at batch 1 (fp32 x ~ N(0,1), y = W x). The weights are copied into
    64 distinct device buffers (604 MB, more than twice the 256 MB last-level cache), and one graph
    holds 64 launches, launch i reading copy i, so every launch streams its weights from HBM.
    A step is one replay of that graph; the launch time is the replay time over 64. The same 64
    buffers are then read by a plain streaming-read kernel (libtq_readref.so) in a graph of 64
    launches, which gives the read-only time of the same bytes in the same launch setting."""
    import ctypes as C

    import numpy as np

    n = k = 4096
    g = synth.rng(args.seed, "c1")
    wh = synth.blob("q4_k", g, n, k)
    xh = synth.normal_f32(g, (1, k))
    copies = [torch.from_numpy(wh).cuda() for _ in range(C1_COPIES)]
    x = torch.from_numpy(xh).cuda()
    ys = [torch.empty((1, n), dtype=torch.float32, device="cuda") for _ in range(C1_COPIES)]
    ws = torch.zeros(max(tq.gemv_workspace_bytes("q4_k", n, k, 1), 256), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.Stream()

    def step():
        for w, y in zip(copies, ys):
            tq.gemv("q4_k", w, n, k, x, out=y, ws=ws)

    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(args.warmup):
            graph.replay()
        wall, per = timed_replays(torch, graph, stream, args.steps)
    y0 = ys[0].cpu().numpy()
    assert all(np.array_equal(y0, y.cpu().numpy()) for y in ys[1:]), "copies disagree"
    launches = args.steps * C1_COPIES
    launch_s = wall / launches
    kernel_s = sum(per) / 1000 / launches
    algo = wh.size + 4 * (n + k)
    assert algo == C1_BYTES_PER_LAUNCH
    achieved = algo / kernel_s / 1e9

    # the plain streaming read of the same 64 buffers
    R = C.CDLL(os.path.join(ROOT, "moe_expert_ffn_q4_amd", "libtq_readref.so"))
    R.tq_read_ref.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
    R.tq_read_ref.restype = C.c_int
    R.tq_read_ref_sink_words.argtypes = [C.c_int64]
    R.tq_read_ref_sink_words.restype = C.c_int64
    sink = torch.empty(int(R.tq_read_ref_sink_words(wh.size)), dtype=torch.int32, device="cuda")

    def read_step():
        st = torch.cuda.current_stream().cuda_stream
        for w in copies:
            if R.tq_read_ref(w.data_ptr(), wh.size, sink.data_ptr(), st):
                raise RuntimeError("tq_read_ref failed")

    with torch.cuda.stream(stream):
        read_step()
        torch.cuda.synchronize()
        rgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(rgraph, stream=stream):
            read_step()
        for _ in range(args.warmup):
            rgraph.replay()
        _, rper = timed_replays(torch, rgraph, stream, args.steps)
    read_s = sum(rper) / 1000 / launches
    out = {
        "metric": METRIC, "value": round(algo / launch_s / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1000 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "q4_k weights, f32 activations and accumulation",
        "data": "synthetic (seeded random Q4_K blocks, N(0,1) activations)",
        "config": {"workload": "single Q4_K GEMV at batch 1, W 4096x4096, 64 distinct weight "
                               "copies cycled (one launch per copy)", "global_batch": 1,
                   "seq_len": 1, "parallelism": "none (1 GPU)"},
        "launches_per_step": C1_COPIES,
        "launch_us": trial_stats([m * 1000 for m in per], C1_COPIES),
        "plain_read": {"launch_us": round(read_s * 1e6, 3),
                       "achieved": round(wh.size / read_s / 1e9, 1), "unit": "GB/s",
                       "gemv_over_read_time": round(kernel_s / read_s, 3),
                       "what": "tq_read_ref over the same 64 buffers, 64 launches per graph"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(C1_COUNTERS),
                     "kernel": gemv_kernel_name(tq, 1),
                     "avg_launch_us": round(kernel_s * 1e6, 3)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = c1_cpu_baseline(wh, xh, y0, n, k, args.cpu_seconds)
    return out


def llama70b_bench(args, torch, tq, synth):
    """One Llama-3-70B-shaped layer (q, k, v, o, gate, up, down) in each of Q4_K, Q6_K and Q8_0,
    at batch 1, 4 and 16: q/k/v as one tq_gemv_multi call, o, gate/up as one tq_gemv_swiglu
    call, down; the layer captured as a HIP graph and replayed. Reports per (format, batch) the
    layer time and the blob bytes over that time. value: Q4_K tokens/s of the layer at batch 1."""
    import ctypes as C

    shape = synth.LLAMA70B
    H, F = shape["hidden"], shape["ffn"]
    L = tq.lib()
    results = {}
    stream = torch.cuda.Stream()
    host_q4k = {}  # the Q4_K layer's host blobs, for the oracle's CPU baseline
    act_bytes = {}
    for t in ("q4_k", "q6_k", "q8_0"):
        T = tq._type(t)
        projs = {}
        for name, n, k in synth.dense_projections(shape):
            w = synth.blob(t, synth.rng(args.seed, "70b", t, name), n, k)
            projs[name] = (torch.from_numpy(w).to("cuda"), n, k)
            if t == "q4_k":
                host_q4k[name] = (w, n, k)
        blob_bytes = sum(w.numel() for w, _, _ in projs.values())
        for batch in (1, 4, 16):
            g = synth.rng(args.seed, "70b-act", t, batch)
            x = torch.from_numpy(synth.normal_f32(g, (batch, H))).cuda()
            a = torch.from_numpy(synth.normal_f32(g, (batch, H))).cuda()
            out = {m: torch.empty(batch, n, device="cuda") for m, (_, n, _) in projs.items()}
            hbuf = torch.empty(batch, F, device="cuda")
            need = [tq.gemv_workspace_bytes(t, n, k, batch) for _, n, k in projs.values()]
            narr = (C.c_int64 * 3)(H, shape["kv"], shape["kv"])
            need.append(int(L.tq_gemv_multi_workspace_bytes(T, 3, narr, H, batch)))
            need.append(int(L.tq_gemv_swiglu_workspace_bytes(T, F, H, batch)))
            ws = torch.zeros(max(max(need), 256), dtype=torch.uint8, device="cuda")
            wsn = ws.numel()

            def step():
                st = torch.cuda.current_stream().cuda_stream
                w3 = (C.c_void_p * 3)(*[projs[m][0].data_ptr() for m in ("q", "k", "v")])
                y3 = (C.c_void_p * 3)(*[out[m].data_ptr() for m in ("q", "k", "v")])
                rc = L.tq_gemv_multi(T, 3, w3, narr, y3, H, x.data_ptr(), batch, ws.data_ptr(),
                                     wsn, st)
                rc = rc or L.tq_gemv(T, projs["o"][0].data_ptr(), H, H, a.data_ptr(), batch,
                                     out["o"].data_ptr(), ws.data_ptr(), wsn, st)
                rc = rc or L.tq_gemv_swiglu(T, projs["gate"][0].data_ptr(),
                                            projs["up"][0].data_ptr(), F, H, x.data_ptr(), batch,
                                            hbuf.data_ptr(), ws.data_ptr(), wsn, st)
                rc = rc or L.tq_gemv(T, projs["down"][0].data_ptr(), H, F, hbuf.data_ptr(), batch,
                                     out["down"].data_ptr(), ws.data_ptr(), wsn, st)
                if rc:
                    raise tq.TQError(rc, L.tq_last_error().decode())

            with torch.cuda.stream(stream):
                step()
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    step()
                for _ in range(args.warmup):
                    graph.replay()
                wall, per = timed_replays(torch, graph, stream, args.steps)
                dt = wall / args.steps
            # algorithmic bytes: every blob once, plus fp32 activations in and out
            algo = blob_bytes + 4 * batch * sum(n + k for _, n, k in projs.values())
            act_bytes[f"{t} b{batch}"] = algo
            results[f"{t} b{batch}"] = {"ms_per_layer": round(dt * 1000, 4),
                                        "layer_ms": trial_stats(per),
                                        "tokens_s_one_layer": round(batch / dt, 1),
                                        "blob_gbs": round(blob_bytes / dt / 1e9, 1),
                                        "hbm_frac": round(algo / dt / 1e9 / HBM_PEAK_GBS, 4)}
        del projs
        torch.cuda.empty_cache()
    q = results["q4_k b1"]
    achieved = act_bytes["q4_k b1"] / (q["ms_per_layer"] / 1000) / 1e9
    out = {
        "metric": METRIC, "value": q["tokens_s_one_layer"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": q["ms_per_layer"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "q4_k / q6_k / q8_0 weights, f32 activations and accumulation",
        "data": "synthetic (seeded random blocks, N(0,1) activations)",
        "config": {"workload": "llama3-70b-shaped layer (hidden 8192, kv 1024, ffn 28672), one "
                               "layer per format, batch 1 / 4 / 16", "global_batch": 1,
                   "seq_len": 1, "parallelism": "none (1 GPU)"},
        "per_format_batch": results,
        # the layer's four launches (q|k|v, o, gate|up + SwiGLU, down), Q4_K at batch 1: bytes
        # and time summed over the launches, i.e. per-launch bytes over the average launch time
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": f"Q4_K batch-1 layer (tq::{b1_kernel(tq)}; down in k slices)"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = llama70b_cpu_baseline(host_q4k, args.cpu_seconds, tq, torch)
    return out


def llama70b_cpu_baseline(projs, budget_s, tq, torch):
    """The oracle (as it is) on the same Q4_K layer at batch 1: whole layers on all the host's
    threads until about budget_s, then on one thread for about a third of that. The all-core
    outputs are checked element by element against tq_gemv's for the same inputs."""
    import oracle
    import synth

    xs = {name: synth.normal_f32(synth.rng(7, "70b-cpu-x", name), (1, k))
          for name, (_, _, k) in projs.items()}
    refs = {}

    def layer():
        for name, (w, n, k) in projs.items():
            refs[name] = oracle.gemv("q4_k", w, n, k, xs[name])

    layers, elapsed = oracle_repeat(layer, budget_s, 1000)
    cores = oracle.num_threads()
    checks = []
    for name, (w, n, k) in projs.items():
        y = tq.gemv("q4_k", torch.from_numpy(w).cuda(), n, k, torch.from_numpy(xs[name]).cuda())
        checks.append(check_against(y.cpu().numpy(), *refs[name]))
    w, n, k = projs["o"]
    reps1, el1 = single_thread(lambda: oracle.gemv("q4_k", w, n, k, xs["o"]), budget_s / 3,
                               10000)
    frac = w.size / sum(p[0].size for p in projs.values())
    return {"value": round(layers / elapsed, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{layers} full Q4_K layers (7 projections each, batch 1) in {elapsed:.1f} s "
                      f"on {cores} threads",
            "single_thread": {"value": round(frac / (el1 / reps1), 5), "unit": "tokens/s",
                              "sample": f"{reps1} x the o projection in {el1:.1f} s on 1 thread, "
                                        f"scaled by blob bytes to the layer"},
            "checked_vs_gpu": {"elements": sum(c["elements"] for c in checks),
                               "max_err_over_bound": max(c["max_err_over_bound"] for c in checks),
                               "pass": all(c["pass"] for c in checks),
                               "what": "the Q4_K layer's 7 projections at batch 1, every output "
                                       "element, the all-core oracle's against tq_gemv's"}}


def host_bench(args, torch, tq, synth):
    """DeepSeek-shaped decode layer with the routed experts in pinned host memory: every step
    reads the selected experts' blobs over PCIe (a host sync on the routing, then per-expert
    copies on a side stream overlapped with the kernels). Not graph-capturable (host sync), so
    steps are timed eagerly. Reports the layer rate, the achieved host-to-device rate of the
    expert copies and that of one plain pinned copy of the same size on the same box."""
    shape = synth.DEEPSEEK
    k, T = shape["top_k"], args.batch
    layer = synth.moe_layer(shape, "q4_k", seed=args.seed, tag="deepseek")
    pinned = [tuple(torch.from_numpy(b).pin_memory() for b in e) for e in layer["experts"]]
    shared = tuple(torch.from_numpy(b).cuda() for b in layer["shared"])
    copy_stream = torch.cuda.Stream()
    moe = tq.MoeLayer("q4_k", shape["hidden"], shape["ffn"], torch.from_numpy(layer["router"]).cuda(),
                      pinned, shared, top_k=k, copy_stream=copy_stream)
    x = torch.from_numpy(synth.normal_f32(synth.rng(args.seed, "bench-x", T), (T, shape["hidden"]))).cuda()
    y = torch.empty_like(x)
    ws = torch.empty(moe.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    counts = torch.empty(shape["n_experts"], dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        moe(x, out=y, ws=ws, routing=dict(counts=counts))
        for _ in range(args.warmup):
            moe(x, out=y, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            moe(x, out=y, ws=ws)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    c = counts.cpu().numpy()
    eb = sum(b.numel() for b in pinned[0])
    routed = int((c > 0).sum())
    h2d_bytes = routed * eb
    # one plain pinned host-to-device copy of the same number of bytes
    src = torch.empty(h2d_bytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(h2d_bytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    plain = h2d_bytes * args.steps / (time.perf_counter() - t1) / 1e9
    ms = elapsed * 1000 / args.steps
    achieved = h2d_bytes / (ms / 1000) / 1e9
    out = {
        "metric": METRIC, "value": round(T * args.steps / elapsed, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "q4_k weights, f32 activations and accumulation",
        "data": "synthetic (seeded random Q4_K experts in pinned host memory, N(0,1) activations)",
        "config": {"workload": f"deepseek-shaped MoE layer, top-{k} of {shape['n_experts']} routed "
                               f"experts in pinned host memory + device-resident shared expert, "
                               f"{T} tokens", "global_batch": T, "seq_len": 1,
                   "parallelism": "none (1 GPU)"},
        "routed_experts_copied": routed,
        "h2d": {"bytes_per_step": h2d_bytes, "achieved": round(achieved, 2),
                "plain_pinned_copy": round(plain, 2), "unit": "GB/s",
                "frac": round(achieved / plain, 4)},
    }
    if args.cache_slots:
        out["cache_sweep"] = {
            "trace": f"Zipf-skewed routing (synth.zipf_router), one new x per step, {T} token(s) "
                     f"per step, {args.steps} timed steps after {args.warmup}",
            "rows": cache_sweep(args, torch, tq, synth)}
    return out


def cache_sweep(args, torch, tq, synth):
    """The DeepSeek-shaped decode layer (T = --batch) with its routed experts in pinned host
    memory and a router whose routing favours some experts (synth.zipf_router: the hottest 32 of
    256 experts take about 3/4 of the selections), one new activation vector per step (x = z + v).
    For each slot count (0: no cache) the same trace of steps runs after --warmup steps; reported
    per configuration: time and tokens/s per step, host-to-device bytes per step, and the cache's
    hit rate and prefetches."""
    shape = synth.DEEPSEEK
    k, T, E, H = shape["top_k"], args.batch, shape["n_experts"], shape["hidden"]
    layer = synth.moe_layer(shape, "q4_k", seed=args.seed, tag="deepseek")
    wr, v = synth.zipf_router(synth.rng(args.seed, "zipf-router"), E, H)
    pinned = [tuple(torch.from_numpy(b).pin_memory() for b in e) for e in layer["experts"]]
    shared = tuple(torch.from_numpy(b).cuda() for b in layer["shared"])
    expert_bytes = sum(b.numel() for b in pinned[0])
    g = synth.rng(args.seed, "zipf-trace", T)
    n = args.warmup + args.steps
    xs = torch.from_numpy(synth.normal_f32(g, (n, T, H)) + v).cuda()
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    rows = []
    configs = [(0, 0)] if 0 in args.cache_slots else []
    configs += [(s, min(p, s)) for s in args.cache_slots if s > 0 for p in args.prefetch]
    for slots, prefetch in dict.fromkeys(configs):
        moe = tq.MoeLayer("q4_k", H, shape["ffn"], torch.from_numpy(wr).cuda(), pinned, shared,
                          top_k=k, copy_stream=torch.cuda.Stream())
        ws = torch.empty(moe.workspace_bytes(T), dtype=torch.uint8, device="cuda")
        cache = moe.attach_cache(slots, prefetch) if slots else None
        stream = torch.cuda.Stream()
        routed = 0
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                moe(xs[i], out=y, ws=ws)
            torch.cuda.synchronize()
            s0 = cache.stats() if cache else None
            t0 = time.perf_counter()
            for i in range(args.warmup, n):
                moe(xs[i], out=y, ws=ws)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / args.steps
            if not cache:  # the experts each step routes to (all copied without a cache)
                for i in range(args.warmup, n):
                    moe(xs[i], out=y, ws=ws, routing=dict(counts=counts))
                    routed += int((counts > 0).sum().item())
        row = {"slots": slots, "prefetch": prefetch,
               "device_gb": round(slots * expert_bytes / 1e9, 2),
               "ms_per_step": round(dt * 1000, 3), "tokens_s": round(T / dt, 1)}
        if cache:
            s1 = cache.stats()
            d = {f: s1[f] - s0[f] for f in s1}
            routed = d["hits"] + d["misses"] + d["fallbacks"]
            row.update(h2d_mb_per_step=round(d["bytes_copied"] / args.steps / 1e6, 1),
                       hit_rate=round(d["hits"] / max(routed, 1), 4),
                       prefetched_per_step=round(d["prefetched"] / args.steps, 2),
                       prefetch_hits_per_step=round(d["prefetch_hits"] / args.steps, 2))
            moe.detach_cache()
        else:
            row.update(h2d_mb_per_step=round(routed * expert_bytes / args.steps / 1e6, 1),
                       hit_rate=0.0)
        rows.append(row)
        del moe, ws
        torch.cuda.empty_cache()
    return rows


def calibrate_copy(torch):
    """One plain 1 GiB device-to-device copy: the reading that the HBM counters of the same run
    are scaled by (bytes copied / counter value)."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def main():
    args = _args()
    if args.summarize:
        print(summarize(*args.summarize, workload=args.workload, batch=args.batch))
        return
    if args.kernel_summary:
        print(kernel_summary(*args.kernel_summary))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(no multi-GPU path in this build)", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_expert_ffn_q4_amd as tq
    import synth

    torch.cuda.set_device(0)
    for kv in args.knob:
        name, value = kv.split("=", 1)
        tq.set_knob(name, int(value))
    other = {"deepseek-host": host_bench, "llama70b": llama70b_bench,
             "c1": c1_bench}.get(args.workload)
    if other is None and args.workload != "llama8b":
        other = moe_bench
    if other is not None:
        out = other(args, torch, tq, synth)
        if args.calibrate_copy:
            calibrate_copy(torch)
        print(json.dumps(out), flush=True)
        return
    layers = build_dense_model(tq, synth, torch, args.batch, args.seed)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step = make_step(tq, torch, layers, args.batch)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        # the whole decode step as one HIP graph, replayed once per step
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(args.warmup):
            graph.replay()
        elapsed, per_step = timed_replays(torch, graph, stream, args.steps)
    ms_per_step = elapsed * 1000 / args.steps
    tokens_s = args.batch * args.steps / elapsed

    # Roofline of the Q4_K GEMV: the step's GEMV launches alone (no SwiGLU), captured as their
    # own graph on the same stream and replayed back to back between two events on that stream;
    # the average launch duration is the elapsed time over the number of launches.
    events = []
    with torch.cuda.stream(stream):
        gstep = make_step(tq, torch, layers, args.batch, events=events, gemv_only=True)
        gstep()
        torch.cuda.synchronize()
        ggraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ggraph, stream=stream):
            gstep()
        ggraph.replay()
        _, gper = timed_replays(torch, ggraph, stream, max(5, args.steps // 4))
    launches = len(events) // 2  # the eager call and the captured one each appended
    kernel_bytes = sum(events[:launches])
    avg_launch_s = sum(gper) / 1000 / (len(gper) * launches)
    achieved = kernel_bytes / launches / avg_launch_s / 1e9
    step_bytes = kernel_bytes
    traffic = (recorded_traffic() if args.batch == 1 else
               recorded_traffic(B8_COUNTERS, QMM_SOURCES) if args.batch == 8 else None)

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_k weights, f32 activations and accumulation",
        "data": "synthetic (seeded random Q4_K blocks, N(0,1) activations)",
        "config": {"workload": f"llama3-8b-shaped decode, 32 layers x 7 Q4_K projections + "
                               f"SwiGLU, batch {args.batch}",
                   "global_batch": args.batch, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "step_gbs": round(step_bytes / (ms_per_step / 1000) / 1e9, 1),
        "step_ms": trial_stats(per_step),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": gemv_kernel_name(tq, args.batch),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3)},
    }
    if args.calibrate_copy:
        calibrate_copy(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(synth, args.batch, args.seed, args.cpu_seconds, tq,
                                           torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
