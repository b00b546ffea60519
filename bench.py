"""Benchmark of the sparse MoE layer forward on one MI355X.

One step = one whole layer forward (route, grouping, gate/up experts, down
experts, combine, and the balance statistics written by the grouping step), on
seeded synthetic inputs that
are resident in HBM before timing starts.  Prints ONE JSON line; its
"backward" object times the layer's backward on the same inputs (bf16/fp32
expert weights).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-tokens N]
    python bench.py --pass backward [--workload NAME] ...
                                              # the layer backward, its own JSON line
    python bench.py --copy-probe MIB          # counter calibration copy
    python bench.py --summarize-profiles DIR --workload NAME
                                              # rocprofv3 output -> profiles/

Workloads (random weights of the named models' shapes, no checkpoints):
deepseek_v3 (default: the largest single-GPU workload), mixtral_prefill,
mixtral_decode, qwen3_skew, tiny_f32, and FP8-weight variants.  The default run
also times mixtral_prefill, mixtral_decode and qwen3_skew on the same GPU and
reports them under "other_workloads" (--also "" turns that off).
"""

from __future__ import annotations

import argparse
import re
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec; active TFLOP/s and HBM GB/s as % of MI355X peak"
PEAK_BF16_TFLOPS = 2500.0     # dense MFMA bf16, MI355X
PEAK_F32_TFLOPS = 157.3       # dense MFMA fp32
PEAK_HBM_GBS = 8000.0         # HBM3E
# first CPU-oracle sample per workload; when it finishes in under CPU_MIN_S the
# sample grows so that the reported run takes about CPU_TARGET_S
DEFAULT_CPU_TOKENS = {"mixtral_prefill": 256, "mixtral_decode": 32, "deepseek_v3": 8,
                      "qwen3_skew": 256, "tiny_f32": 64}
CPU_MIN_S, CPU_TARGET_S = 8.0, 15.0
# host memory the CPU baseline may fill with float64 expert weights; past it the
# token sample stops growing and is repeated instead
CPU_F64_WEIGHT_BUDGET = 40 << 30
CSRC = os.path.join(ROOT, "sparse_mixture_experts_router_amd", "csrc")
# the sources that decide the expert GEMMs' memory traffic
GEMM_SRCS = ("expert_gemm.hip", "expert_tile.h", "grouped_gemm.hip", "route_tile.h", "mfma.h",
             "lds_ring.h")
PROFILE_STEPS, PROFILE_WARMUP, PMC_STEPS, PMC_WARMUP, COPY_MIB = 20, 20, 3, 1, 1024
# matrix-core counters of the expert GEMMs, one --pmc pass (2 SQ + 1 GRBM):
# busy cycles of the MFMA units summed over the SIMDs, MFMA bf16 operations / 512,
# and the GPU's active cycles summed over the 8 XCDs
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")
SIMDS, XCDS = 1024, 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="deepseek_v3")
    ap.add_argument("--also", default="mixtral_prefill,mixtral_decode,qwen3_skew",
                    help="comma-separated workloads timed after the headline one "
                         "(compact entries under other_workloads; empty: none)")
    ap.add_argument("--pass", dest="pass_", choices=("forward", "backward"), default="forward",
                    help="backward: time moe_layer_backward instead (one JSON line of its own)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="forward line without its compact backward measurement")
    ap.add_argument("--cpu-tokens", type=int, default=0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="turn the rocprofv3 runs under DIR (trace/, fetch/, write/, "
                         "copy_fetch/, copy_write/) into profiles/ summaries and exit")
    return ap.parse_args()


def copy_probe(mib):
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}), flush=True)


def mark_stride(steps):
    """One timed step in this many carries the gate/up HIP events: every step
    of a short run, one in ten of a run of 50 or more (at least 5 samples)."""
    return max(1, min(10, steps // 5))


def algorithmic(shape, active):
    """Layer and gate/up-kernel algorithmic FLOPs and bytes (inputs once, outputs once)."""
    T, d, N, k, F, S, b = shape.T, shape.d, shape.N, shape.k, shape.F, shape.S, shape.elem_bytes
    wb = 1 if shape.fp8 else b          # expert weight bytes per element
    sb = 4 if shape.fp8 else 0          # fp32 scale bytes per output channel
    rows = T * k + S * T
    layer_flops = 2 * rows * 3 * d * F + 2 * T * d * N
    layer_bytes = ((active + S) * (3 * d * F * wb + (2 * F + d) * sb) + N * d * b + 2 * T * d * b
                   + T * k * 8)
    up_flops = 2 * rows * d * 2 * F
    up_bytes = (active + S) * 2 * F * (d * wb + sb) + T * d * b + rows * F * b
    return layer_flops, layer_bytes, up_flops, up_bytes


def gemm_source_hash():
    h = hashlib.sha256()
    for name in GEMM_SRCS:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"expert_up_gemm_{workload}_traffic.json")


def load_traffic(workload):
    """The committed rocprofv3 --pmc record of the gate/up launch, or None.

    None also when the GEMM sources changed since the counters were taken.
    """
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return rec


def mfma_path(workload):
    return os.path.join(ROOT, "profiles", f"expert_gemm_{workload}_mfma.json")


def load_mfma(workload):
    """The committed rocprofv3 --pmc record of the expert GEMMs' matrix-core
    counters, or None (also when the GEMM sources changed since)."""
    path = mfma_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return rec


def cpu_baseline(shape, inputs, n_tok, gpu_idx):
    """The CPU oracle, as it stands, on the first n_tok tokens of the same batch.

    The experts those tokens use are widened to float64 on the host before the
    timed runs (widening the inputs' bits is not the oracle's arithmetic), so
    each run times the oracle's forward alone.  The sample grows until one run
    takes CPU_MIN_S, while the float64 weights it needs fit
    CPU_F64_WEIGHT_BUDGET; past that the sample is repeated instead."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()}))
    except Exception:  # threadpoolctl missing: report the affinity set
        threads, blas = len(os.sched_getaffinity(0)), "unknown"

    def f64(t):
        return t.double().cpu().numpy()

    n_tok = min(n_tok, shape.T)
    x = f64(inputs["x"])
    wr = f64(inputs["w_router"])
    lb = None if inputs["logit_bias"] is None else inputs["logit_bias"].cpu().numpy()
    sb = None if inputs["select_bias"] is None else inputs["select_bias"].cpu().numpy()

    def weight(name, e=None):
        w = inputs[name] if e is None else inputs[name][e]
        if not shape.fp8:
            return f64(w)
        sc = inputs[name + "_scale"] if e is None else inputs[name + "_scale"][e]
        return oracle.dequantize(w.cpu().numpy(), sc.cpu().numpy())   # O9, part of the oracle

    def load(e):
        return (weight("w_gate", e), weight("w_up", e), weight("w_down", e))

    per_expert = 3 * shape.d * shape.F * 8
    cache = {}

    def need(n):
        return sorted(set(gpu_idx[:n].reshape(-1).tolist()))

    def prepare(n):
        for e in need(n):
            if e not in cache:
                cache[e] = load(e)

    fetched = []

    def expert(e):
        if e not in cache:   # a selection flip against the GPU's routing: fetch on demand
            fetched.append(e)
            cache[e] = load(e)
        return cache[e]

    shared = None
    if shape.S:
        shared = tuple(weight(n) for n in ("ws_gate", "ws_up", "ws_down"))

    def run(n):
        t0 = time.perf_counter()
        oracle.moe_forward(x[:n], wr, expert, shape.k, logit_bias=lb,
                           select_bias=sb, shared=shared, n_experts=shape.N)
        return time.perf_counter() - t0

    prepare(n_tok)
    dt = run(n_tok)
    first = (n_tok, dt)
    reps = 1
    while dt < CPU_MIN_S and n_tok < shape.T:   # too short to time: grow the sample
        nxt = min(shape.T, int(np.ceil(n_tok * CPU_TARGET_S / max(dt, 1e-3))))
        if len(need(nxt)) * per_expert > CPU_F64_WEIGHT_BUDGET:
            break
        n_tok = nxt
        prepare(n_tok)
        dt = run(n_tok)
    if dt < CPU_MIN_S:                       # quick (or capped) sample: repeat it
        reps, dt = 0, 0.0
        while dt < CPU_TARGET_S:
            dt += run(n_tok)
            reps += 1
    return {"value": n_tok * reps / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"first {n_tok} of {shape.T} tokens with all their experts"
                       f"{f', {reps} runs' if reps > 1 else ''}, NumPy float64 ({blas}), "
                       f"{dt:.1f} s in all (sized from a {first[0]}-token run of "
                       f"{first[1]:.1f} s); weights widened to float64 before timing "
                       f"({len(cache)} experts); host affinity "
                       f"{len(os.sched_getaffinity(0))} cpus"
                       f"{f'; {len(fetched)} experts fetched during timing' if fetched else ''}"),
            "seconds": round(dt, 2)}


def profile_commands(d, workload):
    """The rocprofv3 runs that --summarize-profiles reads (d: their output root)."""
    run = f"python3 bench.py --workload {workload} --also= --no-cpu-baseline --no-backward"
    return {
        "trace": (f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- {run} "
                  f"--steps {PROFILE_STEPS} --warmup {PROFILE_WARMUP} > {d}/trace_bench.json"),
        "fetch": (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o run -- {run} "
                  f"--steps {PMC_STEPS} --warmup {PMC_WARMUP}"),
        "write": (f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o run -- {run} "
                  f"--steps {PMC_STEPS} --warmup {PMC_WARMUP}"),
        "mfma": (f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d {d}/mfma "
                 f"-o run -- {run} --steps {PMC_STEPS} --warmup {PMC_WARMUP}"),
        "copy_fetch": (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/copy_fetch -o run -- "
                       f"python3 bench.py --copy-probe {COPY_MIB}"),
        "copy_write": (f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/copy_write -o run -- "
                       f"python3 bench.py --copy-probe {COPY_MIB}"),
    }


def gemm_template_args(name):
    """(kernel, [template arguments]) of a grouped GEMM kernel name, or None."""
    m = re.search(r"(expert_gemm_pp_kernel|expert_gemm_kernel|grouped_gemm_kernel)<([^>]*)>", name)
    return None if m is None else (m.group(1), [a.strip() for a in m.group(2).split(",")])


def is_up_gemm(name):
    """The gate/up launch: a grouped GEMM kernel instantiated with GATED = true
    (the first template argument of expert_gemm_kernel and expert_gemm_pp_kernel,
    grouped_gemm_kernel's third)."""
    ka = gemm_template_args(name)
    if ka is None:
        return False
    kern, args = ka
    i = 0 if kern.startswith("expert_gemm") else 2
    return len(args) > i and args[i] == "true"


def is_grad_w_gemm(name):
    """The weight-gradient launches: expert_gemm_pp_kernel with KMAJ (its
    sixth template argument) = true."""
    ka = gemm_template_args(name)
    return (ka is not None and ka[0] == "expert_gemm_pp_kernel" and len(ka[1]) >= 6
            and ka[1][5] == "true")


def is_down_gemm(name):
    """The down launch: a forward grouped GEMM kernel with GATED = false (and,
    for the large-tile kernel, neither the weight-gradient nor the K-row mode)."""
    ka = gemm_template_args(name)
    if ka is None:
        return False
    kern, args = ka
    if kern == "expert_gemm_pp_kernel":
        # <GATED, DENSE, NARROW, FP8W, BT, KMAJ>: DENSE is the router GEMM
        return args[0] == "false" and all(a == "false" for i, a in enumerate(args) if i in (1, 4, 5))
    if kern == "expert_gemm_kernel":  # <GATED, BM, BNE, NBUF, FP8W, BT, TRIPB>
        return args[0] == "false" and all(a == "false" for a in args[5:6])
    return len(args) > 2 and args[2] == "false"


def short_name(name):
    return name.replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(")[0]


def read_counters(path, counter):
    """{kernel name: [value per dispatch]} for one counter of a --pmc run (KiB)."""
    import csv
    import glob

    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (f, r["Dispatch_Id"])
                per.setdefault(key, [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
    out = {}
    for name, v in per.values():
        out.setdefault(name, []).append(v)
    return out


def summarize_profiles(d, workload):
    """Write profiles/expert_up_gemm_<workload>.md and the _traffic.json that
    the bench reads, from the five rocprofv3 runs of profile_commands()."""
    import csv
    import glob

    import numpy as np

    from workloads import CONFIGS

    shape = CONFIGS[workload]
    cmds = profile_commands(d.rstrip("/"), workload)
    # kernel trace
    stats = glob.glob(os.path.join(d, "trace", "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {d}/trace")
    rows = []
    with open(stats[0]) as fh:
        for r in csv.DictReader(fh):
            if "moe::" in r["Name"]:
                rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]),
                             float(r["MinNs"]), float(r["MaxNs"]), float(r["Percentage"])))
    up = [r for r in rows if is_up_gemm(r[0])]
    if len(up) != 1:
        raise SystemExit(f"expected one gate/up GEMM kernel in the trace, found {len(up)}")
    up = up[0]
    bench = None
    bpath = os.path.join(d, "trace_bench.json")
    if os.path.exists(bpath):
        with open(bpath) as fh:
            lines = [ln for ln in fh if ln.startswith("{")]
        bench = json.loads(lines[-1]) if lines else None
    # counters, calibrated on a plain copy of known size
    copy_bytes = COPY_MIB * (1 << 20)

    def copy_scale(sub, counter):
        vals = [v for n, vs in read_counters(os.path.join(d, sub), counter).items()
                if "copyBuffer" in n for v in vs]
        if not vals:
            raise SystemExit(f"no copy dispatch in {sub}")
        return copy_bytes / (float(np.median(vals)) * 1024.0), len(vals)

    fscale, nf = copy_scale("copy_fetch", "FETCH_SIZE")
    wscale, nw = copy_scale("copy_write", "WRITE_SIZE")

    def up_kib(sub, counter):
        vals = [v for n, vs in read_counters(os.path.join(d, sub), counter).items()
                if is_up_gemm(short_name(n)) for v in vs]
        if not vals:
            raise SystemExit(f"no gate/up dispatch in {sub}")
        return float(np.mean(vals)), len(vals)

    fk, nfk = up_kib("fetch", "FETCH_SIZE")
    wk, nwk = up_kib("write", "WRITE_SIZE")
    fetch_b = fk * 1024.0 * fscale
    write_b = wk * 1024.0 * wscale
    alg = bench["roofline"]["algorithmic_bytes"] if bench else None
    rec = {
        "workload": workload,
        "kernel": up[0],
        "gemm_source_sha256_16": gemm_source_hash(),
        "fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wk, 1),
        "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
        "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
        "fetch_bytes_per_launch": int(round(fetch_b)),
        "write_bytes_per_launch": int(round(write_b)),
        "algorithmic_bytes_per_launch": alg,
        "dispatches": {"fetch": nfk, "write": nwk, "copy_fetch": nf, "copy_write": nw},
        "commands": {k: v for k, v in cmds.items() if k != "trace"},
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(traffic_path(workload), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    # matrix-core counters of both expert GEMMs (bf16 layers only)
    mrec = None
    if os.path.isdir(os.path.join(d, "mfma")) and shape.dtype == "bf16":
        rows_all = shape.T * (shape.k + shape.S)
        alg_flops = {"up": 4 * rows_all * shape.d * shape.F, "down": 2 * rows_all * shape.d * shape.F}
        trace_us = {"up": up[2] / 1e3}
        dn = [r_ for r_ in rows if is_down_gemm(r_[0])]
        if len(dn) == 1:
            trace_us["down"] = dn[0][2] / 1e3
        mrec = {"workload": workload, "gemm_source_sha256_16": gemm_source_hash(),
                "counters": list(MFMA_COUNTERS), "command": cmds["mfma"]}
        for role, pick in (("up", is_up_gemm), ("down", is_down_gemm)):
            vals = {}
            for c in MFMA_COUNTERS:
                v = [x_ for n_, xs in read_counters(os.path.join(d, "mfma"), c).items()
                     if pick(short_name(n_)) for x_ in xs]
                if not v:
                    raise SystemExit(f"no {role} dispatch with {c} in {d}/mfma")
                vals[c] = float(np.mean(v))
            cycles = vals["GRBM_GUI_ACTIVE"] / XCDS
            issued = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            ent = {"kernel": (up[0] if role == "up" else (dn[0][0] if len(dn) == 1 else None)),
                   "gpu_active_cycles": round(cycles),
                   "mfma_busy_frac": round(vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS), 4),
                   "mfma_flops_issued": int(issued),
                   "algorithmic_flops": alg_flops[role],
                   "issued_over_algorithmic": round(issued / alg_flops[role], 4)}
            if role in trace_us:
                ent["trace_avg_us"] = round(trace_us[role], 1)
                ent["clock_ghz"] = round(cycles / (trace_us[role] * 1e3), 3)
            mrec[role] = ent
        with open(mfma_path(workload), "w") as fh:
            json.dump(mrec, fh, indent=1)
            fh.write("\n")
    md = [f"# Gate/up expert GEMM, {workload}: rocprofv3 summary", "",
          f"Workload: {shape.describe()}.", "",
          "Commands (run from the repository root; the summary below is",
          f"`python3 bench.py --summarize-profiles {d.rstrip('/')} --workload {workload}`):", ""]
    md += [f"    {c}" for c in cmds.values()]
    md += ["", "## Kernel trace (--kernel-trace --stats), this library's kernels", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    md += [f"| `{n}` | {c} | {a / 1e3:.1f} | {lo / 1e3:.1f} | {hi / 1e3:.1f} | {p:.2f} |"
           for n, c, a, lo, hi, p in rows]
    if bench:
        r = bench["roofline"]
        md += ["", f"The bench line of the traced run timed the same launch at "
               f"{r['avg_launch_ms'] * 1e3:.1f} us on average with HIP events on its stream "
               f"(trace: {up[2] / 1e3:.1f} us); layer {bench['ms_per_step']} ms per step, "
               f"{bench['value']} tokens/s; roofline {r['bound']} {r['achieved']} {r['unit']} "
               f"= {r['frac']:.3f} of peak."]
    md += ["", "## HBM traffic of the gate/up launch (--pmc)", "",
           "FETCH_SIZE and WRITE_SIZE are in KiB per dispatch. Each is scaled by the factor",
           f"that makes a plain {COPY_MIB} MiB device copy read and write {COPY_MIB} MiB.", "",
           "| quantity | value |", "|---|---:|",
           f"| FETCH_SIZE per launch (KiB, mean of {nfk}) | {fk:.0f} |",
           f"| WRITE_SIZE per launch (KiB, mean of {nwk}) | {wk:.0f} |",
           f"| fetch scale (copy of {COPY_MIB} MiB) | {fscale:.3f} |",
           f"| write scale (copy of {COPY_MIB} MiB) | {wscale:.3f} |",
           f"| HBM bytes read per launch | {fetch_b / 1e6:.1f} MB |",
           f"| HBM bytes written per launch | {write_b / 1e6:.1f} MB |"]
    if alg:
        md += [f"| algorithmic bytes per launch | {alg / 1e6:.1f} MB |",
               f"| measured / algorithmic | {(fetch_b + write_b) / alg:.2f} |"]
    if mrec is not None:
        md += ["", "## Matrix-core counters of the expert GEMMs (--pmc)", "",
               f"Counters {', '.join(MFMA_COUNTERS)}, one pass. MFMA busy = "
               f"SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs); issued FLOPs ="
               " SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, against the algorithmic"
               " 4 rows d F (gate/up) or 2 rows d F (down); clock = active cycles per XCD over"
               " the kernel trace's mean duration.", "",
               "| launch | MFMA busy | issued / algorithmic FLOPs | clock (GHz) |",
               "|---|---:|---:|---:|"]
        for role in ("up", "down"):
            e_ = mrec[role]
            md.append(f"| {role} `{e_['kernel']}` | {e_['mfma_busy_frac']:.3f} | "
                      f"{e_['issued_over_algorithmic']:.3f} | "
                      f"{e_.get('clock_ghz', float('nan')):.2f} |")
    with open(os.path.join(ROOT, "profiles", f"expert_up_gemm_{workload}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps(rec))


def backward_profile_commands(d, workload):
    """The rocprofv3 runs that --summarize-profiles --pass backward reads."""
    run = f"python3 bench.py --pass backward --workload {workload} --no-cpu-baseline"
    return {
        "trace": (f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/btrace -o run -- "
                  f"{run} --steps 10 --warmup 2 > {d}/btrace_bench.json"),
        "fetch": (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/bfetch -o run -- {run} "
                  f"--steps {PMC_STEPS} --warmup {PMC_WARMUP}"),
        "write": (f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/bwrite -o run -- {run} "
                  f"--steps {PMC_STEPS} --warmup {PMC_WARMUP}"),
        "copy_fetch": (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/copy_fetch -o run -- "
                       f"python3 bench.py --copy-probe {COPY_MIB}"),
        "copy_write": (f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/copy_write -o run -- "
                       f"python3 bench.py --copy-probe {COPY_MIB}"),
    }


def read_counters_ordered(path, counter, keep):
    """Values (KiB) of one counter for the dispatches whose kernel name passes
    keep(), in dispatch order."""
    import csv
    import glob

    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and keep(short_name(r["Kernel_Name"])):
                    key = int(r["Dispatch_Id"])
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def summarize_backward_profiles(d, workload):
    """Write profiles/grad_w_gemm_backward_<workload>.md and the _traffic.json
    that the backward bench reads, from backward_profile_commands()' runs."""
    import csv
    import glob

    import numpy as np

    from workloads import CONFIGS

    shape = CONFIGS[workload]
    cmds = backward_profile_commands(d.rstrip("/"), workload)
    stats = glob.glob(os.path.join(d, "btrace", "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {d}/btrace")
    rows = []
    with open(stats[0]) as fh:
        for r in csv.DictReader(fh):
            if "moe::" in r["Name"]:
                rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]),
                             float(r["MinNs"]), float(r["MaxNs"]), float(r["Percentage"])))
    gw = [r for r in rows if is_grad_w_gemm(r[0])]
    if len(gw) != 1:
        raise SystemExit(f"expected one weight-gradient GEMM kernel in the trace, found {len(gw)}")
    gw = gw[0]
    bench = None
    bpath = os.path.join(d, "btrace_bench.json")
    if os.path.exists(bpath):
        with open(bpath) as fh:
            lines = [ln for ln in fh if ln.startswith("{")]
        bench = json.loads(lines[-1]) if lines else None
    copy_bytes = COPY_MIB * (1 << 20)

    def copy_scale(sub, counter):
        vals = [v for n, vs in read_counters(os.path.join(d, sub), counter).items()
                if "copyBuffer" in n for v in vs]
        if not vals:
            raise SystemExit(f"no copy dispatch in {sub}")
        return copy_bytes / (float(np.median(vals)) * 1024.0)

    fscale = copy_scale("copy_fetch", "FETCH_SIZE")
    wscale = copy_scale("copy_write", "WRITE_SIZE")
    roles = ("dW_down", "dW_gate", "dW_up")  # launch order inside a backward call

    def by_role(sub, counter):
        vals = read_counters_ordered(os.path.join(d, sub), counter, is_grad_w_gemm)
        if not vals or len(vals) % 3:
            raise SystemExit(f"{sub}: {len(vals)} weight-gradient dispatches, not 3 per call")
        return [float(np.mean(vals[i::3])) for i in range(3)], len(vals)

    fk, nf = by_role("bfetch", "FETCH_SIZE")
    wk, nw = by_role("bwrite", "WRITE_SIZE")
    hbm = [fk[i] * 1024.0 * fscale + wk[i] * 1024.0 * wscale for i in range(3)]
    roof = bench["roofline"] if bench else {}
    alg = roof.get("algorithmic_bytes")
    rec = {
        "workload": workload,
        "kernel": gw[0] + " (" + ", ".join(roles) + ")",
        "backward_source_sha256_16": backward_source_hash(),
        "fetch_kib_per_launch": [round(v, 1) for v in fk],
        "write_kib_per_launch": [round(v, 1) for v in wk],
        "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
        "hbm_bytes_per_launch": [int(round(v)) for v in hbm],
        "hbm_bytes_per_launch_mean": int(round(float(np.mean(hbm)))),
        "algorithmic_bytes_per_launch": alg,
        "dispatches": {"fetch": nf, "write": nw},
        "commands": {k: v for k, v in cmds.items() if k != "trace"},
    }
    with open(backward_traffic_path(workload), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    md = [f"# Weight-gradient GEMMs of the layer backward, {workload}: rocprofv3 summary", "",
          f"Workload: {shape.describe()}; one `moe_layer_backward` per step (routing and "
          "gate/up recomputed, every gradient written).", "",
          "Commands (run from the repository root; the summary below is",
          f"`python3 bench.py --summarize-profiles {d.rstrip('/')} --workload {workload} "
          "--pass backward`):", ""]
    md += [f"    {c}" for c in cmds.values()]
    md += ["", "## Kernel trace (--kernel-trace --stats), this library's kernels", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    md += [f"| `{n}` | {c} | {a / 1e3:.1f} | {lo / 1e3:.1f} | {hi / 1e3:.1f} | {p:.2f} |"
           for n, c, a, lo, hi, p in rows]
    md += ["", f"`{gw[0]}` is the three weight-gradient launches of every call "
           f"({', '.join(roles)}); the trace averages them ({gw[2] / 1e3:.1f} us)."]
    if bench:
        st = ", ".join(f"{k} {v:.3f}" for k, v in bench["stages_ms"].items())
        md += ["", f"The bench line of the traced run: {bench['ms_per_step']} ms per backward step, "
               f"{bench['value']} tokens/s. Stages (ms, HIP events on the library's stream, "
               f"markers included): {st}. Slowest GEMM stage {roof.get('stage')}: "
               f"{roof.get('avg_launch_ms', 0) * 1e3:.1f} us per launch, {roof.get('achieved')} "
               f"TFLOP/s = {roof.get('frac', 0):.3f} of peak."]
    md += ["", "## HBM traffic of the weight-gradient launches (--pmc)", "",
           "FETCH_SIZE and WRITE_SIZE are in KiB per dispatch (means over the calls of the",
           f"runs: {nf // 3} and {nw // 3}). Each is scaled by the factor that makes a plain "
           f"{COPY_MIB} MiB device", f"copy read and write {COPY_MIB} MiB (fetch "
           f"{fscale:.3f}, write {wscale:.3f}).", "",
           "| launch | FETCH_SIZE (KiB) | HBM read (GB) | WRITE_SIZE (KiB) | HBM written (GB) |",
           "|---|---:|---:|---:|---:|"]
    md += [f"| {roles[i]} | {fk[i]:,.0f} | {fk[i] * 1024 * fscale / 1e9:.2f} | {wk[i]:,.0f} | "
           f"{wk[i] * 1024 * wscale / 1e9:.2f} |" for i in range(3)]
    if alg:
        md += ["", f"Algorithmic bytes per launch (both transposed operands in, one weight "
               f"gradient per expert out): {alg / 1e9:.2f} GB; measured / algorithmic "
               f"{float(np.mean(hbm)) / alg:.2f} (mean over the three launches)."]
    with open(os.path.join(ROOT, "profiles", f"grad_w_gemm_backward_{workload}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps(rec))


def backward_traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"grad_w_gemm_backward_{workload}_traffic.json")


def backward_source_hash():
    """Hash of the sources of the weight-gradient launches (the backward's
    host code and the large-tile GEMM it runs them on)."""
    h = hashlib.sha256()
    for name in ("backward.hip",) + GEMM_SRCS:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_backward_traffic(workload):
    """The committed rocprofv3 --pmc record of the weight-gradient GEMM
    launches, or None (also when their sources changed since it was taken)."""
    path = backward_traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    return rec if rec.get("backward_source_sha256_16") == backward_source_hash() else None


BWD_CPU_MAX_F64_BYTES = 32 << 30   # oracle backward baseline only when its fp64 weights and
                                   # weight gradients fit in this much host memory


def backward_flops(shape):
    """Algorithmic FLOPs of one backward call per stage (GEMM stages only) and in all."""
    T, d, N, k, F, S = shape.T, shape.d, shape.N, shape.k, shape.F, shape.S
    rows = T * k + S * T
    stage = {"recompute": 4 * rows * d * F, "grad_h": 2 * rows * d * F,
             "grad_x": 4 * rows * d * F + 2 * T * N * d, "grad_w": 6 * rows * d * F,
             "grad_wr": 2 * T * N * d}
    total = sum(stage.values()) + 2 * T * N * d  # + the recomputed router GEMM
    return stage, total


def cpu_backward_baseline(shape, inputs, dy, idx_all, n_tok):
    """The oracle's backward (O10), as it stands, on the first n tokens (with the
    GPU's choice of experts for them), grown until one call takes >= CPU_MIN_S."""
    import numpy as np
    import torch

    import oracle
    if shape.fp8 or shape.dtype != "bf16" and shape.dtype != "f32":
        return None
    wbytes = 3 * shape.N * shape.F * shape.d * 8
    if 2 * wbytes > BWD_CPU_MAX_F64_BYTES:
        return {"skipped": f"float64 weights and gradients would take {2 * wbytes / 2**30:.0f} GiB"}
    host = {n: inputs[n].float().cpu().numpy().astype(np.float64) for n in
            ("w_router", "w_gate", "w_up", "w_down") if inputs.get(n) is not None}
    shared = None
    if shape.S:
        shared = tuple(inputs[n].float().cpu().numpy().astype(np.float64)
                       for n in ("ws_gate", "ws_up", "ws_down"))
    lb = inputs["logit_bias"].cpu().numpy() if inputs.get("logit_bias") is not None else None
    sb = inputs["select_bias"].cpu().numpy() if inputs.get("select_bias") is not None else None
    threads = torch.get_num_threads()

    def run(n):
        x = inputs["x"][:n].float().cpu().numpy().astype(np.float64)
        g = dy[:n].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.moe_backward(x, host["w_router"], (host["w_gate"], host["w_up"], host["w_down"]),
                            shape.k, g, logit_bias=lb, select_bias=sb, shared=shared,
                            route_idx=idx_all[:n])
        return time.perf_counter() - t0

    n = min(n_tok, shape.T)
    el = run(n)
    while el < CPU_MIN_S and n < shape.T:
        n = min(shape.T, max(n + 1, int(n * min(8.0, CPU_TARGET_S / max(el, 1e-3)))))
        el = run(n)
    return {"value": round(n / el, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle backward (float64 NumPy) on the first {n} of {shape.T} tokens, "
                      f"one call, {el:.1f} s, the GPU's expert choice for those tokens"}


def time_backward(shape, inputs, steps, warmup, seed=0):
    """K timed moe_layer_backward calls on resident inputs (dy seeded): the
    backward's ms per step, tokens/s and GEMM rate, for the forward's line."""
    import torch

    import sparse_mixture_experts_router_amd as moe
    dev = inputs["x"].device
    T, d, N, k, F, S = shape.T, shape.d, shape.N, shape.k, shape.F, shape.S
    dt = shape.torch_dtype
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 7919 + 17)
    dy = torch.randn((T, d), generator=gen, device=dev).to(dt)
    cfg = moe.make_config(T, d, N, k, F, S, dt)
    ws = moe.alloc_backward_workspace(cfg, dev)
    g = {"dx": torch.empty((T, d), dtype=dt, device=dev),
         "dw_router": torch.empty((N, d), dtype=dt, device=dev),
         "dlogit_bias": torch.empty(N, dtype=torch.float32, device=dev),
         "dw_gate": torch.empty((N, F, d), dtype=dt, device=dev),
         "dw_up": torch.empty((N, F, d), dtype=dt, device=dev),
         "dw_down": torch.empty((N, d, F), dtype=dt, device=dev)}
    if S:
        g.update(dws_gate=torch.empty((S, F, d), dtype=dt, device=dev),
                 dws_up=torch.empty((S, F, d), dtype=dt, device=dev),
                 dws_down=torch.empty((S, d, F), dtype=dt, device=dev))

    def step():
        moe.moe_layer_backward(cfg, inputs["x"], inputs, dy, g, workspace=ws)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    _, total = backward_flops(shape)
    peak = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    del ws, g
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "tflops": round(total / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(total / (ms * 1e-3) / 1e12 / peak, 4), "steps": steps,
            "note": "moe_layer_backward on the same inputs (seeded dy): routing and gate/up "
                    "recomputed, every gradient written; details: bench.py --pass backward"}


def bench_backward(args, shape):
    """One step = one moe_layer_backward call (routing and gate/up recomputed,
    every gradient written) on resident inputs; prints one JSON line."""
    import numpy as np
    import torch

    import sparse_mixture_experts_router_amd as moe
    from workloads import make_inputs

    if shape.fp8:
        print("bench.py: the backward takes expert weights in the layer dtype", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    print(f"[bench] backward, drawing inputs: {shape.describe()}", file=sys.stderr, flush=True)
    inputs = make_inputs(shape, seed=args.seed, device=dev)
    T, d, N, k, F, S = shape.T, shape.d, shape.N, shape.k, shape.F, shape.S
    dt = shape.torch_dtype
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed * 7919 + 17)
    dy = torch.randn((T, d), generator=gen, device=dev).to(dt)
    cfg = moe.make_config(T, d, N, k, F, S, dt)
    ws = moe.alloc_backward_workspace(cfg, dev)
    g = {"dx": torch.empty((T, d), dtype=dt, device=dev),
         "dw_router": torch.empty((N, d), dtype=dt, device=dev),
         "dlogit_bias": torch.empty(N, dtype=torch.float32, device=dev),
         "dw_gate": torch.empty((N, F, d), dtype=dt, device=dev),
         "dw_up": torch.empty((N, F, d), dtype=dt, device=dev),
         "dw_down": torch.empty((N, d, F), dtype=dt, device=dev)}
    if S:
        g.update(dws_gate=torch.empty((S, F, d), dtype=dt, device=dev),
                 dws_up=torch.empty((S, F, d), dtype=dt, device=dev),
                 dws_down=torch.empty((S, d, F), dtype=dt, device=dev))
    stream = torch.cuda.current_stream()
    nst = len(moe.BACKWARD_STAGES)

    def step(events=None):
        moe.moe_layer_backward(cfg, inputs["x"], inputs, dy, g, workspace=ws,
                               stage_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr,
          flush=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = start.elapsed_time(end) / args.steps
    # per-stage breakdown from K more steps with every marker (HIP events on
    # the library's stream)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                for i, name in enumerate(moe.BACKWARD_STAGES)}
    sflops, total = backward_flops(shape)
    peak = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    dom = max(sflops, key=lambda n_: stage_ms[n_])
    launches = {"recompute": 2, "grad_h": 1, "grad_x": 1, "grad_w": 3, "grad_wr": 1}[dom]
    achieved = sflops[dom] / (stage_ms[dom] * 1e-3) / 1e12
    kernels = {"recompute": "grouped GEMMs of the gate and up projections (2 launches)",
               "grad_h": "grouped GEMM dy W_down + SwiGLU backward",
               "grad_x": "grouped GEMM [dA dB][W_gate; W_up] + router backward + dx",
               "grad_w": "weight-gradient grouped GEMMs, reduction per expert (3 launches)",
               "grad_wr": "router weight gradient"}[dom]
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None, "kernel": kernels,
            "stage": dom, "avg_launch_ms": round(stage_ms[dom] / launches, 4),
            "algorithmic_flops": sflops[dom] // launches,
            "note": "stage time (HIP events on the library's stream) over its launches"}
    if dom == "grad_w":
        # per launch: the two transposed operands (rows x (d + F)) in, one
        # weight gradient per expert out
        rows = T * k + S * T
        b = shape.elem_bytes
        roof["algorithmic_bytes"] = rows * (d + F) * b + (N + S) * d * F * b
        rec = load_backward_traffic(shape.name)
        if rec is not None:
            roof["traffic"] = rec["hbm_bytes_per_launch_mean"]
            roof["traffic_source"] = os.path.relpath(backward_traffic_path(shape.name), ROOT)
            roof["traffic_over_algorithmic"] = round(
                rec["hbm_bytes_per_launch_mean"] / roof["algorithmic_bytes"], 3)
    result = {
        "metric": "MoE layer backward tokens/sec; GEMM TFLOP/s as % of MI355X peak",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens and dy, N(0,0.02^2) random weights)",
        "config": {"workload": shape.name + "_backward", "T": T, "d_model": d, "n_experts": N,
                   "top_k": k, "d_ff": F, "n_shared": S, "parallelism": "single GPU"},
        "layer": {"tflops": round(total / (ms_step * 1e-3) / 1e12, 2),
                  "mfma_frac": round(total / (ms_step * 1e-3) / 1e12 / peak, 4),
                  "algorithmic_flops": total},
        "stages_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        fws = moe.alloc_workspace(cfg, dev)
        y = torch.empty((T, d), dtype=dt, device=dev)
        moe.moe_layer_forward(cfg, inputs["x"], inputs, y, workspace=fws, topk_idx=idx)
        n = args.cpu_tokens or 32
        print(f"[bench] CPU oracle backward from {n} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_backward_baseline(shape, inputs, dy, idx.cpu().numpy(), n)
    print(json.dumps(result), flush=True)


def time_forward(moe, shape, inputs, steps, warmup, extras=True):
    """Time `steps` layer forwards after `warmup`, inputs resident in HBM.

    The timed region is bracketed by HIP events on the library's stream (and
    the wall clock).  Inside it, one step in mark_stride(steps) also records
    events around the gate/up and the down launches, so their durations are
    measured live in the timed region.  With `extras`, K more (untimed) steps
    with every stage marker give the stage breakdown and the per-step spread,
    and the step is replayed K times from a HIP graph."""
    import numpy as np
    import torch

    dev = inputs["x"].device
    T, N, k = shape.T, shape.N, shape.k
    cfg = moe.make_config(T, shape.d, N, k, shape.F, shape.S, shape.torch_dtype,
                          weight_format=(moe.MOE_WEIGHTS_FP8_E4M3 if shape.fp8
                                         else moe.MOE_WEIGHTS_DTYPE))
    ws = moe.alloc_workspace(cfg, dev)
    y = torch.empty((T, shape.d), dtype=shape.torch_dtype, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(N, dtype=torch.int32, device=dev)
    psum = torch.empty(N, dtype=torch.float32, device=dev)
    f = torch.empty(N, dtype=torch.float32, device=dev)
    P = torch.empty(N, dtype=torch.float32, device=dev)
    aux = torch.empty(2, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        # the forward also writes the balance statistics (f, P, aux) from its
        # grouping step, so one call covers the whole path
        moe.moe_layer_forward(cfg, inputs["x"], inputs, y, workspace=ws, topk_idx=idx,
                              topk_gate=gate, counts=counts, prob_sum=psum, f=f, P=P, aux=aux,
                              alpha=0.01, stage_events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {shape.name}: warmup {warmup} done; timing {steps} steps", file=sys.stderr,
          flush=True)
    nst = len(moe.STAGES)
    iu, idn = moe.STAGES.index("expert_up"), moe.STAGES.index("expert_down")

    def gemm_events():
        evs_ = [None] * (nst + 1)
        for i in (iu, iu + 1, idn + 1):
            evs_[i] = torch.cuda.Event(enable_timing=True)
        return evs_

    every = mark_stride(steps)
    marked = list(range(every // 2, steps, every))
    tevs = {i: gemm_events() for i in marked}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(tevs.get(i))
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = start.elapsed_time(end) / steps
    up_ms = sum(e[iu].elapsed_time(e[iu + 1]) for e in tevs.values()) / len(tevs)
    dn_ms = sum(e[idn].elapsed_time(e[idn + 1]) for e in tevs.values()) / len(tevs)
    res = {"cfg": cfg, "ms_step": ms_step, "wall_ms": wall * 1e3 / steps, "up_ms": up_ms,
           "down_ms": dn_ms, "marked": len(tevs), "every": every, "idx": idx,
           "counts": counts.cpu().numpy()}
    if extras:
        # per-stage breakdown from K more (untimed) steps with every marker
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
               for _ in range(steps)]
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        res["stage_ms"] = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps
                           for i, name in enumerate(moe.STAGES)}
        per_step = np.sort(np.array([e[0].elapsed_time(e[nst]) for e in evs]))
        res["pct"] = {q: float(np.percentile(per_step, q)) for q in (10, 50, 90)}
        # the same step captured once in a HIP graph and replayed K times, as a
        # serving loop would run it
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        # the capture leaves the GPU idle for a moment; after any idle spell the
        # GEMMs run up to a third slower for the next ~30 ms while the clock
        # settles, so the replays get the same warm-up as the eager steps
        for _ in range(max(warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()
        gs = torch.cuda.Event(enable_timing=True)
        ge = torch.cuda.Event(enable_timing=True)
        gs.record(stream)
        for _ in range(steps):
            graph.replay()
        ge.record(stream)
        torch.cuda.synchronize()
        res["graph_ms"] = gs.elapsed_time(ge) / steps
        del graph
    del ws
    return res


def plan_of(moe, shape):
    """How the library runs the workload on this device (moe_forward_plan):
    the kernel and tile rows of each grouped GEMM, the router's kernel and
    split, the down pass's split and whether the all-token pass runs."""
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S,
                          shape.torch_dtype,
                          weight_format=(moe.MOE_WEIGHTS_FP8_E4M3 if shape.fp8
                                         else moe.MOE_WEIGHTS_DTYPE))
    p = moe.moe_forward_plan(cfg)
    return {k: p[k] for k in ("up_kernel", "up_tile_rows", "down_kernel", "down_tile_rows",
                              "route_kernel", "route_split", "down_split", "all_token_pass")}


def roofline_of(shape, active, up_ms, workload, plan=None):
    """The gate/up launch against both roofs.  `bound` is the roof that binds
    at its arithmetic intensity (time at the MFMA peak against time at the HBM
    peak); achieved and frac are in that roof's unit, and both fractions are
    reported."""
    _, _, uf, ub = algorithmic(shape, active)
    peak_flops = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    t_mfma = uf / (peak_flops * 1e12)
    t_hbm = ub / (PEAK_HBM_GBS * 1e9)
    tflops = uf / (up_ms * 1e-3) / 1e12
    gbs = ub / (up_ms * 1e-3) / 1e9
    if t_hbm > t_mfma:
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(tflops / peak_flops, 4)}
    roof["mfma_frac"] = round(tflops / peak_flops, 4)
    roof["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4)
    roof["arithmetic_intensity"] = round(uf / ub, 1)
    roof["kernel"] = "grouped gate/up GEMM with SiLU*up (expert_up stage)"
    if plan is not None and plan.get("all_token_pass"):
        roof["kernel"] = ("grouped gate/up GEMM with SiLU*up, every expert on all tokens, and "
                          "the batch's routing in one more workgroup of the same launch "
                          "(expert_up stage, all-token pass)")
    roof["avg_launch_ms"] = round(up_ms, 4)
    roof["algorithmic_bytes"] = ub
    roof["algorithmic_flops"] = uf
    rec = load_traffic(workload)
    roof["traffic"] = None if rec is None else rec["hbm_bytes_per_launch"]
    if rec is not None:
        roof["traffic_source"] = os.path.relpath(traffic_path(workload), ROOT)
        roof["traffic_over_algorithmic"] = round(rec["hbm_bytes_per_launch"] / ub, 3)
    mrec = load_mfma(workload)
    if mrec is not None:
        roof["mfma_busy"] = mrec["up"]["mfma_busy_frac"]
        roof["mfma_flops_issued_over_algorithmic"] = mrec["up"]["issued_over_algorithmic"]
        roof["mfma_source"] = os.path.relpath(mfma_path(workload), ROOT)
    return roof


def layer_of(shape, active, ms_step):
    lf, lb, _, _ = algorithmic(shape, active)
    peak_flops = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    tflops = lf / (ms_step * 1e-3) / 1e12
    gbs = lb / (ms_step * 1e-3) / 1e9
    return {"tflops": round(tflops, 2), "mfma_frac": round(tflops / peak_flops, 4),
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "roofline_ms": round(max(lf / (peak_flops * 1e12), lb / (PEAK_HBM_GBS * 1e9)) * 1e3, 4),
            "algorithmic_flops": lf, "algorithmic_bytes": lb, "active_experts": active}


def config_of(shape):
    return {"workload": shape.name, "T": shape.T, "d_model": shape.d, "n_experts": shape.N,
            "top_k": shape.k, "d_ff": shape.F, "n_shared": shape.S,
            "select_bias": shape.select_bias, "zipf_s": shape.zipf_s,
            "expert_weights": "fp8_e4m3 + fp32 per-channel scales" if shape.fp8 else shape.dtype,
            "parallelism": "single GPU"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards over tokens or experts, but no multi-GPU path exists)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.summarize_profiles:
        if args.pass_ == "backward":
            summarize_backward_profiles(args.summarize_profiles, args.workload)
        else:
            summarize_profiles(args.summarize_profiles, args.workload)
        return

    import numpy as np
    import torch

    import sparse_mixture_experts_router_amd as moe
    from workloads import CONFIGS, make_inputs

    shape = CONFIGS[args.workload]
    if args.pass_ == "backward":
        bench_backward(args, shape)
        return
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    print(f"[bench] drawing inputs: {shape.describe()}", file=sys.stderr, flush=True)
    inputs = make_inputs(shape, seed=args.seed, device=dev)
    T = shape.T
    r = time_forward(moe, shape, inputs, args.steps, args.warmup)
    ms_step = r["ms_step"]
    active = int(np.count_nonzero(r["counts"]))
    plan = plan_of(moe, shape)
    roof = roofline_of(shape, active, r["up_ms"], args.workload, plan)
    roof["timed_launches"] = (f"{r['marked']} of the {args.steps} timed steps "
                              f"(one in {r['every']})")
    result = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02^2) random weights of the model's shape)",
        "config": config_of(shape),
        "plan": plan,
        "layer": layer_of(shape, active, ms_step),
        "stages_ms": {k_: round(v, 4) for k_, v in r["stage_ms"].items()},
        "down_launch_ms": round(r["down_ms"], 4),
        "forward_ms_p10_p50_p90": [round(r["pct"][q], 4) for q in (10, 50, 90)],
        "wall_ms_per_step": round(r["wall_ms"], 4),
        "graph_replay": {"ms_per_step": round(r["graph_ms"], 4),
                         "tokens_per_s": round(T / (r["graph_ms"] * 1e-3), 1),
                         "note": "the same step captured once in a HIP graph, K replays"},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_backward and not shape.fp8:
        print("[bench] backward of the same layer", file=sys.stderr, flush=True)
        result["backward"] = time_backward(shape, inputs, min(args.steps, 20),
                                           min(args.warmup, 3), args.seed)
    if not args.no_cpu_baseline:
        n = args.cpu_tokens or DEFAULT_CPU_TOKENS.get(args.workload, 64)
        print(f"[bench] CPU oracle on {n} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(shape, inputs, n, r["idx"].cpu().numpy())
    del inputs, r
    torch.cuda.empty_cache()

    also = [w for w in args.also.split(",") if w and w != args.workload]
    if also:
        others = {}
        for name in also:
            shp = CONFIGS[name]
            print(f"[bench] also: drawing inputs of {name}: {shp.describe()}", file=sys.stderr,
                  flush=True)
            inp = make_inputs(shp, seed=args.seed, device=dev)
            o = time_forward(moe, shp, inp, args.steps, args.warmup, extras=False)
            act = int(np.count_nonzero(o["counts"]))
            pl = plan_of(moe, shp)
            rf = roofline_of(shp, act, o["up_ms"], name, pl)
            others[name] = {
                "ms_per_step": round(o["ms_step"], 4),
                "tokens_per_s": round(shp.T / (o["ms_step"] * 1e-3), 1),
                "layer": {k_: v for k_, v in layer_of(shp, act, o["ms_step"]).items()
                          if k_ in ("tflops", "mfma_frac", "hbm_gbs", "hbm_frac", "roofline_ms")},
                "gate_up": {k_: rf[k_] for k_ in ("bound", "achieved", "unit", "frac", "mfma_frac",
                                                  "hbm_frac", "avg_launch_ms")},
                "down_launch_ms": round(o["down_ms"], 4),
                "config": {k_: v for k_, v in config_of(shp).items() if k_ != "parallelism"},
                "plan": pl,
            }
            del inp, o
            torch.cuda.empty_cache()
        result["other_workloads"] = {
            "note": ("timed in the same run, same protocol (warm-up, K steps between HIP "
                     "events; gate/up and down launches from markers in one step in "
                     f"{mark_stride(args.steps)})"),
            **others}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
