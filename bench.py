"""Benchmark of the sparse MoE layer forward on one MI355X.

One step = one whole layer forward (route, grouping, gate/up experts, down
experts, combine) plus the balance statistics, on seeded synthetic inputs that
are resident in HBM before timing starts.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-tokens N]

Workloads (random weights of the named models' shapes, no checkpoints):
mixtral_prefill (default), mixtral_decode, deepseek_v3, qwen3_skew, tiny_f32.
"""

from __future__ import annotations

import argparse
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
DEFAULT_CPU_TOKENS = {"mixtral_prefill": 256, "mixtral_decode": 32, "deepseek_v3": 32,
                      "qwen3_skew": 256, "tiny_f32": 64}
GEMM_SRC = os.path.join(ROOT, "sparse_mixture_experts_router_amd", "csrc", "grouped_gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
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


def algorithmic(shape, active):
    """Layer and gate/up-kernel algorithmic FLOPs and bytes (inputs once, outputs once)."""
    T, d, N, k, F, S, b = shape.T, shape.d, shape.N, shape.k, shape.F, shape.S, shape.elem_bytes
    rows = T * k + S * T
    layer_flops = 2 * rows * 3 * d * F + 2 * T * d * N
    layer_bytes = (active + S) * 3 * d * F * b + N * d * b + 2 * T * d * b + T * k * 8
    up_flops = 2 * rows * d * 2 * F
    up_bytes = (active + S) * 2 * F * d * b + T * d * b + rows * F * b
    return layer_flops, layer_bytes, up_flops, up_bytes


def gemm_source_hash():
    with open(GEMM_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per gate/up launch from the committed rocprofv3 --pmc summary.

    Returns None when there is no summary or when the kernel source changed
    since the counters were taken.
    """
    path = os.path.join(ROOT, "profiles", f"expert_up_gemm_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(shape, inputs, n_tok, gpu_idx):
    """The CPU oracle, as it stands, on the first n_tok tokens of the same batch."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()}))
    except Exception:  # threadpoolctl missing: report the affinity set
        threads, blas = len(os.sched_getaffinity(0)), "unknown"

    n_tok = min(n_tok, shape.T)
    x = inputs["x"][:n_tok].float().cpu().numpy()
    wr = inputs["w_router"].float().cpu().numpy()
    lb = None if inputs["logit_bias"] is None else inputs["logit_bias"].cpu().numpy()
    sb = None if inputs["select_bias"] is None else inputs["select_bias"].cpu().numpy()
    need = sorted(set(gpu_idx[:n_tok].reshape(-1).tolist()))
    cache = {e: (inputs["w_gate"][e].float().cpu().numpy(), inputs["w_up"][e].float().cpu().numpy(),
                 inputs["w_down"][e].float().cpu().numpy()) for e in need}
    fetched = []

    def expert(e):
        if e not in cache:   # a selection flip against the GPU's routing: fetch on demand
            fetched.append(e)
            cache[e] = (inputs["w_gate"][e].float().cpu().numpy(),
                        inputs["w_up"][e].float().cpu().numpy(),
                        inputs["w_down"][e].float().cpu().numpy())
        return cache[e]

    shared = None
    if shape.S:
        shared = tuple(inputs[n].float().cpu().numpy() for n in ("ws_gate", "ws_up", "ws_down"))
    t0 = time.perf_counter()
    ref = oracle.moe_forward(x, wr, expert, shape.k, logit_bias=lb, select_bias=sb, shared=shared,
                             n_experts=shape.N)
    dt = time.perf_counter() - t0
    del ref
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"first {n_tok} of {shape.T} tokens, all their experts; NumPy float64 "
                       f"({blas}), {dt:.1f} s; host affinity {len(os.sched_getaffinity(0))} cpus"),
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards over tokens or experts, but no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import numpy as np
    import torch

    import sparse_mixture_experts_router_amd as moe
    from workloads import CONFIGS, make_inputs

    shape = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    print(f"[bench] drawing inputs: {shape.describe()}", file=sys.stderr, flush=True)
    inputs = make_inputs(shape, seed=args.seed, device=dev)
    T, N, k = shape.T, shape.N, shape.k
    cfg = moe.make_config(T, shape.d, N, k, shape.F, shape.S, shape.torch_dtype)
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
        moe.moe_layer_forward(cfg, inputs["x"], inputs, y, workspace=ws, topk_idx=idx,
                              topk_gate=gate, counts=counts, prob_sum=psum,
                              stage_events=events)
        moe.moe_balance_stats(T, N, k, counts, psum, 0.01, f, P, aux)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr,
          flush=True)

    nst = len(moe.STAGES)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    stage_ms = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                for i, name in enumerate(moe.STAGES)}

    counts_h = counts.cpu().numpy()
    active = int(np.count_nonzero(counts_h))
    lf, lb, uf, ub = algorithmic(shape, active)
    tok_s = T / (ms_step * 1e-3)
    peak_flops = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    up_ms = stage_ms["expert_up"]
    decode_like = (T * k) / max(1, active) < 64
    if decode_like:
        achieved = ub / (up_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = uf / (up_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4)}
    roof["kernel"] = "grouped gate/up GEMM with SiLU*up (expert_up stage)"
    roof["avg_launch_ms"] = round(up_ms, 4)
    roof["traffic"] = load_traffic(args.workload)

    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
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
        "config": {"workload": shape.name, "T": T, "d_model": shape.d, "n_experts": N,
                   "top_k": k, "d_ff": shape.F, "n_shared": shape.S,
                   "select_bias": shape.select_bias, "zipf_s": shape.zipf_s,
                   "parallelism": "single GPU"},
        "layer": {"tflops": round(lf / (ms_step * 1e-3) / 1e12, 2),
                  "mfma_frac": round(lf / (ms_step * 1e-3) / 1e12 / peak_flops, 4),
                  "hbm_gbs": round(lb / (ms_step * 1e-3) / 1e9, 1),
                  "hbm_frac": round(lb / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "algorithmic_flops": lf, "algorithmic_bytes": lb,
                  "active_experts": active},
        "stages_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        n = args.cpu_tokens or DEFAULT_CPU_TOKENS.get(args.workload, 64)
        print(f"[bench] CPU oracle on {n} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(shape, inputs, n, idx.cpu().numpy())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
