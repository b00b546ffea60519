"""Helpers for the GPU parity tests: run the HIP library on seeded inputs and
check it against the CPU oracle on the same bits.

Routing parity protocol: the library returns its fp32 logits; the oracle
selects and gates on *those* logits, so expert indices and counts must agree
bit for bit, whatever the accumulation order of the router GEMM.  The
oracle's own logits are compared separately (selection flips are counted).
"""

from __future__ import annotations

import sys
import time
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import oracle
import sparse_mixture_experts_router_amd as moe
from workloads import MoEShape, make_inputs

# tolerances: fp32 output max|err| <= 1e-4; bf16 output max|err| <=
# 1e-2 * max|y_ref| + 1e-3 (rounding Y_perm and y to bf16 costs at most
# 2 * 2^-8 of |y|, rounding H a random ~2^-8 / sqrt(3) per element); gates
# 1e-6; f, P, aux 1e-5 relative
TOL_F32 = 1e-4
GATE_TOL = 1e-6
STAT_RTOL = 1e-5


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.cpu().numpy()


def run_layer(shape: MoEShape, inputs: Dict[str, Optional[torch.Tensor]], alpha: float = 0.01,
              events=None, capacity: int = 0):
    """One moe_layer_forward + moe_balance_stats call; returns device outputs."""
    T = shape.T
    dev = inputs["w_gate"].device
    cfg = moe.make_config(T, shape.d, shape.N, shape.k, shape.F, shape.S, shape.torch_dtype,
                          capacity=capacity,
                          weight_format=(moe.MOE_WEIGHTS_FP8_E4M3 if shape.fp8
                                         else moe.MOE_WEIGHTS_DTYPE))
    ws = moe.alloc_workspace(cfg, dev)
    out = {
        "y": torch.empty((T, shape.d), dtype=shape.torch_dtype, device=dev),
        "logits": torch.empty((T, shape.N), dtype=torch.float32, device=dev),
        "topk_idx": torch.empty((T, shape.k), dtype=torch.int32, device=dev),
        "topk_gate": torch.empty((T, shape.k), dtype=torch.float32, device=dev),
        "counts": torch.zeros(shape.N, dtype=torch.int32, device=dev),
        "prob_sum": torch.zeros(shape.N, dtype=torch.float32, device=dev),
        "f": torch.empty(shape.N, dtype=torch.float32, device=dev),
        "P": torch.empty(shape.N, dtype=torch.float32, device=dev),
        "aux": torch.empty(2, dtype=torch.float32, device=dev),
    }
    moe.moe_layer_forward(cfg, inputs["x"], inputs, out["y"], workspace=ws,
                          logits=out["logits"], topk_idx=out["topk_idx"],
                          topk_gate=out["topk_gate"], counts=out["counts"],
                          prob_sum=out["prob_sum"], stage_events=events)
    moe.moe_balance_stats(T, shape.N, shape.k, out["counts"], out["prob_sum"], alpha,
                          out["f"], out["P"], out["aux"])
    torch.cuda.synchronize()
    return out


def bf16_bound(y_ref: np.ndarray) -> float:
    return 1e-2 * float(np.max(np.abs(y_ref))) + 1e-3 if y_ref.size else 1e-3


def check_routing(shape: MoEShape, host: Dict[str, np.ndarray], gpu: Dict[str, np.ndarray]):
    """Bit-exact idx/counts on the GPU's logits, gates to 1e-6."""
    logits = gpu["logits"].astype(np.float32)
    idx_ref, g_ref = oracle.route_from_logits(logits, shape.k, host.get("select_bias"))
    mism = np.nonzero(np.any(gpu["topk_idx"] != idx_ref, axis=1))[0]
    assert mism.size == 0, (f"{mism.size} tokens routed differently, first {mism[:5].tolist()}: "
                            f"gpu {gpu['topk_idx'][mism[:3]].tolist()} ref "
                            f"{idx_ref[mism[:3]].tolist()}")
    gerr = float(np.max(np.abs(gpu["topk_gate"] - g_ref))) if g_ref.size else 0.0
    assert gerr <= GATE_TOL, f"gate error {gerr}"
    counts_ref = np.bincount(idx_ref.reshape(-1), minlength=shape.N)
    assert np.array_equal(gpu["counts"], counts_ref), "counts differ"
    return idx_ref, g_ref


def check_stats(shape: MoEShape, gpu: Dict[str, np.ndarray]):
    logits = gpu["logits"].astype(np.float32)
    idx = gpu["topk_idx"]
    counts, f, P = oracle.stats(idx, logits, shape.N)
    raw, aux = oracle.balance(f, P)
    np.testing.assert_allclose(gpu["f"], f, rtol=STAT_RTOL, atol=1e-7)
    np.testing.assert_allclose(gpu["prob_sum"] / max(shape.T, 1), P, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(gpu["P"], P, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(gpu["aux"][0], raw, rtol=STAT_RTOL)
    np.testing.assert_allclose(gpu["aux"][1], aux, rtol=STAT_RTOL)
    return raw


def host_inputs(inputs: Dict[str, Optional[torch.Tensor]], names: Sequence[str]):
    return {n: to_np(inputs[n]) for n in names if inputs.get(n) is not None}


def full_parity(shape: MoEShape, seed: int = 0, inputs=None, label: str = "",
                capacity: int = 0):
    """Element-wise parity of the whole layer against the oracle (small shapes)."""
    say(f"[parity] {label or shape.name}: {shape.describe()} seed={seed} capacity={capacity}")
    if inputs is None:
        inputs = make_inputs(shape, seed=seed, device="cuda")
    out = run_layer(shape, inputs, capacity=capacity)
    gpu = {k_: to_np(v) for k_, v in out.items()}
    host = host_inputs(inputs, ["x", "w_router", "w_gate", "w_up", "w_down", "ws_gate",
                                "ws_up", "ws_down", "logit_bias", "select_bias"])
    if shape.fp8:  # the oracle decodes the codes and applies the scales (O9)
        for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
            if host.get(n) is not None:
                host[n] = oracle.dequantize(host[n], to_np(inputs[n + "_scale"]))
    check_routing(shape, host, gpu)
    shared = ((host["ws_gate"], host["ws_up"], host["ws_down"]) if shape.S else None)
    ref = oracle.moe_forward(host["x"], host["w_router"],
                             (host["w_gate"], host["w_up"], host["w_down"]), shape.k,
                             select_bias=host.get("select_bias"), shared=shared,
                             route_logits=gpu["logits"], logit_bias=host.get("logit_bias"),
                             capacity=capacity)
    # the oracle's own fp64 logits agree with the GPU's to fp32 accumulation error
    own = oracle.router_logits(host["x"], host["w_router"], host.get("logit_bias"))
    if own.size:
        scale = float(np.max(np.abs(own))) + 1e-30
        assert float(np.max(np.abs(own - gpu["logits"]))) <= 1e-4 * scale + 1e-6
    err = float(np.max(np.abs(gpu["y"] - ref["y"]))) if ref["y"].size else 0.0
    bound = TOL_F32 if shape.dtype == "f32" else bf16_bound(ref["y"])
    say(f"[parity] {label or shape.name}: max|err| {err:.3e} bound {bound:.3e}")
    assert err <= bound, f"y error {err} > {bound}"
    check_stats(shape, gpu)
    return inputs, out, ref


def sampled_parity(shape: MoEShape, seed: int = 0, n_samples: int = 8):
    """Parity at full size: routing for every token, y for sampled tokens."""
    t0 = time.time()
    say(f"[full] {shape.name}: {shape.describe()} seed={seed}")
    inputs = make_inputs(shape, seed=seed, device="cuda")
    torch.cuda.synchronize()
    say(f"[full] inputs drawn in {time.time() - t0:.1f}s")
    out = run_layer(shape, inputs)
    say(f"[full] forward done in {time.time() - t0:.1f}s")
    gpu = {k_: to_np(out[k_]) for k_ in ("logits", "topk_idx", "topk_gate", "counts",
                                         "prob_sum", "f", "P", "aux")}
    host = host_inputs(inputs, ["logit_bias", "select_bias"])
    check_routing(shape, host, gpu)
    raw = check_stats(shape, gpu)
    say(f"[full] routing bit-exact, aux_raw {raw:.4f}, {time.time() - t0:.1f}s")

    rng = np.random.default_rng(seed + 99)
    T = shape.T
    toks = sorted(set([0, T - 1] + rng.choice(T, size=min(T, n_samples), replace=False).tolist()))
    sel = torch.tensor(toks, dtype=torch.long, device="cuda")
    x_s = to_np(inputs["x"].index_select(0, sel))
    y_s = to_np(out["y"].index_select(0, sel))
    lg_s = gpu["logits"][toks]

    def weight(name, e=None):
        w = inputs[name] if e is None else inputs[name][e]
        if not shape.fp8:
            return to_np(w)
        s = inputs[name + "_scale"] if e is None else inputs[name + "_scale"][e]
        return oracle.dequantize(to_np(w), to_np(s))

    def expert(e):
        return (weight("w_gate", e), weight("w_up", e), weight("w_down", e))

    shared = None
    if shape.S:
        shared = (weight("ws_gate"), weight("ws_up"), weight("ws_down"))
    ref = oracle.moe_forward(x_s, None, expert, shape.k, select_bias=host.get("select_bias"),
                             shared=shared, route_logits=lg_s, n_experts=shape.N)
    err = float(np.max(np.abs(y_s - ref["y"])))
    bound = bf16_bound(ref["y"])
    say(f"[full] {shape.name}: {len(toks)} sampled tokens max|err| {err:.3e} bound {bound:.3e}"
        f" ({time.time() - t0:.1f}s)")
    assert err <= bound
    yf = out["y"].float()
    assert bool(torch.isfinite(yf).all()), "non-finite output"
    return out
