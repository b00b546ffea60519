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
# 1e-6; f, P, prob_sum / T and aux 1e-5 relative.
# P's bound: each softmax term carries at most ~25 units of fp32 rounding
# (u = 2^-24): the exponential's argument |r - max r| <= ~15 costs that many
# u, the N-term sum of exponentials log2(N) + N/16 more, the division one.
# The terms are positive, so sums of them keep the relative error of their
# worst term plus one u per addition on the longest chain: 4 tokens per lane,
# 2 butterfly levels and 4 wavefronts inside a 64-token block, then at most
# ceil(B / P) blocks per thread and P thread partials per expert in the
# grouping step (P = min(1024 / N, B) threads per expert, B blocks): at most
# 64 + 2 additions at every workload here.  25 + 8 + 66 = 99 u = 5.9e-6.
# Below fp32's smallest normal number (FLT_MIN = 1.18e-38) there is no relative
# precision: an expert whose probability is e^-100 gets 0 from the GPU's
# exponential (its subnormal result flushes to zero) and ~1e-43 from the
# float64 oracle.  Each term's absolute error is then at most FLT_MIN, and so
# is that of their mean: P and prob_sum / T take FLT_MIN as absolute term.
TOL_F32 = 1e-4
GATE_TOL = 1e-6
STAT_RTOL = 1e-5
STAT_ATOL = float(np.finfo(np.float32).tiny)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.cpu().numpy()


def poisoned_workspace(cfg, dev) -> torch.Tensor:
    """A workspace filled with 0xFF bytes, so a region the kernels read before
    writing (or never write) shows up as garbage instead of a stale value."""
    ws = moe.alloc_workspace(cfg, dev)
    ws.fill_(0xFF)
    return ws


def run_layer(shape: MoEShape, inputs: Dict[str, Optional[torch.Tensor]], alpha: float = 0.01,
              events=None, capacity: int = 0):
    """One moe_layer_forward + moe_balance_stats call; returns device outputs.

    Every output starts as NaN (floating point) or -1 (integer) and the
    workspace as 0xFF bytes, so an element the library never writes cannot
    pass as a stale value from an earlier allocation."""
    T = shape.T
    dev = inputs["w_gate"].device
    cfg = moe.make_config(T, shape.d, shape.N, shape.k, shape.F, shape.S, shape.torch_dtype,
                          capacity=capacity,
                          weight_format=(moe.MOE_WEIGHTS_FP8_E4M3 if shape.fp8
                                         else moe.MOE_WEIGHTS_DTYPE))
    ws = poisoned_workspace(cfg, dev)
    nan = float("nan")
    out = {
        "y": torch.full((T, shape.d), nan, dtype=shape.torch_dtype, device=dev),
        "logits": torch.full((T, shape.N), nan, dtype=torch.float32, device=dev),
        "topk_idx": torch.full((T, shape.k), -1, dtype=torch.int32, device=dev),
        "topk_gate": torch.full((T, shape.k), nan, dtype=torch.float32, device=dev),
        "counts": torch.full((shape.N,), -1, dtype=torch.int32, device=dev),
        "prob_sum": torch.full((shape.N,), nan, dtype=torch.float32, device=dev),
        "f": torch.full((shape.N,), nan, dtype=torch.float32, device=dev),
        "P": torch.full((shape.N,), nan, dtype=torch.float32, device=dev),
        "aux": torch.full((2,), nan, dtype=torch.float32, device=dev),
    }
    moe.moe_layer_forward(cfg, inputs["x"], inputs, out["y"], workspace=ws,
                          logits=out["logits"], topk_idx=out["topk_idx"],
                          topk_gate=out["topk_gate"], counts=out["counts"],
                          prob_sum=out["prob_sum"], stage_events=events)
    moe.moe_balance_stats(T, shape.N, shape.k, out["counts"], out["prob_sum"], alpha,
                          out["f"], out["P"], out["aux"])
    torch.cuda.synchronize()
    # the down pass's split plan as the forward wrote it into the workspace:
    # [pieces, first split row, rows per piece, split row tiles]
    off = moe.moe_forward_plan(cfg)["split_plan_offset"]
    out["split_plan"] = ws[off:off + 16].view(torch.int32).clone()
    return out


_E4M3_TABLE = None


def fast_dequantize(codes: torch.Tensor, scale: torch.Tensor) -> np.ndarray:
    """oracle.dequantize (O9) through a 256-entry table: the table holds the
    oracle's own e4m3_decode of every code, gathered on the host with torch's
    multithreaded indexing and multiplied by the float64 scale per output
    channel.  Bitwise the same float64 values as oracle.dequantize (a CPU
    test checks it), about a hundred times faster on the DeepSeek-V3-shaped
    weights (11 billion codes)."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = torch.from_numpy(oracle.e4m3_decode(np.arange(256, dtype=np.uint8)))
    c = codes.cpu().long()
    s = scale.cpu().double()
    return (_E4M3_TABLE[c] * s[..., :, None]).numpy()


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
    np.testing.assert_allclose(gpu["f"], f, rtol=STAT_RTOL, atol=0)
    np.testing.assert_allclose(gpu["prob_sum"].astype(np.float64) / max(shape.T, 1), P,
                               rtol=STAT_RTOL, atol=STAT_ATOL)
    np.testing.assert_allclose(gpu["P"], P, rtol=STAT_RTOL, atol=STAT_ATOL)
    if P.size:
        say(f"[stats] P max relative error "
            f"{float(np.max(np.abs(gpu['P'] - P) / np.maximum(P, STAT_ATOL))):.2e}")
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


def full_size_parity(shape: MoEShape, seed: int = 0):
    """Parity at a workload's full size, in the launch configuration the
    benchmark times: routing bit-exact for every token, then EVERY element of
    y against the oracle's float64 forward of the whole batch (routed on the
    library's logits), the experts handed to the oracle one at a time."""
    t0 = time.time()
    say(f"[full] {shape.name}: {shape.describe()} seed={seed}")
    inputs = make_inputs(shape, seed=seed, device="cuda")
    torch.cuda.synchronize()
    say(f"[full] inputs drawn in {time.time() - t0:.1f}s")
    out = run_layer(shape, inputs)
    say(f"[full] forward done in {time.time() - t0:.1f}s")
    gpu = {k_: to_np(out[k_]) for k_ in ("logits", "topk_idx", "topk_gate", "counts",
                                         "prob_sum", "f", "P", "aux")}
    host = host_inputs(inputs, ["x", "w_router", "logit_bias", "select_bias"])
    check_routing(shape, host, gpu)
    raw = check_stats(shape, gpu)
    # the oracle's own logits (O1) against the library's, and the selections
    # they would make
    own = oracle.router_logits(host["x"], host["w_router"], host.get("logit_bias"))
    scale = float(np.max(np.abs(own))) + 1e-30
    lerr = float(np.max(np.abs(own - gpu["logits"])))
    assert lerr <= 1e-4 * scale + 1e-6, f"logits differ from O1 by {lerr}"
    own_idx, _ = oracle.route_from_logits(own, shape.k, host.get("select_bias"))
    flips = int(np.count_nonzero(np.any(own_idx != gpu["topk_idx"], axis=1)))
    say(f"[full] routing bit-exact, aux_raw {raw:.4f}, logits max|diff| from O1 {lerr:.2e}, "
        f"{flips} of {shape.T} tokens would route differently on O1's logits, "
        f"{time.time() - t0:.1f}s")

    def weight(name, e=None):
        w = inputs[name] if e is None else inputs[name][e]
        if not shape.fp8:
            return to_np(w)
        s_ = inputs[name + "_scale"] if e is None else inputs[name + "_scale"][e]
        return fast_dequantize(w, s_)

    done = [0]

    def expert(e):
        done[0] += 1
        if done[0] % 32 == 0:
            say(f"[full] oracle: {done[0]} experts run, {time.time() - t0:.1f}s")
        return (weight("w_gate", e), weight("w_up", e), weight("w_down", e))

    shared = None
    if shape.S:
        shared = (weight("ws_gate"), weight("ws_up"), weight("ws_down"))
    ref = oracle.moe_forward(host["x"], None, expert, shape.k,
                             select_bias=host.get("select_bias"), shared=shared,
                             route_logits=gpu["logits"], n_experts=shape.N)
    say(f"[full] oracle forward of all {shape.T} tokens done, {time.time() - t0:.1f}s")
    y = to_np(out["y"])
    assert bool(np.all(np.isfinite(y))), "non-finite (or unwritten) output elements"
    diff = np.abs(y - ref["y"])
    err = float(np.max(diff))
    bound = bf16_bound(ref["y"]) if shape.dtype == "bf16" else TOL_F32
    worst = np.unravel_index(int(np.argmax(diff)), diff.shape)
    say(f"[full] {shape.name}: every element of y ({y.size}) max|err| {err:.3e} at token "
        f"{worst[0]} column {worst[1]}, bound {bound:.3e}, max|y_ref| "
        f"{float(np.max(np.abs(ref['y']))):.3e} ({time.time() - t0:.1f}s)")
    assert err <= bound, f"y error {err} > {bound}"
    return out
