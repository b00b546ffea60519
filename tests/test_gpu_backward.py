"""GPU parity of the layer backward (moe_layer_backward) and of the
selection-bias update (moe_update_select_bias) against the CPU oracle (O10,
O11), element by element.

Routing protocol: a forward call gives the library's fp32 logits and its
choice of experts; check_routing confirms that choice is exactly the
oracle's on those logits, and the oracle's backward then takes it
(route_idx), so a near-tie taken differently by the two float64 / float32
logit sums cannot change which gradient is compared.

Tolerances.  fp32 layers: 1e-4 of each gradient's largest magnitude (fp32
accumulation; the oracle is float64).  bf16 layers: the path to every
gradient passes a few tensors held in bf16 (the recomputed gate/up
projections, dy W_down, the SwiGLU gradients, each row's dx contribution,
the router gradient), each rounding adding at most 2^-9 relative error to its
terms; the bound 2^-6 of the gradient's largest magnitude leaves room for
sums of many such terms of mixed sign.  The selection-bias update is
bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_router_amd as moe
from gpu_harness import check_routing, host_inputs, say, to_np
from workloads import MoEShape, make_inputs

pytestmark = pytest.mark.gpu

ALPHA, AUX_GRAD = 0.05, 3.0
GRADS = ("dx", "dw_router", "dlogit_bias", "dw_gate", "dw_up", "dw_down")
SHARED = {"ds_gate": "dws_gate", "ds_up": "dws_up", "ds_down": "dws_down"}


def run_backward(shape: MoEShape, inputs, dy, capacity=0, logit_bias_grad=True):
    T, d, N, F, S = shape.T, shape.d, shape.N, shape.F, shape.S
    dt, dev = shape.torch_dtype, "cuda"
    cfg = moe.make_config(T, d, N, shape.k, F, S, dt, capacity=capacity)
    ws = moe.alloc_backward_workspace(cfg, dev)
    ws.fill_(0xFF)  # stale bytes must not leak into any result
    g = {
        "dx": torch.empty((T, d), dtype=dt, device=dev),
        "dw_router": torch.empty((N, d), dtype=dt, device=dev),
        "dlogit_bias": (torch.empty(N, dtype=torch.float32, device=dev)
                        if logit_bias_grad else None),
        "dw_gate": torch.empty((N, F, d), dtype=dt, device=dev),
        "dw_up": torch.empty((N, F, d), dtype=dt, device=dev),
        "dw_down": torch.empty((N, d, F), dtype=dt, device=dev),
    }
    if S:
        g["dws_gate"] = torch.empty((S, F, d), dtype=dt, device=dev)
        g["dws_up"] = torch.empty((S, F, d), dtype=dt, device=dev)
        g["dws_down"] = torch.empty((S, d, F), dtype=dt, device=dev)
    for v in g.values():
        if v is not None:
            v.fill_(float("nan"))  # every element must be written
    moe.moe_layer_backward(cfg, inputs["x"], inputs, dy, g, workspace=ws, alpha=ALPHA,
                           aux_grad=AUX_GRAD)
    torch.cuda.synchronize()
    return g


def forward_routing(shape, inputs, capacity=0):
    T = shape.T
    cfg = moe.make_config(T, shape.d, shape.N, shape.k, shape.F, shape.S, shape.torch_dtype,
                          capacity=capacity)
    ws = moe.alloc_workspace(cfg, "cuda")
    out = {"y": torch.empty((T, shape.d), dtype=shape.torch_dtype, device="cuda"),
           "logits": torch.empty((T, shape.N), dtype=torch.float32, device="cuda"),
           "topk_idx": torch.empty((T, shape.k), dtype=torch.int32, device="cuda"),
           "topk_gate": torch.empty((T, shape.k), dtype=torch.float32, device="cuda"),
           "counts": torch.zeros(shape.N, dtype=torch.int32, device="cuda")}
    moe.moe_layer_forward(cfg, inputs["x"], inputs, out["y"], workspace=ws,
                          logits=out["logits"], topk_idx=out["topk_idx"],
                          topk_gate=out["topk_gate"], counts=out["counts"])
    torch.cuda.synchronize()
    return {k_: to_np(v) for k_, v in out.items()}


def draw_dy(shape, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed * 7919 + 17)
    return torch.randn((shape.T, shape.d), generator=gen, device="cuda").to(shape.torch_dtype)


def check_backward(shape: MoEShape, seed=0, capacity=0, label=""):
    say(f"[bwd] {label or shape.name}: {shape.describe()} seed={seed} capacity={capacity}")
    inputs = make_inputs(shape, seed=seed, device="cuda", weight_std=0.05)
    dy = draw_dy(shape, seed)
    fwd = forward_routing(shape, inputs, capacity)
    host = host_inputs(inputs, ["x", "w_router", "w_gate", "w_up", "w_down", "ws_gate",
                                "ws_up", "ws_down", "logit_bias", "select_bias"])
    check_routing(shape, host, fwd)
    g = run_backward(shape, inputs, dy, capacity)
    shared = (host["ws_gate"], host["ws_up"], host["ws_down"]) if shape.S else None
    ref = oracle.moe_backward(host["x"], host["w_router"],
                              (host["w_gate"], host["w_up"], host["w_down"]), shape.k,
                              to_np(dy), logit_bias=host.get("logit_bias"),
                              select_bias=host.get("select_bias"), shared=shared, alpha=ALPHA,
                              aux_grad=AUX_GRAD, capacity=capacity, route_idx=fwd["topk_idx"])
    rtol = 1e-4 if shape.dtype == "f32" else 2.0 ** -6
    names = list(GRADS) + (list(SHARED) if shape.S else [])
    for n in names:
        got = to_np(g[SHARED.get(n, n)])
        exp = ref[n]
        assert np.all(np.isfinite(got)), f"{n}: non-finite values (unwritten elements?)"
        scale = float(np.max(np.abs(exp))) if exp.size else 0.0
        err = float(np.max(np.abs(got - exp))) if exp.size else 0.0
        say(f"[bwd]   {n:12s} max|ref| {scale:.3e} max|err| {err:.3e} ({err / (scale + 1e-30):.2e})")
        assert err <= rtol * scale + 1e-30, f"{n}: error {err} > {rtol} * {scale}"
    return g, ref


BACKWARD_CASES = [
    # 128-row large tiles, ragged T and F (partial row and column tiles)
    ("tiles128_ragged", MoEShape("bwd_t128", T=300, d=256, N=8, k=2, F=320)),
    # shared expert, selection bias, Zipf logit offset (logit-bias gradient)
    ("shared_bias", MoEShape("bwd_shared", T=200, d=128, N=16, k=4, F=192, S=1,
                             select_bias=True, zipf_s=1.2)),
    # large-tile plain passes (>= 512 rows per expert: 256-row tiles)
    ("large_tiles", MoEShape("bwd_large", T=1100, d=512, N=4, k=2, F=384)),
    # decode-sized: 32-row tiles, most experts with a handful of rows
    ("decode", MoEShape("bwd_decode", T=24, d=256, N=8, k=2, F=640)),
    # experts no token chose: their weight gradients are exactly zero
    ("unused_experts", MoEShape("bwd_unused", T=6, d=128, N=32, k=1, F=128)),
    ("fp32", MoEShape("bwd_f32", T=96, d=128, N=4, k=2, F=256, S=1, dtype="f32")),
    # few rows per weight matrix (128 per expert): D and dXp read the weights
    # as K-rows on the large-tile kernel; dXp's 768-long reduction takes 6
    # buffers from W_gate, then 6 from W_up; D's 384 columns end in a part tile
    ("kmajor_rows", MoEShape("bwd_krows", T=512, d=512, N=16, k=4, F=384, S=1)),
    # the same on 256-row tiles (~256 rows per expert, groups under 384 rows
    # on average with the shared expert): the ping-pong kernel's K-row mode.
    # dXp's 640-long reduction takes 5 buffers from W_gate, then 5 from W_up;
    # D (320 columns) and dXp (640) both end in a part column tile
    ("kmajor_rows_256", MoEShape("bwd_krows256", T=1024, d=640, N=8, k=2, F=320, S=1)),
    # DeepSeek-V3's routing structure: 256 experts, top-8, shared expert and
    # selection bias (257 segments, most a few rows long or empty)
    ("many_experts", MoEShape("bwd_many", T=100, d=128, N=256, k=8, F=128, S=1,
                              select_bias=True)),
]


@pytest.mark.parametrize("label,shape", BACKWARD_CASES, ids=[c[0] for c in BACKWARD_CASES])
def test_backward_parity(label, shape):
    g, ref = check_backward(shape, seed=5, label=label)
    if label == "unused_experts":
        used = np.unique(ref["idx"])
        unused = np.setdiff1d(np.arange(shape.N), used)
        assert unused.size > 0
        for n in ("dw_gate", "dw_up", "dw_down"):
            assert np.all(to_np(g[n])[unused] == 0.0), f"{n} of an unused expert"


def test_backward_capacity():
    shape = MoEShape("bwd_capacity", T=256, d=128, N=4, k=2, F=192)
    check_backward(shape, seed=9, capacity=100, label="capacity 100 of ~128 per expert")


def test_backward_deterministic():
    shape = MoEShape("bwd_det", T=300, d=256, N=8, k=2, F=320, S=1)
    inputs = make_inputs(shape, seed=2, device="cuda", weight_std=0.05)
    dy = draw_dy(shape, 2)
    a = run_backward(shape, inputs, dy)
    b = run_backward(shape, inputs, dy)
    for n, v in a.items():
        if v is not None:
            assert torch.equal(v, b[n]), f"{n} differs between two identical calls"


def test_backward_empty_batch_zero_gradients():
    shape = MoEShape("bwd_empty", T=0, d=128, N=4, k=2, F=128, S=1)
    inputs = make_inputs(MoEShape("bwd_w", T=1, d=128, N=4, k=2, F=128, S=1), seed=1,
                         device="cuda")
    inputs["x"] = inputs["x"][:0]
    dy = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    g = run_backward(shape, inputs, dy)
    for n, v in g.items():
        if v is not None and v.numel():
            assert bool((v == 0).all()), f"{n} not zero for an empty batch"


@pytest.mark.parametrize("N", [1, 8, 256, 512])
def test_select_bias_update_exact(N):
    rng = np.random.default_rng(N)
    counts = rng.integers(0, 50, size=N).astype(np.int32)
    if N > 1:
        counts[0] = int(round(counts.mean()))  # may sit exactly on the mean
        counts[-1] = counts.sum() // N if counts.sum() % N == 0 else counts[-1]
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
    rate = np.float32(1e-3)
    exp = oracle.update_select_bias(bias, counts, float(rate))
    b = torch.from_numpy(bias.copy()).cuda()
    moe.moe_update_select_bias(torch.from_numpy(counts).cuda(), float(rate), b)
    torch.cuda.synchronize()
    got = b.cpu().numpy()
    assert np.array_equal(got, exp), f"max diff {np.max(np.abs(got - exp))}"


def test_backward_full_size_mixtral_prefill():
    """The bench's backward workload at full size (T = 4096, d = 4096, 8 experts,
    top-2, d_ff = 14336, bf16), every gradient element against the oracle's
    float64 backward (about 9 TFLOP of NumPy on the host, ~10-30 s)."""
    import time
    from workloads import CONFIGS
    t0 = time.time()
    shape = CONFIGS["mixtral_prefill"]
    inputs = make_inputs(shape, seed=0, device="cuda")
    dy = draw_dy(shape, 0)
    fwd = forward_routing(shape, inputs)
    say(f"[bwd-full] {shape.describe()}: forward done {time.time() - t0:.1f}s")
    check_routing(shape, {}, fwd)
    g = run_backward(shape, inputs, dy)
    say(f"[bwd-full] backward done {time.time() - t0:.1f}s")
    host = {n: inputs[n].float().cpu().numpy().astype(np.float64)
            for n in ("x", "w_router", "w_gate", "w_up", "w_down")}
    ref = oracle.moe_backward(host["x"], host["w_router"],
                              (host["w_gate"], host["w_up"], host["w_down"]), shape.k,
                              dy.float().cpu().numpy().astype(np.float64), alpha=ALPHA,
                              aux_grad=AUX_GRAD, route_idx=fwd["topk_idx"])
    del host
    say(f"[bwd-full] oracle done {time.time() - t0:.1f}s")
    for n in GRADS:
        got = g[n].float().cpu().numpy()
        exp = ref[n]
        assert np.all(np.isfinite(got)), f"{n}: non-finite values"
        scale = float(np.max(np.abs(exp)))
        err = float(np.max(np.abs(got - exp)))
        say(f"[bwd-full]   {n:12s} max|ref| {scale:.3e} max|err| {err:.3e} ({err / scale:.2e})")
        assert err <= 2.0 ** -6 * scale, f"{n}: error {err} > 2^-6 * {scale}"
        del got
