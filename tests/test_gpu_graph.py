"""The layer forward and backward captured once in a HIP graph and replayed
(needs an MI355X).

The library allocates, frees and synchronises nothing and launches only on the
caller's stream, so a serving loop may capture a whole step.  Every replay is
checked bit for bit against an eager call on the same inputs, with eager work
and synchronisation between the replays.
"""
import pytest
import torch

import sparse_mixture_experts_router_amd as moe
from gpu_harness import say
from workloads import CONFIGS, make_inputs, reduced

pytestmark = pytest.mark.gpu

CASES = [
    ("large_tiles", reduced(CONFIGS["mixtral_prefill"], T=300, d=512, F=1024)),
    ("decode_split_k", reduced(CONFIGS["mixtral_decode"], T=24, d=256, F=2496)),
    ("shared_and_bias", reduced(CONFIGS["deepseek_v3"], T=200, d=512, F=256, N=64)),
]


@pytest.mark.parametrize("label,shape", CASES, ids=[c[0] for c in CASES])
def test_forward_replays_from_a_graph(label, shape):
    say(f"[graph] {label}: {shape.describe()}")
    inputs = make_inputs(shape, seed=11, device="cuda")
    T, N, k = shape.T, shape.N, shape.k
    cfg = moe.make_config(T, shape.d, N, k, shape.F, shape.S, shape.torch_dtype)
    ws = moe.alloc_workspace(cfg)
    x = inputs["x"].clone()
    outs = {
        "y": torch.empty((T, shape.d), dtype=shape.torch_dtype, device="cuda"),
        "idx": torch.empty((T, k), dtype=torch.int32, device="cuda"),
        "gate": torch.empty((T, k), dtype=torch.float32, device="cuda"),
        "counts": torch.empty(N, dtype=torch.int32, device="cuda"),
        "psum": torch.empty(N, dtype=torch.float32, device="cuda"),
        "f": torch.empty(N, dtype=torch.float32, device="cuda"),
        "P": torch.empty(N, dtype=torch.float32, device="cuda"),
        "aux": torch.empty(2, dtype=torch.float32, device="cuda"),
    }

    def step():
        moe.moe_layer_forward(cfg, x, inputs, outs["y"], workspace=ws, topk_idx=outs["idx"],
                              topk_gate=outs["gate"], counts=outs["counts"],
                              prob_sum=outs["psum"])
        moe.moe_balance_stats(T, N, k, outs["counts"], outs["psum"], 0.01, outs["f"],
                              outs["P"], outs["aux"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for rep in range(3):
        x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        graph.replay()
        torch.cuda.synchronize()
        got = {key: t.clone() for key, t in outs.items()}
        for t in outs.values():
            t.fill_(0)
        step()
        torch.cuda.synchronize()
        for key, t in outs.items():
            assert torch.equal(got[key], t), f"replay {rep}: {key} differs from the eager call"
        say(f"[graph] {label}: replay {rep} matches the eager call")


BACKWARD_CASES = [
    ("large_tiles", reduced(CONFIGS["mixtral_prefill"], T=300, d=512, F=1024)),
    ("shared_and_bias", reduced(CONFIGS["deepseek_v3"], T=200, d=512, F=256, N=64)),
]


@pytest.mark.parametrize("label,shape", BACKWARD_CASES, ids=[c[0] for c in BACKWARD_CASES])
def test_backward_replays_from_a_graph(label, shape):
    """The backward captured once and replayed with new x and dy each time,
    every gradient bit for bit against an eager call."""
    say(f"[graph-bwd] {label}: {shape.describe()}")
    inputs = make_inputs(shape, seed=13, device="cuda")
    T, d, N, k, F, S = shape.T, shape.d, shape.N, shape.k, shape.F, shape.S
    dt = shape.torch_dtype
    cfg = moe.make_config(T, d, N, k, F, S, dt)
    ws = moe.alloc_backward_workspace(cfg)
    x = inputs["x"].clone()
    dy = torch.zeros((T, d), dtype=dt, device="cuda")
    g = {"dx": torch.empty((T, d), dtype=dt, device="cuda"),
         "dw_router": torch.empty((N, d), dtype=dt, device="cuda"),
         "dlogit_bias": torch.empty(N, dtype=torch.float32, device="cuda"),
         "dw_gate": torch.empty((N, F, d), dtype=dt, device="cuda"),
         "dw_up": torch.empty((N, F, d), dtype=dt, device="cuda"),
         "dw_down": torch.empty((N, d, F), dtype=dt, device="cuda")}
    if S:
        g.update(dws_gate=torch.empty((S, F, d), dtype=dt, device="cuda"),
                 dws_up=torch.empty((S, F, d), dtype=dt, device="cuda"),
                 dws_down=torch.empty((S, d, F), dtype=dt, device="cuda"))

    def step():
        moe.moe_layer_backward(cfg, x, inputs, dy, g, workspace=ws, alpha=0.05, aux_grad=2.0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for rep in range(3):
        x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(dt))
        dy.copy_(torch.randn(dy.shape, generator=gen, device="cuda").to(dt))
        graph.replay()
        torch.cuda.synchronize()
        got = {key: t.clone() for key, t in g.items()}
        for t in g.values():
            t.fill_(0)
        step()
        torch.cuda.synchronize()
        for key, t in g.items():
            assert torch.equal(got[key], t), f"replay {rep}: {key} differs from the eager call"
        say(f"[graph-bwd] {label}: replay {rep} matches the eager call")
