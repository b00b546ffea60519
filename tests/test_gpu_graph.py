"""The layer forward captured once in a HIP graph and replayed (needs an MI355X).

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
