"""The no-allocation forward (moe_layer_forward_noalloc) against
moe_layer_forward: the same kernels on a library-owned per-GPU workspace, so
every output must be bitwise the one the workspace-argument entry point gives.
Two calls in a row on one GPU, the second with a smaller batch, on each of the
GEMM paths (large tiles, and register-staged tiles with a split reduction)."""
import pytest
import torch

import sparse_mixture_experts_router_amd as moe
from gpu_harness import full_parity, run_layer, say
from workloads import CONFIGS, MoEShape, make_inputs, reduced

pytestmark = pytest.mark.gpu

OUTPUTS = ("y", "logits", "topk_idx", "topk_gate", "counts", "prob_sum", "f", "P", "aux")


def run_noalloc(shape, inputs):
    T, dev = shape.T, inputs["x"].device
    cfg = moe.make_config(T, shape.d, shape.N, shape.k, shape.F, shape.S, shape.torch_dtype)
    nan = float("nan")
    out = {"y": torch.full((T, shape.d), nan, dtype=shape.torch_dtype, device=dev),
           "logits": torch.full((T, shape.N), nan, device=dev),
           "topk_idx": torch.full((T, shape.k), -1, dtype=torch.int32, device=dev),
           "topk_gate": torch.full((T, shape.k), nan, device=dev),
           "counts": torch.full((shape.N,), -1, dtype=torch.int32, device=dev),
           "prob_sum": torch.full((shape.N,), nan, device=dev),
           "f": torch.full((shape.N,), nan, device=dev),
           "P": torch.full((shape.N,), nan, device=dev),
           "aux": torch.full((2,), nan, device=dev)}
    moe.moe_layer_forward_noalloc(cfg, inputs["x"], inputs, out["y"], logits=out["logits"],
                                  topk_idx=out["topk_idx"], topk_gate=out["topk_gate"],
                                  counts=out["counts"], prob_sum=out["prob_sum"], f=out["f"],
                                  P=out["P"], aux=out["aux"], alpha=0.01)
    torch.cuda.synchronize()
    return out


def reference(shape, inputs):
    """moe_layer_forward (workspace argument) plus the f, P, aux it writes."""
    T, dev = shape.T, inputs["x"].device
    cfg = moe.make_config(T, shape.d, shape.N, shape.k, shape.F, shape.S, shape.torch_dtype)
    ref = run_layer(shape, inputs)
    f, P = torch.empty(shape.N, device=dev), torch.empty(shape.N, device=dev)
    aux = torch.empty(2, device=dev)
    y = torch.empty_like(ref["y"])
    moe.moe_layer_forward(cfg, inputs["x"], inputs, y,
                          workspace=moe.alloc_workspace(cfg, dev), f=f, P=P, aux=aux,
                          alpha=0.01)
    torch.cuda.synchronize()
    ref["f"], ref["P"], ref["aux"] = f, P, aux
    return ref


@pytest.mark.parametrize("big,small", [
    # large-tile GEMMs (256-row tiles), then a smaller batch of the same layer
    (reduced(CONFIGS["mixtral_prefill"], T=600, d=512, F=1024),
     reduced(CONFIGS["mixtral_prefill"], T=200, d=512, F=1024)),
    # the Mixtral-shaped decode layer (register-staged tiles, down pass split
    # over its reduction; the all-token pass), then 8 tokens (routed rows)
    (CONFIGS["mixtral_decode"], reduced(CONFIGS["mixtral_decode"], T=8, d=4096, F=14336)),
    # the all-token pass with a shared expert and a selection bias, then a
    # batch of 12 tokens that takes the routed rows
    (MoEShape("ats24", T=24, d=512, N=16, k=4, F=256, S=1, select_bias=True),
     MoEShape("ats12", T=12, d=512, N=16, k=4, F=256, S=1, select_bias=True)),
    # shared expert and selection bias, 256 experts top-8
    (reduced(CONFIGS["deepseek_v3"], T=160, d=512, F=256),
     reduced(CONFIGS["deepseek_v3"], T=33, d=512, F=256)),
    # 256 experts and 2048+ tokens: the router GEMM on the large-tile kernel
    # (8 parts of the reduction), then a batch on the router kernel
    (reduced(CONFIGS["deepseek_v3"], T=2048, d=512, F=128),
     reduced(CONFIGS["deepseek_v3"], T=300, d=512, F=128)),
], ids=["large_tiles", "decode_split_k", "all_token_shared", "shared_bias", "router_tiles"])
def test_noalloc_matches_forward_on_two_calls(big, small):
    for i, shape in enumerate((big, small)):
        cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S)
        need = moe.moe_workspace_size(cfg)
        assert need <= moe.NOALLOC_SCRATCH_BYTES
        plan = moe.moe_forward_plan(cfg)
        say(f"[noalloc] call {i + 1}: router kernel {plan['route_kernel']}, all-token pass "
            f"{plan['all_token_pass']}")
        inputs = make_inputs(shape, seed=21 + i, device="cuda")
        got = run_noalloc(shape, inputs)
        ref = reference(shape, inputs)
        for key in OUTPUTS:
            assert torch.equal(got[key], ref[key]), f"call {i + 1} ({shape.name}): {key} differs"
        say(f"[noalloc] call {i + 1}: {shape.describe()} ({need} bytes of workspace) bitwise "
            f"equal to moe_layer_forward")
    # and the second (smaller) call against the oracle, to the parity bar
    full_parity(small, seed=22, inputs=inputs, label=f"noalloc_{small.name}")


def test_noalloc_rejects_a_workspace_past_its_array():
    shape = CONFIGS["mixtral_prefill"]
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F)
    assert moe.moe_workspace_size(cfg) > moe.NOALLOC_SCRATCH_BYTES
    small = MoEShape("w", T=shape.T, d=shape.d, N=shape.N, k=shape.k, F=64)
    inputs = make_inputs(small, seed=0, device="cuda")
    inputs["w_gate"] = torch.empty((shape.N, shape.F, shape.d), dtype=torch.bfloat16,
                                   device="cuda")
    inputs["w_up"] = torch.empty_like(inputs["w_gate"])
    inputs["w_down"] = torch.empty((shape.N, shape.d, shape.F), dtype=torch.bfloat16,
                                   device="cuda")
    y = torch.empty((shape.T, shape.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward_noalloc(cfg, inputs["x"], inputs, y)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    assert "MOE_NOALLOC_SCRATCH_BYTES" in str(ei.value)
