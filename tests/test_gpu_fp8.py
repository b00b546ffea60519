"""GPU parity of FP8 (OCP E4M3) expert weights with per-output-channel scales
against the oracle's decode (O9).  Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_router_amd as moe
from gpu_harness import full_parity, full_size_parity, run_layer, say, to_np
from workloads import CONFIGS, MoEShape, make_inputs, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()  # the HIP library must be built; no fallback


def test_every_finite_code_decodes_exactly():
    """One expert, x = identity rows, gate codes all 1.0, down = identity on
    the first F channels: y[t, n] = SiLU(1) * decode(up[n, t]), so every
    finite code reaches the output through its own element."""
    T = d = 256
    F = 64
    shp = MoEShape("fp8_codes", T=T, d=d, N=1, k=1, F=F, fp8=True)
    inputs = make_inputs(shp, seed=3, device="cuda")
    one = 0x38  # E4M3 1.0
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    reps = math.ceil(F * d / len(codes))
    up = torch.tensor((codes * reps)[:F * d], dtype=torch.uint8).reshape(1, F, d)
    down = torch.zeros((1, d, F), dtype=torch.uint8)
    down[0, torch.arange(F), torch.arange(F)] = one
    inputs.update({
        "x": torch.eye(T, d, dtype=torch.bfloat16, device="cuda"),
        "w_gate": torch.full((1, F, d), one, dtype=torch.uint8, device="cuda"),
        "w_up": up.cuda(), "w_down": down.cuda(),
        "w_gate_scale": torch.ones((1, F), device="cuda"),
        "w_up_scale": torch.ones((1, F), device="cuda"),
        "w_down_scale": torch.ones((1, d), device="cuda"),
    })
    out = run_layer(shp, inputs)
    y = to_np(out["y"]).astype(np.float64)
    ref = oracle.silu(np.ones(1))[0] * oracle.e4m3_decode(up[0].numpy()).T  # [T, F]
    err = np.abs(y[:, :F] - ref)
    bad = err > 2.0 ** -7 * np.abs(ref)
    say(f"[fp8] codes: max rel err {float(np.max(err / np.maximum(np.abs(ref), 1e-30))):.3e}")
    assert not bad.any(), f"{int(bad.sum())} codes decoded wrongly, e.g. " \
        f"{[hex(int(up[0, n, t])) for t, n in zip(*np.nonzero(bad))][:8]}"
    assert np.all(y[:, F:] == 0.0)


FP8_CASES = [
    # few rows per expert: 32-row tiles, down pass split over K (39 steps)
    ("decode_split_k", reduced(CONFIGS["mixtral_decode_fp8"], T=24, d=256, F=2496)),
    # prefill rows: 128-row register-staged tiles, ragged T and F
    ("prefill", reduced(CONFIGS["mixtral_decode_fp8"], T=300, d=512, F=1088,
                        name="fp8_prefill")),
    # shared expert and selection bias
    ("shared_and_bias", MoEShape("fp8_ds", T=200, d=512, N=64, k=8, F=256, S=1,
                                 select_bias=True, fp8=True)),
    # large-tile kernel: 128-row tiles with a shared expert, 256-row tiles
    ("large_tiles_shared", MoEShape("fp8_l128", T=600, d=512, N=8, k=2, F=512, S=1, fp8=True)),
    ("large_tiles_256", MoEShape("fp8_l256", T=1100, d=512, N=4, k=2, F=1024, fp8=True)),
]


@pytest.mark.parametrize("label,shape", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_parity(label, shape):
    full_parity(shape, seed=4, label=f"fp8_{label}")


# Narrow tail tiles with FP8 weights: 257 rows per expert (1-row tails), and
# ~300 rows per expert (assorted tails on both passes, a shared expert's
# 5-tile group beside them).
FP8_NARROW_CASES = [
    ("one_row_tails", MoEShape("fp8_nar1", T=257, d=512, N=4, k=4, F=512, fp8=True)),
    ("assorted_tails_shared", MoEShape("fp8_nar", T=1200, d=512, N=8, k=2, F=512, S=1,
                                       fp8=True)),
]


@pytest.mark.parametrize("label,shape", FP8_NARROW_CASES, ids=[c[0] for c in FP8_NARROW_CASES])
def test_fp8_narrow_tail_tiles(label, shape):
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S,
                          weight_format=moe.MOE_WEIGHTS_FP8_E4M3)
    info = moe.moe_forward_plan(cfg)
    assert (info["up_kernel"], info["up_tile_rows"]) == (1, 256)
    assert (info["up_narrow_tails"], info["down_narrow_tails"]) == (1, 1)
    _, out, _ = full_parity(shape, seed=4, label=f"fp8_{label}")
    tails = [int(c) % 256 for c in to_np(out["counts"]) if int(c) > 0]
    say(f"[fp8 narrow] {label}: last-tile rows {tails}")
    assert any(0 < t <= 64 for t in tails), "no narrow tail in this case"


@pytest.mark.parametrize("S", [0, 1])
def test_fp8_tail_tiles_split_over_k(S):
    """The large-tile down pass's tail split with FP8 weights: every token on
    expert 7, 20 (40) row tiles of 256, the last 4 (8) split in 2 pieces
    (on 256 compute units) whose fp32 partial sums are scaled per piece."""
    shp = MoEShape("fp8_tail", T=5000, d=4096, N=8, k=1, F=1024, S=S, fp8=True)
    inputs = make_inputs(shp, seed=8, device="cuda")
    inputs["logit_bias"] = torch.tensor([0.0] * 7 + [100.0], device="cuda")
    _, out, _ = full_parity(shp, inputs=inputs, label=f"fp8_tail_split_S{S}")
    assert int(out["counts"][7]) == 5000
    pieces, _, _, tail = to_np(out["split_plan"]).tolist()
    assert pieces >= 2 and tail >= 1, "the tail split was not taken"
    cfg = moe.make_config(5000, 4096, 8, 1, 1024, S,
                          weight_format=moe.MOE_WEIGHTS_FP8_E4M3)
    if moe.moe_forward_plan(cfg)["compute_units"] == 256:
        assert (pieces, tail) == ((2, 4) if S == 0 else (2, 8))


@pytest.mark.parametrize("shape,capacity", [
    (MoEShape("fp8_part256", T=1100, d=512, N=4, k=2, F=1024, fp8=True), 264),
    (MoEShape("fp8_part128", T=1000, d=512, N=4, k=2, F=512, fp8=True), 280),
], ids=["bm256_C264", "bm128_C280"])
def test_fp8_partial_last_tiles(shape, capacity):
    _, out, _ = full_parity(shape, seed=11, label=f"fp8_partial_C{capacity}", capacity=capacity)
    assert np.all(to_np(out["counts"]) >= capacity)


def test_fp8_capacity():
    shp = MoEShape("fp8_cap", T=300, d=256, N=8, k=2, F=512, fp8=True)
    _, out, ref = full_parity(shp, seed=5, label="fp8_capacity_60", capacity=60)
    assert int(np.sum(~ref["keep"])) > 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_decode_fp8", "mixtral_prefill_fp8", "deepseek_v3_fp8"])
def test_fp8_full_size_every_element(name):
    full_size_parity(CONFIGS[name], seed=0)
