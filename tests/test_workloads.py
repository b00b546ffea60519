"""Seeded input generation: shapes, dtypes, determinism (CPU)."""
import math

import torch

from workloads import CONFIGS, make_inputs, reduced, zipf_offsets


def test_shapes_and_determinism():
    shp = reduced(CONFIGS["deepseek_v3"], T=20, d=64, F=128, N=16)
    a = make_inputs(shp, seed=3)
    b = make_inputs(shp, seed=3)
    c = make_inputs(shp, seed=4)
    assert a["x"].shape == (20, 64) and a["x"].dtype == torch.bfloat16
    assert a["w_gate"].shape == (16, 128, 64) and a["w_down"].shape == (16, 64, 128)
    assert a["ws_gate"].shape == (1, 128, 64)
    assert a["select_bias"].shape == (16,) and float(a["select_bias"].abs().max()) <= 0.1
    assert a["logit_bias"] is None
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key])
    assert not torch.equal(a["x"], c["x"])


def test_weight_std_and_zipf():
    shp = reduced(CONFIGS["qwen3_skew"], T=8, d=256, F=256, N=8)
    inp = make_inputs(shp, seed=0)
    std = inp["w_gate"].float().std().item()
    assert abs(std - 0.02) < 0.001
    assert torch.allclose(inp["logit_bias"], zipf_offsets(8, 1.2))
    assert inp["logit_bias"][0] == 0.0 and math.isclose(inp["logit_bias"][7].item(),
                                                        -1.2 * math.log(8), rel_tol=1e-6)


def test_fp32_config():
    inp = make_inputs(CONFIGS["tiny_f32"], seed=0)
    assert inp["x"].dtype == torch.float32 and inp["ws_gate"] is None
