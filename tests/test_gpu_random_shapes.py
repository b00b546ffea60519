"""Seeded random layer shapes inside the supported envelope (needs an MI355X):
the forward element by element against the oracle (full_parity), and for some
of them the backward (check_backward).  The shapes mix ragged T, d and F that
are multiples of 64 but not of 128 or 256, odd expert counts, k up to 8,
shared experts, capacities that drop, both biases and both dtypes, so that
every GEMM path (32-row decode tiles, register-staged tiles, 128- and
256-row large tiles) meets sizes the hand-picked cases do not; a second set of
small batches takes the all-token decode pass.
"""
import numpy as np
import pytest

import sparse_mixture_experts_router_amd as moe
from gpu_harness import full_parity, say
from test_gpu_backward import check_backward
from workloads import MoEShape

pytestmark = pytest.mark.gpu


def _shapes(seed=2024, n=14):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if i % 5 == 4 else "bf16"
        N = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 33, 64]))
        k = int(rng.integers(1, min(N, 8) + 1))
        d = int(rng.choice([64, 128, 192, 320, 512]))
        F = int(rng.choice([64, 128, 192, 320, 576]))
        S = int(rng.choice([0, 0, 1, 2]))
        T = int(rng.choice([1, 5, 63, 64, 65, 130, 257, 700, 1100]))
        cap = 0
        if N > 1 and rng.random() < 0.3:
            cap = max(1, int(T * k / N * 0.7))
        shape = MoEShape(f"rand{i}", T=T, d=d, N=N, k=k, F=F, S=S, dtype=dtype,
                         select_bias=bool(rng.random() < 0.4),
                         zipf_s=float(rng.choice([0.0, 0.0, 1.2])))
        out.append((shape, cap))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("shape,cap", SHAPES, ids=[s.name for s, _ in SHAPES])
def test_random_shape_forward(shape, cap):
    full_parity(shape, seed=100 + int(shape.name[4:]), capacity=cap, label=shape.name)


def _all_token_shapes(seed=77, n=10):
    """Small batches (T <= 32, N <= 64) where (nearly) every expert is chosen,
    so the forward runs every expert on every token (the all-token pass)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype = "f32" if len(out) % 4 == 3 else "bf16"
        N = int(rng.choice([2, 3, 5, 8, 12, 17, 24, 40, 64]))
        k = int(rng.integers(1, min(N, 16) + 1))
        T = int(rng.integers(1, 33))
        if N * (1.0 - k / N) ** T > 0.5:  # the plan would take the routed rows
            continue
        d = int(rng.choice([64, 128, 192, 320, 512]))
        F = int(rng.choice([64, 128, 192, 320, 576, 2048]))
        S = int(rng.choice([0, 0, 1, 2]))
        cap = 0
        if rng.random() < 0.3:
            cap = max(1, int(T * k / N * 0.7))
        shape = MoEShape(f"at_rand{len(out)}", T=T, d=d, N=N, k=k, F=F, S=S, dtype=dtype,
                         select_bias=bool(rng.random() < 0.4),
                         zipf_s=float(rng.choice([0.0, 0.0, 1.2])))
        out.append((shape, cap))
    return out


ALL_TOKEN_SHAPES = _all_token_shapes()


@pytest.mark.parametrize("shape,cap", ALL_TOKEN_SHAPES, ids=[s.name for s, _ in ALL_TOKEN_SHAPES])
def test_random_all_token_forward(shape, cap):
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S,
                          shape.torch_dtype, capacity=cap)
    assert moe.moe_forward_plan(cfg)["all_token_pass"] == 1
    full_parity(shape, seed=200 + int(shape.name[7:]), capacity=cap, label=shape.name)


@pytest.mark.parametrize("shape,cap", SHAPES[::2], ids=[s.name for s, _ in SHAPES[::2]])
def test_random_shape_backward(shape, cap):
    say(f"[rand-bwd] {shape.name} capacity={cap}")
    check_backward(shape, seed=3, capacity=cap, label=shape.name)


# A second seeded set, and two batches with several 256-row tiles per expert
# (narrow tail tiles, weight-gradient segments of an odd number of 64-row
# pairs)
SHAPES_B = _shapes(seed=9001, n=24) + [
    (MoEShape("big0", T=2000, d=320, N=8, k=2, F=576, S=1, select_bias=True), 0),
    (MoEShape("big1", T=1500, d=512, N=5, k=2, F=320, S=0), 0),
]


@pytest.mark.parametrize("i", range(len(SHAPES_B)), ids=[f"b_{s.name}" for s, _ in SHAPES_B])
def test_random_shape_forward_second_set(i):
    shape, cap = SHAPES_B[i]
    full_parity(shape, seed=500 + i, capacity=cap, label=f"b_{shape.name}")


@pytest.mark.parametrize("i", [i for i, (s, _) in enumerate(SHAPES_B)
                               if i % 2 == 0 or s.name.startswith("big")],
                         ids=[f"b_{s.name}" for i, (s, _) in enumerate(SHAPES_B)
                              if i % 2 == 0 or s.name.startswith("big")])
def test_random_shape_backward_second_set(i):
    shape, cap = SHAPES_B[i]
    say(f"[rand-bwd] b_{shape.name} capacity={cap}")
    check_backward(shape, seed=7, capacity=cap, label=f"b_{shape.name}")
