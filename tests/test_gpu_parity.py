"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Element-wise on shapes the oracle finishes in seconds (several tiles, ragged
tails, every routing variant), and on sampled tokens at the full workload
sizes in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_router_amd as moe
from gpu_harness import full_parity, full_size_parity, run_layer, say, to_np
from workloads import CONFIGS, MoEShape, make_inputs, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()  # the HIP library must be built; no fallback


def test_tiny_f32_config():
    full_parity(CONFIGS["tiny_f32"], seed=0)


def test_deterministic_bitwise():
    shp = reduced(CONFIGS["deepseek_v3"], T=130, d=256, F=256, N=32)
    inputs = make_inputs(shp, seed=5, device="cuda")
    a = run_layer(shp, inputs)
    b = run_layer(shp, inputs)
    for key in a:
        assert torch.equal(a[key], b[key]), key


REDUCED = [
    ("mixtral_like", reduced(CONFIGS["mixtral_prefill"], T=300, d=512, F=1024)),
    ("decode_like", reduced(CONFIGS["mixtral_decode"], T=32, d=512, F=1024)),
    ("deepseek_like", reduced(CONFIGS["deepseek_v3"], T=200, d=512, F=256, N=64)),
    ("qwen_like_ntail", reduced(CONFIGS["qwen3_skew"], T=333, d=256, F=192, N=128)),
    ("max_experts_topk", MoEShape("max_experts", T=100, d=128, N=512, k=16, F=128)),
    ("single_expert", MoEShape("single", T=70, d=128, N=1, k=1, F=64)),
    ("f32_ragged", MoEShape("f32_ragged", T=77, d=192, N=6, k=3, F=320, dtype="f32")),
    ("f32_shared_bias", MoEShape("f32_sb", T=65, d=128, N=8, k=2, F=128, S=2, dtype="f32",
                                 select_bias=True)),
    ("one_token", reduced(CONFIGS["deepseek_v3"], T=1, d=256, F=128, N=16)),
    ("bf16_k_equals_n", MoEShape("dense", T=40, d=128, N=4, k=4, F=128)),
    # few rows per expert and a long reduction: the down pass splits its K
    # steps over workgroups (39 steps -> 20 + 19; 50 steps -> 17 + 17 + 16)
    ("decode_split_k", reduced(CONFIGS["mixtral_decode"], T=24, d=256, F=2496)),
    ("f32_split_k_shared", MoEShape("f32_split", T=9, d=128, N=4, k=2, F=1600, S=1,
                                    dtype="f32")),
]


@pytest.mark.parametrize("label,shape", REDUCED, ids=[r[0] for r in REDUCED])
def test_reduced_parity(label, shape):
    full_parity(shape, seed=1, label=label)


def test_empty_batch_is_noop():
    shp = MoEShape("empty", T=0, d=128, N=4, k=2, F=128)
    cfg = moe.make_config(0, 128, 4, 2, 128)
    inputs = make_inputs(MoEShape("w", T=1, d=128, N=4, k=2, F=128), device="cuda")
    y = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward(cfg, inputs["x"][:0], inputs, y, workspace=torch.empty(
        256, dtype=torch.uint8, device="cuda"))
    f = torch.full((4,), 7.0, device="cuda")
    P = torch.full((4,), 7.0, device="cuda")
    aux = torch.full((2,), 7.0, device="cuda")
    moe.moe_balance_stats(0, 4, 2, torch.zeros(4, dtype=torch.int32, device="cuda"),
                          torch.zeros(4, device="cuda"), 0.01, f, P, aux)
    torch.cuda.synchronize()
    assert float(f.abs().sum() + P.abs().sum() + aux.abs().sum()) == 0.0
    del shp


def test_all_tokens_one_expert():
    shp = MoEShape("hot", T=300, d=256, N=4, k=1, F=256)
    inputs = make_inputs(shp, seed=2, device="cuda")
    inputs["logit_bias"] = torch.tensor([0.0, 0.0, 0.0, 100.0], device="cuda")
    _, out, _ = full_parity(shp, inputs=inputs, label="all_to_expert_3")
    assert to_np(out["counts"]).tolist() == [0, 0, 0, 300]


# (label, T, F, {S: (pieces, split row tiles)} on 256 compute units): every
# token goes to expert 7, so the down pass (256-row tiles, 16 column tiles of
# 256) has ceil(T / 256) row tiles, twice that with S = 1, i.e. W = 16 x tiles
# workgroups.  The last round holds r = W mod 256 of them; the scan splits the
# last ceil(r / 16) row tiles over their reduction into min(256 / (16 x those
# tiles), the most pieces the reduction allows) pieces, each at least 8 pairs
# of K steps:
#  base  : T = 5000, 20 (40) row tiles: r = 64 (128), the last 4 (8) row tiles
#          split in 2 pieces (d_ff = 1024: 16 pairs of K steps, 8 + 8).
#  odd_k : the same with d_ff = 1152, 18 pairs split 10 + 8.
#  long  : T = 4200, d_ff = 4096, 17 (34) row tiles: r = 16 (32), the last 1
#          (2) row tiles split in 8 pieces of 8 pairs.
# The combine adds the fp32 pieces.
TAIL_SPLIT_CASES = [("base", 5000, 1024, {0: (2, 4), 1: (2, 8)}),
                    ("odd_k", 5000, 1152, {0: (2, 4), 1: (2, 8)}),
                    ("long", 4200, 4096, {0: (8, 1), 1: (8, 2)})]


@pytest.mark.parametrize("S", [0, 1])
@pytest.mark.parametrize("label,T,F,plan", TAIL_SPLIT_CASES, ids=[c[0] for c in TAIL_SPLIT_CASES])
def test_tail_tiles_split_over_k(label, T, F, plan, S):
    """Last-round tail split of the large-tile down GEMM, and that the scan
    actually took it."""
    shp = MoEShape("tail", T=T, d=4096, N=8, k=1, F=F, S=S)
    cfg = moe.make_config(T, 4096, 8, 1, F, S)
    info = moe.moe_forward_plan(cfg)
    assert info["down_kernel"] == 1 and info["down_tile_rows"] == 256
    inputs = make_inputs(shp, seed=8, device="cuda")
    inputs["logit_bias"] = torch.tensor([0.0] * 7 + [100.0], device="cuda")
    _, out, _ = full_parity(shp, inputs=inputs, label=f"tail_split_{label}_S{S}")
    assert int(out["counts"][7]) == T
    pieces, first_row, stride, tail = to_np(out["split_plan"]).tolist()
    say(f"[tail] {label} S={S}: {pieces} pieces over the last {tail} row tiles from row "
        f"{first_row} ({info['compute_units']} CUs)")
    assert pieces >= 2 and tail >= 1, "the tail split was not taken"
    assert stride == tail * 256
    if info["compute_units"] == 256:
        assert (pieces, tail) == plan[S]


CAPACITY_CASES = [
    # (label, shape, capacity): mean rows per expert vs the cap
    ("large_tiles", reduced(CONFIGS["mixtral_prefill"], T=300, d=512, F=1024), 60),
    ("shared_and_bias", reduced(CONFIGS["deepseek_v3"], T=200, d=512, F=256, N=64), 20),
    ("decode_split_k", reduced(CONFIGS["mixtral_decode"], T=24, d=256, F=2496), 3),
    ("f32", MoEShape("f32_cap", T=77, d=192, N=6, k=3, F=320, dtype="f32"), 25),
]


@pytest.mark.parametrize("label,shape,capacity", CAPACITY_CASES,
                         ids=[c[0] for c in CAPACITY_CASES])
def test_capacity_parity(label, shape, capacity):
    """Expert capacity: the first C assignments per expert in token order are
    kept, the rest dropped (oracle O8); shared experts are untouched."""
    _, out, ref = full_parity(shape, seed=3, label=f"capacity_{label}", capacity=capacity)
    assert int(np.sum(~ref["keep"])) > 0, "the case should drop something"
    # routing statistics describe the router's choice before dropping
    assert to_np(out["counts"]).sum() == shape.T * shape.k


# Exact row counts per expert: with every expert's demand above the capacity C,
# each gets exactly C rows, so its last row tile holds C mod BM rows.  The C
# values put the tile's live 16-row blocks per wavefront (the large-tile
# kernel skips the MFMAs of empty ones) into every class it distinguishes:
# all, half, a quarter and none of a wavefront's row blocks.  bm256: >= 512
# rows per expert, 256-row tiles; bm128: fewer rows, 128-row tiles; odd_k:
# the same with reductions that are odd multiples of 128.
PARTIAL_TILE_CASES = (
    [("bm256", MoEShape("part256", T=1100, d=512, N=4, k=2, F=1024), c)
     for c in (264, 296, 356, 396, 436)] +
    [("bm128", MoEShape("part128", T=1000, d=512, N=4, k=2, F=512), c)
     for c in (264, 280, 296, 376, 456)] +
    [("odd_k", MoEShape("part_odd", T=600, d=384, N=4, k=2, F=640), c)
     for c in (136, 158, 178, 200, 228)])


@pytest.mark.parametrize("label,shape,capacity", PARTIAL_TILE_CASES,
                         ids=[f"{c[0]}_C{c[2]}" for c in PARTIAL_TILE_CASES])
def test_partial_last_tiles(label, shape, capacity):
    _, out, ref = full_parity(shape, seed=11, label=f"partial_{label}_C{capacity}",
                              capacity=capacity)
    counts = to_np(out["counts"])
    assert np.all(counts >= capacity), "every expert must be capped at exactly C rows"


def test_capacity_drops_extra_tokens_of_a_hot_expert():
    shp = MoEShape("hot_cap", T=300, d=256, N=4, k=1, F=256)
    inputs = make_inputs(shp, seed=2, device="cuda")
    inputs["logit_bias"] = torch.tensor([0.0, 0.0, 0.0, 100.0], device="cuda")
    _, out, _ = full_parity(shp, inputs=inputs, label="hot_expert_capacity_100", capacity=100)
    y = to_np(out["y"])
    assert np.all(y[100:] == 0.0), "tokens past the capacity must get nothing"
    assert np.any(y[:100] != 0.0)


def test_capacity_at_least_every_count_is_a_no_op():
    shp = reduced(CONFIGS["qwen3_skew"], T=200, d=256, F=128, N=32)
    inputs = make_inputs(shp, seed=6, device="cuda")
    free = run_layer(shp, inputs)
    capped = run_layer(shp, inputs, capacity=shp.T)
    for key in free:
        assert torch.equal(free[key], capped[key]), key


def test_unchosen_expert_weights_never_read():
    shp = MoEShape("nan_cold", T=150, d=128, N=6, k=2, F=128)
    inputs = make_inputs(shp, seed=3, device="cuda")
    inputs["logit_bias"] = torch.tensor([0, 0, 0, 0, 0, -1.0e4], dtype=torch.float32,
                                        device="cuda")
    for name in ("w_gate", "w_up", "w_down"):
        inputs[name][5] = float("nan")
    _, out, _ = full_parity(shp, inputs=inputs, label="nan_in_unused_expert")
    assert int(out["counts"][5]) == 0
    assert bool(torch.isfinite(out["y"].float()).all())


ALL_TOKEN_CASES = [
    # (label, shape, capacity): batches of at most 32 tokens where (nearly)
    # every expert is chosen, so every expert runs on every token and the
    # routing runs inside the gate/up launch
    ("n8_k2", reduced(CONFIGS["mixtral_decode"], T=32, d=256, F=512), 0),
    ("n20_k6_shared_bias", MoEShape("at20", T=32, d=192, N=20, k=6, F=256, S=1,
                                    select_bias=True), 0),
    ("n40_k10_zipf", MoEShape("at40", T=30, d=128, N=40, k=10, F=192, zipf_s=1.2), 0),
    ("n64_k16", MoEShape("at64", T=32, d=128, N=64, k=16, F=128), 0),
    ("one_token_k_equals_n", MoEShape("at1", T=1, d=256, N=4, k=4, F=256), 0),
    ("capacity_split_k", reduced(CONFIGS["mixtral_decode"], T=28, d=256, F=2048), 5),
    ("f32_shared", MoEShape("at32", T=17, d=128, N=4, k=2, F=320, S=2, dtype="f32"), 3),
]


@pytest.mark.parametrize("label,shape,capacity", ALL_TOKEN_CASES,
                         ids=[c[0] for c in ALL_TOKEN_CASES])
def test_all_token_pass(label, shape, capacity):
    """The all-token expert pass of small batches: the plan takes it, and y,
    the routing and the statistics match the oracle, capacity drops and the
    down pass's split included."""
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S,
                          shape.torch_dtype, capacity=capacity)
    info = moe.moe_forward_plan(cfg)
    assert info["all_token_pass"] == 1
    _, out, _ = full_parity(shape, seed=6, label=f"all_token_{label}", capacity=capacity)
    pieces = int(out["split_plan"][0])
    say(f"[all-token] {label}: down pass in {max(pieces, 1)} pieces")
    assert pieces == (info["down_split"] if info["down_split"] > 1 else 0)


def test_all_token_pass_never_reads_unchosen_rows():
    """Under the all-token pass an expert no token chose still runs (its
    weights here are NaN), and the combine never reads its rows."""
    shp = MoEShape("at_nan", T=32, d=128, N=6, k=2, F=128)
    cfg = moe.make_config(shp.T, shp.d, shp.N, shp.k, shp.F)
    assert moe.moe_forward_plan(cfg)["all_token_pass"] == 1
    inputs = make_inputs(shp, seed=3, device="cuda")
    inputs["logit_bias"] = torch.tensor([0, 0, 0, 0, 0, -1.0e4], dtype=torch.float32,
                                        device="cuda")
    for name in ("w_gate", "w_up", "w_down"):
        inputs[name][5] = float("nan")
    _, out, _ = full_parity(shp, inputs=inputs, label="all_token_nan_in_unused_expert")
    assert int(out["counts"][5]) == 0
    assert bool(torch.isfinite(out["y"].float()).all())


def test_exact_ties_go_to_lower_index():
    # small integers make every logit an exact integer, so many keys tie exactly;
    # experts 1 and 2 have identical router rows and always tie
    shp = MoEShape("ties", T=256, d=128, N=8, k=3, F=128)
    inputs = make_inputs(shp, seed=4, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    inputs["x"] = torch.randint(-2, 3, (256, 128), generator=g, device="cuda").to(torch.bfloat16)
    wr = torch.randint(-1, 2, (8, 128), generator=g, device="cuda").to(torch.bfloat16)
    wr[2] = wr[1]
    inputs["w_router"] = wr.contiguous()
    _, out, _ = full_parity(shp, inputs=inputs, label="exact_ties")
    lg = to_np(out["logits"])
    assert np.array_equal(lg[:, 1], lg[:, 2])
    idx = to_np(out["topk_idx"])
    both = np.sum(np.any(idx == 1, axis=1) & ~np.any(idx == 2, axis=1))
    only2 = np.sum(np.any(idx == 2, axis=1) & ~np.any(idx == 1, axis=1))
    say(f"[ties] tokens with 1 but not 2: {both}, with 2 but not 1: {only2}")
    assert only2 == 0 and both > 0


def test_route_entry_point_matches_forward():
    shp = reduced(CONFIGS["qwen3_skew"], T=200, d=256, F=128, N=32)
    inputs = make_inputs(shp, seed=6, device="cuda")
    full = run_layer(shp, inputs)
    cfg = moe.make_config(shp.T, shp.d, shp.N, shp.k, shp.F, shp.S)
    ws = moe.alloc_workspace(cfg)
    idx = torch.empty_like(full["topk_idx"])
    gate = torch.empty_like(full["topk_gate"])
    counts = torch.empty_like(full["counts"])
    ps = torch.empty_like(full["prob_sum"])
    lg = torch.empty_like(full["logits"])
    moe.moe_route(cfg, inputs["x"], inputs, topk_idx=idx, topk_gate=gate, workspace=ws,
                  logits=lg, counts=counts, prob_sum=ps)
    torch.cuda.synchronize()
    for a, b in ((idx, full["topk_idx"]), (gate, full["topk_gate"]), (counts, full["counts"]),
                 (ps, full["prob_sum"]), (lg, full["logits"])):
        assert torch.equal(a, b)


# Narrow tail tiles: an expert's last row tile of at most 64 rows runs as one
# tile over two column tiles, next to its expert's full tiles.  k = N gives
# every expert 257 rows (a 256-row tile and a 1-row tail); ~300 rows per
# expert give tails of assorted sizes on both passes; an odd number of down
# column tiles (d = 768) keeps them on the gate/up pass only; a shared expert
# adds a 4-tile group with no narrow tail.
NARROW_CASES = [
    ("one_row_tails", MoEShape("nar_k_eq_n", T=257, d=512, N=4, k=4, F=512), (1, 1)),
    ("assorted_tails", MoEShape("nar_mixed", T=1200, d=512, N=8, k=2, F=512), (1, 1)),
    ("odd_down_cols_shared", MoEShape("nar_odd", T=1200, d=768, N=8, k=2, F=512, S=1,
                                      select_bias=True), (1, 0)),
]


@pytest.mark.parametrize("label,shape,flags", NARROW_CASES, ids=[c[0] for c in NARROW_CASES])
def test_narrow_tail_tiles(label, shape, flags):
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S)
    info = moe.moe_forward_plan(cfg)
    assert (info["up_kernel"], info["up_tile_rows"]) == (1, 256)
    assert (info["up_narrow_tails"], info["down_narrow_tails"]) == flags
    _, out, _ = full_parity(shape, seed=4, label=label)
    counts = to_np(out["counts"])
    tails = [int(c) % 256 for c in counts if int(c) > 0]
    say(f"[narrow] {label}: rows per expert {counts.tolist()}, last-tile rows {tails}")
    assert any(0 < t <= 64 for t in tails), "no narrow tail in this case"


@pytest.mark.parametrize("S,fp8", [(0, False), (1, False), (1, True)],
                         ids=["S0", "S1", "S1_fp8"])
def test_narrow_tails_beside_the_down_pass_tail_split(S, fp8):
    """A down pass with narrow tail items and a last-round split over K:
    expert 14 gets 300 rows (a 256-row tile and a 44-row narrow tail in the
    paired item layout), expert 15 the other 4000 (16 tiles), and the scan
    splits the last row tiles of the list (expert 15's, or the shared
    expert's) over their reduction.  Routing is fixed by one-hot router rows
    and a large entry of x in the chosen expert's column."""
    T, N = 4300, 16
    shp = MoEShape("nar_split", T=T, d=4096, N=N, k=1, F=1024, S=S, fp8=fp8)
    cfg = moe.make_config(T, 4096, N, 1, 1024, S,
                          weight_format=moe.MOE_WEIGHTS_FP8_E4M3 if fp8 else moe.MOE_WEIGHTS_DTYPE)
    info = moe.moe_forward_plan(cfg)
    assert info["down_narrow_tails"] == 1 and info["tail_split_cols"] > 0
    inputs = make_inputs(shp, seed=9, device="cuda")
    x = torch.randn((T, 4096), generator=torch.Generator(device="cuda").manual_seed(9),
                    device="cuda")
    expert = torch.full((T,), 15, dtype=torch.long, device="cuda")
    expert[:300] = 14
    x[torch.arange(T, device="cuda"), expert] = 30.0
    wr = torch.zeros((N, 4096), device="cuda")
    wr[torch.arange(N), torch.arange(N)] = 1.0
    inputs["x"] = x.to(torch.bfloat16)
    inputs["w_router"] = wr.to(torch.bfloat16)
    _, out, _ = full_parity(shp, inputs=inputs, label=f"narrow_split_S{S}{'_fp8' if fp8 else ''}")
    counts = to_np(out["counts"]).tolist()
    assert counts[14] == 300 and counts[15] == T - 300 and sum(counts) == T
    pieces, first_row, stride, tail = to_np(out["split_plan"]).tolist()
    say(f"[narrow+split] S={S} fp8={fp8}: {pieces} pieces over the last {tail} row tiles from row "
        f"{first_row} ({info['compute_units']} CUs)")
    if info["compute_units"] == 256:
        assert pieces >= 2 and tail >= 1, "the tail split was not taken"


# Batches of 2048 or more bf16 tokens and 129-256 experts run the router GEMM
# on the large-tile expert GEMM kernel (256-token tiles, the reduction split
# into parts that the selection kernel adds in order): a ragged last tile,
# an expert count that is no multiple of 16, 4 and 8 parts.
ROUTER_TILE_CASES = [
    ("n128_shared", MoEShape("rt128s", T=2600, d=768, N=128, k=4, F=256, S=1, select_bias=True), 6),
    ("n128", MoEShape("rt128", T=2048, d=512, N=128, k=8, F=256), 4),
    ("ragged_160", MoEShape("rt160", T=2500, d=512, N=160, k=6, F=128, select_bias=True), 4),
    ("full_256_shared", MoEShape("rt256", T=2048, d=1024, N=256, k=8, F=128, S=1,
                                 select_bias=True), 8),
]


@pytest.mark.parametrize("label,shape,parts", ROUTER_TILE_CASES,
                         ids=[c[0] for c in ROUTER_TILE_CASES])
def test_router_gemm_on_the_large_tile_kernel(label, shape, parts):
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S)
    info = moe.moe_forward_plan(cfg)
    assert info["route_kernel"] == 1
    if info["compute_units"] == 256:
        assert info["route_split"] == parts
    full_parity(shape, seed=3, label=label)


@pytest.mark.parametrize("shape", [
    reduced(CONFIGS["mixtral_decode"], T=24, d=256, F=256),
    reduced(CONFIGS["qwen3_skew"], T=1000, d=256, F=128, N=128),
    MoEShape("n512", T=70, d=128, N=512, k=4, F=64),
], ids=["decode", "qwen_skew", "N512"])
def test_balance_outputs_of_the_forward(shape):
    """f, P and aux written by the forward's grouping step are bitwise the
    values moe_balance_stats computes from the same counts and sums, and the
    same again from moe_route."""
    inputs = make_inputs(shape, seed=4, device="cuda")
    out = run_layer(shape, inputs, alpha=0.03)
    cfg = moe.make_config(shape.T, shape.d, shape.N, shape.k, shape.F, shape.S)
    ws = moe.alloc_workspace(cfg)
    N = shape.N
    f, P = (torch.empty(N, device="cuda") for _ in range(2))
    aux = torch.empty(2, device="cuda")
    y = torch.empty_like(inputs["x"])
    moe.moe_layer_forward(cfg, inputs["x"], inputs, y, workspace=ws, f=f, P=P, aux=aux,
                          alpha=0.03)
    torch.cuda.synchronize()
    for a, b in ((f, out["f"]), (P, out["P"]), (aux, out["aux"])):
        assert torch.equal(a, b)
    idx = torch.empty_like(out["topk_idx"])
    gate = torch.empty_like(out["topk_gate"])
    f2, P2 = (torch.empty(N, device="cuda") for _ in range(2))
    aux2 = torch.empty(2, device="cuda")
    moe.moe_route(cfg, inputs["x"], inputs, topk_idx=idx, topk_gate=gate, workspace=ws, f=f2,
                  P=P2, aux=aux2, alpha=0.03)
    torch.cuda.synchronize()
    for a, b in ((f2, out["f"]), (P2, out["P"]), (aux2, out["aux"])):
        assert torch.equal(a, b)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_decode", "mixtral_prefill", "qwen3_skew",
                                  "deepseek_v3"])
def test_full_size_every_element(name):
    out = full_size_parity(CONFIGS[name], seed=0)
    if name == "qwen3_skew":
        counts = to_np(out["counts"])
        say(f"[full] qwen3_skew counts max {counts.max()} min {counts.min()} "
            f"aux_raw {float(out['aux'][0]):.3f}")
        assert counts.max() > 8 * counts.mean()   # the Zipf offset skews the load
    del out
    torch.cuda.empty_cache()
