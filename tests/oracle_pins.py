"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes the oracle module ``O`` and raises when the
oracle disagrees with: a value printed on the pages (fixtures in
``tests/golden/worked_examples.json``, each carrying its citation), a closed
form, an exhaustive search on tiny inputs, or a library routine that the layer
reduces to in a special case (PyTorch / SciPy, float64, CPU).

The functions are shared by ``test_oracle_pins.py`` (the real oracle must pass
every pin) and ``test_oracle_mutations.py`` (oracles with a planted mistake
must fail at least one pin).
"""

from __future__ import annotations

import itertools
import json
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as Fnn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def _close(a, b, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape or not np.all(np.abs(a - b) <= atol):
        raise AssertionError(f"{what}: got {a.tolist()} expected {b.tolist()} (atol {atol})")


def _half_ulp(dec):
    return 0.5 * 10.0 ** (-dec) + 1e-12


# ----------------------------------------------------------- printed examples
def pin_e1_top2(O):
    ex = golden()["E1_top2_single_token"]
    r = np.array([ex["logits"]], dtype=np.float32)
    idx, g = O.route_from_logits(r, ex["k"])
    want = [e - 1 for e in ex["kept_experts_1based"]]
    if idx[0].tolist() != want:
        raise AssertionError(f"E1 experts {idx[0].tolist()} != {want}")
    _close(g[0], ex["gates"], _half_ulp(ex["decimals"]), "E1 gates")
    p = O.full_softmax(r)[0]
    _close(p[want], ex["softmax_all_for_kept"], _half_ulp(ex["decimals"]), "E1 softmax-all")
    _close(p[want] / p[want].sum(), g[0], 1e-12, "E1 renormalised softmax-all")


def pin_e2_blend(O):
    ex = golden()["E2_blend"]
    y = O.combine(ex["gates"], ex["expert_outputs"])
    _close(y, ex["y"], _half_ulp(ex["decimals"]), "E2 blend (page gates)")
    # the same blend with the exact E1 gates still rounds to the printed row
    e1 = golden()["E1_top2_single_token"]
    _, g = O.route_from_logits(np.array([e1["logits"]], np.float32), e1["k"])
    _close(O.combine(g[0], ex["expert_outputs"]), ex["y"], _half_ulp(ex["decimals"]),
           "E2 blend (exact gates)")


def pin_e3_top2(O):
    ex = golden()["E3_top2_guided_page"]
    r = np.array([ex["logits"]], dtype=np.float32)
    idx, g = O.route_from_logits(r, ex["k"])
    want = [e - 1 for e in ex["kept_experts_1based"]]
    if idx[0].tolist() != want:
        raise AssertionError(f"E3 experts {idx[0].tolist()} != {want}")
    _close(g[0], ex["gates"], _half_ulp(ex["decimals"]), "E3 gates")
    dense = np.zeros(4)
    dense[idx[0]] = g[0]
    _close(dense, ex["final_weights"], _half_ulp(ex["decimals"]), "E3 final weights")


def pin_e4_dense(O):
    ex = golden()["E4_dense_gate"]
    y = O.combine(ex["G"], np.array(ex["E"])[:, None])
    _close(y, [ex["y"]], 1e-12, "E4 dense gate")
    ex = golden()["E4b_dense_softmax"]
    p = O.full_softmax(np.array([ex["logits"]], np.float32))[0]
    _close(p, ex["softmax_printed"], ex["tolerance"], "E4b dense softmax")
    # dense MoE is the k = N special case: gates are the full softmax
    idx, g = O.route_from_logits(np.array([ex["logits"]], np.float32), 4)
    _close(g[0], p[idx[0]], 1e-12, "k = N gates vs full softmax")


def pin_e5_balance(O):
    ex = golden()["E5_balance_loss"]
    for case in ("balanced", "collapsed"):
        c = ex[case]
        raw, aux = O.balance(c["f"], c["P"], ex["alpha_switch"])
        _close(raw, c["loss_over_alpha"], 1e-12, f"E5 {case} loss/alpha")
        _close(aux, ex["alpha_switch"] * c["loss_over_alpha"], 1e-14, f"E5 {case} loss")


def pin_e6_toy_routing(O):
    """Replays the toy layer's random draws with torch's CPU generator.

    Construction order of the toy: eight experts, each a Linear(d, h) then a
    Linear(h, d), then the bias-free router Linear(d, N); then the token batch.
    Only the router weights and the tokens matter for the routing; the expert
    layers are drawn to advance the generator exactly as the toy does.
    """
    ex = golden()["E6_toy_layer"]
    d, h, N, k, T = ex["d_model"], ex["d_hidden"], ex["n_experts"], ex["top_k"], ex["tokens"]
    torch.manual_seed(ex["torch_seed"])
    experts = [(torch.nn.Linear(d, h), torch.nn.Linear(h, d)) for _ in range(N)]
    router = torch.nn.Linear(d, N, bias=False)
    x = torch.randn(T, d)
    total = sum(p.numel() for a, b in experts for p in list(a.parameters()) + list(b.parameters()))
    total += router.weight.numel()
    active = k * sum(p.numel() for p in list(experts[0][0].parameters()) +
                     list(experts[0][1].parameters())) + router.weight.numel()
    if (total, active) != (ex["total_params"], ex["active_params"]):
        raise AssertionError(f"toy parameter counts {(total, active)}")
    r32 = O.router_logits(x.numpy(), router.weight.detach().numpy())
    idx = O.topk_by_rank(O.selection_keys(r32), k)
    hist = np.bincount(idx.reshape(-1), minlength=N).tolist()
    if hist != ex["tokens_per_expert"]:
        raise AssertionError(f"toy tokens per expert {hist} != {ex['tokens_per_expert']}")


# ---------------------------------------------------------- exhaustive search
def _brute_topk(keys_row, k):
    """Top-k of one row by trying every k-subset (higher key wins, ties to lower index)."""
    keys_row = np.asarray(keys_row, dtype=np.float32)
    N = keys_row.shape[0]

    def beats(a, b):
        return keys_row[a] > keys_row[b] or (keys_row[a] == keys_row[b] and a < b)

    hits = [S for S in itertools.combinations(range(N), k)
            if all(beats(a, b) for a in S for b in range(N) if b not in S)]
    assert len(hits) == 1
    members, ordered = list(hits[0]), []
    while members:
        best = members[0]
        for m in members[1:]:
            if beats(m, best):
                best = m
        ordered.append(best)
        members.remove(best)
    return ordered


def pin_topk_brute_force(O):
    rng = np.random.default_rng(1234)
    for trial in range(300):
        N = int(rng.integers(1, 9))
        k = int(rng.integers(1, N + 1))
        mode = trial % 3
        if mode == 0:
            keys = rng.standard_normal(N).astype(np.float32)
        elif mode == 1:   # many exact ties
            keys = rng.integers(-2, 3, N).astype(np.float32)
        else:             # signed zeros compare equal
            keys = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), N)
        got = O.topk_by_rank(keys[None, :], k)[0].tolist()
        want = _brute_topk(keys, k)
        if got != want:
            raise AssertionError(f"top-k {keys.tolist()} k={k}: {got} != {want}")


def pin_select_bias_semantics(O):
    # the bias moves the choice, the gates come from the unbiased logits
    r = np.array([[1.0, 0.9, 0.0]], np.float32)
    idx, g = O.route_from_logits(r, 2, select_bias=np.array([0.0, 0.0, 2.0], np.float32))
    if idx[0].tolist() != [2, 0]:
        raise AssertionError(f"biased selection {idx[0].tolist()}")
    _close(g[0], scipy.special.softmax([0.0, 1.0]), 1e-12, "gates use unbiased logits")
    # the key is one fp32 addition: 1 + 2^-25 rounds to 1, so the tie goes to expert 0
    r = np.array([[1.0, 1.0]], np.float32)
    idx, _ = O.route_from_logits(r, 1, select_bias=np.array([0.0, 2.0 ** -25], np.float32))
    if idx[0].tolist() != [0]:
        raise AssertionError("selection key is not a single fp32 addition")


# ------------------------------------------------------------ library routes
def _torch_swiglu(x, wg, wu, wd):
    x, wg, wu, wd = (torch.as_tensor(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return Fnn.linear(Fnn.silu(Fnn.linear(x, wg)) * Fnn.linear(x, wu), wd).numpy()


def _layer(rng, T, d, F, N, S=0):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((N, d)) * 0.3
    wg = rng.standard_normal((N, F, d)) * 0.2
    wu = rng.standard_normal((N, F, d)) * 0.2
    wd = rng.standard_normal((N, d, F)) * 0.2
    sh = None
    if S:
        sh = (rng.standard_normal((S, F, d)) * 0.2, rng.standard_normal((S, F, d)) * 0.2,
              rng.standard_normal((S, d, F)) * 0.2)
    return x, wr, (wg, wu, wd), sh


def pin_swiglu_closed_form(O):
    # one unit: y = w_d * SiLU(w_g x) * (w_u x); SiLU(2) = 2 * sigmoid(2)
    y = O.swiglu_expert([[1.0]], [[2.0]], [[-1.0]], [[0.5]])
    _close(y, [[-0.5 * 2.0 * scipy.special.expit(2.0)]], 1e-15, "SwiGLU closed form")


def pin_single_expert_is_swiglu(O):
    rng = np.random.default_rng(7)
    x, wr, (wg, wu, wd), _ = _layer(rng, 9, 12, 20, 1)
    out = O.moe_forward(x, wr, (wg, wu, wd), 1)
    _close(out["gates"], np.ones((9, 1)), 0, "N = 1 gates")
    _close(out["y"], _torch_swiglu(x, wg[0], wu[0], wd[0]), 1e-12, "N = 1 layer vs SwiGLU")


def pin_router_linear(O):
    x = np.array([[1.0, 2.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    _close(O.router_logits(x, w), [[1.0, 2.0, 3.0]], 0, "router hand example")
    rng = np.random.default_rng(3)
    x = rng.standard_normal((11, 13))
    w = rng.standard_normal((5, 13))
    lb = rng.standard_normal(5)
    ref = Fnn.linear(torch.as_tensor(x), torch.as_tensor(w)).numpy()
    _close(O.router_logits(x, w), ref.astype(np.float32), 1e-6, "router vs linear")
    _close(O.router_logits(x, w, lb), (ref + lb).astype(np.float32), 1e-6,
           "router with logit offset")


def pin_dense_crosspath(O):
    """Dense formulation: every expert on every token, gate zero outside the top-k."""
    rng = np.random.default_rng(11)
    T, d, F, N, k = 37, 24, 40, 6, 3
    x, wr, (wg, wu, wd), _ = _layer(rng, T, d, F, N)
    out = O.moe_forward(x, wr, (wg, wu, wd), k)
    logits = torch.as_tensor(out["logits"].astype(np.float64))
    top_v, top_i = torch.topk(logits, k, dim=1)
    G = torch.zeros(T, N, dtype=torch.float64).scatter(1, top_i, torch.softmax(top_v, dim=1))
    y = np.zeros((T, d))
    for e in range(N):
        y += G[:, e].numpy()[:, None] * _torch_swiglu(x, wg[e], wu[e], wd[e])
    _close(out["y"], y, 1e-12, "per-expert loop vs dense gate")
    if not np.array_equal(out["idx"], top_i.numpy()):
        raise AssertionError("idx vs torch.topk")


def pin_k_equals_n_is_dense_softmax(O):
    rng = np.random.default_rng(5)
    T, d, F, N = 8, 10, 14, 4
    x, wr, (wg, wu, wd), _ = _layer(rng, T, d, F, N)
    out = O.moe_forward(x, wr, (wg, wu, wd), N)
    p = scipy.special.softmax(out["logits"].astype(np.float64), axis=1)
    y = sum(p[:, e:e + 1] * _torch_swiglu(x, wg[e], wu[e], wd[e]) for e in range(N))
    _close(out["y"], y, 1e-12, "k = N layer vs dense softmax MoE")


def pin_shared_expert(O):
    rng = np.random.default_rng(9)
    x, wr, ex, sh = _layer(rng, 10, 16, 24, 5, S=1)
    with_s = O.moe_forward(x, wr, ex, 2, shared=sh)
    without = O.moe_forward(x, wr, ex, 2)
    _close(with_s["y"] - without["y"], _torch_swiglu(x, sh[0][0], sh[1][0], sh[2][0]), 1e-12,
           "shared expert adds with gate 1")
    for key in ("counts", "f", "P"):
        _close(with_s[key], without[key], 0, f"shared expert leaves {key}")


def pin_relabel_and_chunking(O):
    rng = np.random.default_rng(21)
    T, d, F, N, k = 30, 16, 24, 7, 3
    x, wr, (wg, wu, wd), _ = _layer(rng, T, d, F, N)
    base = O.moe_forward(x, wr, (wg, wu, wd), k)
    perm = rng.permutation(N)
    inv = np.argsort(perm)
    rel = O.moe_forward(x, wr[perm], (wg[perm], wu[perm], wd[perm]), k)
    _close(rel["y"], base["y"], 1e-12, "expert relabelling leaves y")
    if not np.array_equal(perm[rel["idx"]], base["idx"]):
        raise AssertionError("relabelled idx")
    tperm = rng.permutation(T)
    sh = O.moe_forward(x[tperm], wr, (wg, wu, wd), k)
    _close(sh["y"], base["y"][tperm], 1e-12, "token shuffle commutes")
    a = O.moe_forward(x[:11], wr, (wg, wu, wd), k)
    b = O.moe_forward(x[11:], wr, (wg, wu, wd), k)
    _close(np.concatenate([a["y"], b["y"]]), base["y"], 1e-12, "token chunking")


def pin_stats(O):
    idx = np.array([[0, 1], [0, 2]], np.int32)
    r = np.array([[0.0, 0.0, 0.0, 0.0], [np.log(2.0), 0.0, 0.0, 0.0]], np.float32)
    counts, f, P = O.stats(idx, r, 4)
    _close(counts, [2, 1, 1, 0], 0, "counts")
    _close(f, [0.5, 0.25, 0.25, 0.0], 0, "f = counts / (T k)")
    _close(P, [(0.25 + 0.4) / 2, (0.25 + 0.2) / 2, (0.25 + 0.2) / 2, (0.25 + 0.2) / 2],
           1e-7, "P = mean full softmax")


def pin_invariants(O):
    rng = np.random.default_rng(17)
    for (T, N, k) in [(40, 8, 2), (25, 5, 1), (16, 16, 16), (33, 12, 5)]:
        x, wr, ex, _ = _layer(rng, T, 8, 16, N)
        out = O.moe_forward(x, wr, ex, k)
        g = out["gates"]
        _close(g.sum(axis=1), np.ones(T), 1e-12, "gates sum to 1")
        if not (np.all(g > 0) and np.all(g <= 1)):
            raise AssertionError("gates outside (0, 1]")
        if int(out["counts"].sum()) != T * k:
            raise AssertionError("counts do not add to T k")
        _close(out["f"].sum(), 1.0, 1e-12, "sum f")
        _close(out["P"].sum(), 1.0, 1e-12, "sum P")
        p = scipy.special.softmax(out["logits"].astype(np.float64), axis=1).mean(axis=0)
        _close(out["P"], p, 1e-12, "P vs scipy softmax")
        raw, _ = O.balance(np.full(N, 1.0 / N), out["P"])
        _close(raw, 1.0, 1e-12, "uniform f gives loss/alpha = 1")
        if k == 1 and np.allclose(out["P"], out["f"]):
            raise AssertionError("P must come from the full softmax, not the hard choice")
        srt = out["idx"]
        keys = out["logits"]
        kept = np.take_along_axis(keys, srt.astype(np.int64), axis=1)
        if np.any(np.diff(kept, axis=1) > 0):
            raise AssertionError("slots not in descending key order")


def pin_unused_expert_never_read(O):
    rng = np.random.default_rng(23)
    T, d, F, N, k = 12, 8, 16, 6, 2
    x, wr, (wg, wu, wd), _ = _layer(rng, T, d, F, N)
    lb = np.zeros(N)
    lb[5] = -1.0e4                      # expert 5 can never be among the top k
    base = O.moe_forward(x, wr, (wg, wu, wd), k, logit_bias=lb)
    if base["counts"][5] != 0:
        raise AssertionError("setup: expert 5 was chosen")
    wg[5] = np.nan
    wu[5] = np.nan
    wd[5] = np.nan
    out = O.moe_forward(x, wr, (wg, wu, wd), k, logit_bias=lb)
    _close(out["y"], base["y"], 0, "unchosen expert's weights are never read")


def pin_empty_batch(O):
    out = O.moe_forward(np.zeros((0, 8)), np.ones((4, 8)),
                        (np.ones((4, 16, 8)), np.ones((4, 16, 8)), np.ones((4, 8, 16))), 2)
    if out["y"].shape != (0, 8) or out["counts"].sum() != 0 or out["aux_raw"] != 0.0:
        raise AssertionError("T = 0")


def _brute_keep(idx, N, C):
    """Per expert, walk the tokens in order and keep its first C assignments."""
    T, k = idx.shape
    keep = np.ones((T, k), dtype=bool)
    if C <= 0:
        return keep
    seen = [0] * N
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            seen[e] += 1
            if seen[e] > C:
                keep[t, s] = False
    return keep


def pin_capacity_brute_force(O):
    """Expert capacity ("Keeping the experts busy"): the first C assignments per
    expert in token order are kept, by a plain walk over the batch."""
    rng = np.random.default_rng(21)
    for _ in range(200):
        T, N = int(rng.integers(1, 13)), int(rng.integers(1, 6))
        k = int(rng.integers(1, N + 1))
        idx = np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
        C = int(rng.integers(0, 5))
        keep = O.capacity_keep(idx, N, C)
        if not np.array_equal(keep, _brute_keep(idx, N, C)):
            raise AssertionError(f"capacity keep mask differs (T={T} N={N} k={k} C={C})")
        for e in range(N):
            n_e = int(np.sum(idx == e))
            if int(np.sum(keep & (idx == e))) != (min(n_e, C) if C > 0 else n_e):
                raise AssertionError("kept count is not min(count, C)")


def pin_capacity_layer(O):
    """Capacity in the layer: no effect when C covers every count; with k = 1
    and C = 1 each expert runs on the first token that chose it only, and the
    dropped tokens get nothing; routing statistics ignore the capacity."""
    rng = np.random.default_rng(23)
    T, d, F, N = 10, 12, 16, 3
    x, wr, (wg, wu, wd), _ = _layer(rng, T, d, F, N)
    free = O.moe_forward(x, wr, (wg, wu, wd), 2)
    full = O.moe_forward(x, wr, (wg, wu, wd), 2, capacity=T)
    _close(full["y"], free["y"], 0, "capacity >= every count changes nothing")
    one = O.moe_forward(x, wr, (wg, wu, wd), 1, capacity=1)
    idx = one["idx"][:, 0]
    y = np.zeros((T, d))
    for e in range(N):
        ts = np.nonzero(idx == e)[0]
        if ts.size:
            t = int(ts[0])
            y[t] = _torch_swiglu(x[t:t + 1], wg[e], wu[e], wd[e])[0]
    _close(one["y"], y, 1e-12, "k = 1, C = 1: first token per expert only")
    ref = O.moe_forward(x, wr, (wg, wu, wd), 1)
    for key in ("counts", "f", "P"):
        _close(one[key], ref[key], 0, f"{key} independent of capacity")


def pin_e4m3_closed_form(O):
    """O9: E4M3 codes whose values follow from the format's definition alone
    (bias 7, 3 mantissa bits, subnormals at exponent field 0, S.1111.111 NaN,
    no infinities)."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0,
             0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    got = O.e4m3_decode(np.array(list(table), dtype=np.uint8))
    _close(got, list(table.values()), 0, "E4M3 closed-form codes")
    if not np.signbit(O.e4m3_decode(np.array([0x80], dtype=np.uint8))[0]):
        raise AssertionError("0x80 must decode to -0.0")
    nan = O.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))
    if not np.all(np.isnan(nan)):
        raise AssertionError("S.1111.111 must decode to NaN")


def pin_e4m3_library(O):
    """O9: all 256 codes against PyTorch's float8_e4m3fn (the OCP E4M3 type),
    widened to float64; the 127 positive finite codes strictly increase and a
    set sign bit negates."""
    codes = np.arange(256, dtype=np.uint8)
    got = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    if not np.array_equal(np.isnan(got), np.isnan(ref)):
        raise AssertionError("NaN codes differ from float8_e4m3fn")
    fin = ~np.isnan(ref)
    _close(got[fin], ref[fin], 0, "E4M3 against float8_e4m3fn")
    pos = got[:127]
    if not np.all(np.diff(pos) > 0):
        raise AssertionError("positive E4M3 codes must increase")
    _close(got[128:255], -pos, 0, "sign bit negates")


def pin_dequantize_per_output_channel(O):
    """O9: a scale belongs to an output channel: x (Q s)^T = (x Q^T) s over
    the rows n of the [out, in] matrix, for any x; a layer with FP8 weights
    equals the layer with the decoded, scaled weights written out by the
    library decode."""
    rng = np.random.default_rng(31)
    E, n_out, n_in = 2, 6, 8
    codes = rng.integers(0, 0x7F, size=(E, n_out, n_in)).astype(np.uint8)
    codes |= (rng.random((E, n_out, n_in)) < 0.5).astype(np.uint8) << 7
    scale = rng.uniform(0.5, 2.0, size=(E, n_out))
    W = O.dequantize(codes, scale)
    x = rng.standard_normal((5, n_in))
    q = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    for e in range(E):
        _close(x @ W[e].T, (x @ q[e].T) * scale[e][None, :], 1e-12, "scale per output channel")
    T, d, F, N = 7, 8, 6, 2
    xl = rng.standard_normal((T, d))
    wr = rng.standard_normal((N, d))
    cg = rng.integers(0, 0x7F, size=(N, F, d)).astype(np.uint8)
    cu = rng.integers(0, 0x7F, size=(N, F, d)).astype(np.uint8)
    cd = rng.integers(0, 0x7F, size=(N, d, F)).astype(np.uint8)
    sg, su, sd = (rng.uniform(0.01, 0.02, size=s) for s in ((N, F), (N, F), (N, d)))
    dec = lambda c: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()
    ref = O.moe_forward(xl, wr, (dec(cg) * sg[..., None], dec(cu) * su[..., None],
                                 dec(cd) * sd[..., None]), 1)
    got = O.moe_forward(xl, wr, (O.dequantize(cg, sg), O.dequantize(cu, su),
                                 O.dequantize(cd, sd)), 1)
    _close(got["y"], ref["y"], 1e-12, "FP8 layer")


# ------------------------------------------------------------------ backward
def _fd_grad(fun, arrays, h=1e-6):
    """Central differences of the scalar fun(*arrays) w.r.t. every element."""
    grads = []
    for a_i, a in enumerate(arrays):
        g = np.zeros_like(a)
        for pos in np.ndindex(a.shape):
            old = a[pos]
            a[pos] = old + h
            up = fun(*arrays)
            a[pos] = old - h
            dn = fun(*arrays)
            a[pos] = old
            g[pos] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


def pin_backward_finite_differences(O):
    """O10 against central differences of the exact-logit forward: every
    gradient (x, W_r, logit offset, routed and shared expert weights), with a
    selection bias, a shared expert, an aux-loss weight and a capacity."""
    rng = np.random.default_rng(41)
    T, d, F, N, k = 7, 5, 3, 4, 2
    x, wr, (wg, wu, wd), sh = _layer(rng, T, d, F, N, S=1)
    wr = wr * 3.0
    lb = rng.standard_normal(N) * 0.3
    sb = (rng.standard_normal(N) * 0.3).astype(np.float32)
    dy = rng.standard_normal((T, d))
    alpha, aux_grad = 0.3, 2.5
    for cap in (0, 3):
        B = O.moe_backward(x, wr, (wg, wu, wd), k, dy, logit_bias=lb, select_bias=sb,
                           shared=sh, alpha=alpha, aux_grad=aux_grad, capacity=cap)
        if cap and B["keep"].all():
            raise AssertionError("capacity case drops nothing")

        def loss(x_, wr_, lb_, wg_, wu_, wd_, sg_, su_, sd_):
            out = O.moe_forward(x_, wr_, (wg_, wu_, wd_), k, logit_bias=lb_, select_bias=sb,
                                shared=(sg_, su_, sd_), alpha=alpha, capacity=cap,
                                exact_logits=True)
            if not np.array_equal(out["idx"], B["idx"]):
                raise AssertionError("finite-difference step changed the routing")
            return float(np.sum(out["y"] * dy)) + aux_grad * out["aux"]

        arrays = [x.copy(), wr.copy(), lb.copy(), wg.copy(), wu.copy(), wd.copy(),
                  sh[0].copy(), sh[1].copy(), sh[2].copy()]
        fd = _fd_grad(loss, arrays)
        names = ["dx", "dw_router", "dlogit_bias", "dw_gate", "dw_up", "dw_down",
                 "ds_gate", "ds_up", "ds_down"]
        for name, ref in zip(names, fd):
            _close(B[name], ref, 1e-6, f"{name} vs finite differences (capacity {cap})")


def pin_backward_one_expert_is_swiglu_autograd(O):
    """N = 1, k = 1: the layer is a dense SwiGLU with gate 1 and a constant
    balance loss, so the expert gradients are PyTorch autograd's and the
    router gets exactly zero."""
    rng = np.random.default_rng(43)
    x, wr, (wg, wu, wd), _ = _layer(rng, 9, 6, 8, 1)
    dy = rng.standard_normal((9, 6))
    B = O.moe_backward(x, wr, (wg, wu, wd), 1, dy)
    X, Wg, Wu, Wd = (torch.tensor(np.asarray(a, np.float64), requires_grad=True)
                     for a in (x, wg[0], wu[0], wd[0]))
    y = Fnn.linear(Fnn.silu(Fnn.linear(X, Wg)) * Fnn.linear(X, Wu), Wd)
    (y * torch.as_tensor(dy)).sum().backward()
    _close(B["dx"], X.grad.numpy(), 1e-12, "one expert dx vs autograd")
    _close(B["dw_gate"][0], Wg.grad.numpy(), 1e-12, "one expert dW_gate vs autograd")
    _close(B["dw_up"][0], Wu.grad.numpy(), 1e-12, "one expert dW_up vs autograd")
    _close(B["dw_down"][0], Wd.grad.numpy(), 1e-12, "one expert dW_down vs autograd")
    _close(B["dw_router"], np.zeros_like(wr), 0, "one expert router gradient")


def pin_backward_uniform_router_balance(O):
    """W_r = 0 and dy = 0: every logit is 0, the selection takes experts
    0..k-1 (ties to the lower index), p = 1/N, and the only gradient is the
    balance loss's: dr[t, j] = (c_j - mean c) / N with c_j = aux_grad alpha N
    f_j / T, f_j = 1/k for j < k."""
    rng = np.random.default_rng(47)
    T, d, F, N, k = 5, 4, 3, 6, 2
    x, _, (wg, wu, wd), _ = _layer(rng, T, d, F, N)
    wr = np.zeros((N, d))
    alpha, aux_grad = 0.01, 3.0
    B = O.moe_backward(x, wr, (wg, wu, wd), k, np.zeros((T, d)), alpha=alpha,
                       aux_grad=aux_grad)
    f = np.array([1.0 / k] * k + [0.0] * (N - k))
    c = aux_grad * alpha * N * f / T
    dr = np.tile((c - c.mean()) / N, (T, 1))
    _close(B["dlogits"], dr, 1e-15, "balance-loss logit gradient")
    _close(B["dw_router"], dr.T @ x, 1e-14, "router weight gradient")
    _close(B["dx"], np.zeros((T, d)), 0, "dx with W_r = 0 and dy = 0")


def pin_select_bias_update(O):
    """O11 sign cases: above the mean load -> bias - rate, below -> + rate,
    at the mean -> unchanged; one float32 addition (1 + 1e-8 stays 1)."""
    got = O.update_select_bias([0.0, 0.5, -1.0, 1e-8], [10, 2, 6, 6], 0.25)
    exp = np.array([-0.25, 0.75, -1.0, 1e-8], dtype=np.float32)
    if got.dtype != np.float32 or not np.array_equal(got, exp):
        raise AssertionError(f"bias update {got} expected {exp}")
    got = O.update_select_bias([1.0, 1.0], [0, 4], 1e-8)
    if not np.array_equal(got, np.array([1.0, 1.0], np.float32)):
        raise AssertionError("bias update must be a float32 addition")


ALL_PINS = [
    pin_e1_top2, pin_e2_blend, pin_e3_top2, pin_e4_dense, pin_e5_balance, pin_e6_toy_routing,
    pin_topk_brute_force, pin_select_bias_semantics, pin_swiglu_closed_form,
    pin_single_expert_is_swiglu, pin_router_linear, pin_dense_crosspath,
    pin_k_equals_n_is_dense_softmax, pin_shared_expert, pin_relabel_and_chunking, pin_stats,
    pin_invariants, pin_unused_expert_never_read, pin_empty_batch, pin_capacity_brute_force,
    pin_capacity_layer, pin_e4m3_closed_form, pin_e4m3_library, pin_dequantize_per_output_channel,
    pin_backward_finite_differences, pin_backward_one_expert_is_swiglu_autograd,
    pin_backward_uniform_router_balance, pin_select_bias_update,
]
