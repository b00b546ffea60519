"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each case rewrites one fragment of the oracle's source (a dropped term, a wrong
sign, a wrong index, a transposed operand, a wrong normalisation), loads the
result as a separate module and checks that at least one pin fails on it.
"""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "moe_oracle.py")

MUTATIONS = {
    "ties_to_higher_index": (
        "lower = np.tri(N, N, -1, dtype=bool)", "lower = np.tri(N, N, -1, dtype=bool).T"),
    "keeps_smallest": ("beats = (other > mine)", "beats = (other < mine)"),
    "gates_not_renormalised": (
        "    return z / z.sum(axis=1, keepdims=True)\n\n\ndef full_softmax",
        "    return z / np.exp(r - kept.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)"
        "\n\n\ndef full_softmax"),
    "silu_sign": ("return a / (1.0 + np.exp(-a))", "return a / (1.0 + np.exp(a))"),
    "silu_on_up": ("h = silu(a) * b", "h = a * silu(b)"),
    "down_transposed": ("return h @ _f64(w_down).T", "return h @ _f64(w_down)"),
    "gates_from_biased_keys": ("return idx, kept_softmax(r32, idx)",
                               "return idx, kept_softmax(keys, idx)"),
    "f_divided_by_T": ("f = counts.astype(np.float64) / float(T * k)",
                       "f = counts.astype(np.float64) / float(T)"),
    "P_from_hard_choice": ("P = full_softmax(r32).mean(axis=0)",
                           "P = f.copy()"),
    "loss_without_N": ("raw = float(f.shape[0]) * float(np.sum(f * P))",
                       "raw = float(np.sum(f * P))"),
    "combine_drops_gate": ("y[tok] += g[tok, slot][:, None] * E", "y[tok] += E"),
    "combine_wrong_slot": ("y[tok] += g[tok, slot][:, None] * E",
                           "y[tok] += g[tok, 0][:, None] * E"),
    "shared_dropped": ("y += swiglu_expert(x64, sg[s], su[s], sd[s])", "pass"),
    "logit_offset_dropped": ("r = r + _f64(logit_bias)[None, :]", "r = r"),
    "combine_drops_term": ("    for j in range(g.shape[0]):", "    for j in range(g.shape[0] - 1):"),
    "capacity_keeps_last": ("keep[tok[capacity:], slot[capacity:]] = False",
                            "keep[tok[:-capacity], slot[:-capacity]] = False"),
    "capacity_off_by_one": ("keep[tok[capacity:], slot[capacity:]] = False",
                            "keep[tok[capacity + 1:], slot[capacity + 1:]] = False"),
    "capacity_ignored_in_layer": ("tok, slot = np.nonzero((idx == e) & keep)",
                                  "tok, slot = np.nonzero(idx == e)"),
    "e4m3_bias_8": ("np.ldexp(1.0 + m / 8.0, e - 7))", "np.ldexp(1.0 + m / 8.0, e - 8))"),
    "e4m3_subnormal_as_normal": ("mag = np.where(e == 0, np.ldexp(m / 8.0, -6),",
                                 "mag = np.where(e < 0, np.ldexp(m / 8.0, -6),"),
    "e4m3_no_nan": ("mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)", "pass"),
    "scale_on_input_channel": ("return e4m3_decode(codes) * _f64(scale)[..., :, None]",
                               "return e4m3_decode(codes) * _f64(scale)[..., None, :]"),
    "bwd_silu_derivative": ("da = dh * b * (s + a * s * (1.0 - s))", "da = dh * b * s"),
    "bwd_gate_not_applied": ("wd_all[e],\n                                                  gate * dy[tok])",
                             "wd_all[e],\n                                                  dy[tok])"),
    "bwd_gate_gradient_wrong": ("dgate[tok, slot] = np.sum(dy[tok] * out, axis=1)",
                                "dgate[tok, slot] = np.sum(dy[tok], axis=1)"),
    "bwd_softmax_not_centred": ("dz = g * (dgate - np.sum(g * dgate, axis=1, keepdims=True))",
                                "dz = g * dgate"),
    "bwd_balance_sign": ("dr += p * (c[None, :] - np.sum(p * c[None, :], axis=1, keepdims=True))",
                         "dr -= p * (c[None, :] - np.sum(p * c[None, :], axis=1, keepdims=True))"),
    "bwd_balance_not_over_T": ("c = aux_grad * alpha * N * f / T", "c = aux_grad * alpha * N * f"),
    "bwd_router_term_missing": ("    dx += dr @ wr\n", "    pass\n"),
    "bwd_shared_dx_dropped": ("            dx += dX\n            ds[0][s_] += dWg",
                              "            ds[0][s_] += dWg"),
    "bwd_capacity_ignored": ("tok, slot = np.nonzero(keep & (idx == e))",
                             "tok, slot = np.nonzero(idx == e)"),
    "bwd_down_grad_transposed": ("return da @ wg + db @ wu, da.T @ X, db.T @ X, dout.T @ h, out",
                                 "return da @ wg + db @ wu, da.T @ X, db.T @ X, (h.T @ dout).T[::-1], out"),
    "bias_update_sign": ("step = np.sign(mean - c)", "step = np.sign(c - mean)"),
    "keys_compared_in_fp64": [
        ("return (r32 + b32[None, :]).astype(np.float32)",
         "return r32.astype(np.float64) + b32.astype(np.float64)[None, :]"),
        ("    keys = np.asarray(keys, dtype=np.float32)\n    T, N = keys.shape",
         "    keys = np.asarray(keys, dtype=np.float64)\n    T, N = keys.shape"),
    ],
}


def _mutant(name):
    edits = MUTATIONS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    with open(SRC) as fh:
        src = fh.read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation {name}: fragment not found exactly once"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # a pin may fail by assertion or by a shape error
            failures.append(f"{pin.__name__}: {type(exc).__name__}")
    assert failures, f"planted mistake {name} passed every pin"
