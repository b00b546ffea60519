"""Plain CPU oracle for the sparse mixture-of-experts layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library; it takes plain NumPy arrays (already decoded to
float32/float64 by the caller) and computes everything in float64 except the
two places where floating point decides an integer (the routing keys), which it
takes in float32 exactly as the pages' method would on fp32 logits.

What it computes, and where the pages define it:

* O1 router scores ``r = x W_r`` -- one linear layer, no bias, one score per
  expert.  "Mixture of experts and speculative decoding", section "Opening the
  hood: the MoE layer precisely" (equation for r) and step 1 of "Following one
  token through an MoE layer"; "MoE inference: the call centre with 256
  specialists ...", section "The bare mechanism" (Router).
* O2 selection keys: the logits plus an optional per-expert bias that only
  influences which experts are picked ("The bare mechanism", auxiliary-loss-free
  routing variant).
* O3 top-k: the k highest keys; ties go to the lower expert index; slot 0 holds
  the highest key ("Opening the hood", TopK; step 2 of "Following one token").
* O4 gates: softmax over the k kept *unbiased* logits, so they sum to one
  ("Opening the hood", g(x) = softmax(r_TopK); "The bare mechanism", Top-k
  selection).
* O5 experts: SwiGLU feed-forward networks, down( SiLU(gate(x)) * up(x) )
  ("The bare mechanism", the dense FFN it replaces), evaluated only on the
  tokens routed to each expert ("A toy MoE layer in PyTorch": an expert no
  token picked never runs).
* O6 combine: y = sum over the kept experts of g_i(x) E_i(x), plus every
  always-on shared expert with weight one ("Opening the hood", equation for y;
  "The bare mechanism", Weighted combination and Shared experts).
* O7 balance statistics: f_i = share of routed (token, slot) assignments that
  went to expert i, P_i = mean over tokens of the router's softmax probability
  for i, loss = alpha * N * sum_i f_i P_i ("Keeping the experts busy", balance
  loss equation; "Mixture of Experts and Guided Decoding", routing-collapse
  passage and its auxiliary-loss equation and worked example).
* O8 expert capacity (optional): an expert accepts at most C of a batch's
  (token, slot) assignments; the extras are dropped ("Keeping the experts
  busy", expert capacity).  The pages do not say which ones; here the first C
  in token order are kept, a dropped assignment contributes nothing to y (the
  token's other gates are not renormalised), and f, counts and P still
  describe the router's choice before dropping.

* O9 FP8 expert weights (optional): the pages size expert weights at one byte
  per parameter in FP8 ("MoE inference: the call centre with 256 specialists
  ...", weight-memory estimate under "Total memory") without defining the
  format.  Here a weight is an OCP FP8 E4M3 code (sign, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 = subnormal; S.1111.111 = NaN; no
  infinities) times a per-output-channel scale, decoded exactly to float64.

* O10 backward (training side): the gradients of L = sum(y * dy) + c * aux
  with respect to x, W_r, the logit offset and every expert weight, for a
  given output gradient dy and aux-loss weight c.  The pages train the router
  through P_i only, f_i coming from a hard choice ("Mixture of Experts and
  Guided Decoding", routing-collapse passage after the auxiliary-loss
  equation); everything else is the chain rule through O1..O8 with the
  selection (O2, O3) and the capacity mask (O8) held fixed, which is the
  derivative wherever no two keys tie.
* O11 selection-bias update (auxiliary-loss-free routing): the pages say only
  that the bias is adjusted as training runs to keep the experts balanced
  ("MoE inference: the call centre with 256 specialists ...", "The bare
  mechanism", auxiliary-loss-free variant).  Reading taken: after a batch,
  b_i <- b_i + rate * sign(mean load - load_i), one float32 step per expert,
  the load being the expert's count of (token, slot) assignments.

Readings taken where the pages are silent (each is listed in the design notes):
ties in top-k go to the lower index under IEEE comparison (+0 == -0); f_i
divides by T*k so that sum f = 1 for any k; P_i uses the full N-way softmax of
the unbiased logits; shared experts have gate 1 and count in neither k, f nor
P; no biases inside experts or router.

Parity status: every function here (O9 included: closed-form codes, all 256
codes against PyTorch's float8_e4m3fn, the output-channel scale identity; O10
against central finite differences of the float64 forward and, for one expert,
PyTorch autograd of a dense SwiGLU; O11 against its sign cases) is pinned by
``tests/test_oracle_pins.py``
(worked examples of the pages, closed forms, brute force, library special
cases).  SwiGLU numerics at the real layer shapes have no printed values on the
pages; they are pinned only through the N = 1, k = 1 reduction to a library
SwiGLU and the dense cross-path.
"""

from __future__ import annotations

from typing import Callable, Optional, Sequence, Tuple, Union

import numpy as np

__all__ = [
    "e4m3_decode",
    "dequantize",
    "router_logits",
    "selection_keys",
    "capacity_keep",
    "topk_by_rank",
    "kept_softmax",
    "full_softmax",
    "silu",
    "swiglu_expert",
    "route_from_logits",
    "combine",
    "stats",
    "balance",
    "moe_forward",
    "moe_backward",
    "update_select_bias",
    "BALANCE_ALPHA",
]

# Switch Transformer's coefficient, quoted on "Mixture of Experts and Guided
# Decoding" (auxiliary-loss passage).
BALANCE_ALPHA = 0.01

ExpertSource = Union[
    Tuple[np.ndarray, np.ndarray, np.ndarray],
    Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]],
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- O1
def router_logits(x, w_router, logit_bias=None) -> np.ndarray:
    """O1: r[t, e] = sum_j x[t, j] * W_r[e, j] (+ logit_bias[e]), rounded to fp32.

    W_r is stored one row per expert (the linear layer's [out, in] layout).
    The sum is formed in float64, then rounded once to float32 (the precision
    the routing decision is taken in).  The optional ``logit_bias`` is a
    per-expert offset that is part of the logits themselves (it moves
    selection, gates and P alike).
    """
    x64 = _f64(x)
    w64 = _f64(w_router)
    r = x64 @ w64.T
    if logit_bias is not None:
        r = r + _f64(logit_bias)[None, :]
    return r.astype(np.float32)


# --------------------------------------------------------------------------- O2
def selection_keys(r32, select_bias=None) -> np.ndarray:
    """O2: key = fp32(r + b) with one round-to-nearest-even float32 addition.

    Without a selection bias the key is the logit itself.  The bias steers only
    which experts are chosen ("The bare mechanism", auxiliary-loss-free
    routing); gates and P keep using the unbiased logits.
    """
    r32 = np.asarray(r32, dtype=np.float32)
    if select_bias is None:
        return r32.copy()
    b32 = np.asarray(select_bias, dtype=np.float32)
    return (r32 + b32[None, :]).astype(np.float32)


# --------------------------------------------------------------------------- O3
def topk_by_rank(keys, k: int, chunk: int = 256) -> np.ndarray:
    """O3: the k experts with the highest keys, ties to the lower index.

    Definition used: the rank of expert e for token t is the number of experts
    that beat it, where e' beats e when key[e'] > key[e], or the keys compare
    equal (IEEE, so +0 == -0) and e' < e.  Expert e is kept when its rank is
    below k, and it lands in slot rank(e).  Slot 0 therefore holds the highest
    key.  Returns int32 [T, k].
    """
    keys = np.asarray(keys, dtype=np.float32)
    T, N = keys.shape
    if not 1 <= k <= N:
        raise ValueError("need 1 <= k <= n_experts")
    out = np.empty((T, k), dtype=np.int32)
    lower = np.tri(N, N, -1, dtype=bool)  # lower[e, e2] is True when e2 < e
    step = max(1, min(chunk, (1 << 24) // max(1, N * N)))
    for t0 in range(0, T, step):
        kk = keys[t0:t0 + step]
        mine = kk[:, :, None]     # key[e]
        other = kk[:, None, :]    # key[e']
        beats = (other > mine) | ((other == mine) & lower[None, :, :])
        rank = beats.sum(axis=2)  # [t, e]
        for t in range(kk.shape[0]):
            sel = np.nonzero(rank[t] < k)[0]
            out[t0 + t, rank[t, sel]] = sel
    return out


# --------------------------------------------------------------------------- O4
def kept_softmax(r32, idx) -> np.ndarray:
    """O4: g[t, j] = exp(r[t, idx[t, j]]) / sum_l exp(r[t, idx[t, l]]) in float64.

    The unbiased logits of the kept experts only; the largest kept logit is
    subtracted first (it cancels in the ratio).
    """
    r = _f64(r32)
    idx = np.asarray(idx)
    kept = np.take_along_axis(r, idx.astype(np.int64), axis=1)
    if kept.shape[0] == 0:
        return kept
    z = np.exp(kept - kept.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def full_softmax(r32) -> np.ndarray:
    """Softmax over all N experts per token (float64): the router's probabilities."""
    r = _f64(r32)
    if r.shape[0] == 0:
        return r
    z = np.exp(r - r.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------- O5
def silu(a) -> np.ndarray:
    """SiLU (swish with beta = 1): a * sigmoid(a) = a / (1 + e^-a)."""
    a = _f64(a)
    return a / (1.0 + np.exp(-a))


def swiglu_expert(X, w_gate, w_up, w_down) -> np.ndarray:
    """O5: one SwiGLU expert on a block of rows.

    a = X W_gate^T, b = X W_up^T (both [rows, F]); h = SiLU(a) * b;
    out = h W_down^T ([rows, d]).  W_gate and W_up are [F, d] and W_down is
    [d, F], each in the linear layer's [out, in] layout.
    """
    X = _f64(X)
    a = X @ _f64(w_gate).T
    b = X @ _f64(w_up).T
    h = silu(a) * b
    return h @ _f64(w_down).T


# ------------------------------------------------------------------ O2+O3+O4
def route_from_logits(r32, k: int, select_bias=None):
    """Selection and gates from given fp32 logits: returns (idx int32 [T,k], g f64 [T,k])."""
    keys = selection_keys(r32, select_bias)
    idx = topk_by_rank(keys, k)
    return idx, kept_softmax(r32, idx)


# --------------------------------------------------------------------------- O8
def capacity_keep(idx, n_experts: int, capacity: int) -> np.ndarray:
    """O8: bool [T, k], True where assignment (t, slot) is kept.

    Expert e keeps the first ``capacity`` of the assignments that chose it,
    counted in token order (a token picks an expert at most once).
    ``capacity`` <= 0 means no limit.
    """
    idx = np.asarray(idx)
    keep = np.ones(idx.shape, dtype=bool)
    if capacity <= 0:
        return keep
    for e in range(n_experts):
        tok, slot = np.nonzero(idx == e)  # row-major: ascending token
        keep[tok[capacity:], slot[capacity:]] = False
    return keep


# --------------------------------------------------------------------------- O6
def combine(gates, expert_outputs) -> np.ndarray:
    """O6 for one token: sum_j gates[j] * expert_outputs[j] (float64).

    ``gates`` has shape [k] and ``expert_outputs`` [k, dim].
    """
    g = _f64(gates)
    E = _f64(expert_outputs)
    out = np.zeros(E.shape[1:], dtype=np.float64)
    for j in range(g.shape[0]):
        out += g[j] * E[j]
    return out


# --------------------------------------------------------------------------- O7
def stats(idx, r32, n_experts: int):
    """O7 counts, f and P.

    counts[e] = number of (token, slot) assignments to expert e;
    f[e] = counts[e] / (T * k); P[e] = mean over tokens of the full softmax of
    the (unbiased) logits.  With T = 0 every value is 0.
    """
    idx = np.asarray(idx)
    T = idx.shape[0]
    k = idx.shape[1] if idx.ndim == 2 else 0
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in idx.reshape(-1):
        counts[int(e)] += 1
    if T == 0:
        return counts, np.zeros(n_experts), np.zeros(n_experts)
    f = counts.astype(np.float64) / float(T * k)
    P = full_softmax(r32).mean(axis=0)
    return counts, f, P


def balance(f, P, alpha: float = BALANCE_ALPHA):
    """Balance loss: returns (N * sum_i f_i P_i, alpha * that)."""
    f = _f64(f)
    P = _f64(P)
    raw = float(f.shape[0]) * float(np.sum(f * P))
    return raw, alpha * raw


# ------------------------------------------------------------------ O1..O7
def e4m3_decode(codes) -> np.ndarray:
    """O9: the float64 value of each OCP FP8 E4M3 code (uint8 array).

    value = (-1)^s * 2^(e - 7) * (1 + m / 8)   for exponent field e >= 1,
            (-1)^s * 2^(-6) * (m / 8)          for e = 0 (subnormal),
    NaN for e = 15 and m = 7.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def dequantize(codes, scale) -> np.ndarray:
    """O9: weights [..., out, in] = e4m3_decode(codes) * scale[..., out] (one
    scale per output channel, i.e. per row of the [out, in] matrix)."""
    return e4m3_decode(codes) * _f64(scale)[..., :, None]


def _expert_getter(experts: ExpertSource):
    if callable(experts):
        return experts
    wg, wu, wd = experts
    return lambda e: (wg[e], wu[e], wd[e])


def moe_forward(
    x,
    w_router,
    experts: ExpertSource,
    k: int,
    *,
    logit_bias=None,
    select_bias=None,
    shared: Optional[Sequence[np.ndarray]] = None,
    route_logits=None,
    alpha: float = BALANCE_ALPHA,
    n_experts: Optional[int] = None,
    capacity: int = 0,
    exact_logits: bool = False,
):
    """The whole layer forward, O1..O8, with the experts looped one at a time.

    ``experts`` is either a tuple (W_gate [N,F,d], W_up [N,F,d], W_down [N,d,F])
    or a callable e -> (W_gate[e], W_up[e], W_down[e]) so that large layers can
    hand over one expert's weights at a time.  ``shared`` is an optional tuple
    of [S,F,d], [S,F,d], [S,d,F] arrays for always-on experts.

    ``route_logits`` (fp32 [T, N]) replaces O1 when given: the routing is then
    taken on those logits, which is how a caller checks another implementation's
    routing bit for bit on its own logits.

    ``capacity`` > 0 applies O8 (per-expert capacity, extras dropped).

    ``exact_logits``: gates and P take the float64 logits instead of their
    float32 rounding (the selection still compares float32 keys), which makes
    the output a smooth function of the weights between ties -- the function
    whose derivative O10 is.

    Returns a dict with y (float64 [T, d]), logits, idx, gates, keep (the O8
    mask), counts, f, P, aux_raw and aux.
    """
    x64 = _f64(x)
    T, d = x64.shape
    if route_logits is None:
        r32 = router_logits(x64, w_router, logit_bias)
    else:
        r32 = np.asarray(route_logits, dtype=np.float32)
    r_soft = r32
    if exact_logits and route_logits is None:
        r_soft = x64 @ _f64(w_router).T
        if logit_bias is not None:
            r_soft = r_soft + _f64(logit_bias)[None, :]
    N = r32.shape[1] if n_experts is None else n_experts
    idx, g = route_from_logits(r32, k, select_bias) if T else (
        np.zeros((0, k), np.int32), np.zeros((0, k)))
    if T and r_soft is not r32:
        g = kept_softmax(r_soft, idx)
    get = _expert_getter(experts)
    keep = capacity_keep(idx, N, capacity)

    y = np.zeros((T, d), dtype=np.float64)
    for e in range(N):
        tok, slot = np.nonzero((idx == e) & keep)
        if tok.size == 0:
            continue  # an expert that no token picked does no work
        wg, wu, wd = get(e)
        E = swiglu_expert(x64[tok], wg, wu, wd)
        y[tok] += g[tok, slot][:, None] * E
    if shared is not None:
        sg, su, sd = shared
        for s in range(np.asarray(sg).shape[0]):
            y += swiglu_expert(x64, sg[s], su[s], sd[s])

    counts, f, P = stats(idx, r_soft, N)
    aux_raw, aux = balance(f, P, alpha)
    return {
        "y": y,
        "logits": r32,
        "idx": idx,
        "gates": g,
        "keep": keep,
        "counts": counts,
        "f": f,
        "P": P,
        "aux_raw": aux_raw,
        "aux": aux,
    }


# -------------------------------------------------------------------------- O10
def _sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def _swiglu_backward(X, w_gate, w_up, w_down, dout):
    """Chain rule through one SwiGLU expert (O5) for rows X and output
    gradient dout: returns (dX, dW_gate, dW_up, dW_down, out)."""
    X = _f64(X)
    wg, wu, wd = _f64(w_gate), _f64(w_up), _f64(w_down)
    a = X @ wg.T
    b = X @ wu.T
    s = _sigmoid(a)
    h = a * s * b                        # SiLU(a) * b
    out = h @ wd.T
    dh = dout @ wd                       # [rows, F]
    da = dh * b * (s + a * s * (1.0 - s))  # d SiLU(a) / da = s + a s (1 - s)
    db = dh * a * s
    return da @ wg + db @ wu, da.T @ X, db.T @ X, dout.T @ h, out


def moe_backward(
    x,
    w_router,
    experts: Tuple[np.ndarray, np.ndarray, np.ndarray],
    k: int,
    dy,
    *,
    logit_bias=None,
    select_bias=None,
    shared: Optional[Sequence[np.ndarray]] = None,
    alpha: float = BALANCE_ALPHA,
    aux_grad: float = 1.0,
    capacity: int = 0,
    route_idx=None,
):
    """O10: gradients of L = sum(y * dy) + aux_grad * aux (float64).

    The forward is O1..O8 with float64 logits for the gates and P (the
    ``exact_logits`` forward); the selection is taken on the float32 keys and,
    like the capacity mask, held fixed.  In order, reversing the forward:

    * combine (O6): a kept slot j of token t passes g_tj * dy_t to its expert
      and receives dg_tj = <dy_t, E_e(x_t)>; a shared expert gets dy_t;
    * experts (O5): the chain rule through down, the SiLU product and gate/up,
      giving the weight gradients and each row's contribution to dx;
    * gates (O4): the softmax over the token's k kept logits,
      dr_t[idx_tj] += g_tj (dg_tj - sum_l g_tl dg_tl), dropped slots included
      with dg = 0 (their gate stays in the normalisation);
    * balance (O7): only P depends on the weights; with c_i = aux_grad * alpha
      * N * f_i / T, dr_t[i] += p_ti (c_i - sum_j c_j p_tj), p_t the full
      softmax;
    * router (O1): dW_r = dr^T x, dx += dr W_r, d logit_bias = sum_t dr_t.

    ``route_idx`` (int [T, k]) replaces the selection when given, which is how
    a caller checks another implementation's backward on that
    implementation's own choice of experts (near-ties in the logits may be
    taken either way by two correct implementations).

    Returns a dict: dx [T, d], dw_router [N, d], dlogit_bias [N], dw_gate,
    dw_up [N, F, d], dw_down [N, d, F], and with shared experts ds_gate, ds_up,
    ds_down; also dgate [T, k] (the gate gradients) and dlogits [T, N].
    """
    x64 = _f64(x)
    T, d = x64.shape
    wr = _f64(w_router)
    N = wr.shape[0]
    wg_all, wu_all, wd_all = (_f64(w) for w in experts)
    dy = _f64(dy)
    r = x64 @ wr.T
    if logit_bias is not None:
        r += _f64(logit_bias)[None, :]
    r32 = r.astype(np.float32)
    if route_idx is not None:
        idx = np.asarray(route_idx).astype(np.int32).reshape(T, k)
    elif T:
        idx = topk_by_rank(selection_keys(r32, select_bias), k)
    else:
        idx = np.zeros((0, k), np.int32)
    keep = capacity_keep(idx, N, capacity)
    g = kept_softmax(r, idx)

    dx = np.zeros_like(x64)
    dwg, dwu, dwd = np.zeros_like(wg_all), np.zeros_like(wu_all), np.zeros_like(wd_all)
    dgate = np.zeros((T, k))
    for e in range(N):
        tok, slot = np.nonzero(keep & (idx == e))
        if tok.size == 0:
            continue
        gate = g[tok, slot][:, None]
        dX, dWg, dWu, dWd, out = _swiglu_backward(x64[tok], wg_all[e], wu_all[e], wd_all[e],
                                                  gate * dy[tok])
        dgate[tok, slot] = np.sum(dy[tok] * out, axis=1)
        dx[tok] += dX  # a token picks an expert at most once
        dwg[e] += dWg
        dwu[e] += dWu
        dwd[e] += dWd
    res = {}
    if shared is not None:
        sg, su, sd = (_f64(w) for w in shared)
        ds = [np.zeros_like(sg), np.zeros_like(su), np.zeros_like(sd)]
        for s_ in range(sg.shape[0]):
            dX, dWg, dWu, dWd, _ = _swiglu_backward(x64, sg[s_], su[s_], sd[s_], dy)
            dx += dX
            ds[0][s_] += dWg
            ds[1][s_] += dWu
            ds[2][s_] += dWd
        res.update(ds_gate=ds[0], ds_up=ds[1], ds_down=ds[2])

    dr = np.zeros((T, N))
    if T:
        # kept softmax (O4)
        dz = g * (dgate - np.sum(g * dgate, axis=1, keepdims=True))
        np.add.at(dr, (np.repeat(np.arange(T), k), idx.reshape(-1).astype(np.int64)),
                  dz.reshape(-1))
        # balance loss through P (O7)
        counts = np.bincount(idx.reshape(-1).astype(np.int64), minlength=N).astype(np.float64)
        f = counts / float(T * k)
        c = aux_grad * alpha * N * f / T
        p = full_softmax(r)
        dr += p * (c[None, :] - np.sum(p * c[None, :], axis=1, keepdims=True))
    dx += dr @ wr
    res.update(dx=dx, dw_router=dr.T @ x64, dlogit_bias=dr.sum(axis=0), dw_gate=dwg,
               dw_up=dwu, dw_down=dwd, dgate=dgate, dlogits=dr, idx=idx, keep=keep)
    return res


# -------------------------------------------------------------------------- O11
def update_select_bias(select_bias, counts, rate: float) -> np.ndarray:
    """O11: b_i + rate * sign(mean(counts) - counts_i), in float32.

    An expert that took more than the mean load has its selection bias
    lowered by ``rate``, one that took less has it raised, one exactly at the
    mean keeps it.  The mean is sum(counts) / N; the step is one float32
    addition of +rate, -rate or 0.
    """
    b = np.asarray(select_bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.float64)
    mean = c.sum() / c.shape[0]
    step = np.sign(mean - c).astype(np.float32) * np.float32(rate)
    return (b + step).astype(np.float32)
