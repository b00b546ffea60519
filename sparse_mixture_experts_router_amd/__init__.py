"""Sparse mixture-of-experts layer (forward and backward) on AMD MI355X (gfx950).

A thin ctypes binding of ``libmoe.so``: every function below only marshals
PyTorch tensors (device memory) and the current HIP stream into the C ABI
declared in ``include/moe.h``; every step of the layer runs in the library's
HIP kernels.  There is no CPU fallback: if the library is not built, calls
raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

__all__ = [
    "LIB_PATH", "MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
    "MOE_ERR_HIP", "MOE_F32", "MOE_BF16", "MOE_WEIGHTS_DTYPE", "MOE_WEIGHTS_FP8_E4M3", "STAGES", "BACKWARD_STAGES",
    "MoEError", "MoEConfig", "MoEWeights",
    "MoERouting", "lib", "make_config", "moe_workspace_size", "moe_status_string",
    "alloc_workspace", "moe_route", "moe_layer_forward", "moe_balance_stats", "MoELayer",
    "MoEGrads", "moe_backward_workspace_size", "alloc_backward_workspace", "moe_layer_backward",
    "moe_update_select_bias", "MoEPlanInfo", "moe_forward_plan", "moe_layer_forward_noalloc",
    "NOALLOC_SCRATCH_BYTES",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_WEIGHTS_DTYPE, MOE_WEIGHTS_FP8_E4M3 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h
_SCALES = ("w_gate_scale", "w_up_scale", "w_down_scale", "ws_gate_scale", "ws_up_scale",
           "ws_down_scale")
STAGES = ("route", "permute", "expert_up", "expert_down", "combine")
BACKWARD_STAGES = ("route", "transpose_w", "recompute", "grad_h", "grad_x", "segments", "grad_w",
                   "grad_wr")


class MoEError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        self.status = status
        msg = moe_status_string(status)
        super().__init__(f"{msg} ({detail})" if detail else msg)


class MoEConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("weight_format", ctypes.c_int32)]


class MoEWeights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("ws_gate", ctypes.c_void_p), ("ws_up", ctypes.c_void_p),
                ("ws_down", ctypes.c_void_p), ("logit_bias", ctypes.c_void_p),
                ("select_bias", ctypes.c_void_p)] + [(n, ctypes.c_void_p) for n in _SCALES]


class MoERouting(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p),
                ("topk_gate", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("prob_sum", ctypes.c_void_p), ("f", ctypes.c_void_p), ("P", ctypes.c_void_p),
                ("aux", ctypes.c_void_p), ("balance_alpha", ctypes.c_float)]


class MoEPlanInfo(ctypes.Structure):
    _fields_ = [("up_kernel", ctypes.c_int32), ("up_tile_rows", ctypes.c_int32),
                ("down_kernel", ctypes.c_int32), ("down_tile_rows", ctypes.c_int32),
                ("route_split", ctypes.c_int32), ("route_kernel", ctypes.c_int32),
                ("down_split", ctypes.c_int32),
                ("tail_split_cols", ctypes.c_int32), ("up_narrow_tails", ctypes.c_int32),
                ("down_narrow_tails", ctypes.c_int32), ("compute_units", ctypes.c_int32),
                ("all_token_pass", ctypes.c_int32),
                ("split_plan_offset", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64)]


class MoEGrads(ctypes.Structure):
    _fields_ = [("dx", ctypes.c_void_p), ("dw_router", ctypes.c_void_p),
                ("dlogit_bias", ctypes.c_void_p), ("dw_gate", ctypes.c_void_p),
                ("dw_up", ctypes.c_void_p), ("dw_down", ctypes.c_void_p),
                ("dws_gate", ctypes.c_void_p), ("dws_up", ctypes.c_void_p),
                ("dws_down", ctypes.c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m sparse_mixture_experts_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        cfgp, wp, rp = (ctypes.POINTER(MoEConfig), ctypes.POINTER(MoEWeights),
                        ctypes.POINTER(MoERouting))
        L.moe_workspace_size.argtypes = [cfgp]
        L.moe_workspace_size.restype = sz
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_route.argtypes = [cfgp, vp, wp, rp, vp, sz, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [cfgp, vp, wp, vp, rp, vp, sz, vp]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward_timed.argtypes = [cfgp, vp, wp, vp, rp, vp, sz, vp,
                                              ctypes.POINTER(vp)]
        L.moe_layer_forward_timed.restype = ctypes.c_int
        L.moe_balance_stats.argtypes = [i32, i32, i32, vp, vp, ctypes.c_float, vp, vp, vp, vp]
        L.moe_balance_stats.restype = ctypes.c_int
        L.moe_backward_workspace_size.argtypes = [cfgp]
        L.moe_backward_workspace_size.restype = sz
        L.moe_layer_backward.argtypes = [cfgp, vp, wp, vp, ctypes.c_float, ctypes.c_float,
                                         ctypes.POINTER(MoEGrads), vp, sz, vp]
        L.moe_layer_backward.restype = ctypes.c_int
        L.moe_layer_backward_timed.argtypes = L.moe_layer_backward.argtypes + [ctypes.POINTER(vp)]
        L.moe_layer_backward_timed.restype = ctypes.c_int
        L.moe_update_select_bias.argtypes = [i32, vp, ctypes.c_float, vp, vp]
        L.moe_update_select_bias.restype = ctypes.c_int
        L.moe_forward_plan.argtypes = [cfgp, ctypes.POINTER(MoEPlanInfo)]
        L.moe_forward_plan.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [cfgp, vp, wp, vp, rp, vp]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        _LIB = L
    return _LIB


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error().decode())


_TORCH_DTYPE = {MOE_BF16: torch.bfloat16, MOE_F32: torch.float32}


def make_config(T: int, d_model: int, n_experts: int, top_k: int, d_ff: int,
                n_shared: int = 0, dtype=torch.bfloat16, capacity: int = 0,
                weight_format: int = MOE_WEIGHTS_DTYPE) -> MoEConfig:
    """``capacity``: 0 = dropless, else the most (token, slot) assignments a
    routed expert takes per call (the rest are dropped).  ``weight_format``:
    MOE_WEIGHTS_FP8_E4M3 for expert weights given as uint8 E4M3 codes plus
    fp32 per-output-channel scales (``*_scale`` entries of the weights)."""
    code = MOE_BF16 if dtype in (torch.bfloat16, "bf16", MOE_BF16) else MOE_F32
    return MoEConfig(int(T), int(d_model), int(n_experts), int(top_k), int(d_ff),
                     int(n_shared), code, int(capacity), int(weight_format))


def moe_workspace_size(cfg: MoEConfig) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(cfg)))


def alloc_workspace(cfg: MoEConfig, device="cuda") -> torch.Tensor:
    n = moe_workspace_size(cfg)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARG, "configuration rejected")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_forward_plan(cfg: MoEConfig) -> Dict[str, int]:
    """How moe_layer_forward runs ``cfg`` on the current device (kernel
    choices, tile rows, reduction splits, and the workspace offset of the
    device-side split plan); see ``moe_forward_plan`` in include/moe.h."""
    info = MoEPlanInfo()
    _check(lib().moe_forward_plan(ctypes.byref(cfg), ctypes.byref(info)))
    return {name: int(getattr(info, name)) for name, _ in MoEPlanInfo._fields_}


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor",
         numel: Optional[int] = None) -> Optional[int]:
    """Device address of ``t`` after checking placement, layout, dtype and,
    when ``numel`` is given, its element count: the C ABI sees only pointers,
    so a tensor of the wrong size would be read or written out of bounds."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the configuration needs {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _weight_numels(cfg: MoEConfig) -> Dict[str, int]:
    """Element count of every weight, bias and scale that ``cfg`` implies."""
    N, d, F, S = cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.n_shared
    return {"w_router": N * d, "w_gate": N * F * d, "w_up": N * F * d, "w_down": N * d * F,
            "ws_gate": S * F * d, "ws_up": S * F * d, "ws_down": S * d * F,
            "logit_bias": N, "select_bias": N,
            "w_gate_scale": N * F, "w_up_scale": N * F, "w_down_scale": N * d,
            "ws_gate_scale": S * F, "ws_up_scale": S * F, "ws_down_scale": S * d}


def _weights(cfg: MoEConfig, w: Dict[str, Optional[torch.Tensor]], experts=True) -> MoEWeights:
    dt = _TORCH_DTYPE[cfg.dtype]
    fp8 = cfg.weight_format == MOE_WEIGHTS_FP8_E4M3
    n = _weight_numels(cfg)
    args = {"w_router": _ptr(w.get("w_router"), dt, "w_router", n["w_router"])}
    if experts:
        for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
            args[name] = _ptr(w.get(name), torch.uint8 if fp8 else dt, name, n[name])
        if fp8:
            for name in _SCALES:
                args[name] = _ptr(w.get(name), torch.float32, name, n[name])
    args["logit_bias"] = _ptr(w.get("logit_bias"), torch.float32, "logit_bias", n["logit_bias"])
    args["select_bias"] = _ptr(w.get("select_bias"), torch.float32, "select_bias",
                               n["select_bias"])
    return MoEWeights(**args)


def _routing(cfg: MoEConfig, logits=None, topk_idx=None, topk_gate=None, counts=None,
             prob_sum=None, f=None, P=None, aux=None, alpha=0.01):
    T, N, k = cfg.T, cfg.n_experts, cfg.top_k
    return MoERouting(_ptr(logits, torch.float32, "logits", T * N),
                      _ptr(topk_idx, torch.int32, "topk_idx", T * k),
                      _ptr(topk_gate, torch.float32, "topk_gate", T * k),
                      _ptr(counts, torch.int32, "counts", N),
                      _ptr(prob_sum, torch.float32, "prob_sum", N),
                      _ptr(f, torch.float32, "f", N), _ptr(P, torch.float32, "P", N),
                      _ptr(aux, torch.float32, "aux", 2), float(alpha))


def moe_route(cfg: MoEConfig, x: torch.Tensor, weights: Dict[str, Optional[torch.Tensor]], *,
              topk_idx: torch.Tensor, topk_gate: torch.Tensor, workspace: torch.Tensor,
              logits=None, counts=None, prob_sum=None, f=None, P=None, aux=None, alpha=0.01,
              stream=None) -> None:
    """Routing only; see ``moe_route`` in include/moe.h."""
    w = _weights(cfg, weights, experts=False)
    r = _routing(cfg, logits, topk_idx, topk_gate, counts, prob_sum, f, P, aux, alpha)
    _check(lib().moe_route(ctypes.byref(cfg),
                           _ptr(x, _TORCH_DTYPE[cfg.dtype], "x", cfg.T * cfg.d_model),
                           ctypes.byref(w), ctypes.byref(r), _ptr(workspace, None, "workspace"),
                           workspace.numel(), _stream(stream)))


def moe_layer_forward(cfg: MoEConfig, x: torch.Tensor, weights: Dict[str, Optional[torch.Tensor]],
                      y: torch.Tensor, *, workspace: torch.Tensor, logits=None, topk_idx=None,
                      topk_gate=None, counts=None, prob_sum=None, f=None, P=None, aux=None,
                      alpha=0.01, stream=None,
                      stage_events: Optional[Sequence[torch.cuda.Event]] = None) -> None:
    """Whole layer forward into ``y``; see ``moe_layer_forward`` in include/moe.h.

    ``f``, ``P``, ``aux``: optional balance statistics written by the same
    call (``aux`` = [N sum f P, alpha N sum f P]).
    ``stage_events``: optional list of len(STAGES) + 1 ``torch.cuda.Event``
    (enable_timing=True) or None, recorded before each stage and after the
    last; None entries are skipped.
    """
    dt = _TORCH_DTYPE[cfg.dtype]
    w = _weights(cfg, weights)
    r = _routing(cfg, logits, topk_idx, topk_gate, counts, prob_sum, f, P, aux, alpha)
    td = cfg.T * cfg.d_model
    args = (ctypes.byref(cfg), _ptr(x, dt, "x", td), ctypes.byref(w), _ptr(y, dt, "y", td),
            ctypes.byref(r), _ptr(workspace, None, "workspace"), workspace.numel(),
            _stream(stream))
    if stage_events is None:
        _check(lib().moe_layer_forward(*args))
        return
    if len(stage_events) != len(STAGES) + 1:
        raise ValueError("need one event per stage plus one")
    s = torch.cuda.current_stream() if stream is None else stream
    for ev in stage_events:      # torch creates the HIP event on first record
        if ev is not None and not ev.cuda_event:
            ev.record(s)
    arr = (ctypes.c_void_p * len(stage_events))(
        *[None if ev is None else ev.cuda_event for ev in stage_events])
    _check(lib().moe_layer_forward_timed(*args, arr))


def moe_layer_forward_noalloc(cfg: MoEConfig, x: torch.Tensor,
                              weights: Dict[str, Optional[torch.Tensor]], y: torch.Tensor, *,
                              logits=None, topk_idx=None, topk_gate=None, counts=None,
                              prob_sum=None, f=None, P=None, aux=None, alpha=0.01,
                              stream=None) -> None:
    """moe_layer_forward without a workspace argument: the library's own
    per-GPU device array of NOALLOC_SCRATCH_BYTES serves as the workspace, so
    the call allocates nothing; see ``moe_layer_forward_noalloc`` in
    include/moe.h (larger configurations raise MOE_ERR_WORKSPACE; calls that
    overlap on one GPU race)."""
    dt = _TORCH_DTYPE[cfg.dtype]
    w = _weights(cfg, weights)
    r = _routing(cfg, logits, topk_idx, topk_gate, counts, prob_sum, f, P, aux, alpha)
    td = cfg.T * cfg.d_model
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(cfg), _ptr(x, dt, "x", td),
                                           ctypes.byref(w), _ptr(y, dt, "y", td),
                                           ctypes.byref(r), _stream(stream)))


def moe_balance_stats(T: int, N: int, k: int, counts: torch.Tensor, prob_sum: torch.Tensor,
                      alpha: float, f: torch.Tensor, P: torch.Tensor, aux: torch.Tensor,
                      stream=None) -> None:
    """f = counts / (T k), P = prob_sum / T, aux = [N sum f P, alpha N sum f P]."""
    _check(lib().moe_balance_stats(
        int(T), int(N), int(k), _ptr(counts, torch.int32, "counts", N),
        _ptr(prob_sum, torch.float32, "prob_sum", N), float(alpha),
        _ptr(f, torch.float32, "f", N), _ptr(P, torch.float32, "P", N),
        _ptr(aux, torch.float32, "aux", 2), _stream(stream)))


def moe_backward_workspace_size(cfg: MoEConfig) -> int:
    return int(lib().moe_backward_workspace_size(ctypes.byref(cfg)))


def alloc_backward_workspace(cfg: MoEConfig, device="cuda") -> torch.Tensor:
    n = moe_backward_workspace_size(cfg)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARG, "configuration rejected")
    return torch.empty(n, dtype=torch.uint8, device=device)


_GRADS = ("dx", "dw_router", "dlogit_bias", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up",
          "dws_down")


def _event_array(stage_events, n, stream):
    if len(stage_events) != n + 1:
        raise ValueError("need one event per stage plus one")
    s = torch.cuda.current_stream() if stream is None else stream
    for ev in stage_events:      # torch creates the HIP event on first record
        if ev is not None and not ev.cuda_event:
            ev.record(s)
    return (ctypes.c_void_p * len(stage_events))(
        *[None if ev is None else ev.cuda_event for ev in stage_events])


def moe_layer_backward(cfg: MoEConfig, x: torch.Tensor, weights: Dict[str, Optional[torch.Tensor]],
                       dy: torch.Tensor, grads: Dict[str, Optional[torch.Tensor]], *,
                       workspace: torch.Tensor, alpha: float = 0.01, aux_grad: float = 1.0,
                       stream=None,
                       stage_events: Optional[Sequence[torch.cuda.Event]] = None) -> None:
    """Gradients of sum(y * dy) + aux_grad * aux into ``grads`` (keys dx,
    dw_router, dlogit_bias, dw_gate, dw_up, dw_down, dws_*); see
    ``moe_layer_backward`` in include/moe.h.  ``stage_events``: as for
    moe_layer_forward, one per BACKWARD_STAGES entry plus one."""
    dt = _TORCH_DTYPE[cfg.dtype]
    w = _weights(cfg, weights)
    wn = _weight_numels(cfg)
    td = cfg.T * cfg.d_model
    gn = {"dx": td, "dw_router": wn["w_router"], "dlogit_bias": cfg.n_experts,
          "dw_gate": wn["w_gate"], "dw_up": wn["w_up"], "dw_down": wn["w_down"],
          "dws_gate": wn["ws_gate"], "dws_up": wn["ws_up"], "dws_down": wn["ws_down"]}
    g = MoEGrads(**{n: _ptr(grads.get(n), torch.float32 if n == "dlogit_bias" else dt, n, gn[n])
                    for n in _GRADS})
    args = (ctypes.byref(cfg), _ptr(x, dt, "x", td), ctypes.byref(w), _ptr(dy, dt, "dy", td),
            float(alpha), float(aux_grad), ctypes.byref(g), _ptr(workspace, None, "workspace"),
            workspace.numel(), _stream(stream))
    if stage_events is None:
        _check(lib().moe_layer_backward(*args))
    else:
        _check(lib().moe_layer_backward_timed(
            *args, _event_array(stage_events, len(BACKWARD_STAGES), stream)))


def moe_update_select_bias(counts: torch.Tensor, rate: float, select_bias: torch.Tensor,
                           stream=None) -> None:
    """select_bias += rate * sign(mean(counts) - counts), in place (fp32)."""
    n = int(counts.numel())
    _check(lib().moe_update_select_bias(
        n, _ptr(counts, torch.int32, "counts"), float(rate),
        _ptr(select_bias, torch.float32, "select_bias", n), _stream(stream)))


class MoELayer:
    """Convenience holder: config, device weights and a workspace sized once.

    ``forward(x)`` allocates the outputs with torch (device memory only) and
    calls ``moe_layer_forward``, which also writes the balance statistics.
    """

    def __init__(self, weights: Dict[str, Optional[torch.Tensor]], top_k: int,
                 alpha: float = 0.01):
        wg = weights["w_gate"]
        self.weights = weights
        self.N, self.F, self.d = wg.shape
        self.S = 0 if weights.get("ws_gate") is None else weights["ws_gate"].shape[0]
        self.k = int(top_k)
        self.dtype = wg.dtype
        self.alpha = alpha
        self._ws = None
        self._ws_T = -1

    def config(self, T: int) -> MoEConfig:
        return make_config(T, self.d, self.N, self.k, self.F, self.S, self.dtype)

    def forward(self, x: torch.Tensor, want_logits: bool = False):
        T = x.shape[0]
        cfg = self.config(T)
        if self._ws is None or self._ws_T < T:
            self._ws = alloc_workspace(cfg, x.device)
            self._ws_T = T
        dev = x.device
        out = {
            "y": torch.empty_like(x),
            "topk_idx": torch.empty((T, self.k), dtype=torch.int32, device=dev),
            "topk_gate": torch.empty((T, self.k), dtype=torch.float32, device=dev),
            "counts": torch.zeros(self.N, dtype=torch.int32, device=dev),
            "prob_sum": torch.zeros(self.N, dtype=torch.float32, device=dev),
            "logits": (torch.empty((T, self.N), dtype=torch.float32, device=dev)
                       if want_logits else None),
            "f": torch.empty(self.N, dtype=torch.float32, device=dev),
            "P": torch.empty(self.N, dtype=torch.float32, device=dev),
            "aux": torch.empty(2, dtype=torch.float32, device=dev),
        }
        moe_layer_forward(cfg, x, self.weights, out["y"], workspace=self._ws,
                          logits=out["logits"], topk_idx=out["topk_idx"],
                          topk_gate=out["topk_gate"], counts=out["counts"],
                          prob_sum=out["prob_sum"], f=out["f"], P=out["P"], aux=out["aux"],
                          alpha=self.alpha)
        return out
