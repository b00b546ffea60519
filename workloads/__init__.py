"""Seeded synthetic workloads for the sparse MoE layer forward.

This module only *draws inputs*: shapes, dtypes and seeded random tensors.  It
holds none of the layer's arithmetic, so both the HIP library's callers and the
CPU oracle's tests may use it.  Every tensor is drawn with its own
``torch.Generator`` (seed, tensor tag) so the bits do not depend on which other
tensors were drawn; bf16 tensors are drawn in fp32 and rounded to bf16 with
round-to-nearest-even by ``Tensor.to``.

The shapes follow the model families the pages tabulate ("MoE inference: the
call centre with 256 specialists ...", table "The relevant MoE models in May
2026": Mixtral 8x7B with 8 experts and top-2, DeepSeek-V3 with 256 routed + 1
shared expert and top-8, Qwen3-235B-A22B with 128 experts and top-8).  The
weights are random stand-ins: no trained checkpoint is used.

Distributions: x ~ N(0, 1); router and expert weights ~ N(0, 0.02^2) (std
0.02); the selection bias of the DeepSeek-V3-shaped layer ~ U(-0.1, 0.1); the
skewed Qwen3-shaped layer adds to the logits a per-expert offset
-s * ln(rank) with s = 1.2 and rank = e + 1 (the log of an unnormalised Zipf
profile, expert 0 hottest).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["MoEShape", "CONFIGS", "make_inputs", "reduced", "zipf_offsets", "to_e4m3"]


@dataclasses.dataclass(frozen=True)
class MoEShape:
    name: str
    T: int            # tokens
    d: int            # d_model
    N: int            # routed experts
    k: int            # experts kept per token
    F: int            # expert hidden size (d_ff)
    S: int = 0        # always-on shared experts (same d_ff as routed ones)
    dtype: str = "bf16"   # "bf16" or "f32": x, all weights and y
    select_bias: bool = False   # per-expert U(-0.1, 0.1) bias on the selection key only
    zipf_s: float = 0.0         # > 0: add -s*ln(e+1) to the logits
    fp8: bool = False           # expert weights as E4M3 codes + fp32 per-output-channel scales

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def describe(self) -> str:
        extra = []
        if self.S:
            extra.append(f"{self.S} shared")
        if self.select_bias:
            extra.append("selection bias U(-0.1,0.1)")
        if self.zipf_s:
            extra.append(f"Zipf(s={self.zipf_s}) logit offset")
        if self.fp8:
            extra.append("FP8 E4M3 expert weights, per-channel scales")
        tail = (", " + ", ".join(extra)) if extra else ""
        return (f"T={self.T} d_model={self.d} experts={self.N} top-{self.k} "
                f"d_ff={self.F} {self.dtype}{tail}")


CONFIGS: Dict[str, MoEShape] = {
    "tiny_f32": MoEShape("tiny_f32", T=64, d=128, N=4, k=2, F=256, dtype="f32"),
    "mixtral_prefill": MoEShape("mixtral_prefill", T=4096, d=4096, N=8, k=2, F=14336),
    "mixtral_decode": MoEShape("mixtral_decode", T=32, d=4096, N=8, k=2, F=14336),
    "mixtral_decode_fp8": MoEShape("mixtral_decode_fp8", T=32, d=4096, N=8, k=2, F=14336,
                                   fp8=True),
    "mixtral_prefill_fp8": MoEShape("mixtral_prefill_fp8", T=4096, d=4096, N=8, k=2, F=14336,
                                    fp8=True),
    "deepseek_v3_fp8": MoEShape("deepseek_v3_fp8", T=8192, d=7168, N=256, k=8, F=2048, S=1,
                                select_bias=True, fp8=True),
    "deepseek_v3": MoEShape("deepseek_v3", T=8192, d=7168, N=256, k=8, F=2048, S=1,
                            select_bias=True),
    "qwen3_skew": MoEShape("qwen3_skew", T=16384, d=4096, N=128, k=8, F=1536,
                           zipf_s=1.2),
}


def reduced(shape: MoEShape, T: int, d: int, F: int, N: Optional[int] = None,
            name: Optional[str] = None) -> MoEShape:
    """The same routing structure (k, shared, biases, dtype) at smaller sizes."""
    return dataclasses.replace(shape, T=T, d=d, F=F, N=shape.N if N is None else N,
                               name=name or f"{shape.name}_T{T}_d{d}_F{F}")


def zipf_offsets(N: int, s: float) -> torch.Tensor:
    """Per-expert logit offsets -s * ln(rank), rank = 1..N (fp32)."""
    return torch.tensor([-s * math.log(e + 1) for e in range(N)], dtype=torch.float32)


_TAGS = {"x": 1, "w_router": 2, "select_bias": 3, "w_gate": 4, "w_up": 5,
         "w_down": 6, "ws_gate": 7, "ws_up": 8, "ws_down": 9}


def _gen(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + _TAGS[tag])
    return g


def _normal(shape, std, dtype, seed, tag, device, chunk_rows: int = 0):
    """N(0, std^2) drawn in fp32, rounded to ``dtype``; large tensors in row chunks."""
    out = torch.empty(shape, dtype=dtype, device=device)
    g = _gen(seed, tag, device)
    rows = shape[0]
    step = rows if chunk_rows <= 0 else chunk_rows
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        tmp = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                          dtype=torch.float32, device=device)
        if std != 1.0:
            tmp.mul_(std)
        out[r0:r1].copy_(tmp)
        del tmp
    return out


def make_inputs(shape: MoEShape, seed: int = 0, device="cpu",
                weight_std: float = 0.02) -> Dict[str, Optional[torch.Tensor]]:
    """Draw every input of one layer call.

    Returns a dict with x [T,d], w_router [N,d], w_gate/w_up [N,F,d],
    w_down [N,d,F], shared weights ws_gate/ws_up [S,F,d] and ws_down [S,d,F]
    (None when S = 0), logit_bias [N] fp32 or None, select_bias [N] fp32 or None.
    """
    dt = shape.torch_dtype
    T, d, N, F, S = shape.T, shape.d, shape.N, shape.F, shape.S
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal((T, d), 1.0, dt, seed, "x", device)
    out["w_router"] = _normal((N, d), weight_std, dt, seed, "w_router", device)
    per = max(1, (1 << 26) // max(1, F * d))   # experts per fp32 temporary of <= 256 MiB
    out["w_gate"] = _normal((N, F, d), weight_std, dt, seed, "w_gate", device, per)
    out["w_up"] = _normal((N, F, d), weight_std, dt, seed, "w_up", device, per)
    out["w_down"] = _normal((N, d, F), weight_std, dt, seed, "w_down", device, per)
    if S:
        out["ws_gate"] = _normal((S, F, d), weight_std, dt, seed, "ws_gate", device, per)
        out["ws_up"] = _normal((S, F, d), weight_std, dt, seed, "ws_up", device, per)
        out["ws_down"] = _normal((S, d, F), weight_std, dt, seed, "ws_down", device, per)
    else:
        out["ws_gate"] = out["ws_up"] = out["ws_down"] = None
    if shape.select_bias:
        g = _gen(seed, "select_bias", device)
        out["select_bias"] = (torch.rand((N,), generator=g, dtype=torch.float32,
                                         device=device) * 0.2 - 0.1)
    else:
        out["select_bias"] = None
    out["logit_bias"] = (zipf_offsets(N, shape.zipf_s).to(device)
                         if shape.zipf_s > 0 else None)
    if shape.fp8:
        for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
            codes, scale = to_e4m3(out[n]) if out[n] is not None else (None, None)
            out[n], out[n + "_scale"] = codes, scale
    return out


def to_e4m3(w: torch.Tensor, chunk: int = 8):
    """Weights [E, out, in] -> (E4M3 codes as uint8 [E, out, in], fp32 scales
    [E, out]): each output channel scaled so its largest magnitude maps to
    448, the largest finite E4M3 value, then rounded by torch's float8_e4m3fn
    cast.  Input preparation for the FP8 weight format, in chunks of experts."""
    E = w.shape[0]
    codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scale = torch.empty(w.shape[:2], dtype=torch.float32, device=w.device)
    for e0 in range(0, E, chunk):
        wf = w[e0:e0 + chunk].float()
        s = wf.abs().amax(dim=2).clamp_min(1e-30) / 448.0
        codes[e0:e0 + chunk] = (wf / s[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        scale[e0:e0 + chunk] = s
        del wf
    return codes, scale
