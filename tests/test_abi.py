"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH),
                                reason="libmoe.so not built (run __graft_entry__.build())")


def declared_functions():
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_layer_forward", "moe_route", "moe_balance_stats",
                     "moe_workspace_size", "moe_status_string", "moe_layer_backward",
                     "moe_backward_workspace_size", "moe_update_select_bias"):
        assert required in names


def test_every_declared_symbol_is_exported():
    lib = moe.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in moe.h but not exported"


def test_status_strings():
    for code in range(5):
        assert moe.moe_status_string(code).startswith("MOE_")
    assert "unknown" in moe.moe_status_string(99)


def test_config_struct_matches_the_header():
    """The binding's moe_config mirrors include/moe.h field by field."""
    import re
    with open(os.path.join(ROOT, "include", "moe.h")) as fh:
        hdr = fh.read()
    body = re.search(r"typedef struct \{([^}]*)\} moe_config;", hdr).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [f for f, _ in moe.MoEConfig._fields_]
    body = re.search(r"typedef struct \{(.*?)\} moe_weights;", hdr, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    wfields = re.findall(r"const (?:void|float)\*\s+(\w+);", body)
    assert wfields == [f for f, _ in moe.MoEWeights._fields_]
    cap = moe.make_config(64, 128, 4, 2, 256, capacity=7)
    assert cap.capacity == 7 and moe.make_config(64, 128, 4, 2, 256).capacity == 0


def test_workspace_size_validation():
    ok = moe.make_config(64, 128, 4, 2, 256, 0, "f32")
    n = moe.moe_workspace_size(ok)
    assert n > 0 and n % 256 == 0
    # grows with T, never shrinks
    assert moe.moe_workspace_size(moe.make_config(128, 128, 4, 2, 256, 0, "f32")) > n
    for bad in [moe.make_config(64, 100, 4, 2, 256), moe.make_config(64, 128, 4, 5, 256),
                moe.make_config(64, 128, 600, 2, 256), moe.make_config(64, 128, 40, 17, 256),
                moe.make_config(-1, 128, 4, 2, 256), moe.make_config(64, 128, 4, 2, 96),
                moe.make_config(64, 128, 4, 2, 256, n_shared=5),
                moe.make_config(64, 128, 4, 2, 256, capacity=-1),
                moe.make_config(64, 128, 4, 2, 256, weight_format=2),
                moe.make_config(64, 128, 4, 2, 256, 0, "f32",
                                weight_format=moe.MOE_WEIGHTS_FP8_E4M3)]:
        assert moe.moe_workspace_size(bad) == 0
    fp8 = moe.make_config(64, 128, 4, 2, 256, weight_format=moe.MOE_WEIGHTS_FP8_E4M3)
    assert moe.moe_workspace_size(fp8) > 0


def _call_forward(cfg, weights=None, x=1 << 20, y=1 << 20, ws=None, ws_bytes=0):
    lib = moe.lib()
    return lib.moe_layer_forward(ctypes.byref(cfg) if cfg is not None else None, x,
                                 ctypes.byref(weights) if weights is not None else None, y,
                                 None, ws, ws_bytes, None)


FAKE = 1 << 20  # a 256-byte aligned non-null address; never dereferenced on these paths


def _w(**over):
    w = moe.MoEWeights(FAKE, FAKE, FAKE, FAKE, None, None, None, None, None,
                       None, None, None, None, None, None)
    for k_, v in over.items():
        setattr(w, k_, v)
    return w


@pytest.mark.parametrize("case,expect", [
    ("null_cfg", moe.MOE_ERR_INVALID_ARG),
    ("k_gt_n", moe.MOE_ERR_INVALID_ARG),
    ("zero_k", moe.MOE_ERR_INVALID_ARG),
    ("bad_dtype", moe.MOE_ERR_INVALID_ARG),
    ("too_many_experts", moe.MOE_ERR_UNSUPPORTED),
    ("k_above_16", moe.MOE_ERR_UNSUPPORTED),
    ("d_not_64", moe.MOE_ERR_UNSUPPORTED),
    ("null_weights", moe.MOE_ERR_INVALID_ARG),
    ("null_router", moe.MOE_ERR_INVALID_ARG),
    ("null_expert", moe.MOE_ERR_INVALID_ARG),
    ("shared_missing", moe.MOE_ERR_INVALID_ARG),
    ("misaligned_weight", moe.MOE_ERR_INVALID_ARG),
    ("fp8_scale_missing", moe.MOE_ERR_INVALID_ARG),
    ("fp8_with_f32", moe.MOE_ERR_UNSUPPORTED),
    ("bad_weight_format", moe.MOE_ERR_INVALID_ARG),
    ("null_x", moe.MOE_ERR_INVALID_ARG),
    ("no_workspace", moe.MOE_ERR_WORKSPACE),
    ("small_workspace", moe.MOE_ERR_WORKSPACE),
    ("misaligned_workspace", moe.MOE_ERR_WORKSPACE),
    ("empty_batch", moe.MOE_OK),
])
def test_forward_rejects_before_launch(case, expect):
    cfg = moe.make_config(64, 128, 4, 2, 256)
    w = _w()
    kw = {}
    if case == "null_cfg":
        cfg = None
    elif case == "k_gt_n":
        cfg = moe.make_config(64, 128, 4, 5, 256)
    elif case == "zero_k":
        cfg = moe.make_config(64, 128, 4, 0, 256)
    elif case == "bad_dtype":
        cfg.dtype = 7
    elif case == "too_many_experts":
        cfg = moe.make_config(64, 128, 513, 2, 256)
    elif case == "k_above_16":
        cfg = moe.make_config(64, 128, 64, 17, 256)
    elif case == "d_not_64":
        cfg = moe.make_config(64, 96, 4, 2, 256)
    elif case == "null_weights":
        w = None
    elif case == "null_router":
        w = _w(w_router=None)
    elif case == "null_expert":
        w = _w(w_down=None)
    elif case == "shared_missing":
        cfg = moe.make_config(64, 128, 4, 2, 256, n_shared=1)
    elif case == "misaligned_weight":
        w = _w(w_up=FAKE + 2)
    elif case == "fp8_scale_missing":
        cfg.weight_format = moe.MOE_WEIGHTS_FP8_E4M3
        w = _w(w_gate_scale=FAKE, w_up_scale=FAKE)  # down scale missing
    elif case == "fp8_with_f32":
        cfg = moe.make_config(64, 128, 4, 2, 256, 0, "f32",
                              weight_format=moe.MOE_WEIGHTS_FP8_E4M3)
    elif case == "bad_weight_format":
        cfg.weight_format = 5
    elif case == "null_x":
        kw = {"x": None}
    elif case == "no_workspace":
        kw = {"ws": None, "ws_bytes": 10 ** 9}
    elif case == "small_workspace":
        kw = {"ws": FAKE, "ws_bytes": 256}
    elif case == "misaligned_workspace":
        kw = {"ws": FAKE + 64, "ws_bytes": 10 ** 9}
    elif case == "empty_batch":
        cfg = moe.make_config(0, 128, 4, 2, 256)
        kw = {"x": None, "y": None}
    assert _call_forward(cfg, w, **kw) == expect
    if expect != moe.MOE_OK:
        assert moe.lib().moe_last_error()


def test_routing_struct_matches_the_header():
    with open(HEADER) as fh:
        hdr = fh.read()
    body = re.search(r"typedef struct \{([^}]*)\} moe_routing;", hdr).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(?:float|int32_t)\*?\s+(\w+);", body)
    assert fields == [f for f, _ in moe.MoERouting._fields_]


def test_route_requires_outputs():
    lib = moe.lib()
    cfg = moe.make_config(64, 128, 4, 2, 256)
    w = _w()
    r = moe.MoERouting(None, None, None, None, None)
    st = lib.moe_route(ctypes.byref(cfg), FAKE, ctypes.byref(w), ctypes.byref(r), FAKE, 10 ** 9,
                       None)
    assert st == moe.MOE_ERR_INVALID_ARG


def test_balance_stats_validation():
    lib = moe.lib()
    assert lib.moe_balance_stats(10, 4, 5, FAKE, FAKE, 0.01, FAKE, FAKE, FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_balance_stats(10, 4, 2, None, FAKE, 0.01, FAKE, FAKE, FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_balance_stats(10, 600, 2, FAKE, FAKE, 0.01, FAKE, FAKE, FAKE, None) == \
        moe.MOE_ERR_UNSUPPORTED


# ----------------------------------------------------------------- backward
def test_grads_struct_matches_the_header():
    with open(HEADER) as fh:
        hdr = fh.read()
    body = re.search(r"typedef struct \{([^}]*)\} moe_grads;", hdr).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(?:void|float)\*\s+(\w+);", body)
    assert fields == [f for f, _ in moe.MoEGrads._fields_]


def test_backward_workspace_size():
    lib = moe.lib()
    cfg = moe.make_config(64, 128, 4, 2, 256, n_shared=1)
    fwd = lib.moe_workspace_size(ctypes.byref(cfg))
    bwd = lib.moe_backward_workspace_size(ctypes.byref(cfg))
    # at least the transposed expert weights: 3 matrices of F x d per expert
    assert bwd % 256 == 0 and bwd >= 3 * 5 * 256 * 128 * 2 and bwd > fwd
    bad = moe.make_config(64, 96, 4, 2, 256)
    assert lib.moe_backward_workspace_size(ctypes.byref(bad)) == 0
    # bf16 on 256-row tiles reads the expert weights as K-rows: the workspace
    # holds no transposed copies (those alone would be 22.6 GB here)
    big = moe.make_config(8192, 7168, 256, 8, 2048, n_shared=1)
    copies = 3 * 257 * 2048 * 7168 * 2
    assert 0 < lib.moe_backward_workspace_size(ctypes.byref(big)) < copies // 2
    # fp32 layers still transpose them
    big32 = moe.make_config(8192, 7168, 256, 8, 2048, n_shared=1, dtype="f32")
    assert lib.moe_backward_workspace_size(ctypes.byref(big32)) > 2 * copies


def test_workspace_sizes_of_an_empty_batch():
    """T = 0 is a valid size: both queries answer (and do not divide by the
    number of token blocks)."""
    lib = moe.lib()
    cfg = moe.make_config(0, 128, 4, 2, 256, n_shared=1)
    assert lib.moe_workspace_size(ctypes.byref(cfg)) > 0
    assert lib.moe_backward_workspace_size(ctypes.byref(cfg)) > 0


def _grads(**over):
    g = {n: FAKE for n, _ in moe.MoEGrads._fields_}
    g.update(over)
    return moe.MoEGrads(**g)


@pytest.mark.parametrize("case,expect", [
    ("null_grads", moe.MOE_ERR_INVALID_ARG),
    ("null_dx", moe.MOE_ERR_INVALID_ARG),
    ("null_dw_down", moe.MOE_ERR_INVALID_ARG),
    ("misaligned_grad", moe.MOE_ERR_INVALID_ARG),
    ("shared_grad_missing", moe.MOE_ERR_INVALID_ARG),
    ("fp8_weights", moe.MOE_ERR_UNSUPPORTED),
    ("null_dy", moe.MOE_ERR_INVALID_ARG),
    ("small_workspace", moe.MOE_ERR_WORKSPACE),
    ("forward_sized_workspace", moe.MOE_ERR_WORKSPACE),
    ("bad_cfg", moe.MOE_ERR_UNSUPPORTED),
])
def test_backward_rejects_before_launch(case, expect):
    lib = moe.lib()
    cfg = moe.make_config(64, 128, 4, 2, 256)
    w = _w()
    g = _grads()
    x = dy = FAKE
    ws, ws_bytes = FAKE, 10 ** 12
    if case == "null_grads":
        g = None
    elif case == "null_dx":
        g = _grads(dx=None)
    elif case == "null_dw_down":
        g = _grads(dw_down=None)
    elif case == "misaligned_grad":
        g = _grads(dw_up=FAKE + 4)
    elif case == "shared_grad_missing":
        cfg = moe.make_config(64, 128, 4, 2, 256, n_shared=1)
        w = _w(ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE)
        g = _grads(dws_up=None)
    elif case == "fp8_weights":
        cfg.weight_format = moe.MOE_WEIGHTS_FP8_E4M3
        w = _w(w_gate_scale=FAKE, w_up_scale=FAKE, w_down_scale=FAKE)
    elif case == "null_dy":
        dy = None
    elif case == "small_workspace":
        ws_bytes = 256
    elif case == "forward_sized_workspace":
        ws_bytes = lib.moe_workspace_size(ctypes.byref(cfg))
    elif case == "bad_cfg":
        cfg = moe.make_config(64, 96, 4, 2, 256)
    st = lib.moe_layer_backward(ctypes.byref(cfg), x, ctypes.byref(w), dy, 0.01, 1.0,
                                None if g is None else ctypes.byref(g), ws, ws_bytes, None)
    assert st == expect
    assert lib.moe_last_error()


def test_select_bias_update_validation():
    lib = moe.lib()
    assert lib.moe_update_select_bias(0, FAKE, 0.1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_update_select_bias(4, None, 0.1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_update_select_bias(4, FAKE, 0.1, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_update_select_bias(513, FAKE, 0.1, FAKE, None) == moe.MOE_ERR_UNSUPPORTED


def test_forward_plan_reports_the_path():
    """moe_forward_plan: kernel choices, tile rows and splits of the benchmark
    shapes, consistent with the workspace size (no GPU needed)."""
    pre = moe.make_config(4096, 4096, 8, 2, 14336)
    info = moe.moe_forward_plan(pre)
    assert (info["up_kernel"], info["up_tile_rows"]) == (1, 256)
    assert (info["down_kernel"], info["down_tile_rows"]) == (1, 256)
    assert info["down_split"] == 1 and info["tail_split_cols"] == 4096 // 256
    assert info["workspace_bytes"] == moe.moe_workspace_size(pre)
    off = info["split_plan_offset"]
    assert off % 4 == 0 and off + 16 <= info["workspace_bytes"]
    assert info["all_token_pass"] == 0
    dec = moe.moe_forward_plan(moe.make_config(32, 4096, 8, 2, 14336))
    assert (dec["up_kernel"], dec["up_tile_rows"]) == (0, 32) and dec["down_split"] >= 2
    # the decode batch: every expert runs on all 32 tokens (8 (3/4)^32 idle
    # experts expected); its expert rows are (N + S) T, not T (k + S)
    assert dec["all_token_pass"] == 1
    # one token of 8 experts (6 idle expected), 256 experts, or 33 tokens: not
    assert moe.moe_forward_plan(moe.make_config(1, 4096, 8, 2, 14336))["all_token_pass"] == 0
    assert moe.moe_forward_plan(moe.make_config(32, 7168, 256, 8, 2048, 1))["all_token_pass"] == 0
    assert moe.moe_forward_plan(moe.make_config(33, 4096, 8, 2, 14336))["all_token_pass"] == 0
    assert moe.moe_forward_plan(moe.make_config(1, 256, 4, 4, 256))["all_token_pass"] == 1
    fp8 = moe.make_config(32, 4096, 8, 2, 14336, weight_format=moe.MOE_WEIGHTS_FP8_E4M3)
    assert moe.moe_forward_plan(fp8)["all_token_pass"] == 0  # FP8 weights: the routed rows
    assert info["route_kernel"] == 0  # 8 experts: the router kernel
    ds = moe.moe_forward_plan(moe.make_config(8192, 7168, 256, 8, 2048, 1))
    # 256 experts: the router GEMM on the large-tile kernel, 32 tiles of 256
    # tokens x 8 parts of the reduction on 256 compute units
    if ds["compute_units"] == 256:
        assert (ds["route_kernel"], ds["route_split"]) == (1, 8)
    assert ds["route_kernel"] == 1 and 1 <= ds["route_split"] <= 8
    qw = moe.moe_forward_plan(moe.make_config(16384, 4096, 128, 8, 1536))
    assert qw["route_kernel"] == 1  # 128 experts: the large-tile kernel too
    few = moe.moe_forward_plan(moe.make_config(4096, 4096, 96, 8, 1536))
    assert few["route_kernel"] == 0  # 96 experts: the router kernel
    f32 = moe.moe_forward_plan(moe.make_config(64, 128, 4, 2, 256, 0, "f32"))
    assert f32["up_kernel"] == 0 and f32["tail_split_cols"] == 0
    with pytest.raises(moe.MoEError):
        moe.moe_forward_plan(moe.make_config(64, 100, 4, 2, 256))
    assert moe.lib().moe_forward_plan(ctypes.byref(pre), None) == moe.MOE_ERR_INVALID_ARG
