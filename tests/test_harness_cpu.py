"""CPU checks of the GPU harness's own helpers (no GPU)."""
import numpy as np
import torch

import oracle
from gpu_harness import fast_dequantize


def test_fast_dequantize_is_the_oracles_decode_bitwise():
    """The table-driven decode used at full size gives bitwise the float64
    values of oracle.dequantize (O9), NaN codes included, for every code and
    random per-channel scales."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(3, 40, 256), dtype=np.uint8)
    codes[0, 0, :] = np.arange(256, dtype=np.uint8)      # every code once
    scale = (rng.random((3, 40)) * 3.0).astype(np.float32)
    ref = oracle.dequantize(codes, scale)
    got = fast_dequantize(torch.from_numpy(codes), torch.from_numpy(scale))
    assert got.dtype == np.float64 and got.shape == ref.shape
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.nan_to_num(got), np.nan_to_num(ref))
    # one matrix, as the harness hands them over per expert
    one = fast_dequantize(torch.from_numpy(codes[1]), torch.from_numpy(scale[1]))
    assert np.array_equal(np.nan_to_num(one), np.nan_to_num(ref[1]))
