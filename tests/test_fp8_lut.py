"""The table-driven FP8 helpers of the GPU tests agree with the oracle they tabulate (CPU)."""
import numpy as np
import pytest

import oracle.fp8 as f8
from tests import fp8_lut


@pytest.mark.parametrize("scale", [0.02, 0.015, 0.005, 0.05, 1.0])
def test_quantize_table_matches_oracle(scale):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200_000) * rng.choice([1e-4, 1e-2, 1.0, 30.0], 200_000)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncate to bf16 patterns
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(fp8_lut.quantize_bits(bits, scale), f8.quantize(vals, scale))
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(fp8_lut.dequantize(codes, scale), f8.dequantize(codes, scale), equal_nan=True)


def test_every_finite_pattern_within_range():
    # all finite bf16 values whose scaled product stays finite are tabulated
    table = fp8_lut._code_table(0.02)
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        ok = np.isfinite(vals) & np.isfinite(vals * np.float32(1 / np.float32(0.02)))
    assert (table[ok] >= 0).all() and (table[~ok] == -1).all()


def test_non_finite_input_is_refused():
    with pytest.raises(ValueError):
        fp8_lut.quantize_bits(np.array([0x7F80], dtype=np.uint16), 0.02)  # +inf
