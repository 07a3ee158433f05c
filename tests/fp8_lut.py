"""Fast exact stand-ins for oracle.fp8.quantize / dequantize on bf16 inputs.

Test inputs are bf16 values, so quantization is a function of the 65536 bit patterns: the
table holds oracle.fp8.quantize of every pattern it accepts, computed once per scale by the
oracle itself, and is then indexed by the input bits.  Dequantization is likewise
oracle.fp8.dequantize of the 256 codes.  Patterns the oracle does not take (non-finite, or
non-finite after the scale) are marked -1 and must not occur in an input.
"""
import functools

import numpy as np

import oracle.fp8 as f8


@functools.lru_cache(maxsize=8)
def _code_table(scale: float) -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    inv = np.float32(1.0 / float(np.float32(scale)))
    with np.errstate(over="ignore", invalid="ignore"):
        ok = np.isfinite(vals) & np.isfinite(vals * inv)
    table = np.full(65536, -1, dtype=np.int16)
    table[ok] = f8.quantize(vals[ok], scale).astype(np.int16)
    return table


@functools.lru_cache(maxsize=8)
def _value_table(scale: float) -> np.ndarray:
    return f8.dequantize(np.arange(256, dtype=np.uint8), scale)


def quantize_bits(bf16_bits: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes (uint8) of bf16 values given by their bit patterns, as oracle.fp8.quantize."""
    codes = _code_table(scale)[np.asarray(bf16_bits, dtype=np.uint16)]
    if (codes < 0).any():
        raise ValueError("input outside what the oracle quantizes")
    return codes.astype(np.uint8)


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """float64 values of E4M3 codes, as oracle.fp8.dequantize."""
    return _value_table(scale)[np.asarray(codes, dtype=np.uint8)]


def round_trip_bits(bf16_bits: np.ndarray, scale: float) -> np.ndarray:
    """dequantize(quantize(x)) for bf16 bit patterns."""
    return dequantize(quantize_bits(bf16_bits, scale), scale)
