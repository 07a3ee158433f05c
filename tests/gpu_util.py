"""Helpers shared by the GPU tests: device transfer and error metrics."""
from __future__ import annotations

import numpy as np
import torch

from synth import bf16_bits_to_f32

# Parity bar for bf16 inputs with fp32 accumulation (maximum absolute error
# and relative L2 error against the float64 oracle).
MAX_ABS = 2e-2
REL_L2 = 5e-3


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 encodings -> torch bf16 tensor on cuda:0 (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def bits_of(t: torch.Tensor) -> np.ndarray:
    """torch bf16 tensor -> uint16 encodings on the host."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_of(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_to_f32(bits_of(t))


def errors(got: np.ndarray, ref: np.ndarray):
    got = got.astype(np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = errors(got, ref)
    print(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"
    return ma, rl
