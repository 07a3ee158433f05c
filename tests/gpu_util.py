"""Helpers shared by the GPU tests: device transfer and error metrics."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle
from synth import TILE, bf16_bits_to_f32

# Parity bar for bf16 inputs with fp32 accumulation (maximum absolute error
# and relative L2 error against the float64 oracle).
MAX_ABS = 2e-2
REL_L2 = 5e-3


def to_dev(bits: np.ndarray):
    """uint16 bf16 encodings -> torch bf16 tensor on cuda:0 (same bytes)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def bits_of(t) -> np.ndarray:
    """torch bf16 tensor -> uint16 encodings on the host."""
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_of(t) -> np.ndarray:
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


def _host_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def map_row_tiles(fn, rows, tiles_per_call: int = 2):
    """np.concatenate([fn(r) for r in groups]) where the groups cut `rows` at query-tile
    boundaries, `tiles_per_call` tiles each, and run on threads of their own (numpy's matrix
    products and exponentials release the GIL; BLAS runs one thread per call).  Row order is
    kept, so for a row-wise fn the result equals fn(rows)."""
    rows = np.asarray(rows, dtype=np.int64)
    tiles = rows // TILE
    cuts = [0] + [i for i in range(1, len(rows)) if tiles[i] != tiles[i - 1]] + [len(rows)]
    groups = [rows[cuts[i]:cuts[min(i + tiles_per_call, len(cuts) - 1)]]
              for i in range(0, len(cuts) - 1, tiles_per_call)]
    with threadpool_limits(1), ThreadPoolExecutor(_host_threads()) as ex:
        parts = list(ex.map(fn, groups))
    return np.concatenate(parts, axis=0)


def oracle_rows(q, k, v, mask, rows):
    """oracle.attend(q, k, v, mask, rows=rows): the unchanged oracle, called on groups of whole
    query tiles in parallel (map_row_tiles)."""
    return map_row_tiles(lambda r: oracle.attend(q, k, v, mask, rows=r), rows)
