"""The FP8 attention bound of tests/fp8_bound.py holds for an emulation of the kernel's
arithmetic (CPU only).

The emulation follows what the FP8 kernel computes from the dequantized q, k and v: per
query row, probabilities 2^(log2(e) (s_j - max s) + delta) against a reference point delta
in [0, 8] above the row max (the lazy rescaling lets the reference lag by up to 2^8), each
rounded to E4M3 by the oracle's encoder, the output sum_j p_j v_j / sum_j p_j over those
rounded values, then rounded to float32 and to bf16 (nearest even).  Every element must lie
within the bound the GPU tests apply, and the bound must not be vacuous.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.fp8 as f8
from tests.fp8_bound import TILE, bound


def _to_bf16(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def _emulate(q, k, v, mask, rng, delta=None):
    n_q, hq, d = q.shape
    group = hq // k.shape[1]
    out = np.zeros((n_q, hq, d))
    for h in range(hq):
        kh, vh = k[:, h // group], v[:, h // group]
        for qt in range(-(-n_q // TILE)):
            rows = np.arange(qt * TILE, min((qt + 1) * TILE, n_q))
            keys = np.ones(k.shape[0], dtype=bool)
            if mask is not None:
                keys = np.repeat(mask[h, qt] != 0, TILE)[:k.shape[0]]
            s = q[rows, h] @ kh[keys].T / math.sqrt(d)
            dl = rng.uniform(0.0, 8.0, size=(len(rows), 1)) if delta is None else np.full((len(rows), 1), delta)
            p = np.exp2(math.log2(math.e) * (s - s.max(axis=1, keepdims=True)) + dl)
            pr = f8.e4m3_decode(f8.e4m3_encode(p))
            out[rows, h] = (pr @ vh[keys]) / pr.sum(axis=1, keepdims=True)
    return _to_bf16(out)


def _quantized(rng, shape, scale, mult=1.0):
    return f8.dequantize(f8.quantize(rng.standard_normal(shape) * mult, scale), scale)


CASES = [
    # (seed, n_q, n_k, Hq, Hkv, d, q multiplier, mask density %, fixed delta)
    (1, 128, 1000, 2, 2, 128, 1.0, None, None),
    (2, 200, 700, 4, 2, 64, 1.0, 40, None),
    (3, 128, 900, 2, 1, 128, 4.0, None, None),   # sharper attention (q x 4)
    (4, 128, 600, 2, 2, 128, 1.0, None, 0.0),    # reference at the row max
    (5, 128, 600, 2, 2, 128, 1.0, None, 8.0),    # reference lagging by the full 2^8
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_bound_holds_for_emulated_kernel(case):
    seed, n_q, n_k, hq, hkv, d, qmul, pct, delta = case
    rng = np.random.default_rng(seed)
    q = _quantized(rng, (n_q, hq, d), 0.02 * qmul, qmul)
    k = _quantized(rng, (n_k, hkv, d), 0.015)
    v = _quantized(rng, (n_k, hkv, d), 0.02)
    mask = None
    if pct is not None:
        nqt, nkt = -(-n_q // TILE), -(-n_k // TILE)
        mask = (rng.uniform(size=(hq, nqt, nkt)) < pct / 100).astype(np.uint8)
        mask[:, :, 0] = 1  # no empty rows
    ref = oracle.attend(q, k, v, mask)
    got = _emulate(q, k, v, mask, rng, delta)
    b = bound(q, k, v, ref, mask, np.arange(n_q))
    assert np.isfinite(b).all()
    ratio = np.abs(got - ref) / b
    print(f"case {seed}: largest error / bound = {ratio.max():.3f}")
    assert ratio.max() <= 1.0
    assert ratio.max() > 0.01  # the bound is not vacuous for this arithmetic
