"""Per-element error bound of the FP8 attention kernel against the oracle.

The oracle attends in float64 over the dequantized q, k and v.  The kernel differs from it
by rounding the probabilities to E4M3 for the P.V product (and the row sums it divides by),
and by rounding the output to bf16.  With the weights p of a row normalised to a maximum of
1, E4M3 rounding moves each weight by at most e_j = max(2^-4 p_j, 2^-10): half an ulp,
relative 2^-4 for normal codes and absolute 2^-10 below 2^-6.  The kernel's probabilities
are p_j 2^delta for a reference point delta in [0, 8] above the row max (lazy rescaling),
which scales the absolute term by 2^-delta <= 1.  With the same rounded weights in the
numerator and the denominator,
    |out - ref| <= sum_j e_j |v_j - ref| / (sum_j p_j - sum_j e_j)
               <= (sum_j e_j |v_j| + |ref| sum_j e_j) / (sum_j p_j - sum_j e_j),
plus 2^-9 |ref| for the bf16 output and 1e-6 for the fp32 sums.  Where the denominator is
not positive the bound says nothing and is infinite.
"""
import math

import numpy as np

TILE = 128


def bound(q, k, v, ref, mask, rows):
    """[len(rows), Hq, d] bound on |kernel - oracle| for the query rows `rows`.

    q [Nq, Hq, d], k and v [Nk, Hkv, d] are the dequantized values, ref the oracle's output
    for those rows, mask the block mask (or None)."""
    n_q_heads, d = q.shape[1], q.shape[2]
    group = n_q_heads // k.shape[1]
    out = np.zeros_like(ref)
    row_tile = rows // TILE
    for h in range(n_q_heads):
        kh, vh = k[:, h // group, :], v[:, h // group, :]
        for qt in np.unique(row_tile):
            sel = np.nonzero(row_tile == qt)[0]
            keys = np.ones(k.shape[0], dtype=bool)
            if mask is not None:
                keys = np.repeat(mask[0 if mask.shape[0] == 1 else h, qt] != 0, TILE)[:k.shape[0]]
            if not keys.any():
                continue
            s = q[rows[sel], h, :] @ kh[keys].T / math.sqrt(d)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            e = np.maximum(2.0 ** -4 * p, 2.0 ** -10)
            num = e @ np.abs(vh[keys]) + np.abs(ref[sel, h, :]) * e.sum(axis=1)[:, None]
            den = p.sum(axis=1) - e.sum(axis=1)
            with np.errstate(divide="ignore"):
                out[sel, h, :] = np.where(den[:, None] > 0, num / np.maximum(den, 1e-300)[:, None], np.inf)
    return out + 2.0 ** -9 * np.abs(ref) + 1e-6
