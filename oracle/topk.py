"""Block-score top-k mask generation in float64 (oracle, test infrastructure).

What is computed (Ultra Flash notes, key design 3, dynamic block-sparse causal
attention): every attention head rates how related a query block is to a key
block by the dot product of the two blocks' mean-pooled query and key
vectors, and keeps the best-rated key blocks beside a local sliding window.
Readings taken where the notes stop short:
  * Blocks are contiguous 128-token tiles of the step's query rows and of the
    visible keys in key order (the same tiles the attention consumes); the
    last tile may be partial and is averaged over its own tokens only.
  * The block score is the plain dot product of the two means, without the
    1/sqrt(d) attention scale (a positive factor, so the ranking is the same).
    A query head h reads the keys of KV group floor(h * Hkv / Hq).
  * The causal part needs no mask here: every visible key is causally allowed
    (the window holds only past and current frames).  The local window is
    the "diagonal" key tiles, those overlapping the query tile's own key
    positions (the step's queries are the newest n_q of the n_k keys), widened
    by `local_blocks` tiles on each side.  These are always kept.
  * top_k further key tiles are chosen per (head, query tile) row among the
    tiles the local window does not already keep: highest score first, equal
    scores to the lower tile index.  With fewer candidates, all are kept.

Float64 throughout; numpy's mean, matrix product and sort are the only
library steps.
"""
from __future__ import annotations

import numpy as np


def _group_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    return (h * n_kv_heads) // n_q_heads


def pooled_tiles(x: np.ndarray, tile: int = 128) -> np.ndarray:
    """Per-head mean of each tile of consecutive tokens.

    x: [N, H, d] (token-major).  Returns float64 [H, ceil(N/tile), d]; the last
    tile averages only the tokens it has.
    """
    n, h, d = x.shape
    n_t = -(-n // tile)
    out = np.zeros((h, n_t, d), dtype=np.float64)
    for t in range(n_t):
        rows = x[t * tile:min((t + 1) * tile, n)].astype(np.float64)
        out[:, t, :] = rows.mean(axis=0)
    return out


def block_scores(q: np.ndarray, k: np.ndarray, tile: int = 128) -> np.ndarray:
    """Dot products of mean-pooled query and key tiles.

    q: [Nq, Hq, d], k: [Nk, Hkv, d] in key order.  Returns float64
    [Hq, ceil(Nq/tile), ceil(Nk/tile)].
    """
    n_q_heads, n_kv_heads = q.shape[1], k.shape[1]
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    qp = pooled_tiles(q, tile)
    kp = pooled_tiles(k, tile)
    out = np.empty((n_q_heads, qp.shape[1], kp.shape[1]), dtype=np.float64)
    for h in range(n_q_heads):
        out[h] = qp[h] @ kp[_group_of(h, n_q_heads, n_kv_heads)].T
    return out


def local_tiles(q_tile: int, n_q: int, n_k: int, local_blocks: int, tile: int = 128) -> list:
    """Key tiles kept unconditionally for one query tile: the tiles overlapping
    its key positions [n_k - n_q + q_tile*tile, n_k - n_q + min((q_tile+1)*tile, n_q)),
    widened by local_blocks tiles on each side and clipped to the keys."""
    first = n_k - n_q + q_tile * tile
    last = n_k - n_q + min((q_tile + 1) * tile, n_q) - 1
    n_kt = -(-n_k // tile)
    lo = max(0, first // tile - local_blocks)
    hi = min(n_kt - 1, last // tile + local_blocks)
    return list(range(lo, hi + 1))


def topk_block_mask(scores: np.ndarray, n_q: int, n_k: int, top_k: int, local_blocks: int,
                    tile: int = 128) -> np.ndarray:
    """uint8 mask [Hq, n_q_tiles, n_k_tiles]: the local window of every row plus
    its top_k best-scoring other tiles (ties to the lower tile index)."""
    n_heads, n_qt, n_kt = scores.shape
    if n_qt != -(-n_q // tile) or n_kt != -(-n_k // tile):
        raise ValueError("score shape does not match the step")
    if n_q > n_k:
        raise ValueError("more queries than keys")
    mask = np.zeros(scores.shape, dtype=np.uint8)
    for qt in range(n_qt):
        forced = local_tiles(qt, n_q, n_k, local_blocks, tile)
        others = np.setdiff1d(np.arange(n_kt), np.asarray(forced, dtype=np.int64))
        for h in range(n_heads):
            mask[h, qt, forced] = 1
            # stable sort on the negated score: descending score, ascending index among equals
            order = others[np.argsort(-scores[h, qt, others], kind="stable")]
            mask[h, qt, order[:max(0, top_k)]] = 1
    return mask
