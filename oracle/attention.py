"""softmax(Q K^T / sqrt(d)) V in float64 (oracle, test infrastructure).

Definition followed (the operation the pages name, with these readings):
  * Scores are q . k / sqrt(d), softmax over the visible keys, output the
    softmax-weighted sum of values.  The 1/sqrt(d) scale is the standard
    attention scale; the pages name the operation without restating it.
  * FlashDecoder review, Eq. 4 and the model-components table: keys and
    values are held per KV group (grouped-query attention, G groups for N
    query heads).  Read here as consecutive query heads sharing a group:
    query head h uses group floor(h * G / N).
  * Ultra Flash notes, key design 3 (dynamic block-sparse causal attention):
    tokens are grouped into 128-token blocks (2x8x8) and each head keeps only
    some (query block, key block) pairs.  Read here as contiguous 128-token
    tiles of the query rows and of the keys in key order; a query row sees
    exactly the keys of the key tiles its (head, query tile) row keeps.
  * A query row that keeps no key at all outputs zeros.

Everything is float64; the only library steps are numpy's matrix product,
exp and reductions.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .window import sliding_window_allowed


def _group_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    return (h * n_kv_heads) // n_q_heads


def _softmax_rows(s: np.ndarray, vh: np.ndarray) -> np.ndarray:
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ vh) / w.sum(axis=1, keepdims=True)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_mask: Optional[np.ndarray] = None,
           rows: Optional[Sequence[int]] = None, tile: int = 128) -> np.ndarray:
    """Attention of queries q [Nq, Hq, d] over keys k, values v [Nk, Hkv, d].

    block_mask: None (every query sees every key) or uint8/bool
      [Hm, ceil(Nq/tile), ceil(Nk/tile)] with Hm == 1 (shared by all heads) or
      Hm == Hq; nonzero keeps the (query tile, key tile) pair.
    rows: optional query row indices; the result then has len(rows) rows in
      that order.
    Returns float64 [n_rows, Hq, d].
    """
    n_q, n_q_heads, d = q.shape
    n_k, n_kv_heads, d_k = k.shape
    if d_k != d or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if n_k == 0:
        raise ValueError("no keys")
    n_qt, n_kt = -(-n_q // tile), -(-n_k // tile)
    if block_mask is not None:
        block_mask = np.asarray(block_mask)
        if block_mask.shape[1:] != (n_qt, n_kt) or block_mask.shape[0] not in (1, n_q_heads):
            raise ValueError("block mask shape does not match the step")
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), n_q_heads, d), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    row_tile = rows // tile
    for h in range(n_q_heads):
        g = _group_of(h, n_q_heads, n_kv_heads)
        kh = k[:, g, :].astype(np.float64)
        vh = v[:, g, :].astype(np.float64)
        for qt in np.unique(row_tile):
            sel = np.nonzero(row_tile == qt)[0]
            qh = q[rows[sel], h, :].astype(np.float64)
            if block_mask is None:
                keys = slice(None)
            else:
                kept_tiles = block_mask[0 if block_mask.shape[0] == 1 else h, qt] != 0
                keys = np.repeat(kept_tiles, tile)[:n_k]
                if not keys.any():
                    continue  # no visible key: the output row stays zero
            s = (qh @ kh[keys].T) * scale
            out[sel, h, :] = _softmax_rows(s, vh[keys])
    return out


def attend_full_sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray, tokens_per_frame: int,
                         frames_per_step: int, window_frames: int, anchor_frames: int) -> np.ndarray:
    """Attention over a whole stream at once under the equivalent sliding-window mask.

    q, k, v hold every token of the stream, frame-major ([T * L, heads, d]).
    Query token t (frame t // L) sees key token u iff sliding_window_allowed
    holds for their frames.  This is the non-streaming statement of the same
    operation; streaming frame by frame must give the same rows.
    """
    n, n_q_heads, d = q.shape
    n_kv_heads = k.shape[1]
    frame = np.arange(n) // tokens_per_frame
    allowed = sliding_window_allowed(frame, frame, frames_per_step, window_frames, anchor_frames)
    out = np.zeros((n, n_q_heads, d), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    for h in range(n_q_heads):
        g = _group_of(h, n_q_heads, n_kv_heads)
        s = (q[:, h, :].astype(np.float64) @ k[:, g, :].astype(np.float64).T) * scale
        s[~allowed] = -np.inf
        out[:, h, :] = _softmax_rows(s, v[:, g, :].astype(np.float64))
    return out


def executed_pairs(n_q: int, n_k: int, n_q_heads: int, block_mask: Optional[np.ndarray] = None,
                   tile: int = 128) -> int:
    """Number of (query row, key, head) score entries the operation defines.

    Dense: n_q * n_k * Hq.  Masked: for every kept (head, query tile, key
    tile), valid rows times valid columns of that tile.  Multiply by 4 * d
    for the floating-point operations of QK^T plus PV.
    """
    if block_mask is None:
        return n_q * n_k * n_q_heads
    bm = np.asarray(block_mask) != 0
    n_qt, n_kt = -(-n_q // tile), -(-n_k // tile)
    rows = np.minimum(tile, n_q - tile * np.arange(n_qt))
    cols = np.minimum(tile, n_k - tile * np.arange(n_kt))
    per_head = (bm * rows[None, :, None] * cols[None, None, :]).sum()
    if bm.shape[0] == 1:
        per_head = per_head * n_q_heads
    return int(per_head)
