"""The streaming key window as a plain list of frames (oracle, test infrastructure).

Readings of the pages followed here:
  * FlashDecoder review, "Rolling KV cache" and the model-components table:
    each latent frame attends to a fixed window of W_frm frames that holds
    the frame itself and the frames just before it (W_frm = 2 means itself
    plus one previous frame); Eq. 4 sizes the cache at W_frm * L_frm keys.
    So W counts frames *including* the current ones.
  * FlashDecoder review, "causality by processing order": there is no mask
    inside the window; a frame sees every key in the window, its own frame
    included, and never a frame that has not been appended yet.
  * HiStream summary, innovation 2 (anchor-guided sliding window): one anchor
    chunk stays in context next to the recent frames, so the context stays a
    fixed size.  Read here as: the first A frames ever appended are pinned,
    come first in key order, and are never also counted in the recent window.
  * Ultra Flash notes, key design 4 (dynamic cache management, item iii): the
    recent window may be cropped at run time; a crop to `active` frames keeps
    the newest `active` recent frames.
  * FlashDecoder review, Algorithm 1: the cache update keeps the tail of the
    old cache and appends the new frame's K/V after it, so keys are ordered
    oldest to newest.
"""
from __future__ import annotations

from typing import List

import numpy as np


class FrameListWindow:
    """Keys and values of a stream held as a list of whole frames.

    k and v of one frame are arrays [tokens_per_frame, n_kv_heads, head_dim];
    they are stored as given (bf16 values are exact in float32) and widened
    to float64 only by the attention routine.
    """

    def __init__(self, tokens_per_frame: int, window_frames: int, anchor_frames: int = 0):
        if tokens_per_frame <= 0 or window_frames <= 0 or anchor_frames < 0:
            raise ValueError("bad window description")
        self.L = tokens_per_frame
        self.W = window_frames
        self.A = anchor_frames
        self.active = window_frames
        self.frames = {}          # global frame index -> (k, v)
        self.count = 0            # frames appended so far
        self.last_append = 0

    def _split(self, x: np.ndarray, n_frames: int):
        if x.shape[0] != n_frames * self.L:
            raise ValueError("token count is not n_frames * tokens_per_frame")
        return [x[f * self.L:(f + 1) * self.L] for f in range(n_frames)]

    def append(self, k: np.ndarray, v: np.ndarray, n_frames: int) -> None:
        """Append n_frames new frames (oldest first)."""
        if n_frames <= 0:
            raise ValueError("n_frames must be positive")
        ks, vs = self._split(k, n_frames), self._split(v, n_frames)
        for f in range(n_frames):
            self.frames[self.count] = (ks[f], vs[f])
            self.count += 1
        self.last_append = n_frames
        self._forget()

    def overwrite_newest(self, k: np.ndarray, v: np.ndarray, n_frames: int) -> None:
        """Replace the K/V of the newest n_frames frames (same frame count as the last append)."""
        if n_frames != self.last_append or n_frames <= 0:
            raise ValueError("overwrite must cover exactly the newest append")
        ks, vs = self._split(k, n_frames), self._split(v, n_frames)
        for f in range(n_frames):
            self.frames[self.count - n_frames + f] = (ks[f], vs[f])

    def set_active(self, active_frames: int) -> None:
        """Crop the recent window to its newest `active_frames` frames (1..W)."""
        if not 1 <= active_frames <= self.W:
            raise ValueError("active window must lie in 1..W")
        self.active = active_frames

    def visible(self) -> List[int]:
        return visible_frames_after(self.count, self.W, self.A, self.active)

    def _forget(self) -> None:
        keep = set(range(min(self.A, self.count)))
        keep.update(range(max(self.A, self.count - self.W), self.count))
        for f in list(self.frames):
            if f not in keep:
                del self.frames[f]

    def keys_values(self):
        """(K, V) of the visible frames in key order, each [n_keys, n_kv_heads, head_dim]."""
        vis = self.visible()
        if not vis:
            raise ValueError("no frame appended yet")
        k = np.concatenate([self.frames[f][0] for f in vis], axis=0)
        v = np.concatenate([self.frames[f][1] for f in vis], axis=0)
        return k, v


def visible_frames_after(count: int, window_frames: int, anchor_frames: int,
                         active_frames: int = None) -> List[int]:
    """Global indices of the frames visible once `count` frames have been appended.

    The anchor frames (the first `anchor_frames` appended) come first, then
    the newest min(active, W) of the other frames, oldest to newest.
    """
    active = window_frames if active_frames is None else active_frames
    anchors = list(range(min(anchor_frames, count)))
    recent_lo = max(anchor_frames, count - min(active, window_frames))
    return anchors + list(range(recent_lo, count))


def sliding_window_allowed(frame_q: np.ndarray, frame_k: np.ndarray, frames_per_step: int,
                           window_frames: int, anchor_frames: int) -> np.ndarray:
    """Full-sequence mask equivalent to streaming in steps of `frames_per_step` frames.

    A query in frame fq is processed in step s = fq // F, after frames
    [0, (s+1) F) have been appended.  It may see key frame fk iff fk has been
    appended and is an anchor frame or one of the newest W non-anchor frames:
        fk < min(A, end)  or  max(A, end - W) <= fk < end,   end = (s+1) F.
    Broadcasts over frame_q (rows) and frame_k (columns).
    """
    fq = np.asarray(frame_q)[:, None]
    fk = np.asarray(frame_k)[None, :]
    end = (fq // frames_per_step + 1) * frames_per_step
    anchor = fk < np.minimum(anchor_frames, end)
    recent = (fk >= np.maximum(anchor_frames, end - window_frames)) & (fk < end)
    return anchor | recent
