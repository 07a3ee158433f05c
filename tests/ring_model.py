"""Independent model of the cache's storage layout, written from include/uf.h.

Storage per KV head is [(A + W) * L rows][d]: rows [0, A*L) hold the anchor
frames in append order, and non-anchor frame r (counting from 0) sits in
ring slot r mod W, i.e. rows A*L + (r mod W)*L ... + L.  This module tracks
which frame each slot holds, frame by frame, with no modular row arithmetic
of the library's kind (recent-key rotation), so that tests can predict the
storage bytes and the physical row of every visible key independently.
"""
from __future__ import annotations

import numpy as np


class RingModel:
    def __init__(self, n_kv_heads, head_dim, tokens_per_frame, window_frames, anchor_frames):
        self.H, self.d, self.L, self.W, self.A = n_kv_heads, head_dim, tokens_per_frame, window_frames, anchor_frames
        rows = (anchor_frames + window_frames) * tokens_per_frame
        self.k = np.zeros((n_kv_heads, rows, head_dim), dtype=np.uint16)
        self.v = np.zeros_like(self.k)
        self.slot_frame = [None] * (anchor_frames + window_frames)  # global frame held by each slot
        self.count = 0
        self.last = 0

    def _slot_for(self, frame):
        if frame < self.A:
            return frame
        ring_index = frame - self.A
        # walk the ring slot by slot instead of taking a modulus
        slot = 0
        for _ in range(ring_index):
            slot = slot + 1 if slot + 1 < self.W else 0
        return self.A + slot

    def first_row(self, frame):
        return self._slot_for(frame) * self.L

    def write(self, frames, k_tok, v_tok):
        """k_tok, v_tok: uint16 [len(frames) * L, H, d] token-major."""
        for i, f in enumerate(frames):
            slot = self._slot_for(f)
            rows = slice(slot * self.L, (slot + 1) * self.L)
            self.k[:, rows, :] = k_tok[i * self.L:(i + 1) * self.L].transpose(1, 0, 2)
            self.v[:, rows, :] = v_tok[i * self.L:(i + 1) * self.L].transpose(1, 0, 2)
            self.slot_frame[slot] = f

    def append(self, n_frames, k_tok=None, v_tok=None):
        frames = list(range(self.count, self.count + n_frames))
        if k_tok is not None:
            self.write(frames, k_tok, v_tok)
        else:
            for f in frames:
                self.slot_frame[self._slot_for(f)] = f
        self.count += n_frames
        self.last = n_frames
        return frames

    def overwrite_newest(self, k_tok, v_tok):
        frames = list(range(self.count - self.last, self.count))
        self.write(frames, k_tok, v_tok)
        return frames

    def visible_rows(self, visible_frames):
        """Physical row of every visible key, in key order, given the visible frames."""
        rows = []
        for f in visible_frames:
            slot = self.slot_frame.index(f)
            rows.extend(range(slot * self.L, (slot + 1) * self.L))
        return np.asarray(rows, dtype=np.int64)
