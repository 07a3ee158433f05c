"""Workload shapes and seeded generators for the streaming-attention path.

Every tensor is drawn from numpy's PCG64 seeded with
``SeedSequence([workload_index, step, tensor_id])`` (tensor ids: q=0, k=1,
v=2, block mask=3), as float32 standard normals in token-major layout
``[tokens, heads, head_dim]``.  The HIP side receives the bf16 (round to
nearest even) encoding of those draws and the oracle receives the very same
values widened to float64, so both sides see identical inputs.

Shapes follow the latents the pages describe:
  * 480P: the Ultra Flash README mirror's pipeline diagram gives a
    16x60x104 low-resolution latent; 2x2 patches give a 30x52 token grid.
  * 1K / 2K: the same diagram gives a 16x120x208 high-resolution latent
    (60x104 tokens); 1440x2496 pixels at 8x spatial compression and 2x2
    patches give 90x156 tokens.
  * Streaming decoder: FlashDecoder review, model-components table (rolling
    cache of W_frm = 2 frames, G = 3 KV groups) with 12 query heads of 128.
  * FlashDecoder-XL shapes: the model-scaling table's XL row (width 1536,
    24 heads, 3 KV groups, so head_dim 64 and 8 query heads per KV head) on
    720p latents, whose 16x spatial factor (model-components table, spatial
    upsampling) gives a 45x80 token grid.  "decoder-xl" is the backbone's
    per-frame window of W_frm = 2 frames; "refine-xl" is the temporal
    refinement blocks, which take r_t = 4 frames per latent frame and keep a
    window of r_t * W_frm = 8 frames (model-components table; Algorithm 1's
    refinement cache update).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

TILE = 128  # block-mask granularity in tokens (128 = the 2x8x8 block size)

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_MASK = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    dtype: str               # precision the workload is specified in
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    grid: tuple              # latent token grid (H', W') of one frame
    frames_per_step: int     # F: frames appended and queried per step
    window_frames: int       # W: ring frames visible, the current step included
    anchor_frames: int       # A: first frames pinned for the whole stream
    steps: int               # steps streamed
    mask_pct: Optional[int]  # block-mask density in percent, None = dense

    @property
    def tokens_per_frame(self) -> int:
        return self.grid[0] * self.grid[1]

    @property
    def q_tokens(self) -> int:
        return self.frames_per_step * self.tokens_per_frame


WORKLOADS = [
    Workload(0, "tiny", "f32", 2, 2, 64, (8, 8), 1, 3, 0, 6, None),
    Workload(1, "480p", "bf16", 12, 12, 128, (30, 52), 3, 9, 3, 8, None),
    Workload(2, "decoder", "bf16", 12, 3, 128, (30, 52), 1, 2, 0, 120, None),
    Workload(3, "1k", "bf16", 12, 12, 128, (60, 104), 3, 6, 0, 4, 25),
    Workload(4, "2k", "bf16", 12, 12, 128, (90, 156), 3, 6, 0, 4, 15),
    Workload(5, "decoder-xl", "bf16", 24, 3, 64, (45, 80), 1, 2, 0, 24, None),
    Workload(6, "refine-xl", "bf16", 24, 3, 64, (45, 80), 4, 8, 0, 6, None),
]
WORKLOAD = {w.name: w for w in WORKLOADS}  # by name


def _rng(workload_index: int, step: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_index, step, tensor_id])))


def draw_normal(workload_index: int, step: int, tensor_id: int, shape: Sequence[int]) -> np.ndarray:
    """float32 standard normals of `shape` from the (config, step, tensor) stream."""
    return _rng(workload_index, step, tensor_id).standard_normal(tuple(shape), dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 encodings."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((bits[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 encodings to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_step_tensors(cfg: Workload, step: int, scale_q: float = 1.0):
    """q, k, v of one step as bf16 encodings (uint16) in [tokens, heads, head_dim].

    q has n_q_heads heads, k and v have n_kv_heads heads; each holds the
    frames_per_step frames of this step.  `scale_q` multiplies the float32 q
    draw before rounding (a sharper-attention stress variant).
    """
    n = cfg.q_tokens
    q = draw_normal(cfg.index, step, TENSOR_Q, (n, cfg.n_q_heads, cfg.head_dim))
    if scale_q != 1.0:
        q = q * np.float32(scale_q)
    k = draw_normal(cfg.index, step, TENSOR_K, (n, cfg.n_kv_heads, cfg.head_dim))
    v = draw_normal(cfg.index, step, TENSOR_V, (n, cfg.n_kv_heads, cfg.head_dim))
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def diagonal_tiles(q_tile: int, n_q: int, n_k: int, tile: int = TILE) -> list:
    """Key tiles whose token range overlaps the absolute range of query tile `q_tile`.

    The step's queries are the newest n_q of the n_k keys, so query row i sits
    at key position n_k - n_q + i.
    """
    lo = n_k - n_q + q_tile * tile
    hi = n_k - n_q + min((q_tile + 1) * tile, n_q)  # exclusive
    return list(range(lo // tile, (hi - 1) // tile + 1))


def make_block_mask(workload_index: int, step: int, n_heads: int, n_q: int, n_k: int,
                    pct: int, tile: int = TILE) -> np.ndarray:
    """Seeded block mask, uint8 [n_heads, ceil(n_q/tile), ceil(n_k/tile)] (1 = keep).

    Each row (head, query tile) keeps k = max(#diagonal, round(pct * n_k_tiles / 100))
    key tiles: every diagonal tile, plus the rest drawn uniformly without
    replacement from the other tiles.  Rows are drawn in (head, query tile)
    order from the config/step's mask stream.
    """
    nqb = -(-n_q // tile)
    nkb = -(-n_k // tile)
    rng = _rng(workload_index, step, TENSOR_MASK)
    mask = np.zeros((n_heads, nqb, nkb), dtype=np.uint8)
    target = (pct * nkb + 50) // 100
    for h in range(n_heads):
        for qb in range(nqb):
            diag = diagonal_tiles(qb, n_q, n_k, tile)
            keep = max(len(diag), target)
            mask[h, qb, diag] = 1
            others = np.setdiff1d(np.arange(nkb), np.asarray(diag, dtype=np.int64))
            extra = keep - len(diag)
            if extra > 0:
                mask[h, qb, rng.choice(others, size=extra, replace=False)] = 1
    return mask
