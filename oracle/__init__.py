"""Reference oracle for chunk-causal rolling-window attention (TEST INFRASTRUCTURE).

Plain, slow, float64 numpy code that states what the streaming attention
path computes, so that the HIP library can be checked against it.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import this
package; the product path never calls it and shares no code with it.

Contents
  window.py     the streaming window as a plain list of frames (anchor frames
                plus the newest W frames) and the equivalent full-sequence
                sliding-window mask.
  attention.py  softmax(Q K^T / sqrt(d)) V in float64 over a key set, with the
                optional 128x128 block mask and grouped-query heads.
  topk.py       the block mask a head chooses for itself: mean-pooled query and
                key tiles, their dot-product scores, and the local window plus
                the top-k best-scoring other key tiles of every row.
  fp8.py        FP8 E4M3 encoding and static-scale quantization of q, k, v;
                the FP8 path's attention is attend() on the dequantized values.
  blocks.py     the (2, 8, 8) spatio-temporal block order of a step's tokens.

Every function is pinned by tests in tests/test_oracle_pins.py,
tests/test_oracle_topk.py, tests/test_oracle_fp8.py and
tests/test_oracle_blocks.py (closed forms,
invariants, the window tables derived from the pages, hand-worked top-k and
E4M3 examples, brute force over subsets and over all E4M3 codes, and
PyTorch's scaled_dot_product_attention in float64 on small cases).  Parity unpinned:
none.
"""
from .window import FrameListWindow, sliding_window_allowed, visible_frames_after
from .attention import attend, attend_full_sequence, executed_pairs
from .topk import block_scores, local_tiles, pooled_tiles, topk_block_mask

__all__ = [
    "FrameListWindow",
    "sliding_window_allowed",
    "visible_frames_after",
    "attend",
    "attend_full_sequence",
    "executed_pairs",
    "block_scores",
    "local_tiles",
    "pooled_tiles",
    "topk_block_mask",
]
