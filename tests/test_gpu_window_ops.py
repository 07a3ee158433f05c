"""Attention after the window operations, on the GPU against the oracle.

A stream with an anchor, a per-head block mask and GQA goes through:
  * a re-write of the newest chunk in place (UF_APPEND_OVERWRITE_NEWEST: the multi-step
    denoising of one chunk and the reuse of its last step's K/V, Ultra Flash notes, key
    design 4, item ii);
  * a crop of the recent window (uf_kvcache_set_window, key design 4, item iii), then its
    restoration;
for a bf16 cache, an FP8 cache and a cache held in block order.  The oracle's frame list
takes the same operations (overwrite_newest, set_active).
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8
import oracle.blocks as ob
from synth import Workload, bf16_bits_to_f32, draw_step_tensors, make_block_mask
from tests import fp8_lut
from tests.gpu_util import assert_close, f32_of, to_dev
from tests.fp8_bound import bound as _bound
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu

SCALES = (0.02, 0.015, 0.02)
# 4 query heads on 2 KV heads, 10x20 tokens per frame, 2-frame steps, window of 6 frames after an
# anchor of 2, 7 steps, 40% of the key tiles kept per (head, query tile)
CFG = Workload(80, "w-ops", "bf16", 4, 2, 128, (10, 20), 2, 6, 2, 7, 40)
OVERWRITE_AT, CROP_AT, RESTORE_AT = 2, 4, 5


@pytest.mark.parametrize("kind", ["bf16", "fp8", "block-order"])
def test_overwrite_and_crop(kind):
    cfg, F = CFG, CFG.frames_per_step
    kw = {}
    if kind == "fp8":
        kw = dict(kv_dtype=uf.UF_FP8_E4M3, q_scale=SCALES[0], k_scale=SCALES[1], v_scale=SCALES[2])
    if kind == "block-order":
        kw = dict(block_grid=cfg.grid)
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames, **kw)
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    order = ob.block_order(F, cfg.grid[0], cfg.grid[1]) if kind == "block-order" else np.arange(F * cfg.tokens_per_frame)

    def kv_for_oracle(kb, vb):
        if kind == "fp8":
            return fp8_lut.round_trip_bits(kb, SCALES[1]), fp8_lut.round_trip_bits(vb, SCALES[2])
        return bf16_bits_to_f32(kb)[order], bf16_bits_to_f32(vb)[order]

    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        cache.append(to_dev(kb), to_dev(vb), F)
        win.append(*kv_for_oracle(kb, vb), F)
        what = f"{kind} step {s}"
        if s == OVERWRITE_AT:  # the chunk's next denoising step: new K/V for the same frames
            _, kb2, vb2 = draw_step_tensors(cfg, s + 100)
            cache.append(to_dev(kb2), to_dev(vb2), F, uf.UF_APPEND_OVERWRITE_NEWEST)
            win.overwrite_newest(*kv_for_oracle(kb2, vb2), F)
            what += " (newest chunk re-written)"
        if s == CROP_AT:
            cache.set_window(cfg.window_frames - F)
            win.set_active(cfg.window_frames - F)
            what += " (window cropped)"
        if s == RESTORE_AT:
            cache.set_window(cfg.window_frames)
            win.set_active(cfg.window_frames)
            what += " (window restored)"
        n_k = cache.window().n_keys
        kk, vv = win.keys_values()
        assert kk.shape[0] == n_k, (what, kk.shape[0], n_k)
        mask_np = make_block_mask(cfg.index, s, cfg.n_q_heads, cfg.q_tokens, n_k, cfg.mask_pct)
        q = to_dev(qb)
        out = torch.empty_like(q)
        print(what, flush=True)
        cache.attn_step(q, out, torch.from_numpy(mask_np).to("cuda:0"))
        torch.cuda.synchronize()
        got = f32_of(out)
        if kind == "fp8":
            qq = fp8_lut.round_trip_bits(qb, f8.attention_q_scale(SCALES[0], SCALES[1], cfg.head_dim))
            rows = np.arange(cfg.q_tokens)
            ref = oracle.attend(qq, kk, vv, mask_np)
            ratio = float((np.abs(got.astype(np.float64) - ref) / _bound(qq, kk, vv, ref, mask_np, rows)).max())
            print(f"  {what}: largest error / E4M3 bound = {ratio:.3f}", flush=True)
            assert ratio <= 1.0, what
        else:
            ref = oracle.attend(bf16_bits_to_f32(qb)[order], kk, vv, mask_np)
            assert_close(got[order], ref, what)
    cache.close()
