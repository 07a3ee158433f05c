"""Caches held in (2,8,8) block order, on the GPU, against the oracle.

The oracle models block order by permuting each step's tokens with
oracle.blocks.to_block_order before they enter its frame-list window (the
window only counts whole steps, so the order inside a step is free), and by
permuting the step's queries the same way.  Its output rows are then in block
order and go back to raster order with from_block_order; the library returns
raster order directly.  Masks are over the block-ordered tiles on both sides.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.blocks as ob
import oracle.fp8 as f8
from synth import WORKLOAD, TILE, Workload, bf16_bits_to_f32, draw_step_tensors, make_block_mask
from tests.fp8_bound import bound as fp8_bound
from tests.gpu_util import assert_close, bits_of, errors, f32_of, map_row_tiles, oracle_rows, to_dev
from tests.ring_model import RingModel
from tests.test_gpu_topk import check_mask
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu


def _perm(cfg, x):
    return ob.to_block_order(x, cfg.frames_per_step, cfg.grid[0], cfg.grid[1])


def _unperm(cfg, x):
    return ob.from_block_order(x, cfg.frames_per_step, cfg.grid[0], cfg.grid[1])


def test_block_order_storage_bit_exact():
    cfg = Workload(70, "b-store", "bf16", 2, 2, 128, (9, 17), 3, 6, 3, 5, None)
    cache = KVCache(2, 128, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames, block_grid=cfg.grid)
    cache.k_storage.zero_()
    cache.v_storage.zero_()
    model = RingModel(2, 128, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    for s in range(cfg.steps):
        _, kb, vb = draw_step_tensors(cfg, s)
        print(f"block-order append {s}", flush=True)
        cache.append(to_dev(kb), to_dev(vb), cfg.frames_per_step)
        model.append(cfg.frames_per_step, _perm(cfg, kb), _perm(cfg, vb))
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(cache.k_storage), model.k), f"K storage, append {s}"
        assert np.array_equal(bits_of(cache.v_storage), model.v), f"V storage, append {s}"
    cache.close()


def run_block_stream(cfg, fp8=False, scales=(0.02, 0.015, 0.02), **cache_kw):
    F = cfg.frames_per_step
    kw = dict(block_grid=cfg.grid, **cache_kw)
    if fp8:
        kw.update(kv_dtype=uf.UF_FP8_E4M3, q_scale=scales[0], k_scale=scales[1], v_scale=scales[2])
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames, **kw)
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        print(f"{cfg.name} step {s}: block-order append + attend", flush=True)
        cache.append(to_dev(kb), to_dev(vb), F)
        k, v, q = bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), bf16_bits_to_f32(qb)
        if fp8:
            k = f8.dequantize(f8.quantize(k, scales[1]), scales[1])
            v = f8.dequantize(f8.quantize(v, scales[2]), scales[2])
            qs = f8.attention_q_scale(scales[0], scales[1], cfg.head_dim)
            q = f8.dequantize(f8.quantize(q, qs), qs)
        win.append(_perm(cfg, k), _perm(cfg, v), F)
        n_k = cache.window().n_keys
        mask_np = mask_d = None
        if cfg.mask_pct is not None:
            mask_np = make_block_mask(cfg.index, s, cfg.n_q_heads, cfg.q_tokens, n_k, cfg.mask_pct)
            mask_d = torch.from_numpy(mask_np).to("cuda:0")
        out = torch.empty_like(to_dev(qb))
        cache.attn_step(to_dev(qb), out, mask_d)
        torch.cuda.synchronize()
        kk, vv = win.keys_values()
        qp = _perm(cfg, q)
        ref_p = oracle.attend(qp, kk, vv, mask_np)
        ref = _unperm(cfg, ref_p)
        if fp8:
            # every element within the E4M3 probability bound (tests/fp8_bound.py), which is
            # evaluated in the oracle's (block) row order and then put back in raster order
            got = f32_of(out).astype(np.float64)
            bnd = _unperm(cfg, fp8_bound(qp, kk, vv, ref_p, mask_np, np.arange(cfg.q_tokens)))
            ratio = float((np.abs(got - ref) / bnd).max())
            ma, rl = errors(got, ref)
            print(f"  fp8 max_abs={ma:.3e} rel_l2={rl:.3e}, largest error / bound = {ratio:.3f}", flush=True)
            assert np.isfinite(got).all()
            assert ratio <= 1.0, f"{cfg.name} step {s}: error beyond the E4M3 probability bound ({ratio:.3f})"
        else:
            assert_close(f32_of(out), ref, f"{cfg.name} step {s}")
    cache.close()


BLOCK_CASES = [
    # frame pairs, grid 10x20 (edges on both sides), anchor of one step, GQA 2, per-head mask
    Workload(71, "b-pairs", "bf16", 4, 2, 128, (10, 20), 2, 4, 2, 5, 40),
    # 3-frame steps (a pair plus an odd frame), grid 9x17, anchor, dense
    Workload(72, "b-odd", "bf16", 2, 2, 128, (9, 17), 3, 6, 3, 5, None),
    # head_dim 64, grid 16x16 (no edges), GQA 4
    Workload(73, "b-d64", "bf16", 8, 2, 64, (16, 16), 2, 4, 0, 4, None),
]


@pytest.mark.parametrize("cfg", BLOCK_CASES, ids=lambda c: c.name)
def test_block_order_attention(cfg):
    run_block_stream(cfg)


@pytest.mark.parametrize("splits", [2, 5])
def test_block_order_split_key_ranges(splits):
    """Block order with the key range forced into parts (attention partials, then the combine
    kernel, which writes the raster-order output rows)."""
    run_block_stream(Workload(76, "b-split", "bf16", 4, 2, 128, (10, 20), 2, 4, 2, 4, 50), splits=splits)


def test_block_order_fp8_attention():
    run_block_stream(Workload(74, "b-fp8", "bf16", 4, 2, 128, (10, 20), 2, 4, 2, 4, 50), fp8=True)


def test_block_order_topk_mask():
    cfg = Workload(75, "b-topk", "bf16", 4, 2, 128, (12, 20), 2, 4, 0, 3, None)
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, 0, block_grid=cfg.grid)
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, 0)
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        cache.append(to_dev(kb), to_dev(vb), cfg.frames_per_step)
        win.append(_perm(cfg, bf16_bits_to_f32(kb)), _perm(cfg, bf16_bits_to_f32(vb)), cfg.frames_per_step)
    n_k = cache.window().n_keys
    scores = torch.empty((cfg.n_q_heads, -(-cfg.q_tokens // TILE), -(-n_k // TILE)), dtype=torch.float32,
                         device="cuda:0")
    print("block-order top-k", flush=True)
    mask = cache.block_mask_topk(to_dev(qb), 3, 1, scores=scores)
    torch.cuda.synchronize()
    kk, _ = win.keys_values()
    check_mask(mask.cpu().numpy(), scores.cpu().numpy(), _perm(cfg, bf16_bits_to_f32(qb)), kk, 3, 1, "block-order")
    cache.close()


@pytest.mark.timeout(600)
def test_block_order_2k_sampled():
    """The 2K chunk held in block order at full size: 4 steps, each compared on 32 seeded query
    tiles per head (the first, the last and 30 drawn; tile t of the block order holds raster
    tokens order[128 t ...])."""
    cfg = WORKLOAD["2k"]
    F = cfg.frames_per_step
    order = ob.block_order(F, cfg.grid[0], cfg.grid[1])
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames,
                    block_grid=cfg.grid)
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    nqt = -(-cfg.q_tokens // TILE)
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        print(f"2k block order step {s}", flush=True)
        cache.append(to_dev(kb), to_dev(vb), F)
        win.append(bf16_bits_to_f32(kb)[order], bf16_bits_to_f32(vb)[order], F)
        n_k = cache.window().n_keys
        mask_np = make_block_mask(cfg.index, s, cfg.n_q_heads, cfg.q_tokens, n_k, cfg.mask_pct)
        out = torch.empty_like(to_dev(qb))
        cache.attn_step(to_dev(qb), out, torch.from_numpy(mask_np).to("cuda:0"))
        torch.cuda.synchronize()
        tiles = sorted({0, nqt - 1, *np.random.default_rng(s).choice(np.arange(1, nqt - 1), 30, replace=False)})
        rows = np.concatenate([np.arange(t * TILE, min((t + 1) * TILE, cfg.q_tokens)) for t in tiles])
        kk, vv = win.keys_values()
        ref = oracle_rows(bf16_bits_to_f32(qb)[order], kk, vv, mask_np, rows)
        got = f32_of(out)[order[rows]]
        assert_close(got, ref, f"2k block order step {s}, {len(tiles)} tiles")
    cache.close()
