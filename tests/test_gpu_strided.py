"""Strided operands on the GPU against the oracle.

A projection often writes q, k and v side by side in one tensor [tokens, Hq + 2 Hkv, d]
(a fused QKV layout), and the output may land inside a larger buffer.  The library takes
token and head strides for every operand; here q, k_new and v_new are views of one fused
tensor and out is a view into a wider one, for the bf16 and FP8 caches, attention and
top-k mask generation.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8
from synth import TILE, Workload, bf16_bits_to_f32, draw_step_tensors, make_block_mask
from tests import fp8_lut
from tests.fp8_bound import bound
from tests.gpu_util import assert_close, bits_of, to_dev
from tests.test_gpu_topk import check_mask
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu

SCALES = (0.02, 0.015, 0.02)
# 4 query heads on 2 KV heads, 12x20 tokens per frame, 2-frame steps, window 4 frames + anchor 2
CFG = Workload(90, "s-fused", "bf16", 4, 2, 128, (12, 20), 2, 4, 2, 5, 50)


def _fused(qb, kb, vb):
    """One device tensor [N, Hq + 2 Hkv, d] holding q | k | v, and the three views into it."""
    hq, hkv = qb.shape[1], kb.shape[1]
    qkv = to_dev(np.concatenate([qb, kb, vb], axis=1))
    return qkv, qkv[:, :hq], qkv[:, hq:hq + hkv], qkv[:, hq + hkv:]


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_fused_qkv_and_strided_out(kind):
    cfg, F = CFG, CFG.frames_per_step
    kw = {}
    if kind == "fp8":
        kw = dict(kv_dtype=uf.UF_FP8_E4M3, q_scale=SCALES[0], k_scale=SCALES[1], v_scale=SCALES[2])
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames, **kw)
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        qkv, q, k, v = _fused(qb, kb, vb)
        assert not q.is_contiguous() and q.stride(0) == (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
        cache.append(k, v, F)
        if kind == "fp8":
            win.append(fp8_lut.round_trip_bits(kb, SCALES[1]), fp8_lut.round_trip_bits(vb, SCALES[2]), F)
        else:
            win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), F)
        n_k = cache.window().n_keys
        mask_np = make_block_mask(cfg.index, s, cfg.n_q_heads, cfg.q_tokens, n_k, cfg.mask_pct)
        # out: heads 1 .. Hq of a [N, Hq + 2, d] buffer whose other heads must stay untouched
        wide = torch.full((cfg.q_tokens, cfg.n_q_heads + 2, cfg.head_dim), 3.0, dtype=torch.bfloat16, device="cuda:0")
        out = wide[:, 1:1 + cfg.n_q_heads]
        print(f"{kind} step {s}: fused qkv, strided out", flush=True)
        cache.attn_step(q, out, torch.from_numpy(mask_np).to("cuda:0"))
        torch.cuda.synchronize()
        w = bits_of(wide)
        assert (bf16_bits_to_f32(w[:, 0]) == 3.0).all() and (bf16_bits_to_f32(w[:, -1]) == 3.0).all(), \
            "write outside the out view"
        got = bf16_bits_to_f32(w[:, 1:1 + cfg.n_q_heads]).astype(np.float64)
        kk, vv = win.keys_values()
        if kind == "fp8":
            qq = fp8_lut.round_trip_bits(qb, f8.attention_q_scale(SCALES[0], SCALES[1], cfg.head_dim))
            ref = oracle.attend(qq, kk, vv, mask_np)
            ratio = float((np.abs(got - ref) / bound(qq, kk, vv, ref, mask_np, np.arange(cfg.q_tokens))).max())
            print(f"  largest error / E4M3 bound = {ratio:.3f}", flush=True)
            assert ratio <= 1.0
        else:
            assert_close(got, oracle.attend(bf16_bits_to_f32(qb), kk, vv, mask_np), f"{kind} step {s}")
        del qkv
    cache.close()


def test_topk_from_fused_q():
    cfg, F = CFG, CFG.frames_per_step
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        _, q, k, v = _fused(qb, kb, vb)
        cache.append(k, v, F)
        win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), F)
    n_k = cache.window().n_keys
    scores = torch.empty((cfg.n_q_heads, -(-cfg.q_tokens // TILE), -(-n_k // TILE)), dtype=torch.float32,
                         device="cuda:0")
    mask = cache.block_mask_topk(q, 2, 1, scores=scores)
    torch.cuda.synchronize()
    kk, _ = win.keys_values()
    check_mask(mask.cpu().numpy(), scores.cpu().numpy(), bf16_bits_to_f32(qb), kk, 2, 1, "fused q")
    cache.close()
