"""Random small streams on the GPU against the oracle, on every row.

160 stream configurations drawn from a fixed seed: frame size (1 to 300 tokens, so that
the visible keys end anywhere inside a 64-key sub-tile or a 128-key mask tile), window,
anchor, frames per step, KV heads and query heads per KV head, head_dim 64 or 128, dense or
per-head or shared masks of several densities, heads per work-group and forced key-range
splits; along the stream the window is cropped and restored and the newest chunk rewritten in
place.  Every step's attention is compared with the oracle's on every row, to the parity bar.
At head_dim 128 every stream also runs through the software-pipelined attention loop (forced
through the cache description), whose output must equal the one-sub-tile loop's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import Workload, bf16_bits_to_f32, draw_normal, draw_step_tensors, f32_to_bf16_bits, make_block_mask
from tests.gpu_util import assert_close, f32_of, to_dev
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu


def _configs(n=160, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2, 4]))
        W = int(rng.integers(1, 6))
        A = int(rng.integers(0, 3))
        F = int(rng.integers(1, W + 1))
        L = int(rng.integers(1, 301))
        mask = [None, None, 30, 70, 100][int(rng.integers(0, 5))]
        shared = bool(rng.integers(0, 2))
        hpw_choices = [0] + [h for h in (1, 2, 4) if group % h == 0]
        hpw = int(rng.choice(hpw_choices))
        splits = int(rng.choice([0, 0, 1, 3]))
        steps = int(rng.integers(2, 5))
        cfg = Workload(200 + i, f"r{i}", "bf16", hkv * group, hkv, d, (1, L), F, W, A, steps, mask)
        out.append((cfg, shared, hpw, splits))
    return out


CONFIGS = _configs()


def _id(c):
    cfg, shared, hpw, splits = c
    m = "dense" if cfg.mask_pct is None else f"m{cfg.mask_pct}{'s' if shared else 'h'}"
    return (f"{cfg.name}-d{cfg.head_dim}-h{cfg.n_q_heads}x{cfg.n_kv_heads}-L{cfg.tokens_per_frame}-W{cfg.window_frames}"
            f"-A{cfg.anchor_frames}-F{cfg.frames_per_step}-{m}-hpw{hpw}-s{splits}")


@pytest.mark.parametrize("case", CONFIGS, ids=_id)
def test_random_stream(case):
    cfg, shared, hpw, splits = case
    L, F, W, A = cfg.tokens_per_frame, cfg.frames_per_step, cfg.window_frames, cfg.anchor_frames
    print(f"random stream {_id(case)}", flush=True)
    # at head_dim 128 the stream runs through both attention loops: one sub-tile per step in
    # `cache`, software-pipelined in its twin, which must agree bit for bit
    twin_loops = cfg.head_dim == 128
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, L, W, A, heads_per_wg=hpw, splits=splits,
                    pipeline=1 if twin_loops else 0)
    caches = [cache]
    if twin_loops:
        caches.append(KVCache(cfg.n_kv_heads, cfg.head_dim, L, W, A, heads_per_wg=hpw, splits=splits, pipeline=2))
    win = oracle.FrameListWindow(L, W, A)
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        for c in caches:
            c.append(to_dev(kb), to_dev(vb), F)
        win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), F)
        if s == 1:  # rewrite the newest chunk in place (a second denoising pass of the same chunk)
            kb2 = f32_to_bf16_bits(draw_normal(cfg.index, s + 50, 1, kb.shape))
            vb2 = f32_to_bf16_bits(draw_normal(cfg.index, s + 50, 2, vb.shape))
            for c in caches:
                c.append(to_dev(kb2), to_dev(vb2), F, uf.UF_APPEND_OVERWRITE_NEWEST)
            win.overwrite_newest(bf16_bits_to_f32(kb2), bf16_bits_to_f32(vb2), F)
        crop = W > F and s == cfg.steps - 1
        if crop:  # the last step sees a cropped window
            for c in caches:
                c.set_window(F)
            win.set_active(F)
        n_k = cache.window().n_keys
        kk, vv = win.keys_values()
        assert n_k == kk.shape[0]
        mask_np = mask_d = None
        if cfg.mask_pct is not None:
            mask_np = make_block_mask(cfg.index, s, 1 if shared else cfg.n_q_heads, cfg.q_tokens, n_k, cfg.mask_pct)
            mask_d = torch.from_numpy(mask_np).to("cuda:0")
        q = to_dev(qb)
        out = torch.empty_like(q)
        cache.attn_step(q, out, mask_d)
        if twin_loops:
            out2 = torch.empty_like(q)
            caches[1].attn_step(q, out2, mask_d)
        torch.cuda.synchronize()
        ref = oracle.attend(bf16_bits_to_f32(qb), kk, vv, mask_np)
        assert_close(f32_of(out), ref, f"{cfg.name} step {s}")
        if twin_loops:
            assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"{cfg.name} step {s}: loops differ"
        if crop:
            for c in caches:
                c.set_window(W)
            win.set_active(W)
    for c in caches:
        c.close()
