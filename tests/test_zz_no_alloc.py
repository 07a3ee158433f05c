"""The allocation-free attention step (uf_attn_step_static) against uf_attn_step.

uf_attn_step_static puts split partials in the library's own per-device scratch array instead
of the cache's workspace.  On the same inputs and the same split count it runs the same
kernels, so its output must equal uf_attn_step's bit for bit, and both must meet the parity
bar against the float64 oracle.  Two calls in a row, the second with a smaller input, show
that the scratch left by one call does not leak into the next.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import Workload, bf16_bits_to_f32, draw_step_tensors, make_block_mask
from tests.gpu_util import assert_close, f32_of, oracle_rows, to_dev
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu


def _stream(cfg, n_steps, **kw):
    """A cache without workspace (only the static entry point can split) and one with the
    library's workspace, both holding the same frames, plus the oracle's window."""
    L, F, W, A = cfg.tokens_per_frame, cfg.frames_per_step, cfg.window_frames, cfg.anchor_frames
    bare = KVCache(cfg.n_kv_heads, cfg.head_dim, L, W, A, workspace=False, **kw)
    full = KVCache(cfg.n_kv_heads, cfg.head_dim, L, W, A, **kw)
    win = oracle.FrameListWindow(L, W, A)
    for s in range(n_steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        for c in (bare, full):
            c.append(to_dev(kb), to_dev(vb), F)
        win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), F)
    return bare, full, win, qb


def _compare(cfg, bare, full, win, qb, n_q, mask_pct, what):
    q = to_dev(qb[:n_q])
    n_k = full.window().n_keys
    mask_np = mask_d = None
    if mask_pct is not None:
        mask_np = make_block_mask(cfg.index, 99, cfg.n_q_heads, n_q, n_k, mask_pct)
        mask_d = torch.from_numpy(mask_np).to("cuda:0")
    a = torch.full_like(q, 3.0)
    b = torch.full_like(q, -3.0)
    print(f"{what}: {n_q} queries x {cfg.n_q_heads} heads, {n_k} keys", flush=True)
    bare.attn_step_static(q, a, mask_d)
    full.attn_step(q, b, mask_d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{what}: static scratch differs from the workspace"
    kk, vv = win.keys_values()
    ref = oracle_rows(bf16_bits_to_f32(qb[:n_q]), kk, vv, mask_np, np.arange(n_q))
    assert_close(f32_of(a), ref, what)


@pytest.mark.parametrize("splits,pipeline", [(0, 0), (3, 0), (3, 2)])
def test_static_scratch_matches_workspace(splits, pipeline):
    # 12 query heads over 3 KV heads, 1200 queries over 3600 keys: few enough work items that
    # the library splits the key range (forced to 3 parts in the other cases; in the last one
    # the head_dim 128 kernel also takes its software-pipelined loop)
    cfg = Workload(80, "no-alloc", "bf16", 12, 3, 128, (30, 40), 1, 3, 0, 3, None)
    bare, full, win, qb = _stream(cfg, 3, splits=splits, pipeline=pipeline)
    what = f"splits {splits or 'auto'}{', pipelined loop' if pipeline == 2 else ''}"
    _compare(cfg, bare, full, win, qb, 1200, None, f"{what}, first call")
    # the second call is smaller: fewer queries, a per-head mask
    _compare(cfg, bare, full, win, qb, 300, 60, f"{what}, second call, smaller")
    bare.close()
    full.close()


def test_static_scratch_head_dim_64_after_128():
    # a head_dim 64 step right after head_dim 128 steps: the partial layout changes with d
    cfg = Workload(81, "no-alloc-d64", "bf16", 8, 1, 64, (20, 25), 2, 4, 1, 3, None)
    bare, full, win, qb = _stream(cfg, 3)
    _compare(cfg, bare, full, win, qb, 1000, None, "d64, first call")
    _compare(cfg, bare, full, win, qb, 130, None, "d64, second call, smaller")
    bare.close()
    full.close()


def test_forced_splits_beyond_the_scratch_are_refused():
    cfg = Workload(82, "no-alloc-big", "bf16", 16, 1, 128, (50, 82), 1, 2, 0, 1, None)
    bare, full, win, qb = _stream(cfg, 1, splits=16)
    q = to_dev(qb)           # 4100 queries x 16 heads x 16 splits x 130 x 4 bytes > 32 MiB
    out = torch.empty_like(q)
    with pytest.raises(uf.UfError, match="UF_ERR_CAPACITY"):
        bare.attn_step_static(q, out)
    bare.close()
    full.close()


def test_static_scratch_fp8_cache():
    """An E4M3 cache through the static entry point: bit for bit the workspace entry point's
    result (which the FP8 tests hold to the oracle within the derived E4M3 bound), forced to
    3 key-range parts, then a smaller call."""
    cfg = Workload(83, "no-alloc-fp8", "bf16", 12, 3, 128, (30, 40), 1, 3, 0, 3, None)
    kw = dict(kv_dtype=uf.UF_FP8_E4M3, q_scale=0.02, k_scale=0.015, v_scale=0.02, splits=3)
    bare, full, _, qb = _stream(cfg, 3, **kw)
    for n_q in (1200, 300):
        q = to_dev(qb[:n_q])
        a = torch.full_like(q, 3.0)
        b = torch.full_like(q, -3.0)
        print(f"fp8 static: {n_q} queries", flush=True)
        bare.attn_step_static(q, a)
        full.attn_step(q, b)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{n_q} queries: static scratch differs"
    bare.close()
    full.close()
