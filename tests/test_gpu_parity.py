"""GPU attention vs the float64 oracle, element by element, on seeded inputs.

Every test drives the HIP library through its C ABI (ctypes binding).  The
oracle sees the same bf16 values widened to float64.  The bar is
max-abs <= 2e-2 and relative L2 <= 5e-3 on every compared row.

Full-size workloads (480P, decoder, 1K, 2K, FlashDecoder-XL backbone and
refinement) stream all their steps in the library's default launch
configuration.  At every checked step the oracle computes whole query tiles:
every tile when a step has at most 32, else 32 seeded tiles (the first, the
last and 30 drawn without replacement; 4096 rows per head), the same tiles for
all heads.  One steady 2K step is compared on every row.  480P, 1K and 2K
check every step; the decoder and the XL shapes check the steps listed in
their tests.  Reduced shapes are compared on every row of every step.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import (WORKLOAD, TILE, Workload, bf16_bits_to_f32, draw_normal, draw_step_tensors, f32_to_bf16_bits,
                   make_block_mask)
from tests.gpu_util import assert_close, bits_of, errors, f32_of, oracle_rows, to_dev
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu


def _rows_of_tiles(n_q, tiles):
    rows = [np.arange(t * TILE, min((t + 1) * TILE, n_q)) for t in sorted(set(tiles))]
    return np.concatenate(rows)


def _pick_tiles(n_q, n_tiles, seed):
    nqt = -(-n_q // TILE)
    if n_tiles is None or n_tiles >= nqt:
        return list(range(nqt))
    rng = np.random.default_rng(seed)
    extra = rng.choice(np.arange(1, nqt - 1), size=min(n_tiles - 2, nqt - 2), replace=False)
    return sorted({0, nqt - 1, *extra.tolist()})


SAMPLED_TILES = 32  # query tiles per head compared at a checked step of a full-size workload


def run_stream(cfg: Workload, check_steps=None, tiles=None, shared_mask=False, scale_q=1.0, steps=None,
               raw_fp32_oracle=False, full_steps=(), **cache_kw):
    """Stream cfg through the library; compare checked steps against the oracle.

    tiles: query tiles compared per checked step (None = all); steps in full_steps compare
    every row whatever `tiles` says."""
    L, F, W, A = cfg.tokens_per_frame, cfg.frames_per_step, cfg.window_frames, cfg.anchor_frames
    steps = cfg.steps if steps is None else steps
    check_steps = range(steps) if check_steps is None else check_steps
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, L, W, A, **cache_kw)
    win = oracle.FrameListWindow(L, W, A)
    raw = oracle.FrameListWindow(L, W, A) if raw_fp32_oracle else None
    worst = (0.0, 0.0)
    for s in range(steps):
        qb, kb, vb = draw_step_tensors(cfg, s, scale_q)
        q_d, k_d, v_d = to_dev(qb), to_dev(kb), to_dev(vb)
        print(f"{cfg.name} step {s}: append {F} frames, attend {cfg.q_tokens} queries", flush=True)
        cache.append(k_d, v_d, F)
        win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), F)
        info = cache.window()
        kk, vv = win.keys_values()
        assert info.n_keys == kk.shape[0], (info.n_keys, kk.shape)
        mask_np = mask_d = None
        if cfg.mask_pct is not None:
            mh = 1 if shared_mask else cfg.n_q_heads
            mask_np = make_block_mask(cfg.index, s, mh, cfg.q_tokens, info.n_keys, cfg.mask_pct)
            mask_d = torch.from_numpy(mask_np).to("cuda:0")
        out = torch.empty_like(q_d)
        cache.attn_step(q_d, out, mask_d)
        if raw is not None:
            raw.append(draw_normal(cfg.index, s, 1, kb.shape), draw_normal(cfg.index, s, 2, vb.shape), F)
        if s not in check_steps:
            continue
        torch.cuda.synchronize()
        got = f32_of(out)
        picked = _pick_tiles(cfg.q_tokens, None if s in full_steps else tiles, 1000 * cfg.index + s)
        rows = _rows_of_tiles(cfg.q_tokens, picked)
        print(f"  oracle on {len(picked)} query tiles x {cfg.n_q_heads} heads", flush=True)
        ref = oracle_rows(bf16_bits_to_f32(qb), kk, vv, mask_np, rows)
        ma, rl = assert_close(got[rows], ref, f"{cfg.name} step {s} ({len(rows)} rows)")
        worst = (max(worst[0], ma), max(worst[1], rl))
        if raw is not None:
            rk, rv = raw.keys_values()
            q_raw = draw_normal(cfg.index, s, 0, qb.shape) * np.float32(scale_q)
            ref_raw = oracle_rows(q_raw, rk, rv, mask_np, rows)
            ma_raw, rl_raw = errors(got[rows], ref_raw)
            print(f"  vs float32-input oracle: max_abs={ma_raw:.3e} rel_l2={rl_raw:.3e}", flush=True)
            assert ma_raw < 2e-2 and rl_raw < 1e-2
    cache.close()
    return worst


# ---------------------------------------------------------------------------------------------
# the workloads at full size

def test_tiny_all_steps():
    # bf16 path on the tiny workload; also within 1e-2 rel-L2 of the oracle on the raw float32 draws
    run_stream(WORKLOAD["tiny"], raw_fp32_oracle=True)


@pytest.mark.timeout(600)
def test_480p_anchor_stream():
    run_stream(WORKLOAD["480p"], tiles=SAMPLED_TILES)


def test_decoder_gqa_stream():
    # every row of every 8th step (13 query tiles per step) and of the first and last steps
    run_stream(WORKLOAD["decoder"], check_steps=sorted({0, 1, 2, 3, 119, *range(0, 120, 8)}), tiles=None)


@pytest.mark.timeout(600)
def test_1k_masked_stream():
    run_stream(WORKLOAD["1k"], tiles=SAMPLED_TILES)


@pytest.mark.timeout(900)
def test_2k_masked_stream():
    # 32 tiles per head at steps 0-2; the steady step 3 on every row (330 tiles x 12 heads)
    run_stream(WORKLOAD["2k"], tiles=SAMPLED_TILES, full_steps=(3,))


@pytest.mark.timeout(600)
def test_decoder_xl_stream():
    # head_dim 64, 24 query heads over 3 KV heads (8 per group), per-frame steps; 29 query tiles,
    # so every row of each checked step
    run_stream(WORKLOAD["decoder-xl"], check_steps=[0, 1, 2, 5, 11, 17, 23], tiles=SAMPLED_TILES)


@pytest.mark.timeout(600)
def test_refine_xl_stream():
    # temporal refinement: 4-frame steps over an 8-frame window, head_dim 64, GQA 8; every step
    run_stream(WORKLOAD["refine-xl"], tiles=SAMPLED_TILES)


# ---------------------------------------------------------------------------------------------
# reduced shapes, every row

REDUCED = [
    # anchor + ring with frames of 200 tokens: tiles straddle the anchor/ring boundary and the wrap
    Workload(10, "r-anchor", "bf16", 4, 2, 128, (10, 20), 3, 6, 3, 6, None),
    # per-head block mask, GQA 2, ragged tails
    Workload(11, "r-mask", "bf16", 4, 2, 128, (12, 17), 2, 4, 0, 5, 40),
    # head_dim 64 with an anchor frame
    Workload(12, "r-d64", "bf16", 2, 1, 64, (8, 13), 1, 3, 1, 6, None),
    # head_dim 64 with a mask
    Workload(13, "r-d64-mask", "bf16", 3, 3, 64, (9, 31), 2, 4, 2, 5, 30),
    # GQA 8 (two work-groups per group)
    Workload(14, "r-gqa8", "bf16", 8, 1, 128, (11, 11), 1, 3, 0, 4, None),
]


@pytest.mark.parametrize("cfg", REDUCED, ids=lambda c: c.name)
def test_reduced_every_row(cfg):
    run_stream(cfg)


def test_shared_mask_gqa4():
    cfg = Workload(15, "r-shared-mask", "bf16", 8, 2, 128, (13, 20), 3, 6, 0, 4, 35)
    run_stream(cfg, shared_mask=True)


@pytest.mark.parametrize("tail", [8, 16, 24, 32, 48, 64, 72, 88])
def test_query_and_key_tails(tail):
    cfg = Workload(20 + tail, f"r-tail{tail}", "bf16", 2, 2, 128, (1, 128 + tail), 1, 2, 0, 3, None)
    run_stream(cfg)


def test_sharp_attention_stress():
    cfg = Workload(16, "r-stress", "bf16", 4, 4, 128, (16, 25), 1, 3, 1, 4, None)
    run_stream(cfg, scale_q=4.0)


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_forced_splits(splits):
    run_stream(Workload(17, "r-split", "bf16", 4, 1, 128, (10, 30), 2, 4, 1, 5, None), splits=splits)
    run_stream(Workload(18, "r-split-mask", "bf16", 2, 2, 64, (10, 30), 2, 4, 0, 4, 30), splits=splits)


def test_uneven_split_every_row():
    """A dense head_dim 128 step of 320 work items (8 heads x 40 query tiles over 40 key tiles):
    more than half a round and less than one round of 512 resident work-groups, so the library
    cuts every item into a body of 32 key tiles and a tail of 8 and combines the two (the 480P
    case at a size the oracle checks on every row)."""
    run_stream(Workload(38, "r-body-tail", "bf16", 8, 8, 128, (50, 50), 2, 2, 0, 3, None))


@pytest.mark.parametrize("hpw", [1, 2, 4])
def test_heads_per_workgroup(hpw):
    run_stream(Workload(19, "r-hpw", "bf16", 8, 2, 128, (10, 25), 1, 3, 0, 3, None), heads_per_wg=hpw)


@pytest.mark.parametrize("hpw", [2, 4])
def test_per_head_masks_shared_tiles(hpw):
    """Per-head masks with the heads of a KV group sharing staged tiles (the work-group walks the
    union of its heads' mask rows; each wave computes only its own head's kept tiles): GQA 4
    (head_dim 128, anchor, ragged) and GQA 8 (head_dim 64, forced splits)."""
    run_stream(Workload(36, "r-union4", "bf16", 8, 2, 128, (11, 23), 2, 4, 2, 5, 30), heads_per_wg=hpw)
    run_stream(Workload(37, "r-union8", "bf16", 16, 2, 64, (9, 29), 1, 3, 0, 4, 25), heads_per_wg=hpw,
               splits=3)


def test_per_head_masks_shared_tiles_decoder_xl():
    """The FlashDecoder-XL backbone shape (24 query heads over 3 KV heads, head_dim 64) under
    seeded per-head masks of 40% density, four query heads per work-group."""
    cfg = WORKLOAD["decoder-xl"]
    cfg = Workload(38, "decoder-xl-masked", cfg.dtype, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.grid,
                   cfg.frames_per_step, cfg.window_frames, cfg.anchor_frames, 4, 40)
    run_stream(cfg, heads_per_wg=4)


# ---------------------------------------------------------------------------------------------
# special cases with exact answers

def _cache_with(L, W, A, heads, d, frames, seed):
    cache = KVCache(heads, d, L, W, A)
    ks, vs = [], []
    for f in range(frames):
        kb = f32_to_bf16_bits(draw_normal(900 + seed, f, 1, (L, heads, d)))
        vb = f32_to_bf16_bits(draw_normal(900 + seed, f, 2, (L, heads, d)))
        cache.append(to_dev(kb), to_dev(vb), 1)
        ks.append(kb); vs.append(vb)
    return cache, ks, vs


def test_single_key_returns_value_bit_exact():
    """One visible key: softmax weight 1, so out == v exactly (bf16 in, bf16 out)."""
    for d in (64, 128):
        cache, ks, vs = _cache_with(1, 1, 0, 2, d, 3, seed=d)   # W = 1: only the newest frame is visible
        q = to_dev(f32_to_bf16_bits(draw_normal(950, d, 0, (300, 4, d))))
        out = torch.empty_like(q)
        print(f"single key d={d}", flush=True)
        cache.attn_step(q, out)
        got = bits_of(out)
        for h in range(4):
            assert np.array_equal(got[:, h, :], np.broadcast_to(vs[-1][0, h // 2], (300, d)))
        cache.close()


def test_all_ones_mask_is_dense_bit_identical():
    cfg = Workload(30, "ones", "bf16", 4, 2, 128, (10, 20), 2, 4, 1, 1, None)
    cache = KVCache(2, 128, 200, 4, 1)
    for s in range(4):
        qb, kb, vb = draw_step_tensors(cfg, s)
        cache.append(to_dev(kb), to_dev(vb), 2)
    q = to_dev(qb)
    n_k = cache.window().n_keys
    ones = torch.ones((4, -(-400 // 128), -(-n_k // 128)), dtype=torch.uint8, device="cuda:0")
    a, b, c = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    print("all-ones mask vs dense", flush=True)
    cache.attn_step(q, a)
    cache.attn_step(q, b, ones)
    cache.attn_step(q, c, ones[:1])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    cache.close()


def test_empty_mask_rows_output_zero():
    cfg = Workload(31, "empty-rows", "bf16", 2, 2, 128, (10, 30), 1, 2, 0, 2, None)
    cache = KVCache(2, 128, 300, 2, 0)
    win = oracle.FrameListWindow(300, 2, 0)
    for s in range(2):
        qb, kb, vb = draw_step_tensors(cfg, s)
        cache.append(to_dev(kb), to_dev(vb), 1)
        win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), 1)
    mask = make_block_mask(31, 1, 2, 300, 600, 50)
    mask[0, 1, :] = 0
    mask[1, 2, :] = 0
    q = to_dev(qb)
    out = torch.full_like(q, 7.0)
    print("empty mask rows", flush=True)
    cache.attn_step(q, out, torch.from_numpy(mask).to("cuda:0"))
    got = f32_of(out)
    assert np.all(got[128:256, 0] == 0) and np.all(got[256:, 1] == 0)
    kk, vv = win.keys_values()
    assert_close(got, oracle.attend(bf16_bits_to_f32(qb), kk, vv, mask), "empty-rows")
    cache.close()


def test_no_queries_is_a_no_op():
    cache, _, _ = _cache_with(16, 2, 0, 1, 128, 2, seed=5)
    q = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    out = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    cache.attn_step(q, out)
    torch.cuda.synchronize()
    cache.close()


def test_splits_agree():
    """Split-KV partials combine to the unsplit result within fp32 rounding (bf16 output: 1 ulp)."""
    cfg = Workload(32, "split-agree", "bf16", 4, 2, 128, (20, 30), 1, 3, 0, 3, None)
    outs = []
    for splits in (1, 2, 5):
        cache = KVCache(2, 128, 600, 3, 0, splits=splits)
        for s in range(3):
            qb, kb, vb = draw_step_tensors(cfg, s)
            cache.append(to_dev(kb), to_dev(vb), 1)
        q = to_dev(qb)
        o = torch.empty_like(q)
        cache.attn_step(q, o)
        outs.append(f32_of(o))
        cache.close()
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2.0 ** -7 * np.abs(outs[0]).max() + 1e-6
