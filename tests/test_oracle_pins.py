"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each check_* function raises AssertionError when the oracle disagrees with
a closed form, an invariant, a hand-derived window table (tests/golden/) or
PyTorch's scaled_dot_product_attention in float64.  The test_mutant_* tests
plant plausible mistakes in the oracle (on the CPU) and require that some
check catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt
import oracle.window as owin
from synth import WORKLOADS, draw_normal, f32_to_bf16_bits, bf16_bits_to_f32, make_block_mask, diagonal_tiles

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_normal(seed, shape, scale=1.0):
    x = draw_normal(100 + seed, 0, 0, shape) * np.float32(scale)
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _token_mask(block_mask, h, n_q, n_k, tile):
    bm = block_mask[0 if block_mask.shape[0] == 1 else h] != 0
    return np.repeat(np.repeat(bm, tile, axis=0), tile, axis=1)[:n_q, :n_k]


def _sdpa(q, k, v, token_mask_per_head=None):
    """torch SDPA in float64 on the CPU; q [Nq,Hq,d], k/v [Nk,Hkv,d]."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2), dtype=np.float64))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2), dtype=np.float64))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2), dtype=np.float64))[None]
    mask = None if token_mask_per_head is None else torch.from_numpy(token_mask_per_head)[None]
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           enable_gqa=q.shape[1] != k.shape[1])
    return out[0].numpy().transpose(1, 0, 2)


# ----------------------------------------------------------------------------------------------
# checks

def check_two_key_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "two_keys.json")))
    q = np.array(g["q"])[None, None, :]
    k = np.array(g["k"])[:, None, :]
    v = np.array(g["v"])[:, None, :]
    out = oracle.attend(q, k, v)[0, 0]
    assert np.allclose(out, g["out"], rtol=0, atol=1e-15), out


def check_single_key_returns_value():
    q = _bf16_normal(1, (5, 3, 64))
    k = _bf16_normal(2, (1, 3, 64))
    v = _bf16_normal(3, (1, 3, 64))
    out = oracle.attend(q, k, v)
    assert np.array_equal(out, np.broadcast_to(v[0][None].astype(np.float64), out.shape))


def check_identical_keys_give_mean_value():
    q = _bf16_normal(4, (7, 2, 32))
    k = np.repeat(_bf16_normal(5, (1, 2, 32)), 300, axis=0)
    v = _bf16_normal(6, (300, 2, 32))
    out = oracle.attend(q, k, v)
    assert np.allclose(out, v.astype(np.float64).mean(axis=0)[None], rtol=0, atol=1e-13)


def check_window_tables():
    """The frame-list model reproduces the hand-derived window tables (tests/golden/windows.json)."""
    table = json.load(open(os.path.join(GOLDEN, "windows.json")))
    for cfg in WORKLOADS:
        t = table[cfg.name]
        F, L = t["frames_per_step"], t["tokens_per_frame"]
        assert (F, L) == (cfg.frames_per_step, cfg.tokens_per_frame)
        for step, units in enumerate(t["units"]):
            frames = owin.visible_frames_after((step + 1) * F, cfg.window_frames, cfg.anchor_frames)
            expect = [u * F + f for u in units for f in range(F)]
            assert frames == expect, (cfg.name, step, frames, expect)
            assert len(frames) * L == t["n_keys"][step], (cfg.name, step)


def check_uniform_queries_reveal_window():
    """q = 0 gives equal weights, so with one-hot frame codes in V the output
    counts the visible keys of every frame: it must be L/N_k on exactly the
    visible frames of the golden table."""
    table = json.load(open(os.path.join(GOLDEN, "windows.json")))
    for cfg in WORKLOADS:
        t = table[cfg.name]
        L, F = 4, cfg.frames_per_step          # reduced tokens per frame, same frame logic
        n_steps = len(t["units"])
        d = 64
        win = oracle.FrameListWindow(L, cfg.window_frames, cfg.anchor_frames)
        for step in range(n_steps):
            frames = np.arange(step * F, (step + 1) * F)
            v = np.zeros((F * L, 1, d))
            for i, f in enumerate(frames):
                v[i * L:(i + 1) * L, 0, f] = 1.0
            k = _bf16_normal(7 + step, (F * L, 1, d))
            win.append(k, v, F)
            kk, vv = win.keys_values()
            out = oracle.attend(np.zeros((3, 1, d)), kk, vv)
            expect_frames = [u * F + f for u in t["units"][step] for f in range(F)]
            expect = np.zeros(d)
            expect[expect_frames] = 1.0 / len(expect_frames)
            assert np.allclose(out[:, 0, :], expect[None], rtol=0, atol=1e-14), (cfg.name, step)


def _sdpa_case(seed, n_q, n_k, hq, hkv, d, mask_heads=None, density=0.4, tile=128, scale=1.0):
    q = _bf16_normal(seed, (n_q, hq, d), scale)
    k = _bf16_normal(seed + 1, (n_k, hkv, d))
    v = _bf16_normal(seed + 2, (n_k, hkv, d))
    bm = None
    if mask_heads is not None:
        rng = np.random.default_rng(seed)
        bm = (rng.random((mask_heads, -(-n_q // tile), -(-n_k // tile))) < density).astype(np.uint8)
        bm[..., 0] = 1  # every row keeps at least one tile, so SDPA has no empty rows
    out = oracle.attend(q, k, v, bm, tile=tile)
    tm = None
    if bm is not None:
        tm = np.stack([_token_mask(bm, h, n_q, n_k, tile) for h in range(hq)])
    ref = _sdpa(q, k, v, tm)
    return out, ref


def check_against_sdpa():
    cases = [
        dict(seed=10, n_q=200, n_k=333, hq=2, hkv=2, d=64),                  # ragged tiles, MHA
        dict(seed=20, n_q=150, n_k=390, hq=4, hkv=1, d=128),                 # GQA 4
        dict(seed=30, n_q=300, n_k=520, hq=6, hkv=3, d=64, mask_heads=6),    # per-head mask, GQA 2
        dict(seed=40, n_q=260, n_k=700, hq=3, hkv=3, d=32, mask_heads=1),    # shared mask
        dict(seed=50, n_q=90, n_k=150, hq=2, hkv=1, d=64, scale=4.0),        # sharp attention
        dict(seed=60, n_q=70, n_k=90, hq=4, hkv=2, d=16, mask_heads=4, tile=16),
    ]
    for c in cases:
        out, ref = _sdpa_case(**c)
        err = np.abs(out - ref).max()
        assert err < 1e-12, (c, err)


def check_row_subset_matches_sdpa():
    """attend(rows=r) gives row r of SDPA's full output for any subset r: unsorted, repeated,
    spanning several query tiles with their own per-head mask rows, ragged last tiles."""
    cases = [
        dict(seed=80, n_q=300, n_k=520, hq=6, hkv=3, d=64, mask_heads=6),     # per-head mask, GQA 2
        dict(seed=90, n_q=333, n_k=290, hq=4, hkv=1, d=32, mask_heads=1),     # shared mask, GQA 4
        dict(seed=95, n_q=210, n_k=400, hq=2, hkv=2, d=64),                   # dense
    ]
    for c in cases:
        _, ref = _sdpa_case(**c)
        rng = np.random.default_rng(c["seed"])
        rows = np.concatenate([rng.choice(c["n_q"], size=40, replace=False), [c["n_q"] - 1, 0, 0, 129, 128, 127]])
        q = _bf16_normal(c["seed"], (c["n_q"], c["hq"], c["d"]))
        k = _bf16_normal(c["seed"] + 1, (c["n_k"], c["hkv"], c["d"]))
        v = _bf16_normal(c["seed"] + 2, (c["n_k"], c["hkv"], c["d"]))
        bm = None
        if c.get("mask_heads") is not None:
            bm = (np.random.default_rng(c["seed"]).random((c["mask_heads"], -(-c["n_q"] // 128),
                                                            -(-c["n_k"] // 128))) < 0.4).astype(np.uint8)
            bm[..., 0] = 1
        sub = oracle.attend(q, k, v, bm, rows=rows)
        assert sub.shape == (len(rows), c["hq"], c["d"])
        assert np.abs(sub - ref[rows]).max() < 1e-12, c


def check_empty_row_is_zero():
    q = _bf16_normal(70, (256, 2, 64))
    k = _bf16_normal(71, (256, 2, 64))
    v = _bf16_normal(72, (256, 2, 64))
    bm = np.ones((2, 2, 2), dtype=np.uint8)
    bm[1, 0, :] = 0
    out = oracle.attend(q, k, v, bm)
    assert np.all(out[:128, 1] == 0.0)
    assert np.all(out[128:, 1] != 0.0) and np.all(np.abs(out[:, 0]).sum(axis=-1) > 0)


def check_gqa_equals_repeated_mha():
    q = _bf16_normal(80, (100, 8, 64))
    k = _bf16_normal(81, (230, 2, 64))
    v = _bf16_normal(82, (230, 2, 64))
    gqa = oracle.attend(q, k, v)
    mha = oracle.attend(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    assert np.abs(gqa - mha).max() < 1e-14


def check_key_permutation_invariance():
    q = _bf16_normal(90, (64, 2, 64))
    k = _bf16_normal(91, (300, 2, 64))
    v = _bf16_normal(92, (300, 2, 64))
    perm = np.random.default_rng(0).permutation(300)
    a = oracle.attend(q, k, v)
    b = oracle.attend(q, k[perm], v[perm])
    assert np.abs(a - b).max() < 1e-13


def check_all_ones_mask_equals_dense():
    q = _bf16_normal(100, (300, 3, 64))
    k = _bf16_normal(101, (500, 3, 64))
    v = _bf16_normal(102, (500, 3, 64))
    bm = np.ones((3, 3, 4), dtype=np.uint8)
    assert np.array_equal(oracle.attend(q, k, v, bm), oracle.attend(q, k, v))


def check_mask_equals_gathered_dense():
    """A masked query tile equals dense attention over just its kept key tiles."""
    n_q, n_k, t = 300, 700, 128
    q = _bf16_normal(110, (n_q, 2, 64))
    k = _bf16_normal(111, (n_k, 2, 64))
    v = _bf16_normal(112, (n_k, 2, 64))
    bm = make_block_mask(9, 0, 2, n_q, n_k, 30)
    out = oracle.attend(q, k, v, bm)
    for h in range(2):
        for qt in range(bm.shape[1]):
            keys = np.concatenate([np.arange(kt * t, min(kt * t + t, n_k)) for kt in np.nonzero(bm[h, qt])[0]])
            rows = np.arange(qt * t, min(qt * t + t, n_q))
            ref = oracle.attend(q[rows][:, h:h + 1], k[keys][:, h:h + 1], v[keys][:, h:h + 1])
            assert np.abs(out[rows, h:h + 1] - ref).max() < 1e-13


def check_single_tile_uniform_query():
    """q = 0 with one kept key tile gives the mean of that tile's values."""
    n_q, n_k = 128, 640
    v = _bf16_normal(120, (n_k, 1, 64))
    k = _bf16_normal(121, (n_k, 1, 64))
    bm = np.zeros((1, 1, 5), dtype=np.uint8)
    bm[0, 0, 3] = 1
    out = oracle.attend(np.zeros((n_q, 1, 64)), k, v, bm)
    assert np.allclose(out[:, 0], v[384:512, 0].astype(np.float64).mean(axis=0)[None], rtol=0, atol=1e-14)


def _stream(cfg_like, L, hq, hkv, d, n_steps, seed):
    F, W, A = cfg_like
    win = oracle.FrameListWindow(L, W, A)
    qs, ks, vs, outs = [], [], [], []
    for s in range(n_steps):
        q = _bf16_normal(seed + 3 * s, (F * L, hq, d))
        k = _bf16_normal(seed + 3 * s + 1, (F * L, hkv, d))
        v = _bf16_normal(seed + 3 * s + 2, (F * L, hkv, d))
        win.append(k, v, F)
        kk, vv = win.keys_values()
        outs.append(oracle.attend(q, kk, vv))
        qs.append(q); ks.append(k); vs.append(v)
    return np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), np.concatenate(outs)


def check_streaming_equals_full_sequence():
    shapes = [  # (F, W, A), L, Hq, Hkv, d, steps
        ((1, 3, 0), 64, 2, 2, 64, 6),     # tiny at full size
        ((3, 9, 3), 12, 2, 2, 32, 8),     # 480P logic, reduced frame
        ((1, 2, 0), 10, 4, 1, 32, 12),    # decoder logic (GQA 4), reduced
        ((3, 6, 0), 16, 2, 2, 32, 4),     # 1K / 2K logic, reduced
        ((2, 5, 1), 7, 3, 1, 16, 9),      # odd sizes: anchor not a whole step
    ]
    for i, (fwa, L, hq, hkv, d, n) in enumerate(shapes):
        q, k, v, streamed = _stream(fwa, L, hq, hkv, d, n, 200 + 50 * i)
        full = oracle.attend_full_sequence(q, k, v, L, *fwa)
        err = np.abs(full - streamed).max()
        assert err < 1e-12, (fwa, err)


def check_overwrite_and_crop():
    L, d = 8, 16
    win = oracle.FrameListWindow(L, 4, 1)
    k0 = [_bf16_normal(300 + i, (2 * L, 1, d)) for i in range(4)]
    for i in range(3):
        win.append(k0[i], k0[i] * 2, 2)
    assert win.visible() == [0, 2, 3, 4, 5]       # anchor frame 0 + the newest 4 others
    win.overwrite_newest(k0[3], k0[3] * 2, 2)
    kk, vv = win.keys_values()
    assert np.array_equal(kk[3 * L:], k0[3]) and np.array_equal(kk[L:3 * L], k0[1])
    assert np.array_equal(vv[3 * L:], 2 * k0[3]) and np.array_equal(kk[:L], k0[0][:L])
    win.set_active(2)
    assert win.visible() == [0, 4, 5]
    win.set_active(4)
    assert win.visible() == [0, 2, 3, 4, 5]


def check_executed_pairs():
    # dense: the 480P steady step, 4*d*Hq*Nq*Nk = 538.27 GFLOP
    assert 4 * 128 * oracle.executed_pairs(4680, 18720, 12) == 538_273_382_400
    # masked: equals the count of allowed (row, key) entries of the token mask
    bm = make_block_mask(8, 1, 3, 300, 700, 40)
    brute = sum(int(_token_mask(bm, h, 300, 700, 128).sum()) for h in range(3))
    assert oracle.executed_pairs(300, 700, 3, bm) == brute
    bm1 = bm[:1]
    assert oracle.executed_pairs(300, 700, 3, bm1) == 3 * int(_token_mask(bm1, 0, 300, 700, 128).sum())


ALL_CHECKS = [
    check_two_key_worked_example, check_single_key_returns_value, check_identical_keys_give_mean_value,
    check_window_tables, check_uniform_queries_reveal_window, check_against_sdpa, check_row_subset_matches_sdpa,
    check_empty_row_is_zero,
    check_gqa_equals_repeated_mha, check_key_permutation_invariance, check_all_ones_mask_equals_dense,
    check_mask_equals_gathered_dense, check_single_tile_uniform_query, check_streaming_equals_full_sequence,
    check_overwrite_and_crop, check_executed_pairs,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()


# ----------------------------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one check

def _caught(monkeypatch, patches):
    for obj, name, value in patches:
        monkeypatch.setattr(obj, name, value)
    failed = 0
    for check in ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    return failed


def _softmax_no_max(s, vh):
    w = np.exp(s)
    return (w @ vh) / w.sum(axis=1, keepdims=True)


def _softmax_wrong_norm(s, vh):
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ vh) / w.shape[1]


_ORIG_VISIBLE = owin.visible_frames_after

MUTANTS = {
    "group_modulo": [(oatt, "_group_of", lambda h, nq, nkv: h % nkv)],
    "window_one_short": [(owin, "visible_frames_after",
                          lambda c, W, A, a=None: _ORIG_VISIBLE(c, W - 1, A, None if a is None else min(a, W - 1)))],
    "anchor_ignored": [(owin, "visible_frames_after",
                        lambda c, W, A, a=None: list(range(max(0, c - W), c)))],
    "normalise_by_count": [(oatt, "_softmax_rows", _softmax_wrong_norm)],
    "full_mask_off_by_one": [(oatt, "sliding_window_allowed",
                              lambda fq, fk, F, W, A: owin.sliding_window_allowed(fq, fk, F, W + 1, A))],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(monkeypatch, name):
    assert _caught(monkeypatch, MUTANTS[name]) > 0


_ORIG_ATTEND = oracle.attend


def _attend_rows_sorted(q, k, v, block_mask=None, rows=None, tile=128):
    out = _ORIG_ATTEND(q, k, v, block_mask, None, tile)
    return out if rows is None else out[np.sort(np.asarray(rows))]


def _attend_rows_tile_by_position(q, k, v, block_mask=None, rows=None, tile=128):
    # takes each returned row's mask row from its position in `rows`, not from the row itself
    if rows is None:
        return _ORIG_ATTEND(q, k, v, block_mask, None, tile)
    rows = np.asarray(rows)
    out = np.stack([_ORIG_ATTEND(q[[r]], k, v, None if block_mask is None else
                                 block_mask[:, [min(i // tile, block_mask.shape[1] - 1)]], None, tile)[0]
                    for i, r in enumerate(rows)])
    return out


@pytest.mark.parametrize("mutant", [_attend_rows_sorted, _attend_rows_tile_by_position], ids=lambda f: f.__name__)
def test_row_subset_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(oracle, "attend", mutant)
    with pytest.raises(AssertionError):
        check_row_subset_matches_sdpa()


def test_scale_mutant_is_caught(monkeypatch):
    real_sqrt = math.sqrt

    class FakeMath:
        sqrt = staticmethod(lambda x: x)  # 1/d instead of 1/sqrt(d)
        pi = math.pi

    monkeypatch.setattr(oatt, "math", FakeMath)
    assert _caught(monkeypatch, []) > 0
    assert real_sqrt(4.0) == 2.0


def test_mask_generator_counts():
    """Kept tiles per row: 25% of 293 -> 73 (37 at the first 1K step), 15% of 659 -> 99 (50)."""
    for n_q, n_k, pct, want in [(18720, 37440, 25, 73), (18720, 18720, 25, 37),
                                (42120, 84240, 15, 99), (42120, 42120, 15, 50)]:
        bm = make_block_mask(3, 1, 2, n_q, n_k, pct)
        assert np.all(bm.sum(axis=2) == want)
        for qt in range(bm.shape[1]):
            assert np.all(bm[:, qt, diagonal_tiles(qt, n_q, n_k)] == 1)
    # diagonal tiles by absolute position: 1K steady offset is 18720 = 146 tiles + 32
    assert diagonal_tiles(0, 18720, 37440) == [146, 147]
    assert diagonal_tiles(146, 18720, 37440) == [292]
    assert diagonal_tiles(0, 18720, 18720) == [0]


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    b = f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: to even gives 1.0; 1 + 3*2^-8 rounds up to 1 + 2^-6
    assert list(bf16_bits_to_f32(b)[:4]) == [1.0, 1.0, 1.015625, -2.5]
    assert b[0] == 0x3F80 and b[3] == 0xC020
