"""FP8 (E4M3) cache on the GPU against the oracle.

Storage: every appended value is quantized with the cache's static scale; the
stored codes must equal the oracle's E4M3 codes, byte for byte, in the rows
the ring model predicts.

Attention: the oracle attends in float64 over the dequantized q, k and v (its
plain definition).  The kernel differs from it by rounding the probabilities to
E4M3 for the P.V product and the output to bf16; tests/fp8_bound.py derives a
per-element bound for that (and tests/test_fp8_bound.py checks the bound on an
emulation of the kernel's arithmetic).  Every output element must lie within it;
the tests print how much of it was used.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8
from synth import WORKLOAD, TILE, Workload, bf16_bits_to_f32, draw_step_tensors, make_block_mask
from tests import fp8_lut
from tests.fp8_bound import bound as _bound
from tests.gpu_util import errors, f32_of, map_row_tiles, oracle_rows, to_dev
from tests.ring_model import RingModel
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu

SCALES = (0.02, 0.015, 0.02)  # q, k, v: N(0,1) draws use E4M3's range without saturating


def _fp8_cache(cfg, scales=SCALES, **kw):
    q_s, k_s, v_s = scales
    return KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames,
                   kv_dtype=uf.UF_FP8_E4M3, q_scale=q_s, k_scale=k_s, v_scale=v_s, **kw)


@pytest.mark.parametrize("case", [(2, 128, 200, 4, 1, 2, 6), (3, 64, 96, 3, 0, 1, 7)],
                         ids=lambda c: "H%d-d%d-L%d-W%d-A%d-F%d" % c[:6])
def test_fp8_append_codes_bit_exact(case):
    H, d, L, W, A, F, n = case
    print(f"fp8 append case {case}", flush=True)
    cfg = Workload(60, "f8-append", "bf16", H, H, d, (1, L), F, W, A, n, None)
    cache = _fp8_cache(cfg)
    cache.k_storage.zero_()
    cache.v_storage.zero_()
    model = RingModel(H, d, L, W, A)
    for s in range(n):
        _, kb, vb = draw_step_tensors(cfg, s, scale_q=1.0)
        kb = kb.copy()
        kb[0, 0, :4] = [0x4580, 0xC580, 0x3C00, 0x0000]  # +-4096 (saturate at +-448 * scale), 2^-7, 0
        cache.append(to_dev(kb), to_dev(vb), F)
        kc = f8.quantize(bf16_bits_to_f32(kb), SCALES[1]).astype(np.uint16)
        vc = f8.quantize(bf16_bits_to_f32(vb), SCALES[2]).astype(np.uint16)
        model.append(F, kc, vc)
        torch.cuda.synchronize()
        _same_codes(cache.k_storage, model.k, f"K codes, append {s}")
        _same_codes(cache.v_storage, model.v, f"V codes, append {s}")
        if s == n // 2:  # re-write the newest append in place
            _, kb2, vb2 = draw_step_tensors(cfg, s + 100, scale_q=1.0)
            cache.append(to_dev(kb2), to_dev(vb2), F, uf.UF_APPEND_OVERWRITE_NEWEST)
            model.overwrite_newest(f8.quantize(bf16_bits_to_f32(kb2), SCALES[1]).astype(np.uint16),
                                   f8.quantize(bf16_bits_to_f32(vb2), SCALES[2]).astype(np.uint16))
            torch.cuda.synchronize()
            _same_codes(cache.k_storage, model.k, f"K codes, overwrite after append {s}")
            _same_codes(cache.v_storage, model.v, f"V codes, overwrite after append {s}")
    cache.close()


def _same_codes(storage, want, what):
    got = storage.cpu().numpy().astype(np.uint16)
    bad = np.argwhere(got != want)
    for h, r, c in bad[:8]:
        g, w = int(got[h, r, c]), int(want[h, r, c])
        print(f"  {what}: head {h} row {r} ch {c}: got 0x{g:02x} ({f8.e4m3_decode(np.array([g]))[0]}), "
              f"want 0x{w:02x} ({f8.e4m3_decode(np.array([w]))[0]})", flush=True)
    assert len(bad) == 0, f"{what}: {len(bad)} codes differ"


def run_fp8_stream(cfg, check_steps=None, tiles=None, scales=SCALES, scale_q=1.0, **cache_kw):
    q_s, k_s, v_s = scales
    cache = _fp8_cache(cfg, scales, **cache_kw)
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    check_steps = range(cfg.steps) if check_steps is None else check_steps
    worst = 0.0
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s, scale_q)
        q_d = to_dev(qb)
        print(f"{cfg.name} step {s}: fp8 append + attend", flush=True)
        cache.append(to_dev(kb), to_dev(vb), cfg.frames_per_step)
        # oracle.fp8 quantization of bf16 inputs, tabulated over the 65536 bit patterns
        win.append(fp8_lut.round_trip_bits(kb, k_s), fp8_lut.round_trip_bits(vb, v_s), cfg.frames_per_step)
        n_k = cache.window().n_keys
        mask_np = mask_d = None
        if cfg.mask_pct is not None:
            mask_np = make_block_mask(cfg.index, s, cfg.n_q_heads, cfg.q_tokens, n_k, cfg.mask_pct)
            mask_d = torch.from_numpy(mask_np).to("cuda:0")
        out = torch.empty_like(q_d)
        cache.attn_step(q_d, out, mask_d)
        if s not in check_steps:
            continue
        torch.cuda.synchronize()
        got = f32_of(out)
        nqt = -(-cfg.q_tokens // TILE)
        sel_tiles = range(nqt) if tiles is None or tiles >= nqt else \
            sorted({0, nqt - 1, *np.random.default_rng(s).choice(np.arange(1, nqt - 1), tiles - 2, replace=False)})
        rows = np.concatenate([np.arange(t * TILE, min((t + 1) * TILE, cfg.q_tokens)) for t in sel_tiles])
        qq = fp8_lut.round_trip_bits(qb, f8.attention_q_scale(q_s, k_s, cfg.head_dim))
        kk, vv = win.keys_values()
        ref = oracle_rows(qq, kk, vv, mask_np, rows)
        # the bound is row-wise: evaluate it on the same tile groups, each with its rows' ref
        pos = {int(r): i for i, r in enumerate(rows)}
        bound = map_row_tiles(lambda r: _bound(qq, kk, vv, ref[[pos[int(x)] for x in r]], mask_np, r), rows)
        err = np.abs(got[rows].astype(np.float64) - ref)
        ratio = float((err / bound).max())
        ma, rl = errors(got[rows], ref)
        print(f"  {cfg.name} step {s}: max_abs={ma:.3e} rel_l2={rl:.3e}, largest error / bound = {ratio:.3f}",
              flush=True)
        assert np.isfinite(got[rows]).all()
        assert ratio <= 1.0, f"{cfg.name} step {s}: error beyond the E4M3 probability bound ({ratio:.3f})"
        worst = max(worst, ratio)
    cache.close()
    return worst


FP8_CASES = [
    Workload(61, "f8-anchor", "bf16", 4, 2, 128, (10, 20), 3, 6, 3, 6, None),    # anchor + ring, GQA 2
    Workload(62, "f8-mask", "bf16", 4, 4, 128, (12, 17), 2, 4, 0, 5, 40),         # per-head mask, ragged
    Workload(63, "f8-d64", "bf16", 8, 2, 64, (9, 31), 2, 4, 1, 4, None),          # head_dim 64, GQA 4
]


@pytest.mark.parametrize("cfg", FP8_CASES, ids=lambda c: c.name)
def test_fp8_attention_within_bound(cfg):
    run_fp8_stream(cfg)


def test_fp8_forced_splits():
    run_fp8_stream(Workload(64, "f8-split", "bf16", 4, 1, 128, (10, 30), 2, 4, 1, 4, None), splits=3)


@pytest.mark.parametrize("hpw", [2, 4])
def test_fp8_per_head_masks_shared_tiles(hpw):
    # per-head masks with a GQA group's heads sharing staged tiles (union walk), GQA 4
    run_fp8_stream(Workload(66, "f8-union", "bf16", 8, 2, 128, (11, 23), 2, 4, 0, 4, 30), heads_per_wg=hpw)


@pytest.mark.timeout(600)
def test_fp8_uneven_split():
    # 320 dense work items: cut into bodies and tails of the key range, then combined
    run_fp8_stream(Workload(68, "f8-body-tail", "bf16", 8, 8, 128, (50, 50), 2, 2, 0, 3, None), check_steps=[2],
                   tiles=16)


def test_fp8_1k_shape():
    cfg = Workload(3, "1k", "bf16", 12, 12, 128, (60, 104), 3, 6, 0, 2, 25)
    run_fp8_stream(cfg, check_steps=[0, 1], tiles=32)


@pytest.mark.timeout(600)
def test_fp8_2k_shape():
    # the 2K chunk (90x156 tokens per frame, 15% mask) at full size, 32 seeded query tiles per head
    run_fp8_stream(WORKLOAD["2k"], check_steps=[0, 3], tiles=32)


def test_fp8_decoder_shape():
    # the decoder step at full size: 12 query heads on 3 KV heads, 1560 tokens per frame, window of
    # 2 frames; few enough work items that the key range is split (combine kernel)
    cfg = Workload(2, "decoder", "bf16", 12, 3, 128, (30, 52), 1, 2, 0, 5, None)
    run_fp8_stream(cfg, check_steps=[0, 1, 4])


def test_fp8_other_scales():
    # a coarser q scale and a finer v scale
    run_fp8_stream(Workload(65, "f8-scales", "bf16", 2, 2, 128, (8, 25), 1, 3, 0, 4, None), scales=(0.05, 0.01, 0.005))


@pytest.mark.parametrize("scale_q", [12.0, 120.0])
def test_fp8_large_scores(scale_q):
    """Scores of tens to hundreds in log2 units (q scaled up; q's scale 1.0 keeps it in range).
    While the reference point stays within +-96 the kernel converts P with the scaled
    conversion; beyond, with a subtraction per score.  q x 12 stays mostly within, q x 120
    goes beyond on almost every row."""
    cfg = Workload(67, "f8-large", "bf16", 2, 2, 128, (8, 25), 1, 3, 0, 3, None)
    run_fp8_stream(cfg, scales=(1.0, 0.015, 0.02), scale_q=scale_q)
