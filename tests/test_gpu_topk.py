"""GPU block-score top-k masks (uf_block_mask_topk) against the float64 oracle.

The ratings are fp32 on the GPU and float64 in the oracle, and a rating
decides which tiles a row keeps, so the comparison is in two parts:
  * every rating must lie within a bound derived from fp32 summation: the
    tile means are sums of at most 128 rows (8 per lane, then 16 or 32 lane
    partials) and the rating is an fma chain over d, so
        |rating - exact| <= (d + 2 * 48) * 2^-24 * sum_c mean|q_c| * mean|k_c|,
    used here with a factor of 2 to spare (TOL_FACTOR);
  * the mask must keep every local-window tile and exactly top_k (or all
    remaining) other tiles; where the oracle's top_k-th and next rating are
    further apart than twice the bound, the row must equal the oracle's row
    exactly; elsewhere (a near tie that fp32 may order either way) every
    chosen tile must rate within twice the bound of every tile left out.
Inputs come from synth's seeded generators; "biased" inputs add a per-tile
offset vector (drawn from the same generator family, tensor ids 4 and 5) so
that ratings spread out the way real attention's do.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import TILE, Workload, bf16_bits_to_f32, draw_normal, draw_step_tensors, f32_to_bf16_bits
from tests import fp8_lut
from tests.gpu_util import assert_close, to_dev
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
TOL_FACTOR = 2.0


def _abs_means(x, tile=TILE):
    """mean |x| per (head, tile, channel): [H, n_tiles, d] float64."""
    return oracle.pooled_tiles(np.abs(x.astype(np.float64)), tile)


def rating_bound(q, k):
    """[Hq, n_qt, n_kt] bound on |fp32 rating - exact rating|."""
    d = q.shape[2]
    aq, ak = _abs_means(q), _abs_means(k)
    group = q.shape[1] // k.shape[1]
    out = np.empty((q.shape[1], aq.shape[1], ak.shape[1]))
    for h in range(q.shape[1]):
        out[h] = aq[h] @ ak[h // group].T
    return TOL_FACTOR * (d + 2 * 48) * U * out


def check_mask(got_mask, got_scores, q, k, top_k, local, what):
    """Compare one step's GPU mask/ratings with the oracle's; returns (exact rows, near-tie rows)."""
    n_q, n_k = q.shape[0], k.shape[0]
    ref_s = oracle.block_scores(q, k)
    bound = rating_bound(q, k)
    assert got_scores.shape == ref_s.shape
    err = np.abs(got_scores.astype(np.float64) - ref_s)
    assert (err <= bound).all(), f"{what}: rating error {err.max():.3e} beyond bound (worst ratio " \
                                 f"{(err / np.maximum(bound, 1e-300)).max():.2f})"
    ref_m = oracle.topk_block_mask(ref_s, n_q, n_k, top_k, local)
    assert got_mask.shape == ref_m.shape
    assert set(np.unique(got_mask).tolist()) <= {0, 1}
    n_kt = ref_s.shape[2]
    exact = near = 0
    for qt in range(ref_s.shape[1]):
        forced = oracle.local_tiles(qt, n_q, n_k, local)
        is_forced = np.zeros(n_kt, dtype=bool)
        is_forced[forced] = True
        cand = np.nonzero(~is_forced)[0]
        kk = min(top_k, len(cand))
        for h in range(ref_s.shape[0]):
            row = got_mask[h, qt].astype(bool)
            assert row[is_forced].all(), (what, h, qt, "local window tile dropped")
            chosen = cand[row[cand]]
            assert len(chosen) == kk, (what, h, qt, len(chosen), kk)
            s = ref_s[h, qt, cand]
            order = np.sort(s)[::-1]
            gap = order[kk - 1] - order[kk] if 0 < kk < len(cand) else np.inf
            tol = 2 * bound[h, qt, cand].max() if len(cand) else 0.0
            if gap > tol:
                exact += 1
                assert np.array_equal(row, ref_m[h, qt].astype(bool)), (what, h, qt)
            else:
                near += 1
                left = cand[~row[cand]]
                if len(chosen) and len(left):
                    assert ref_s[h, qt, chosen].min() >= ref_s[h, qt, left].max() - tol, (what, h, qt)
    print(f"  {what}: rating err max {err.max():.2e}; rows exact {exact}, near-tie {near}", flush=True)
    return exact, near


def _stream(cfg, biased=False, fp8_scales=None):
    """Yield (step, q bits, cache, window keys) while streaming cfg's steps.  With fp8_scales
    (q, k, v) the cache holds E4M3 codes and the oracle's window the dequantized values."""
    L, F, W, A = cfg.tokens_per_frame, cfg.frames_per_step, cfg.window_frames, cfg.anchor_frames
    kw = {}
    if fp8_scales is not None:
        kw = dict(kv_dtype=uf.UF_FP8_E4M3, q_scale=fp8_scales[0], k_scale=fp8_scales[1], v_scale=fp8_scales[2])
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, L, W, A, **kw)
    win = oracle.FrameListWindow(L, W, A)
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        if biased:
            qb, kb = _biased(cfg, s, qb, kb)
        cache.append(to_dev(kb), to_dev(vb), F)
        if fp8_scales is None:
            win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), F)
        else:
            win.append(fp8_lut.round_trip_bits(kb, fp8_scales[1]), fp8_lut.round_trip_bits(vb, fp8_scales[2]), F)
        yield s, qb, cache, win
    cache.close()


def _biased(cfg, s, qb, kb):
    """Add a per-128-token offset vector (std 2) to q and k, then round to bf16 again."""
    def add(bits, tid):
        x = bf16_bits_to_f32(bits)
        n, h, d = x.shape
        nt = -(-n // TILE)
        off = 2.0 * draw_normal(cfg.index, s, tid, (nt, h, d))
        return f32_to_bf16_bits(x + np.repeat(off, TILE, axis=0)[:n])
    return add(qb, 4), add(kb, 5)


def run_topk(cfg, top_k, local, steps=None, biased=False, fp8_scales=None):
    totals = [0, 0]
    for s, qb, cache, win in _stream(cfg, biased, fp8_scales):
        if steps is not None and s not in steps:
            continue
        q = to_dev(qb)
        n_k = cache.window().n_keys
        scores = torch.empty((cfg.n_q_heads, -(-cfg.q_tokens // TILE), -(-n_k // TILE)), dtype=torch.float32,
                             device="cuda:0")
        print(f"{cfg.name} step {s}: top_k {top_k}, local {local}, {n_k} keys", flush=True)
        mask = cache.block_mask_topk(q, top_k, local, scores=scores)
        torch.cuda.synchronize()
        kk, _ = win.keys_values()
        e, n = check_mask(mask.cpu().numpy(), scores.cpu().numpy(), bf16_bits_to_f32(qb), kk, top_k, local,
                          f"{cfg.name} step {s}")
        totals[0] += e
        totals[1] += n
    return totals


# ---------------------------------------------------------------------------------------------

REDUCED = [
    # anchor + ring: key tiles straddle the anchor/ring boundary and the ring wrap
    (Workload(40, "t-anchor", "bf16", 4, 2, 128, (10, 20), 3, 6, 3, 6, None), 3, 1),
    # head_dim 64, GQA 4, ragged tiles
    (Workload(41, "t-d64", "bf16", 8, 2, 64, (9, 31), 2, 4, 0, 4, None), 2, 0),
    # one KV head, per-frame steps
    (Workload(42, "t-decoder", "bf16", 4, 1, 128, (12, 25), 1, 3, 0, 5, None), 1, 2),
]


@pytest.mark.parametrize("case", REDUCED, ids=lambda c: c[0].name)
def test_topk_reduced(case):
    cfg, top_k, local = case
    run_topk(cfg, top_k, local)


@pytest.mark.parametrize("case", REDUCED, ids=lambda c: c[0].name)
def test_topk_reduced_biased(case):
    cfg, top_k, local = case
    exact, near = run_topk(cfg, top_k, local, biased=True)
    assert exact >= 4 * near, (exact, near)


def test_topk_1k_shape():
    # 1K steady state: 147 query tiles x 293 key tiles per head, 25% of the key tiles chosen
    cfg = Workload(3, "1k", "bf16", 12, 12, 128, (60, 104), 3, 6, 0, 2, None)
    run_topk(cfg, top_k=71, local=0, steps=[0, 1])


def test_topk_2k_shape_biased():
    cfg = Workload(4, "2k", "bf16", 12, 12, 128, (90, 156), 3, 6, 0, 2, None)
    exact, near = run_topk(cfg, top_k=97, local=1, steps=[1], biased=True)
    assert exact > near


@pytest.mark.parametrize("case", REDUCED[:2], ids=lambda c: c[0].name)
def test_topk_from_fp8_cache(case):
    """E4M3 keys (decoded exactly, times k_scale) against the oracle on the dequantized keys."""
    cfg, top_k, local = case
    exact, near = run_topk(cfg, top_k, local, biased=True, fp8_scales=(0.02, 0.03, 0.02))
    assert exact >= 4 * near, (exact, near)


def test_topk_from_fp8_cache_2k_shape():
    cfg = Workload(4, "2k", "bf16", 12, 12, 128, (90, 156), 3, 6, 0, 2, None)
    exact, near = run_topk(cfg, top_k=97, local=1, steps=[1], biased=True, fp8_scales=(0.02, 0.03, 0.02))
    assert exact > near


@pytest.mark.parametrize("top_k,local", [(0, 0), (0, 3), (1000, 0), (5, 1000)])
def test_topk_degenerate_counts(top_k, local):
    cfg = Workload(43, "t-edge", "bf16", 2, 2, 128, (10, 30), 1, 3, 0, 3, None)
    run_topk(cfg, top_k, local)


def test_topk_ties_go_to_lower_tiles():
    """All-zero keys rate every tile 0: the lowest-index candidates are chosen, exactly."""
    L, H, d = 300, 2, 128
    cache = KVCache(H, d, L, 4, 0)
    zeros = torch.zeros((L, H, d), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(4):
        cache.append(zeros, zeros, 1)
    qb = f32_to_bf16_bits(draw_normal(44, 0, 0, (L, 2 * H, d)))
    q = to_dev(qb)
    mask = cache.block_mask_topk(q, 3, 0).cpu().numpy()
    ref = oracle.topk_block_mask(np.zeros(mask.shape), L, 4 * L, 3, 0)
    assert np.array_equal(mask, ref)
    cache.close()


def test_topk_no_queries():
    cache = KVCache(1, 64, 100, 2, 0)
    z = torch.zeros((100, 1, 64), dtype=torch.bfloat16, device="cuda:0")
    cache.append(z, z, 1)
    q = torch.zeros((0, 1, 64), dtype=torch.bfloat16, device="cuda:0")
    mask = torch.empty((1, 0, 1), dtype=torch.uint8, device="cuda:0")
    cache.block_mask_topk(q, 2, 0, mask=mask)
    torch.cuda.synchronize()
    cache.close()


def test_generated_mask_drives_attention():
    """The generated mask, fed to uf_attn_step, gives the oracle's attention under the oracle's mask
    (on the query tiles whose mask rows agree in every head, at least 90% of them)."""
    cfg = Workload(45, "t-e2e", "bf16", 4, 2, 128, (16, 40), 2, 4, 1, 4, None)
    last = None
    for s, qb, cache, win in _stream(cfg, biased=True):
        q = to_dev(qb)
        mask = cache.block_mask_topk(q, 4, 1)
        out = torch.empty_like(q)
        cache.attn_step(q, out, mask)
        torch.cuda.synchronize()
        kk, vv = win.keys_values()
        qf = bf16_bits_to_f32(qb)
        ref_m = oracle.topk_block_mask(oracle.block_scores(qf, kk), cfg.q_tokens, kk.shape[0], 4, 1)
        got_m = mask.cpu().numpy()
        same = [t for t in range(ref_m.shape[1]) if np.array_equal(got_m[:, t], ref_m[:, t])]
        print(f"  step {s}: {len(same)} of {ref_m.shape[1]} query tiles with identical mask rows", flush=True)
        assert len(same) >= 0.9 * ref_m.shape[1]
        rows = np.concatenate([np.arange(t * TILE, min((t + 1) * TILE, cfg.q_tokens)) for t in same])
        ref = oracle.attend(qf, kk, vv, ref_m, rows=rows)
        got = out.float().cpu().numpy()[rows]
        assert_close(got, ref, f"e2e step {s}")
        last = s
    assert last == cfg.steps - 1
