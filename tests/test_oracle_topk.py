"""Pins for the top-k block-mask oracle (oracle/topk.py), CPU only.

Each pin checks the oracle against something other than itself:
  * a hand-worked example (tests/golden/topk_example.json);
  * bilinearity: the dot product of two tile means equals the mean of the
    token-level dot products over the tile pair, computed from the full
    q k^T matrix;
  * brute force over all k-subsets: with distinct scores the chosen tiles
    are the subset of candidates with the largest score sum;
  * closed forms for ragged tiles, ties and the local window at the
    workloads' own shapes;
  * invariances (token order inside a tile, positive scaling of q, GQA
    groups with opposite rankings).
Planted mistakes in the oracle must fail at least one pin.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle.topk as otk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _forced(qt, n_q, n_k, local, tile):
    return set(otk.local_tiles(qt, n_q, n_k, local, tile))


def check_golden_example():
    t = json.load(open(os.path.join(GOLDEN, "topk_example.json")))
    k = np.array(t["keys"], dtype=np.float64)
    q = np.array(t["queries"], dtype=np.float64)
    s = otk.block_scores(q, k, tile=t["tile"])
    assert np.array_equal(s, np.array(t["scores"], dtype=np.float64)), s
    for c in t["cases"]:
        m = otk.topk_block_mask(s, q.shape[0], k.shape[0], c["top_k"], c["local_blocks"], tile=t["tile"])
        assert np.array_equal(m, np.array(c["mask"], dtype=np.uint8)), (c, m)


def check_bilinearity():
    """mean_i q_i . mean_j k_j == mean over (i, j) of q_i . k_j, tile pair by tile pair."""
    rng = np.random.default_rng(7)
    tile = 16
    for n_q, n_k, hq, hkv in [(40, 70, 4, 2), (16, 33, 3, 3), (5, 16, 2, 1)]:
        q = rng.standard_normal((n_q, hq, 8))
        k = rng.standard_normal((n_k, hkv, 8))
        s = otk.block_scores(q, k, tile)
        qb = np.arange(n_q) // tile
        kb = np.arange(n_k) // tile
        for h in range(hq):
            g = h // (hq // hkv)
            full = q[:, h, :] @ k[:, g, :].T          # token-level dot products
            for a in range(qb[-1] + 1):
                for b in range(kb[-1] + 1):
                    blk = full[np.ix_(qb == a, kb == b)]
                    assert abs(s[h, a, b] - blk.mean()) < 1e-12, (n_q, n_k, h, a, b)


def check_ragged_tile_mean():
    """A partial last tile of constant tokens pools to that constant."""
    x = np.zeros((2 * 128 + 5, 1, 4))
    x[256:] = [3.0, -1.0, 0.5, 2.0]
    p = otk.pooled_tiles(x)
    assert p.shape == (1, 3, 4)
    assert np.array_equal(p[0, 2], [3.0, -1.0, 0.5, 2.0])
    assert not p[0, :2].any()


def check_subset_brute_force():
    """Distinct scores: the kept candidates are the k-subset of largest score sum."""
    rng = np.random.default_rng(11)
    tile = 4
    for trial in range(30):
        n_k = int(rng.integers(9, 33))
        n_q = int(rng.integers(1, min(n_k, 12) + 1))
        local = int(rng.integers(0, 2))
        top_k = int(rng.integers(0, 5))
        n_qt, n_kt = -(-n_q // tile), -(-n_k // tile)
        scores = rng.permutation(n_qt * n_kt * 2).reshape(2, n_qt, n_kt).astype(np.float64) - 7.5
        m = otk.topk_block_mask(scores, n_q, n_k, top_k, local, tile)
        for h in range(2):
            for qt in range(n_qt):
                forced = _forced(qt, n_q, n_k, local, tile)
                cands = [j for j in range(n_kt) if j not in forced]
                kk = min(top_k, len(cands))
                best = max(itertools.combinations(cands, kk), key=lambda c: sum(scores[h, qt, j] for j in c))
                expect = np.zeros(n_kt, dtype=np.uint8)
                expect[list(forced)] = 1
                expect[list(best)] = 1
                assert np.array_equal(m[h, qt], expect), (trial, h, qt)


def check_ties_lowest_index():
    """All-zero keys score 0 everywhere: the lowest-index candidates are kept."""
    n_q, n_k, tile = 300, 1300, 128
    q = np.ones((n_q, 2, 8))
    k = np.zeros((n_k, 1, 8))
    s = otk.block_scores(q, k, tile)
    m = otk.topk_block_mask(s, n_q, n_k, 3, 0, tile)
    # queries are keys 1000..1299: tile 0 holds 1000..1127 (key tiles 7, 8); tile 2 holds 1256..1299 (tiles 9, 10)
    assert sorted(np.nonzero(m[0, 0])[0].tolist()) == [0, 1, 2, 7, 8]
    assert sorted(np.nonzero(m[1, 2])[0].tolist()) == [0, 1, 2, 9, 10]


def check_local_window_at_workload_shapes():
    """Diagonal tiles at the 1K/2K steady state (queries are the newest n_q keys)."""
    # 2K: n_q = 42120, n_k = 84240; query tile 0 spans keys 42120..42247 -> tiles 329, 330
    assert otk.local_tiles(0, 42120, 84240, 0) == [329, 330]
    assert otk.local_tiles(0, 42120, 84240, 1) == [328, 329, 330, 331]
    # last query tile: keys 84232..84239 -> tile 658 only, clipped at the end
    assert otk.local_tiles(329, 42120, 84240, 2) == [656, 657, 658]
    # 1K: n_q = 18720, n_k = 37440; tile 146 holds keys 37408..37439 -> tile 292
    assert otk.local_tiles(146, 18720, 37440, 0) == [292]
    # step 0: n_q == n_k, tile i is its own diagonal
    assert otk.local_tiles(5, 18720, 18720, 0) == [5]
    assert otk.local_tiles(0, 18720, 18720, 3) == [0, 1, 2, 3]


def check_counts():
    rng = np.random.default_rng(3)
    n_q, n_k, tile = 700, 2000, 128
    s = rng.standard_normal((3, 6, 16))
    for top_k, local in [(0, 0), (4, 0), (4, 1), (20, 0), (13, 2)]:
        m = otk.topk_block_mask(s, n_q, n_k, top_k, local, tile)
        for qt in range(6):
            nf = len(_forced(qt, n_q, n_k, local, tile))
            assert (m[:, qt].sum(axis=1) == nf + min(top_k, 16 - nf)).all()


def check_invariances():
    rng = np.random.default_rng(5)
    n_q, n_k, tile = 260, 900, 128
    q = rng.standard_normal((n_q, 4, 16))
    k = rng.standard_normal((n_k, 2, 16))
    s = otk.block_scores(q, k, tile)
    m = otk.topk_block_mask(s, n_q, n_k, 2, 0, tile)
    # shuffling tokens inside each tile leaves the means, hence the mask, unchanged
    perm_q = np.concatenate([t * tile + rng.permutation(min(tile, n_q - t * tile)) for t in range(3)])
    perm_k = np.concatenate([t * tile + rng.permutation(min(tile, n_k - t * tile)) for t in range(8)])
    s2 = otk.block_scores(q[perm_q], k[perm_k], tile)
    assert np.allclose(s2, s, rtol=0, atol=1e-12)
    assert np.array_equal(otk.topk_block_mask(s2, n_q, n_k, 2, 0, tile), m)
    # a positive scale of q keeps the ranking
    assert np.array_equal(otk.topk_block_mask(otk.block_scores(3.0 * q, k, tile), n_q, n_k, 2, 0, tile), m)
    # GQA: heads 0, 1 read group 0 and heads 2, 3 read group 1; the groups rank tiles in opposite orders
    qq = np.ones((n_q, 4, 16))
    kk = np.zeros((n_k, 2, 16))
    for t in range(8):
        kk[t * tile:(t + 1) * tile, 0, :] = t
        kk[t * tile:(t + 1) * tile, 1, :] = -t
    mm = otk.topk_block_mask(otk.block_scores(qq, kk, tile), n_q, n_k, 2, 0, tile)
    # query tile 0 keys 640..767 -> diagonal tile 5; group 0 prefers high tiles, group 1 low ones
    for h in (0, 1):
        assert np.nonzero(mm[h, 0])[0].tolist() == [5, 6, 7]
    for h in (2, 3):
        assert np.nonzero(mm[h, 0])[0].tolist() == [0, 1, 5]


ALL_CHECKS = [check_golden_example, check_bilinearity, check_ragged_tile_mean, check_subset_brute_force,
              check_ties_lowest_index, check_local_window_at_workload_shapes, check_counts, check_invariances]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_topk_pin(check):
    check()


# ---------------------------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin

def _pooled_sum(x, tile=128):
    n, h, d = x.shape
    out = np.zeros((h, -(-n // tile), d))
    for t in range(out.shape[1]):
        out[:, t, :] = x[t * tile:(t + 1) * tile].astype(np.float64).sum(axis=0) / tile
    return out


def _mask_ties_high(scores, n_q, n_k, top_k, local_blocks, tile=128):
    m = np.zeros(scores.shape, dtype=np.uint8)
    for qt in range(scores.shape[1]):
        forced = otk.local_tiles(qt, n_q, n_k, local_blocks, tile)
        others = np.setdiff1d(np.arange(scores.shape[2]), forced)[::-1]
        for h in range(scores.shape[0]):
            m[h, qt, forced] = 1
            m[h, qt, others[np.argsort(-scores[h, qt, others], kind="stable")][:top_k]] = 1
    return m


def _mask_lowest(scores, n_q, n_k, top_k, local_blocks, tile=128):
    return ORIG_MASK(-scores, n_q, n_k, top_k, local_blocks, tile)


def _local_shifted(q_tile, n_q, n_k, local_blocks, tile=128):
    return ORIG_LOCAL(q_tile, n_q - 1, n_k, local_blocks, tile)


def _mask_topk_of_all(scores, n_q, n_k, top_k, local_blocks, tile=128):
    # top-k over every tile, then the local window added (the other reading of "top-k plus window")
    m = np.zeros(scores.shape, dtype=np.uint8)
    for qt in range(scores.shape[1]):
        forced = otk.local_tiles(qt, n_q, n_k, local_blocks, tile)
        allt = np.arange(scores.shape[2])
        for h in range(scores.shape[0]):
            m[h, qt, forced] = 1
            m[h, qt, allt[np.argsort(-scores[h, qt], kind="stable")][:top_k]] = 1
    return m


ORIG_MASK = otk.topk_block_mask
ORIG_LOCAL = otk.local_tiles

MUTANTS = {
    "sum_over_full_tile": ("pooled_tiles", _pooled_sum),
    "gqa_modulo": ("_group_of", lambda h, hq, hkv: h % hkv),
    "ties_to_higher_index": ("topk_block_mask", _mask_ties_high),
    "lowest_scores": ("topk_block_mask", _mask_lowest),
    "diagonal_off_by_one": ("local_tiles", _local_shifted),
    "topk_over_all_tiles": ("topk_block_mask", _mask_topk_of_all),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_topk_mutant_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(otk, attr, fn)
    failed = 0
    for check in ALL_CHECKS:
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant {name} passed every pin"
