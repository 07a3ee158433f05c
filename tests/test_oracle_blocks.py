"""Pins for the block order of a step's tokens (oracle/blocks.py), CPU only.

  * small cases worked by hand (a single block is raster order; one frame of
    two patches; a block plus ragged edges);
  * structure at the workload shapes: a permutation; with F even and 8 | H, W
    every tile is one (2, 8, 8) box; with F odd the last frame's tiles are two
    8x8 patches; the leftover tokens come last, in raster order;
  * attention over block-ordered keys equals attention over raster keys, and
    permuting the queries permutes the output rows.
"""
import numpy as np
import pytest

import oracle
import oracle.blocks as ob


def check_hand_examples():
    # F=2, 8x8: one block, frame-major then row then column = raster order
    assert np.array_equal(ob.block_order(2, 8, 8), np.arange(128))
    # F=1, 8x16: two 8x8 patches, left (columns 0-7) then right (8-15)
    left = [16 * y + x for y in range(8) for x in range(8)]
    right = [16 * y + 8 + x for y in range(8) for x in range(8)]
    assert ob.block_order(1, 8, 16).tolist() == left + right
    # F=2, 9x9: the block (frames 0 and 1, rows/columns 0-7), then per frame column 8 of
    # rows 0-7 and all of row 8
    blk = [81 * t + 9 * y + x for t in range(2) for y in range(8) for x in range(8)]
    edges = [81 * t + e for t in range(2) for e in [8, 17, 26, 35, 44, 53, 62, 71, 72, 73, 74, 75, 76, 77, 78, 79, 80]]
    assert ob.block_order(2, 9, 9).tolist() == blk + edges
    # F=2, 16x16: four blocks in row-major block order; block b starts at frame 0, its top-left token
    o = ob.block_order(2, 16, 16)
    assert [int(o[128 * b]) for b in range(4)] == [0, 8, 128, 136]
    assert int(o[64]) == 256  # second half of the first block: frame 1, row 0, column 0


def _coords(idx, h, w):
    return idx // (h * w), (idx // w) % h, idx % w


def check_structure(shape=(3, 90, 156)):
    f, h, w = shape
    order = ob.block_order(f, h, w)
    n = f * h * w
    assert np.array_equal(np.sort(order), np.arange(n))
    hb, wb = h // 8, w // 8
    pair_tokens = (f // 2) * hb * wb * 128
    for t in range(pair_tokens // 128):
        fr, y, x = _coords(order[128 * t:128 * (t + 1)], h, w)
        assert fr.max() - fr.min() == 1 and fr.min() % 2 == 0
        assert y.max() - y.min() == 7 and x.max() - x.min() == 7 and y.min() % 8 == 0 and x.min() % 8 == 0
        assert len({(a, b, c) for a, b, c in zip(fr, y, x)}) == 128
    odd_tokens = (f % 2) * hb * wb * 64
    for pch in range(odd_tokens // 64):
        fr, y, x = _coords(order[pair_tokens + 64 * pch:pair_tokens + 64 * (pch + 1)], h, w)
        assert (fr == f - 1).all() and y.max() - y.min() == 7 and x.max() - x.min() == 7
    rest = order[pair_tokens + odd_tokens:]
    assert np.all(np.diff(rest) > 0)  # raster order
    fr, y, x = _coords(rest, h, w)
    assert np.all((y >= 8 * hb) | (x >= 8 * wb))


def check_all_structures():
    for shape in [(2, 16, 24), (4, 8, 8), (3, 60, 104), (3, 90, 156), (1, 30, 52), (2, 10, 13), (5, 9, 17)]:
        check_structure(shape)


def check_attention_equivariance():
    rng = np.random.default_rng(2)
    f, h, w = 3, 10, 12
    n = f * h * w
    q = rng.standard_normal((n, 2, 16))
    k = rng.standard_normal((n, 1, 16))
    v = rng.standard_normal((n, 1, 16))
    out = oracle.attend(q, k, v)
    perm_out = oracle.attend(ob.to_block_order(q, f, h, w), ob.to_block_order(k, f, h, w), ob.to_block_order(v, f, h, w))
    assert np.allclose(ob.from_block_order(perm_out, f, h, w), out, rtol=0, atol=1e-12)
    x = rng.standard_normal((n, 3))
    assert np.array_equal(ob.from_block_order(ob.to_block_order(x, f, h, w), f, h, w), x)


ALL = [check_hand_examples, check_all_structures, check_attention_equivariance]


@pytest.mark.parametrize("check", ALL, ids=lambda c: c.__name__)
def test_block_order_pin(check):
    check()


def _order_transposed(frames, grid_h, grid_w):
    # planted mistake: blocks taken column-major
    o = ORIG(frames, grid_h, grid_w)
    hb, wb = grid_h // 8, grid_w // 8
    nb = hb * wb
    if nb < 2 or frames < 2:
        return o
    blocks = o[:128 * nb].reshape(hb, wb, 128).transpose(1, 0, 2).reshape(-1)
    return np.concatenate([blocks, o[128 * nb:]])


def _order_time_inner(frames, grid_h, grid_w):
    # planted mistake: inside a block, frames vary fastest
    o = ORIG(frames, grid_h, grid_w).copy()
    n = (frames // 2) * (grid_h // 8) * (grid_w // 8)
    for b in range(n):
        o[128 * b:128 * (b + 1)] = o[128 * b:128 * (b + 1)].reshape(2, 64).T.reshape(-1)
    return o


ORIG = ob.block_order


@pytest.mark.parametrize("mutant", [_order_transposed, _order_time_inner], ids=lambda m: m.__name__)
def test_block_order_mutant_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ob, "block_order", mutant)
    failed = 0
    for check in ALL:
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed > 0
