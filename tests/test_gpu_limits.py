"""The kernels on the largest caches the library accepts, on the GPU against the oracle.

A head's K (or V) storage must stay under 4 GiB: the attention kernels address it with 32-bit
byte offsets from the head's 64-bit base.  Each cache here sits 256 bytes under that limit
(15 frames of L tokens, 2^32 - 256 bytes per head and tensor) and has two KV heads, so that the
second head starts beyond 4 GiB of its allocation.  Fourteen frames are committed without data,
so the first real frame fills ring slot 14, the highest rows of every head:
  * step 0, window cropped to that frame: key tiles at the bottom, in the middle and at the top
    of the frame, the ragged last tile ending 256 bytes below 4 GiB;
  * step 1, one more frame (ring slot 0, the wrap) and a window of two frames: one key tile
    holds the last rows of the storage and the first rows of the ring, and the step's last tile
    is ragged again.
Per-head masks (GQA 2) keep a few of those tiles per query tile, and one query tile keeps none.
The step's key range is split (few work items), so split partials and the combine run too.

Only the rows of the tiles a mask can keep carry seeded data; the rest of each frame is zeros.
The oracle attends over the kept tiles alone, in key order (a masked-out tile adds nothing to
the softmax; Ultra Flash notes, key design 3).  The appended rows are checked bit for bit in
the storage: bf16 as written, E4M3 against the tests' quantization table.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8
from synth import bf16_bits_to_f32, draw_normal, f32_to_bf16_bits
from tests import fp8_lut
from tests.fp8_bound import bound as _bound
from tests.gpu_util import assert_close, bits_of, f32_of, to_dev
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu

TILE = 128
W, HKV, HQ, NQ = 15, 2, 4, 300
SCALES = (0.02, 0.015, 0.02)
# (name, head_dim, kv dtype, tokens per frame): 15 * L rows of 256 (d = 128 bf16) or 128 bytes
CASES = [
    ("bf16-d128", 128, uf.UF_BF16, 1118481),
    ("bf16-d64", 64, uf.UF_BF16, 2236962),
    ("fp8-d128", 128, uf.UF_FP8_E4M3, 2236962),
]
SEED = 91  # synth stream index of this test


def _drawn_rows(L):
    """Rows of a frame that carry data: the first two tiles, a middle tile and the last 300 rows
    (which hold the frame's last full tile and its ragged end)."""
    mid = (L // TILE // 2) * TILE
    return np.unique(np.concatenate([np.arange(0, 2 * TILE), np.arange(mid, mid + TILE), np.arange(L - 300, L)]))


class Frame:
    """One appended frame: seeded bf16 data on its drawn rows, zeros elsewhere."""

    def __init__(self, L, d, frame):
        self.rows = _drawn_rows(L)
        self.k_bits = f32_to_bf16_bits(draw_normal(SEED, frame, 1, (len(self.rows), HKV, d)))
        self.v_bits = f32_to_bf16_bits(draw_normal(SEED, frame, 2, (len(self.rows), HKV, d)))
        self.k_dev = torch.zeros((L, HKV, d), dtype=torch.bfloat16, device="cuda:0")
        self.v_dev = torch.zeros_like(self.k_dev)
        idx = torch.from_numpy(self.rows).to("cuda:0")
        self.k_dev[idx] = to_dev(self.k_bits)
        self.v_dev[idx] = to_dev(self.v_bits)

    def take(self, rows, bits):
        pos = np.searchsorted(self.rows, rows)
        assert (self.rows[pos] == rows).all(), "a kept tile reaches a row without data"
        return bits[pos]


def _mask(rng, n_kt, candidates, empty):
    """Per-head mask [HQ, n_q_tiles, n_kt] keeping a seeded choice of the candidate tiles (at
    least one), except the (head, query tile) `empty`, which keeps none."""
    n_qt = -(-NQ // TILE)
    m = np.zeros((HQ, n_qt, n_kt), dtype=np.uint8)
    for h in range(HQ):
        for qt in range(n_qt):
            if (h, qt) == empty:
                continue
            pick = [c for c in candidates if rng.random() < 0.5] or [candidates[(h + qt) % len(candidates)]]
            m[h, qt, pick] = 1
    return m


@pytest.mark.parametrize("name,d,kv_dtype,L", CASES, ids=[c[0] for c in CASES])
def test_largest_cache(name, d, kv_dtype, L):
    assert W * L * d * (1 if kv_dtype == uf.UF_FP8_E4M3 else 2) == (1 << 32) - 256
    fp8 = kv_dtype == uf.UF_FP8_E4M3
    kw = dict(kv_dtype=kv_dtype, q_scale=SCALES[0], k_scale=SCALES[1], v_scale=SCALES[2]) if fp8 else {}
    cache = KVCache(HKV, d, L, W, 0, **kw)
    rng = np.random.default_rng(SEED)
    try:
        cache.append(None, None, W - 1, uf.UF_APPEND_COMMIT_ONLY)  # ring slots 0..13: no data
        frames = []
        q_bits = f32_to_bf16_bits(draw_normal(SEED, 0, 0, (NQ, HQ, d)))
        q = to_dev(q_bits)
        q_or = fp8_lut.round_trip_bits(q_bits, f8.attention_q_scale(SCALES[0], SCALES[1], d)) if fp8 \
            else bf16_bits_to_f32(q_bits)
        for step in range(2):
            fr = Frame(L, d, step)
            frames.append(fr)
            print(f"{name} step {step}: append into ring slot {(W - 1 + step) % W}", flush=True)
            cache.append(fr.k_dev, fr.v_dev, 1)
            torch.cuda.synchronize()
            # the appended rows, bit for bit, at their storage rows in both heads
            base = ((W - 1 + step) % W) * L
            idx = torch.from_numpy(base + fr.rows).to("cuda:0")
            for stor, bits, sc in ((cache.k_storage, fr.k_bits, SCALES[1]), (cache.v_storage, fr.v_bits, SCALES[2])):
                t = stor.index_select(1, idx).transpose(0, 1).contiguous()  # [rows, HKV, d]
                if fp8:
                    got, want = t.cpu().numpy(), fp8_lut.quantize_bits(bits, sc)
                else:
                    got, want = bits_of(t), bits
                assert np.array_equal(got, want), f"{name} step {step}: storage rows differ"

            cache.set_window(step + 1)
            n_k = cache.window().n_keys
            assert n_k == (step + 1) * L
            n_kt = -(-n_k // TILE)
            mid = L // TILE // 2
            if step == 0:
                cand = [0, 1, mid, n_kt - 2, n_kt - 1]
            else:
                straddle = L // TILE  # keys L - (L mod 128) .. : the storage top, then ring row 0
                cand = [0, straddle - 1, straddle, straddle + 1, n_kt - 2, n_kt - 1]
            mask = _mask(rng, n_kt, cand, empty=(1 + step, 2))
            out = torch.empty_like(q)
            cache.attn_step(q, out, torch.from_numpy(mask).to("cuda:0"))
            torch.cuda.synchronize()
            got = f32_of(out)

            # the oracle over the kept tiles alone, in key order
            tiles = sorted(set(np.nonzero(mask.any(axis=(0, 1)))[0].tolist()))
            keys = np.concatenate([np.arange(t * TILE, min((t + 1) * TILE, n_k)) for t in tiles])
            older = frames[0] if step == 1 else None

            def gather(which):
                out_ = np.empty((len(keys), HKV, d), dtype=np.float64)
                for fr_, off in ((older, 0), (fr, L)) if step == 1 else ((fr, 0),):
                    sel = (keys >= off) & (keys < off + L)
                    if not sel.any():
                        continue
                    b = fr_.take(keys[sel] - off, fr_.k_bits if which == "k" else fr_.v_bits)
                    sc = SCALES[1] if which == "k" else SCALES[2]
                    out_[sel] = fp8_lut.round_trip_bits(b, sc) if fp8 else bf16_bits_to_f32(b)
                return out_

            kk, vv = gather("k"), gather("v")
            sub = mask[:, :, tiles]
            # the kept tiles laid end to end keep their tile boundaries: only the last may be short
            assert all(min((t + 1) * TILE, n_k) - t * TILE == TILE for t in tiles[:-1])
            ref = oracle.attend(q_or, kk, vv, sub)
            what = f"{name} step {step} ({len(tiles)} kept tiles of {n_kt})"
            # the (head, query tile) that keeps no tile gives zeros
            h_e = 1 + step
            assert not got[2 * TILE:, h_e].any(), f"{what}: empty row is not zero"
            if fp8:
                err = np.abs(got.astype(np.float64) - ref)
                b = _bound(q_or, kk, vv, ref, sub, np.arange(NQ))
                assert not err[b == 0].any(), f"{what}: error where the bound is 0 (a row that keeps no tile)"
                ratio = float((err[b > 0] / b[b > 0]).max())
                print(f"  {what}: largest error / E4M3 bound = {ratio:.3f}", flush=True)
                assert ratio <= 1.0, what
            else:
                assert_close(got, ref, what)
    finally:
        cache.close()
        del cache
        torch.cuda.empty_cache()
