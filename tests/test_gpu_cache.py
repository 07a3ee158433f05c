"""Cache appends on the GPU are bit-exact against an independent ring model."""
import numpy as np
import pytest
import torch

from tests.gpu_util import bits_of, to_dev
from tests.ring_model import RingModel
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu

CASES = [  # n_kv_heads, head_dim, tokens_per_frame, W, A, frames per append, appends, strided inputs
    (2, 128, 64, 3, 0, 1, 7, False),
    (3, 128, 200, 4, 2, 2, 8, True),
    (1, 64, 37, 5, 1, 3, 9, False),
    (2, 64, 130, 2, 1, 1, 6, True),
    (12, 128, 1560, 9, 3, 3, 5, False),
]


def _draw(rng, n_tok, heads, d, strided):
    bits = rng.integers(0, 1 << 16, size=(n_tok, heads + (1 if strided else 0), d), dtype=np.uint16)
    dev = to_dev(bits)
    if strided:
        return bits[:, :heads], dev[:, :heads]
    return bits, dev


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H%d-d%d-L%d-W%d-A%d-F%d" % c[:6])
def test_append_bit_exact(case):
    H, d, L, W, A, F, n_appends, strided = case
    print(f"append case {case}", flush=True)
    rng = np.random.default_rng(hash(case) & 0xFFFF)
    cache = KVCache(H, d, L, W, A)
    cache.k_storage.zero_()
    cache.v_storage.zero_()
    model = RingModel(H, d, L, W, A)
    for step in range(n_appends):
        kb, kd = _draw(rng, F * L, H, d, strided)
        vb, vd = _draw(rng, F * L, H, d, strided)
        cache.append(kd, vd, F)
        model.append(F, kb, vb)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(cache.k_storage), model.k), f"K storage differs after append {step}"
        assert np.array_equal(bits_of(cache.v_storage), model.v), f"V storage differs after append {step}"
        if step == n_appends // 2:  # rewrite the newest append in place
            kb, kd = _draw(rng, F * L, H, d, strided)
            vb, vd = _draw(rng, F * L, H, d, strided)
            cache.append(kd, vd, F, uf.UF_APPEND_OVERWRITE_NEWEST)
            model.overwrite_newest(kb, vb)
            torch.cuda.synchronize()
            assert np.array_equal(bits_of(cache.k_storage), model.k)
            assert np.array_equal(bits_of(cache.v_storage), model.v)
    assert cache.window().frames_appended == F * n_appends
    cache.close()
