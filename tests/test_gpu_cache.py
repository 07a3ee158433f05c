"""Cache appends on the GPU are bit-exact against an independent ring model."""
import numpy as np
import pytest
import torch

from synth import f32_to_bf16_bits
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


GUARD = 4096       # bf16 elements of guard before, between and after the two storages
GUARD_BITS = 0x7FA5  # a NaN pattern no append writes from the drawn inputs' positions


def _guarded_storage(H, rows, d):
    """K and V storage as views into one buffer with guard regions around both."""
    n = H * rows * d
    buf = torch.full((3 * GUARD + 2 * n,), GUARD_BITS, dtype=torch.int16, device="cuda:0")
    k = buf[GUARD:GUARD + n].view(torch.bfloat16).view(H, rows, d)
    v = buf[2 * GUARD + n:2 * GUARD + 2 * n].view(torch.bfloat16).view(H, rows, d)
    guards = [(0, GUARD), (GUARD + n, 2 * GUARD + n), (2 * GUARD + 2 * n, 3 * GUARD + 2 * n)]
    return buf, k, v, guards


def _guards_intact(buf, guards, what):
    host = buf.cpu().numpy().view(np.uint16)
    for lo, hi in guards:
        bad = np.nonzero(host[lo:hi] != GUARD_BITS)[0]
        assert len(bad) == 0, f"{what}: {len(bad)} guard elements written, first at {lo + bad[0]}"


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H%d-d%d-L%d-W%d-A%d-F%d" % c[:6])
def test_append_bit_exact(case):
    """Appends and in-place overwrites equal the ring model byte for byte, and nothing outside
    the two storages (guard regions before, between and after them) is ever written."""
    H, d, L, W, A, F, n_appends, strided = case
    print(f"append case {case}", flush=True)
    rng = np.random.default_rng(hash(case) & 0xFFFF)
    buf, k_st, v_st, guards = _guarded_storage(H, (A + W) * L, d)
    cache = KVCache(H, d, L, W, A, k_storage=k_st, v_storage=v_st)
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
        _guards_intact(buf, guards, f"append {step}")
        if step == n_appends // 2:  # rewrite the newest append in place
            kb, kd = _draw(rng, F * L, H, d, strided)
            vb, vd = _draw(rng, F * L, H, d, strided)
            cache.append(kd, vd, F, uf.UF_APPEND_OVERWRITE_NEWEST)
            model.overwrite_newest(kb, vb)
            torch.cuda.synchronize()
            assert np.array_equal(bits_of(cache.k_storage), model.k)
            assert np.array_equal(bits_of(cache.v_storage), model.v)
            _guards_intact(buf, guards, f"overwrite after append {step}")
    assert cache.window().frames_appended == F * n_appends
    cache.close()


def test_attention_reads_leave_guards_intact():
    """A full stream of steps (append, attention, split combine) writes nothing outside the
    storages, and the attention output is independent of what lies outside them."""
    H, d, L, W, A, F = 2, 128, 200, 4, 1, 2
    buf, k_st, v_st, guards = _guarded_storage(H, (A + W) * L, d)
    cache = KVCache(H, d, L, W, A, k_storage=k_st, v_storage=v_st, splits=3)
    ref_cache = KVCache(H, d, L, W, A, splits=3)
    rng = np.random.default_rng(7)

    def normal(shape):
        return to_dev(f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))

    for step in range(6):
        kd, vd, q = normal((F * L, H, d)), normal((F * L, H, d)), normal((F * L, 4, d))
        cache.append(kd, vd, F)
        ref_cache.append(kd, vd, F)
        out, ref = torch.empty_like(q), torch.empty_like(q)
        cache.attn_step(q, out)
        ref_cache.attn_step(q, ref)
        torch.cuda.synchronize()
        _guards_intact(buf, guards, f"step {step}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"step {step}"
    cache.close()
    ref_cache.close()
