"""CPU tests of libuf's host side: exports, validation and window bookkeeping.

No kernel runs here.  Calls that would launch are only made with arguments
that fail validation (which happens before any launch), or with
UF_APPEND_COMMIT_ONLY, which launches nothing.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import visible_frames_after
from tests.ring_model import RingModel
from windowed_attention_amd import uf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = uf.raw_lib()
FAKE = 1 << 20  # an aligned address that is never dereferenced: every call using it fails validation first
KS, VS = 1 << 40, 2 << 40  # fake cache storage, far from every other fake address


def declared_functions():
    text = open(os.path.join(ROOT, "include", "uf.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uf_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 15, names
    assert sorted(uf.EXPORTED) == names
    out = subprocess.run(["nm", "-D", "--defined-only", uf._LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (uf_\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert getattr(LIB, n) is not None


def test_status_strings():
    for code in range(0, -8, -1):
        assert uf.uf_status_string(code).startswith("UF_")
    assert uf.uf_status_string(-5) == "UF_ERR_STATE"


def desc(H=2, d=128, L=64, W=3, A=0, k=KS, v=VS, ws=None, ws_bytes=0, hpw=0, splits=0, max_q_heads=0,
         max_q_tokens=0, pipeline=0):
    dd = uf.uf_kvcache_desc(H, d, L, W, A, k, v, ws, ws_bytes)
    dd.heads_per_wg, dd.splits, dd.max_q_heads, dd.max_q_tokens = hpw, splits, max_q_heads, max_q_tokens
    dd.pipeline = pipeline
    return dd


def create(**kw):
    h = ctypes.c_void_p()
    st = LIB.uf_kvcache_create(ctypes.byref(desc(**kw)), ctypes.byref(h))
    return st, h.value


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), uf.UF_ERR_UNSUPPORTED),
    (dict(H=0), uf.UF_ERR_SHAPE),
    (dict(L=0), uf.UF_ERR_SHAPE),
    (dict(W=0), uf.UF_ERR_SHAPE),
    (dict(A=-1), uf.UF_ERR_SHAPE),
    (dict(k=None), uf.UF_ERR_INVALID_ARG),
    (dict(k=KS + 8), uf.UF_ERR_INVALID_ARG),
    (dict(v=KS + 64), uf.UF_ERR_INVALID_ARG),           # overlaps k storage
    (dict(ws_bytes=1024), uf.UF_ERR_INVALID_ARG),          # size without a pointer
    (dict(ws=FAKE * 8 + 16, ws_bytes=1024), uf.UF_ERR_INVALID_ARG),  # misaligned workspace
    (dict(L=1 << 20, W=4096), uf.UF_ERR_CAPACITY),
    (dict(L=1 << 20, W=16), uf.UF_ERR_CAPACITY),           # 2^24 rows of 256 bytes: 4 GiB per head
    (dict(hpw=3), uf.UF_ERR_INVALID_ARG),
    (dict(hpw=8), uf.UF_ERR_INVALID_ARG),
    (dict(splits=17), uf.UF_ERR_INVALID_ARG),
    (dict(splits=-1), uf.UF_ERR_INVALID_ARG),
    (dict(max_q_heads=-1), uf.UF_ERR_INVALID_ARG),
    (dict(max_q_tokens=-5), uf.UF_ERR_INVALID_ARG),
    (dict(pipeline=3), uf.UF_ERR_INVALID_ARG),
    (dict(pipeline=-1), uf.UF_ERR_INVALID_ARG),
])
def test_create_rejects(kw, status):
    st, h = create(**kw)
    assert st == status, uf.uf_last_error()
    assert h is None
    assert uf.uf_last_error() != ""


def test_sizes():
    d = desc(H=3, d=128, L=1560, W=2, A=0)
    assert uf.uf_kvcache_storage_bytes(d) == 3 * 2 * 1560 * 128 * 2
    d = desc(H=12, d=128, L=1560, W=9, A=3)
    assert uf.uf_kvcache_storage_bytes(d) == 12 * 12 * 1560 * 128 * 2
    # without a GPU the library assumes 256 compute units: 4 rounds of 2 * 256 work-groups of
    # 128 (split, query, head) rows
    full = uf.uf_attn_workspace_bytes(d)
    assert full == 4 * 2 * 256 * 128 * (128 + 2) * 4
    # with the step's largest size given, at most 16 splits of it
    assert uf.uf_attn_workspace_bytes(desc(H=3, d=64, L=1560, W=2, max_q_heads=12, max_q_tokens=100)) == \
        16 * 12 * 100 * (64 + 2) * 4
    assert uf.uf_attn_workspace_bytes(desc(H=12, d=128, L=1560, W=9, A=3, max_q_heads=12, max_q_tokens=4680)) == full
    assert uf.uf_kvcache_storage_bytes(desc(d=80)) == 0


def _window(h):
    return uf.uf_kvcache_window(h).as_dict()


def _check_window(h, model, W, A, L, active):
    w = uf.uf_kvcache_window(h)
    vis = visible_frames_after(model.count, W, A, active)
    assert w.frames_appended == model.count
    assert w.n_keys == len(vis) * L
    assert w.anchor_keys == min(A, model.count) * L
    assert w.ring_keys == w.n_keys - w.anchor_keys
    assert w.ring_capacity_keys == W * L
    # physical row of every visible key, from the header's formula vs the frame-by-frame model
    i = np.arange(w.n_keys)
    rows = np.where(i < w.anchor_keys, i,
                    A * L + (i - w.anchor_keys + w.ring_rotation_keys) % max(1, w.ring_capacity_keys))
    assert np.array_equal(rows, model.visible_rows(vis))


@pytest.mark.parametrize("L,W,A,F", [(64, 3, 0, 1), (1560, 9, 3, 3), (1560, 2, 0, 1), (6240, 6, 0, 3),
                                     (7, 5, 2, 3), (5, 4, 1, 2), (3, 1, 0, 1)])
def test_window_bookkeeping(L, W, A, F):
    st, h = create(H=1, d=64, L=L, W=W, A=A)
    assert st == uf.UF_OK
    model = RingModel(1, 64, L, W, A)
    try:
        for step in range(3 * (W + A) + 2):
            plan = uf.uf_kvcache_plan_append(h, F)
            frames = model.append(F)
            assert [plan.first_row[i] for i in range(F)] == [model.first_row(f) for f in frames]
            uf.uf_kvcache_append(h, None, None, F, uf.UF_APPEND_COMMIT_ONLY, 0)
            assert plan.window_after.as_dict() == _window(h)
            _check_window(h, model, W, A, L, W)
            if W > 1 and step % 3 == 2:           # crop the recent window, then restore it
                uf.uf_kvcache_set_window(h, W - 1)
                _check_window(h, model, W, A, L, W - 1)
                uf.uf_kvcache_set_window(h, W)
        # overwrite of the newest append: same rows, counter unchanged
        before = _window(h)
        plan = uf.uf_kvcache_plan_append(h, F, uf.UF_APPEND_OVERWRITE_NEWEST)
        assert [plan.first_row[i] for i in range(F)] == [model.first_row(f) for f in range(model.count - F, model.count)]
        uf.uf_kvcache_append(h, None, None, F, uf.UF_APPEND_OVERWRITE_NEWEST | uf.UF_APPEND_COMMIT_ONLY, 0)
        assert _window(h) == before
        uf.uf_kvcache_reset(h)
        w = _window(h)
        assert w["frames_appended"] == 0 and w["n_keys"] == 0 and w["active_frames"] == W
    finally:
        uf.uf_kvcache_destroy(h)


def _tensor(n_tok, heads, d=128, data=FAKE, dtype=uf.UF_BF16, st=None, sh=None):
    return uf.uf_tensor(data, dtype, n_tok, heads, d, heads * d if st is None else st, d if sh is None else sh)


def test_append_validation_leaves_state_unchanged():
    st, h = create(H=2, d=128, L=16, W=3, A=1)
    assert st == uf.UF_OK
    try:
        uf.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, 0)
        before = _window(h)
        ok_k, ok_v = _tensor(32, 2), _tensor(32, 2, data=FAKE * 4)
        bad = [
            (ok_k, ok_v, 2, 0x8, uf.UF_ERR_INVALID_ARG),                       # unknown flag
            (ok_k, ok_v, -1, 0, uf.UF_ERR_INVALID_ARG),
            (_tensor(80, 2), _tensor(80, 2), 5, 0, uf.UF_ERR_CAPACITY),       # 4 ring frames > W = 3
            (ok_k, ok_v, 65, 0, uf.UF_ERR_CAPACITY),
            (_tensor(16, 2), _tensor(16, 2), 1, uf.UF_APPEND_OVERWRITE_NEWEST, uf.UF_ERR_STATE),  # newest had 2
            (_tensor(31, 2), ok_v, 2, 0, uf.UF_ERR_SHAPE),                     # token count
            (_tensor(32, 3), ok_v, 2, 0, uf.UF_ERR_SHAPE),                     # head count
            (_tensor(32, 2, d=64), ok_v, 2, 0, uf.UF_ERR_SHAPE),               # head_dim
            (_tensor(32, 2, dtype=7), ok_v, 2, 0, uf.UF_ERR_DTYPE),
            (_tensor(32, 2, data=FAKE + 2), ok_v, 2, 0, uf.UF_ERR_INVALID_ARG),  # misaligned
            (_tensor(32, 2, st=260), ok_v, 2, 0, uf.UF_ERR_INVALID_ARG),        # stride not a multiple of 8
            (_tensor(32, 2, data=None), ok_v, 2, 0, uf.UF_ERR_INVALID_ARG),
            (ok_k, ok_v, 2, uf.UF_APPEND_COMMIT_ONLY, uf.UF_ERR_INVALID_ARG),   # commit-only with tensors
        ]
        for k, v, n, flags, want in bad:
            got = LIB.uf_kvcache_append(h, ctypes.byref(k), ctypes.byref(v), n, flags, None)
            assert got == want, (n, flags, uf.uf_status_string(got), uf.uf_last_error())
            assert _window(h) == before
        assert LIB.uf_kvcache_append(None, None, None, 1, 0, None) == uf.UF_ERR_INVALID_ARG
        assert LIB.uf_kvcache_append(h, None, None, 0, 0, None) == uf.UF_OK   # empty append is a no-op
        assert _window(h) == before
        assert LIB.uf_kvcache_set_window(h, 0) == uf.UF_ERR_SHAPE
        assert LIB.uf_kvcache_set_window(h, 4) == uf.UF_ERR_SHAPE
        assert _window(h) == before
    finally:
        uf.uf_kvcache_destroy(h)


def _mask(n_heads, nqb, nkb, data=FAKE * 16):
    return uf.uf_block_mask(data, n_heads, nqb, nkb, nqb * nkb, nkb)


def test_step_validation():
    st, h = create(H=2, d=128, L=100, W=3, A=0)
    assert st == uf.UF_OK
    q, out = _tensor(200, 4, data=FAKE * 32), _tensor(200, 4, data=FAKE * 64)
    try:
        # no frame appended yet
        assert LIB.uf_attn_step(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_ERR_STATE
        uf.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, 0)  # 200 keys: 2 tiles
        cases = [
            (_tensor(200, 3, data=FAKE * 32), _tensor(200, 3, data=FAKE * 64), None, uf.UF_ERR_SHAPE),  # 3 % 2
            (q, _tensor(199, 4, data=FAKE * 64), None, uf.UF_ERR_SHAPE),
            (q, _tensor(200, 4, d=64, data=FAKE * 64), None, uf.UF_ERR_SHAPE),
            (q, q, None, uf.UF_ERR_INVALID_ARG),                                         # out aliases q
            (q, _tensor(200, 4, data=KS + 256), None, uf.UF_ERR_INVALID_ARG),           # out overlaps K storage
            (q, out, _mask(4, 2, 3), uf.UF_ERR_SHAPE),                                    # 3 key tiles, want 2
            (q, out, _mask(4, 1, 2), uf.UF_ERR_SHAPE),                                    # 1 query tile, want 2
            (q, out, _mask(2, 2, 2), uf.UF_ERR_SHAPE),                                    # heads neither 1 nor 4
            (q, out, _mask(4, 2, 2, data=None), uf.UF_ERR_INVALID_ARG),
            (_tensor(200, 4, data=FAKE * 32, dtype=3), out, None, uf.UF_ERR_DTYPE),
        ]
        for qq, oo, m, want in cases:
            mp = None if m is None else ctypes.byref(m)
            got = LIB.uf_attn_step(ctypes.byref(qq), h, mp, ctypes.byref(oo), None)
            assert got == want, (uf.uf_status_string(got), uf.uf_last_error())
        assert LIB.uf_attn_step(None, h, None, ctypes.byref(out), None) == uf.UF_ERR_INVALID_ARG
        assert LIB.uf_attn_step(ctypes.byref(q), None, None, ctypes.byref(out), None) == uf.UF_ERR_INVALID_ARG
        # an empty query set is valid and launches nothing
        e = _tensor(0, 4, data=FAKE * 32)
        assert LIB.uf_attn_step(ctypes.byref(e), h, None, ctypes.byref(_tensor(0, 4, data=FAKE * 64)), None) == uf.UF_OK
    finally:
        uf.uf_kvcache_destroy(h)


def test_block_mask_workspace_bytes():
    d = desc(H=3, d=64, L=100, W=4, A=1)
    # 250 queries of 6 heads: 2 tiles x 6 heads x 64 floats, rounded to 256 B; keys: ceil(500/128) = 4 tiles x 3 heads
    assert uf.uf_block_mask_workspace_bytes(d, 250, 6) == 3072 + 4 * 3 * 64 * 4
    assert uf.uf_block_mask_workspace_bytes(d, 250, 4) == 0      # 4 heads over 3 KV heads
    assert uf.uf_block_mask_workspace_bytes(d, -1, 6) == 0
    assert uf.uf_block_mask_workspace_bytes(desc(d=96), 10, 2) == 0


def test_block_mask_topk_validation():
    st, h = create(H=2, d=128, L=100, W=3, A=0)
    assert st == uf.UF_OK
    q = _tensor(200, 4, data=FAKE * 32)
    p = uf.uf_topk_params(3, 1)
    ws, ws_bytes = FAKE * 256, 1 << 20
    mask = FAKE * 512

    def call(qq=q, params=p, m=mask, sc=None, w=ws, wb=ws_bytes, handle=h):
        pp = None if params is None else ctypes.byref(params)
        return LIB.uf_block_mask_topk(ctypes.byref(qq), handle, pp, m, sc, w, wb, None)

    try:
        assert call() == uf.UF_ERR_STATE                                   # nothing appended
        uf.uf_kvcache_append(h, None, None, 1, uf.UF_APPEND_COMMIT_ONLY, 0)  # 100 keys
        assert call() == uf.UF_ERR_SHAPE                                   # 200 queries > 100 keys
        uf.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, 0)  # 300 keys
        cases = [
            (dict(handle=None), uf.UF_ERR_INVALID_ARG),
            (dict(params=None), uf.UF_ERR_INVALID_ARG),
            (dict(params=uf.uf_topk_params(-1, 0)), uf.UF_ERR_INVALID_ARG),
            (dict(params=uf.uf_topk_params(2, -3)), uf.UF_ERR_INVALID_ARG),
            (dict(qq=_tensor(200, 3, data=FAKE * 32)), uf.UF_ERR_SHAPE),     # 3 heads over 2 KV heads
            (dict(qq=_tensor(200, 4, d=64, data=FAKE * 32)), uf.UF_ERR_SHAPE),
            (dict(qq=_tensor(200, 4, data=FAKE * 32, dtype=2)), uf.UF_ERR_DTYPE),
            (dict(m=None), uf.UF_ERR_INVALID_ARG),
            (dict(w=None), uf.UF_ERR_INVALID_ARG),
            (dict(wb=1024), uf.UF_ERR_INVALID_ARG),                           # workspace too small
            (dict(w=ws + 64), uf.UF_ERR_INVALID_ARG),                         # misaligned workspace
            (dict(m=ws + 4096), uf.UF_ERR_INVALID_ARG),                       # mask inside the workspace
            (dict(sc=mask + 4), uf.UF_ERR_INVALID_ARG),                       # scores overlap the mask
            (dict(sc=FAKE * 1024 + 2), uf.UF_ERR_INVALID_ARG),                # misaligned scores
        ]
        before = _window(h)
        for kw, want in cases:
            got = call(**kw)
            assert got == want, (kw, uf.uf_status_string(got), uf.uf_last_error())
            assert _window(h) == before
        # no queries: valid, nothing launched
        assert call(qq=_tensor(0, 4, data=FAKE * 32), m=None, w=None, wb=0) == uf.UF_OK
    finally:
        uf.uf_kvcache_destroy(h)


def test_block_mask_topk_key_tile_limit():
    # 3100 key tiles exceed what the selection kernel holds in LDS
    st, h = create(H=1, d=64, L=128 * 3100, W=1, A=0)
    assert st == uf.UF_OK
    try:
        uf.uf_kvcache_append(h, None, None, 1, uf.UF_APPEND_COMMIT_ONLY, 0)
        q = _tensor(128, 1, d=64, data=FAKE * 32)
        got = LIB.uf_block_mask_topk(ctypes.byref(q), h, ctypes.byref(uf.uf_topk_params(4, 0)), FAKE * 512, None,
                                     FAKE * 256, 1 << 30, None)
        assert got == uf.UF_ERR_UNSUPPORTED, uf.uf_last_error()
    finally:
        uf.uf_kvcache_destroy(h)


def fp8_desc(scales=(0.05, 0.02, 0.03), dtype=uf.UF_FP8_E4M3, **kw):
    d = desc(**kw)
    d.kv_dtype = dtype
    d.q_scale, d.k_scale, d.v_scale = scales
    return d


def test_fp8_cache_description():
    assert uf.uf_kvcache_storage_bytes(fp8_desc(H=3, d=64, L=100, W=4, A=1)) == 3 * 500 * 64
    assert uf.uf_kvcache_storage_bytes(desc(H=3, d=64, L=100, W=4, A=1)) == 3 * 500 * 64 * 2
    bad = [
        (fp8_desc(dtype=5), uf.UF_ERR_DTYPE),
        (fp8_desc(scales=(0.0, 1.0, 1.0)), uf.UF_ERR_INVALID_ARG),
        (fp8_desc(scales=(1.0, -1.0, 1.0)), uf.UF_ERR_INVALID_ARG),
        (fp8_desc(scales=(1.0, 1.0, float("inf"))), uf.UF_ERR_INVALID_ARG),
        (fp8_desc(scales=(1.0, 1.0, float("nan"))), uf.UF_ERR_INVALID_ARG),
        (fp8_desc(scales=(1e-45, 1.0, 1.0)), uf.UF_ERR_INVALID_ARG),   # reciprocal overflows float
        (fp8_desc(scales=(1e-30, 1e-30, 1.0)), uf.UF_ERR_INVALID_ARG),  # q k scale product beyond E8M0
    ]
    for d, want in bad:
        h = ctypes.c_void_p()
        got = LIB.uf_kvcache_create(ctypes.byref(d), ctypes.byref(h))
        assert got == want, (uf.uf_status_string(got), uf.uf_last_error())
        assert uf.uf_kvcache_storage_bytes(d) == 0
    # scales are ignored for bf16 caches
    d = fp8_desc(dtype=uf.UF_BF16, scales=(0.0, 0.0, 0.0))
    h = ctypes.c_void_p()
    assert LIB.uf_kvcache_create(ctypes.byref(d), ctypes.byref(h)) == uf.UF_OK
    uf.uf_kvcache_destroy(h.value)


def test_mask_generation_validates_fp8_cache_like_bf16():
    # an FP8 cache is accepted: the request is checked as for bf16 (here: a workspace one byte
    # short), and the rejection happens before any launch
    d = fp8_desc(H=2, d=128, L=100, W=3)
    h = ctypes.c_void_p()
    assert LIB.uf_kvcache_create(ctypes.byref(d), ctypes.byref(h)) == uf.UF_OK
    try:
        uf.uf_kvcache_append(h.value, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, 0)
        q = _tensor(100, 4, data=FAKE * 32)
        need = uf.uf_block_mask_workspace_bytes(d, 100, 4)
        assert need > 0
        got = LIB.uf_block_mask_topk(ctypes.byref(q), h.value, ctypes.byref(uf.uf_topk_params(2, 0)), FAKE * 512,
                                     None, FAKE * 256, need // 2, None)
        assert got == uf.UF_ERR_INVALID_ARG, uf.uf_last_error()
        assert "workspace" in uf.uf_last_error()
    finally:
        uf.uf_kvcache_destroy(h.value)


def test_block_order_validation():
    def mk(**kw):
        d = desc(**kw)
        return d
    d = mk(H=2, d=128, L=200, W=4, A=2)
    d.block_grid_h, d.block_grid_w = 10, 21       # 210 != 200 tokens
    h = ctypes.c_void_p()
    assert LIB.uf_kvcache_create(ctypes.byref(d), ctypes.byref(h)) == uf.UF_ERR_SHAPE
    d.block_grid_h, d.block_grid_w = 10, 0
    assert LIB.uf_kvcache_create(ctypes.byref(d), ctypes.byref(h)) == uf.UF_ERR_SHAPE
    d.block_grid_h, d.block_grid_w = 10, 20
    assert LIB.uf_kvcache_create(ctypes.byref(d), ctypes.byref(h)) == uf.UF_OK
    try:
        # 3 frames do not divide 2 anchor / 4 window frames
        assert LIB.uf_kvcache_append(h, None, None, 3, uf.UF_APPEND_COMMIT_ONLY, None) == uf.UF_ERR_SHAPE
        assert LIB.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, None) == uf.UF_OK
        # the stream's steps keep their frame count
        assert LIB.uf_kvcache_append(h, None, None, 1, uf.UF_APPEND_COMMIT_ONLY, None) == uf.UF_ERR_STATE
        assert LIB.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, None) == uf.UF_OK
        q, out = _tensor(300, 4, data=FAKE * 32), _tensor(300, 4, data=FAKE * 64)
        assert LIB.uf_attn_step(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_ERR_SHAPE  # not 400
        uf.uf_kvcache_reset(h)
        assert LIB.uf_kvcache_append(h, None, None, 1, uf.UF_APPEND_COMMIT_ONLY, None) == uf.UF_OK  # new stream
    finally:
        uf.uf_kvcache_destroy(h)


def test_block_order_crop_keeps_whole_steps():
    """In block order every frame slot of a step holds tokens of all the step's frames, so a
    crop of the recent window must be a whole number of steps."""
    d = desc(H=2, d=128, L=200, W=4, A=0)
    d.block_grid_h, d.block_grid_w = 10, 20
    h = ctypes.c_void_p()
    assert LIB.uf_kvcache_create(ctypes.byref(d), ctypes.byref(h)) == uf.UF_OK
    h = h.value
    q, out = _tensor(400, 4, data=FAKE * 32), _tensor(400, 4, data=FAKE * 64)
    p = uf.uf_topk_params(1, 0)
    try:
        # before the first append the step size is unknown: the crop is accepted here, and the
        # step that would use it refuses
        assert LIB.uf_kvcache_set_window(h, 3) == uf.UF_OK
        for _ in range(3):
            assert LIB.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, None) == uf.UF_OK
        assert LIB.uf_attn_step(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_ERR_SHAPE
        assert "multiple" in uf.uf_last_error()
        assert LIB.uf_block_mask_topk(ctypes.byref(q), h, ctypes.byref(p), FAKE * 512, None, FAKE * 256, 1 << 30,
                                      None) == uf.UF_ERR_SHAPE
        # once the step size is known the crop itself is refused and the window stays as it was
        assert LIB.uf_kvcache_set_window(h, 2) == uf.UF_OK
        before = _window(h)
        assert LIB.uf_kvcache_set_window(h, 1) == uf.UF_ERR_SHAPE
        assert LIB.uf_kvcache_set_window(h, 3) == uf.UF_ERR_SHAPE
        assert _window(h) == before
        assert before["n_keys"] == 2 * 200
        assert LIB.uf_kvcache_set_window(h, 4) == uf.UF_OK
    finally:
        uf.uf_kvcache_destroy(h)


def test_heads_per_wg_must_divide_the_group():
    st, h = create(H=2, d=128, L=100, W=3, hpw=4)
    assert st == uf.UF_OK
    try:
        uf.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, 0)
        q, out = _tensor(200, 4, data=FAKE * 32), _tensor(200, 4, data=FAKE * 64)   # 2 query heads per KV head
        assert LIB.uf_attn_step(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_ERR_SHAPE
        assert "heads_per_wg" in uf.uf_last_error()
    finally:
        uf.uf_kvcache_destroy(h)


def _stub_launches():
    try:
        return LIB.uf_stub_launch_count()
    except AttributeError:
        return None


@pytest.mark.skipif(_stub_launches() is None, reason="only with the host-only build (launch stubs)")
def test_valid_calls_reach_the_launchers():
    """With the host-only build every valid call runs its whole host path (window bookkeeping,
    launch parameters) and reaches the launchers, which check their invariants; each call
    launches what its contract says: append 1, step 1 (2 when split), mask generation 1."""
    ws_bytes = uf.uf_attn_workspace_bytes(desc(H=2, d=128, L=200, W=4, A=1))
    for hpw, splits in ((0, 0), (1, 3), (2, 2), (0, 16)):
        st, h = create(H=2, d=128, L=200, W=4, A=1, ws=FAKE * 1024, ws_bytes=ws_bytes, hpw=hpw, splits=splits)
        assert st == uf.UF_OK, uf.uf_last_error()
        try:
            q, out = _tensor(400, 4, data=FAKE * 32), _tensor(400, 4, data=FAKE * 64)
            for step in range(7):
                n0 = _stub_launches()
                k, v = _tensor(400, 2, data=FAKE * 96), _tensor(400, 2, data=FAKE * 128)
                assert LIB.uf_kvcache_append(h, ctypes.byref(k), ctypes.byref(v), 2, 0, None) == uf.UF_OK
                assert _stub_launches() == n0 + 1
                nkt = -(-_window(h)["n_keys"] // 128)
                m = _mask(4, 4, nkt)
                got = LIB.uf_attn_step(ctypes.byref(q), h, ctypes.byref(m) if step % 2 else None,
                                       ctypes.byref(out), None)
                assert got == uf.UF_OK, uf.uf_last_error()
                assert _stub_launches() in (n0 + 2, n0 + 3)
                if splits > 1:
                    assert _stub_launches() == n0 + 3
                need = uf.uf_block_mask_workspace_bytes(desc(H=2, d=128, L=200, W=4, A=1), 400, 4)
                got = LIB.uf_block_mask_topk(ctypes.byref(q), h, ctypes.byref(uf.uf_topk_params(2, 1)), FAKE * 512,
                                             None, FAKE * 256, need, None)
                assert got == uf.UF_OK, uf.uf_last_error()
        finally:
            uf.uf_kvcache_destroy(h)


def test_static_step_validates_like_the_step():
    """uf_attn_step_static checks its arguments as uf_attn_step does, before any HIP call, and
    refuses a forced split count whose partials exceed its scratch."""
    st, h = create(H=1, d=128, L=4100, W=2, splits=16)
    assert st == uf.UF_OK
    q, out = _tensor(4100, 16, data=FAKE * 32), _tensor(4100, 16, data=FAKE * 64)
    try:
        assert LIB.uf_attn_step_static(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_ERR_STATE
        uf.uf_kvcache_append(h, None, None, 1, uf.UF_APPEND_COMMIT_ONLY, 0)
        # 16 splits x 4100 queries x 16 heads x (128 + 2) x 4 bytes > 32 MiB
        assert LIB.uf_attn_step_static(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_ERR_CAPACITY
        assert "scratch" in uf.uf_last_error()
        assert LIB.uf_attn_step_static(ctypes.byref(q), h, None, ctypes.byref(q), None) == uf.UF_ERR_INVALID_ARG
        assert LIB.uf_attn_step_static(ctypes.byref(q), None, None, ctypes.byref(out), None) == uf.UF_ERR_INVALID_ARG
        bad = _tensor(4100, 16, data=FAKE * 32, dtype=3)
        assert LIB.uf_attn_step_static(ctypes.byref(bad), h, None, ctypes.byref(out), None) == uf.UF_ERR_DTYPE
    finally:
        uf.uf_kvcache_destroy(h)
    assert uf.UF_STATIC_SCRATCH_BYTES == 32 << 20


@pytest.mark.skipif(_stub_launches() is None, reason="only with the host-only build (launch stubs)")
def test_static_step_reaches_the_launchers():
    # no workspace in the description: only the static entry point splits (attention + combine)
    st, h = create(H=3, d=128, L=1200, W=3)
    assert st == uf.UF_OK
    try:
        uf.uf_kvcache_append(h, None, None, 3, uf.UF_APPEND_COMMIT_ONLY, 0)
        q, out = _tensor(1200, 12, data=FAKE * 32), _tensor(1200, 12, data=FAKE * 64)
        n0 = _stub_launches()
        assert LIB.uf_attn_step(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_OK
        assert _stub_launches() == n0 + 1          # no workspace: one launch, no split
        assert LIB.uf_attn_step_static(ctypes.byref(q), h, None, ctypes.byref(out), None) == uf.UF_OK
        assert _stub_launches() == n0 + 3          # split into the static scratch, then combined
    finally:
        uf.uf_kvcache_destroy(h)


@pytest.mark.skipif(_stub_launches() is None, reason="only with the host-only build (launch stubs)")
def test_split_rule_dense_and_masked():
    """Decoder-XL shape (24 heads of 64 over 3 KV heads, 45x80 tokens per frame, 2 frames):
    678 work items fill 1.3 rounds of 512 resident work-groups, so a dense step is split (the
    attention launch and the combine); the same step under a block mask is not."""
    L, H, HQ, d = 45 * 80, 3, 24, 64
    ws_bytes = uf.uf_attn_workspace_bytes(desc(H=H, d=d, L=L, W=2))
    st, h = create(H=H, d=d, L=L, W=2, ws=FAKE * 1024, ws_bytes=ws_bytes)
    assert st == uf.UF_OK, uf.uf_last_error()
    try:
        uf.uf_kvcache_append(h, None, None, 2, uf.UF_APPEND_COMMIT_ONLY, 0)
        q, out = _tensor(L, HQ, d=d, data=FAKE * 32), _tensor(L, HQ, d=d, data=FAKE * 64)
        nqb, nkb = -(-L // 128), -(-2 * L // 128)
        for m, launches in ((None, 2), (_mask(1, nqb, nkb), 1), (_mask(HQ, nqb, nkb), 1)):
            n0 = _stub_launches()
            got = LIB.uf_attn_step(ctypes.byref(q), h, ctypes.byref(m) if m is not None else None,
                                   ctypes.byref(out), None)
            assert got == uf.UF_OK, uf.uf_last_error()
            assert _stub_launches() == n0 + launches
    finally:
        uf.uf_kvcache_destroy(h)


@pytest.mark.skipif(_stub_launches() is None, reason="only with the host-only build (launch stubs)")
def test_uneven_split_rule():
    """480P shape (12 heads of 128, 30x52 tokens per frame, 3 queried frames over 3 anchor and
    9 window frames): 444 work items, more than half a round but less than one round of 512
    resident work-groups, so a dense step is cut into bodies of 119 key tiles and tails of the
    other 28 (attention launch and combine).  Unsplit instead under a block mask, at head_dim 64,
    through the static scratch (the partials do not fit) and when the split count is forced."""
    L, H, d = 30 * 52, 12, 128
    n_q, n_k = 3 * L, 12 * L
    nqb, nkb = -(-n_q // 128), -(-n_k // 128)
    assert (nqb * H, nkb) == (444, 147)
    for kw, dd, mask, static, want in (
            ({}, d, None, False, (2, nkb - (3 * nkb + 8) // 16)),
            ({}, d, _mask(1, nqb, nkb), False, (1, 0)),
            ({}, 64, None, False, (1, 0)),
            ({}, d, None, True, (1, 0)),
            (dict(splits=2), d, None, False, (2, 0))):
        ws_bytes = uf.uf_attn_workspace_bytes(desc(H=H, d=dd, L=L, W=9, A=3))
        st, h = create(H=H, d=dd, L=L, W=9, A=3, ws=FAKE * 1024, ws_bytes=ws_bytes, **kw)
        assert st == uf.UF_OK, uf.uf_last_error()
        try:
            uf.uf_kvcache_append(h, None, None, 12, uf.UF_APPEND_COMMIT_ONLY, 0)
            q, out = _tensor(n_q, H, d=dd, data=FAKE * 32), _tensor(n_q, H, d=dd, data=FAKE * 64)
            call = LIB.uf_attn_step_static if static else LIB.uf_attn_step
            n0 = _stub_launches()
            got = call(ctypes.byref(q), h, ctypes.byref(mask) if mask is not None else None, ctypes.byref(out), None)
            assert got == uf.UF_OK, uf.uf_last_error()
            assert (LIB.uf_stub_last_splits(), LIB.uf_stub_last_split_tile()) == want, (kw, dd, static)
            assert _stub_launches() == n0 + (2 if want[0] > 1 else 1)
        finally:
            uf.uf_kvcache_destroy(h)


@pytest.mark.skipif(_stub_launches() is None, reason="only with the host-only build (launch stubs)")
def test_pipeline_rule():
    """The software-pipelined loop is taken at head_dim 128 when every part of the key range spans
    at least 16 key tiles: the 480P step (bodies of 119 and tails of 28 tiles) and a masked 2K-like
    step take it, the decoder's three 8-tile parts do not, nor a GQA step whose work-groups walk
    the union of per-head mask rows; the descriptor forces either loop; head_dim 64 never takes it."""
    cases = (  # (H, HQ, d, L, W, A, queried frames, mask, heads per work-group, pipeline, want)
        (12, 12, 128, 30 * 52, 9, 3, 3, False, 0, 0, 1),
        (12, 12, 128, 30 * 52, 9, 3, 3, False, 0, 1, 0),
        (3, 12, 128, 1560, 2, 0, 1, False, 0, 0, 0),
        (3, 12, 128, 1560, 2, 0, 1, False, 0, 2, 1),
        (12, 12, 128, 90 * 156, 6, 0, 3, True, 0, 0, 1),
        (3, 12, 128, 90 * 156, 2, 0, 1, True, 4, 0, 0),
        (3, 12, 128, 90 * 156, 2, 0, 1, True, 1, 0, 1),
        (3, 24, 64, 45 * 80, 2, 0, 2, False, 0, 2, 0),
    )
    for H, HQ, d, L, W, A, fq, masked, hpw, pipeline, want in cases:
        ws_bytes = uf.uf_attn_workspace_bytes(desc(H=H, d=d, L=L, W=W, A=A))
        st, h = create(H=H, d=d, L=L, W=W, A=A, ws=FAKE * 1024, ws_bytes=ws_bytes, hpw=hpw, pipeline=pipeline)
        assert st == uf.UF_OK, uf.uf_last_error()
        try:
            uf.uf_kvcache_append(h, None, None, A + W, uf.UF_APPEND_COMMIT_ONLY, 0)
            n_q, n_k = fq * L, (A + W) * L
            # q and out 4 GiB apart, away from the fake workspace: the 2K-like step's q alone spans 129 MB
            q, out = _tensor(n_q, HQ, d=d, data=FAKE * 4096), _tensor(n_q, HQ, d=d, data=FAKE * 8192)
            m = _mask(HQ, -(-n_q // 128), -(-n_k // 128)) if masked else None
            got = LIB.uf_attn_step(ctypes.byref(q), h, ctypes.byref(m) if m is not None else None,
                                   ctypes.byref(out), None)
            assert got == uf.UF_OK, uf.uf_last_error()
            assert LIB.uf_stub_last_pipelined() == want, (H, HQ, d, L, pipeline)
        finally:
            uf.uf_kvcache_destroy(h)


def test_largest_head_storage_is_accepted():
    """Just under 4 GiB of K per head (bf16) is accepted, and so are 2^24 rows of E4M3 codes
    (2 GiB), whose bf16 twin is refused."""
    st, h = create(L=1 << 20, W=15)
    assert st == uf.UF_OK, uf.uf_last_error()
    uf.uf_kvcache_destroy(h)
    dd = desc(L=1 << 20, W=16)
    dd.kv_dtype, dd.q_scale, dd.k_scale, dd.v_scale = uf.UF_FP8_E4M3, 1.0, 1.0, 1.0
    hh = ctypes.c_void_p()
    assert LIB.uf_kvcache_create(ctypes.byref(dd), ctypes.byref(hh)) == uf.UF_OK, uf.uf_last_error()
    uf.uf_kvcache_destroy(hh.value)


def test_header_compiles_as_c(tmp_path):
    """include/uf.h is a C header: the plain-C program that drives the ABI compiles and links
    against the library with -Werror (it runs in the GPU tests)."""
    import shutil
    import subprocess
    from windowed_attention_amd import build as b
    if not shutil.which("gcc"):
        pytest.skip("needs gcc")
    res = subprocess.run(b.c_check_command(str(tmp_path / "uf_c_check"), extra=("-Werror",)),
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr


from hypothesis import HealthCheck, given, settings, strategies as hst  # noqa: E402

_OPS = hst.lists(hst.tuples(hst.sampled_from(["append", "overwrite", "crop", "reset"]), hst.integers(0, 9)),
                 min_size=1, max_size=40)


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(L=hst.integers(1, 40), W=hst.integers(1, 6), A=hst.integers(0, 4), ops=_OPS)
def test_window_bookkeeping_random_sequences(L, W, A, ops):
    """Random sequences of appends (some beyond the ring's capacity), overwrites (some of the
    wrong size), crops (some out of range) and resets.  Each call succeeds exactly when
    include/uf.h says it may, a refused call leaves the window as it was, and after every call
    the window and the storage row of every visible key equal the independent ring model's."""
    st, h = create(H=1, d=64, L=L, W=W, A=A)
    assert st == uf.UF_OK
    model, active = RingModel(1, 64, L, W, A), W
    try:
        for op, n in ops:
            before = _window(h)
            if op == "append":
                ok = max(0, n - max(0, A - model.count)) <= W
                got = LIB.uf_kvcache_append(h, None, None, n, uf.UF_APPEND_COMMIT_ONLY, None)
                if ok and n > 0:
                    model.append(n)
            elif op == "overwrite":
                ok = model.last > 0 and n == model.last
                got = LIB.uf_kvcache_append(h, None, None, n, uf.UF_APPEND_OVERWRITE_NEWEST | uf.UF_APPEND_COMMIT_ONLY,
                                            None)
            elif op == "crop":
                ok = 1 <= n <= W
                got = LIB.uf_kvcache_set_window(h, n)
                if ok:
                    active = n
            else:
                ok = True
                got = LIB.uf_kvcache_reset(h)
                model, active = RingModel(1, 64, L, W, A), W
            assert (got == uf.UF_OK) == ok, (op, n, got, uf.uf_last_error())
            if not ok:
                assert _window(h) == before, (op, n)
            _check_window(h, model, W, A, L, active)
            assert _window(h)["active_frames"] == active
    finally:
        uf.uf_kvcache_destroy(h)
