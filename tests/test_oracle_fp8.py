"""Pins for the FP8 E4M3 oracle (oracle/fp8.py), CPU only.

  * hand-worked values from the format's definition (tests/golden/e4m3_values.json);
  * the 126 positive finite codes decode to strictly increasing values and
    every finite code survives decode -> encode;
  * brute force: the encoder picks the nearest of all 254 finite values, ties
    to the even code, saturating at +-448;
  * planted mistakes (exponent bias, tie rule, saturation, subnormal spacing)
    must each fail a pin.
"""
import json
import os

import numpy as np
import pytest

import oracle.fp8 as f8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.json")


def check_golden():
    t = json.load(open(GOLDEN))
    for code, value in t["decode"].items():
        assert f8.e4m3_decode(np.array([int(code, 16)]))[0] == value, code
    for code in t["nan_codes"]:
        assert np.isnan(f8.e4m3_decode(np.array([int(code, 16)]))[0]), code
    for x, code in t["encode"]:
        assert f8.e4m3_encode(np.array([x], dtype=np.float32))[0] == int(code, 16), (x, code)


def check_order_and_round_trip():
    pos = f8.e4m3_decode(np.arange(0x00, 0x7F))
    assert np.all(np.diff(pos) > 0) and pos[0] == 0 and pos[-1] == 448.0
    neg = f8.e4m3_decode(np.arange(0x80, 0xFF))
    assert np.array_equal(neg, -pos)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = f8.e4m3_decode(finite).astype(np.float32)
    back = f8.e4m3_encode(vals)
    assert np.array_equal(back, finite)


def _brute(x):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = f8.e4m3_decode(codes)
    xs = float(np.clip(x, -448.0, 448.0))
    d = np.abs(vals - xs)
    best = codes[d == d.min()]
    if d.min() == abs(xs) and (np.abs(vals[best]) == 0).any() and len(best) <= 3:
        # the nearest value is zero: +0 and -0 both are; the input's sign decides (ties with
        # the smallest subnormal go to the even code, i.e. to zero)
        return 0x80 if np.signbit(x) else 0x00
    if len(best) > 1:
        best = best[best % 2 == 0]  # a tie: the even code
    return int(best[0])


def check_brute_force():
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.standard_normal(3000) * 3,
        rng.standard_normal(1000) * 0.01,
        rng.uniform(-600, 600, 500),
        f8.e4m3_decode(np.arange(0, 0x7E)) * 0.5 + f8.e4m3_decode(np.arange(1, 0x7F)) * 0.5,  # all midpoints
    ]).astype(np.float32)
    got = f8.e4m3_encode(xs)
    for x, g in zip(xs, got):
        assert g == _brute(x), (x, hex(g), hex(_brute(x)))


def check_static_quantization():
    assert f8.quantize(np.array([3.0]), 0.5)[0] == 0x4C        # 6.0
    assert f8.quantize(np.array([1.0]), 0.25)[0] == 0x48       # 4.0
    assert f8.quantize(np.array([-1000.0]), 1.0)[0] == 0xFE    # saturates
    assert f8.dequantize(np.array([0x4C]), 0.5)[0] == 3.0


def check_attention_q_scale():
    """q's scale for attention: never below q_scale, below twice it, and log2(e)/sqrt(d) times it
    times k_scale a power of two, the smallest such (exponent = ceil of the log2, by math.log2);
    and one value worked by hand: d = 128, q_scale 0.02, k_scale 0.015 give
    log2(log2(e)/sqrt(128) * 0.02 * 0.015) = log2(3.8255e-5) = -14.67, exponent -14, scale
    2^-14 sqrt(128) / (log2(e) 0.015) = 0.0319094."""
    import math
    assert abs(f8.attention_q_scale(0.02, 0.015, 128) / 0.0319094 - 1.0) < 2e-6
    rng = np.random.default_rng(7)
    for _ in range(300):
        d = int(rng.choice([64, 128]))
        qs = float(np.float32(np.exp(rng.uniform(-9, 3))))
        ks = float(np.float32(np.exp(rng.uniform(-9, 3))))
        r = f8.attention_q_scale(qs, ks, d)
        assert qs * (1 - 2.0 ** -22) <= r < 2 * qs * (1 + 2.0 ** -22), (qs, ks, d, r)
        c = math.log2(math.e) / math.sqrt(d)
        lg = math.log2(c * r * ks)
        assert abs(lg - round(lg)) < 1e-6, (qs, ks, d, lg)
        want = math.log2(c * qs * ks)
        if abs(want - round(want)) > 1e-9:
            assert round(lg) == math.ceil(want), (qs, ks, d, lg, want)


ALL = [check_golden, check_order_and_round_trip, check_brute_force, check_static_quantization,
       check_attention_q_scale]


@pytest.mark.parametrize("check", ALL, ids=lambda f: f.__name__)
def test_fp8_pin(check):
    check()


# ---------------------------------------------------------------------------------------------
# planted mistakes

ORIG_DECODE = f8.e4m3_decode
ORIG_ENCODE = f8.e4m3_encode


def _decode_bias8(codes):
    return ORIG_DECODE(codes) / 2.0


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float32)
    out = ORIG_ENCODE(x)
    # nudge every input a hair away from zero before encoding: ties then go away from zero
    return ORIG_ENCODE((x.astype(np.float64) * (1 + 2.0 ** -20)).astype(np.float32)) if x.size else out


def _encode_no_saturation(x):
    x = np.asarray(x, dtype=np.float32)
    out = ORIG_ENCODE(x)
    return np.where(np.abs(x) > 448.0, np.uint8(0x7F) | (out & 0x80), out).astype(np.uint8)


def _decode_sub_spacing(codes):
    c = np.asarray(codes, dtype=np.uint8)
    v = ORIG_DECODE(c)
    return np.where(((c >> 3) & 0xF) == 0, v / 2.0, v)


ORIG_Q_SCALE = f8.attention_q_scale


def _q_scale_floor(q_scale, k_scale, head_dim):
    # rounds the exponent down instead of up
    return ORIG_Q_SCALE(q_scale, k_scale, head_dim) / 2.0


def _q_scale_no_sqrt(q_scale, k_scale, head_dim):
    # softmax factor log2(e)/d instead of log2(e)/sqrt(d)
    return ORIG_Q_SCALE(q_scale, k_scale, head_dim * head_dim)


MUTANTS = {
    "q_scale_exponent_floor": ("attention_q_scale", _q_scale_floor),
    "q_scale_no_sqrt": ("attention_q_scale", _q_scale_no_sqrt),
    "decode_bias_8": ("e4m3_decode", _decode_bias8),
    "encode_ties_away": ("e4m3_encode", _encode_ties_away),
    "encode_no_saturation": ("e4m3_encode", _encode_no_saturation),
    "decode_subnormal_spacing": ("e4m3_decode", _decode_sub_spacing),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutant_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(f8, attr, fn)
    failed = 0
    for check in ALL:
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed > 0, name
