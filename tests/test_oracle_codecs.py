"""Pins for the oracle's KV codecs (CPU only).

The pages name the formats (FP8 E4M3, INT8, FP16 KV with per-layer scales)
but print no encoded values, so the codecs are pinned to the OCP E4M3
reference values, to exhaustive properties of the code table, to exact tie
tables worked by hand, and to library casts (torch float8_e4m3fn and
float16) where those define the same rounding.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs
from tests.conftest import GOLDEN


def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_reference.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_ocp_reference_values():
    for code, val in _golden_e4m3():
        got = codecs.e4m3_value(code)
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_table_monotone_and_symmetric():
    t = codecs.e4m3_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert pos[0] == 0.0 and pos[-1] == 448.0
    neg = t[0x80:0xFF]
    assert np.array_equal(np.abs(neg), pos)
    assert np.all(np.signbit(neg))
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    # every value has at most 4 significant bits: exact in fp32 and fp16
    assert np.array_equal(pos.astype(np.float32).astype(np.float64), pos)


def test_e4m3_exhaustive_round_trip():
    t = codecs.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = t[codes].astype(np.float32)
    assert np.array_equal(codecs.e4m3_encode(vals), codes)


def test_e4m3_midpoints_ties_to_even_and_neighbours():
    t = codecs.e4m3_table()
    for c in range(0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)          # <= 5 significant bits: exact
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert codecs.e4m3_encode(mid) == even, (c, float(mid))
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1000))
        assert codecs.e4m3_encode(below) == c
        assert codecs.e4m3_encode(above) == c + 1
        # negative side mirrors with the sign bit
        assert codecs.e4m3_encode(-mid) == (even | 0x80)
        assert codecs.e4m3_encode(-below) == (c | 0x80)


def test_e4m3_saturation_nan_and_signed_zero():
    big = np.array([448, 449, 463.9, 464, 480, 1e4, 3e38, np.inf], dtype=np.float32)
    assert np.all(codecs.e4m3_encode(big) == 0x7E)
    assert np.all(codecs.e4m3_encode(-big) == 0xFE)
    assert codecs.e4m3_encode(np.float32(np.nan)) == 0x7F
    assert codecs.e4m3_encode(np.float32(-0.0)) == 0x80
    assert codecs.e4m3_encode(np.float32(0.0)) == 0x00
    # below half the smallest subnormal: rounds to a zero of the same sign
    tiny = np.float32(2.0 ** -11)
    assert codecs.e4m3_encode(tiny) == 0x00
    assert codecs.e4m3_encode(-tiny) == 0x80
    # exactly half the smallest subnormal ties to the even code 0
    assert codecs.e4m3_encode(np.float32(2.0 ** -10)) == 0x00
    assert codecs.e4m3_encode(np.float32(3 * 2.0 ** -10)) == 0x02


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 40,
        rng.uniform(-448, 448, 200000).astype(np.float32),
        (rng.standard_normal(100000) * 2.0 ** -8).astype(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3_encode(x), ref)


def test_int8_tie_table():
    y = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.5, -127.5, 0.49999997,
                  300.0, -300.0, np.inf, -np.inf, np.nan, -0.0], dtype=np.float32)
    want = np.array([0, 2, 2, 0, -2, -2, 126, 127, -127, 0, 127, -127, 127, -127, 0, 0],
                    dtype=np.int8)
    assert np.array_equal(codecs.int8_encode(y), want)


def test_int8_nearest_integer_property():
    rng = np.random.default_rng(7)
    y = rng.uniform(-127.49, 127.49, 500000).astype(np.float32)
    y[:1000] = np.round(rng.uniform(-126, 126, 1000)).astype(np.float32) + 0.5
    q = codecs.int8_encode(y).astype(np.float64)
    err = np.abs(y.astype(np.float64) - q)
    assert np.all(err <= 0.5)
    ties = err == 0.5
    assert ties.sum() >= 900
    assert np.all(q[ties] % 2 == 0)
    assert codecs.int8_encode(y).min() >= -127


def test_f16_cast_ties_and_overflow():
    one = 1.0
    x = np.array([one + 2.0 ** -11, one + 3 * 2.0 ** -11, 65504.0, 65519.99, 65520.0,
                  2.0 ** -25, 3 * 2.0 ** -25], dtype=np.float32)
    h = codecs.f16_encode(x)
    assert h[0] == np.float16(1.0)
    assert h[1] == np.float16(one + 2.0 ** -9)
    assert h[2] == np.float16(65504)
    assert h[3] == np.float16(65504)
    assert np.isinf(h[4])
    assert h[5] == 0.0                       # tie at half the min subnormal -> even (0)
    assert float(h[6]) == 2.0 ** -23         # 1.5 * 2^-24 rounds to the even 2^-23
    rng = np.random.default_rng(3)
    r = (rng.standard_normal(100000) * 100).astype(np.float32)
    assert np.array_equal(codecs.f16_encode(r),
                          torch.from_numpy(r).half().numpy())


def test_quantize_uses_correctly_rounded_division():
    # x / s differs from x * (1/s) for these operands; the oracle must divide.
    s = np.float32(0.1)
    xs = np.arange(1, 20000, dtype=np.float32) * np.float32(0.0173)
    div = (xs / s).astype(np.float32)
    mul = (xs * (np.float32(1) / s)).astype(np.float32)
    assert np.any(div != mul)
    q = codecs.quantize(xs, "e4m3", s)
    assert np.array_equal(q, codecs.e4m3_encode(div))
    q8 = codecs.quantize(xs / np.float32(100), "int8", s)
    assert np.array_equal(q8, codecs.int8_encode(((xs / np.float32(100)) / s).astype(np.float32)))


def test_dequantize_is_one_fp32_product():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes != 0x7F) & (codes != 0xFF)]
    s = np.float32(0.0130004883)
    got = codecs.dequantize(codes, "e4m3", s)
    want = np.array([np.float32(codecs.e4m3_value(c)) * s for c in codes], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    i8 = np.arange(-127, 128, dtype=np.int8)
    got = codecs.dequantize(i8, "int8", s)
    assert np.array_equal(got, i8.astype(np.float32) * s)
    h = np.array([1.5, -2.25, 65504], dtype=np.float16)
    assert np.array_equal(codecs.dequantize(h, "f16", 7.0), h.astype(np.float32))


def test_bf16_bits():
    bits = np.array([0x3F80, 0xBFC0, 0x0000, 0x8000, 0x7F80], dtype=np.uint16)
    v = codecs.bf16_bits_to_f32(bits)
    assert list(v[:4]) == [1.0, -1.5, 0.0, -0.0] and np.isinf(v[4])


@pytest.mark.parametrize("kv", ["e4m3", "int8"])
def test_quantize_dequantize_error_bound(kv):
    # with scale = max|x|/qmax, every in-range value is reproduced to within
    # half a code step: relative 2^-4 for E4M3 normals, 0.5*scale for INT8
    rng = np.random.default_rng(11)
    x = rng.standard_normal(100000).astype(np.float32)
    qmax = 448.0 if kv == "e4m3" else 127.0
    s = np.float32(np.abs(x).max()) / np.float32(qmax)
    xh = codecs.dequantize(codecs.quantize(x, kv, s), kv, s).astype(np.float64)
    err = np.abs(xh - x)
    if kv == "int8":
        assert np.all(err <= 0.5 * s * (1 + 1e-6))
    else:
        normal = np.abs(x) >= 2.0 ** -6 * s
        assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4 * (1 + 1e-6))
        assert np.all(err[~normal] <= 2.0 ** -10 * s * (1 + 1e-6))


# ---- INT8 with runtime scales per token and head ('int8_tok')

def test_int8_token_hand_worked_row():
    """max |x| = 2.54 -> scale = fp32(2.54) / 127 (about 0.02); the other
    values sit far from any rounding boundary: 1.0 -> 50, -0.5 -> -25,
    0.26 -> 13, -2.54 -> -127, 0 -> 0."""
    x = np.array([[1.0, -0.5, 0.26, -2.54, 0.0, 2.0]], dtype=np.float32)
    codes, s = codecs.quantize_per_token(x)
    assert s.dtype == np.float32 and s[0] == np.float32(np.float32(2.54) / np.float32(127))
    assert codes.tolist() == [[50, -25, 13, -127, 0, 100]]


def test_int8_token_max_element_codes_127_and_half_step_bound():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((300, 4, 128)) * rng.uniform(1e-3, 50.0, (300, 4, 1))).astype(np.float32)
    codes, s = codecs.quantize_per_token(x)
    assert s.shape == (300, 4)
    idx = np.argmax(np.abs(x), axis=-1)
    top = np.take_along_axis(codes, idx[..., None], axis=-1)[..., 0].astype(np.int64)
    sign = np.sign(np.take_along_axis(x, idx[..., None], axis=-1)[..., 0])
    assert np.all(top == 127 * sign)
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(codecs.dequantize_per_token(codes, s).astype(np.float64) - x.astype(np.float64))
    # half a quantisation step, plus the fp32 roundings of the quotient and the product
    assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 1e-4))


def test_int8_token_zero_row_and_roundtrip_dispatch():
    x = np.zeros((2, 1, 8), dtype=np.float32)
    x[1, 0, 3] = -4.0
    codes, s = codecs.quantize_per_token(x)
    assert s[0, 0] == 0.0 and np.all(codes[0] == 0)
    assert codes[1, 0, 3] == -127 and np.all(np.delete(codes[1, 0], 3) == 0)
    r = codecs.roundtrip(x, "int8_tok")
    assert r[1, 0, 3] == np.float32(-127) * s[1, 0] and np.all(r[0] == 0)
