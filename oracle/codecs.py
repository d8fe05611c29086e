"""Oracle: KV element codecs (FP16, FP8 E4M3, INT8) and exact dequantisation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Passages followed
-----------------
* ReVolta README, intro list: the KV cache is stored as FP8 E4M3, FP16 or
  INT8.
* ReVolta README, "Weight and KV formats": V100 keeps KV compressed and
  converts it to FP16 for the arithmetic; "E4M3 KV" uses calibrated
  per-layer K and V scales and, in strict mode, refuses to run without
  them; "INT8 KV" names runtime scales per token and head (the graded
  workloads instead give INT8 one per-layer scale = max|x|/127, rounded
  half to even and clamped to [-127, 127]).
* "Running FP4-Local on 4 x V100 32 GB (Volta) with ReVolta", "What it
  takes": the scale pack holds the per-layer target K/V scales.

The pages do not print the encoding rules.  E4M3 is read as the OCP 8-bit
floating point format E4M3 ("FN": bias 7, 3 mantissa bits, largest finite
value 448, no infinities, NaN = S.1111.111), which a max of 448 implies.
Readings taken where the pages are silent:

* quantise = correctly rounded fp32 division ``fp32(x) / fp32(scale)``;
* E4M3: saturate to +-448 (so +-inf -> +-448), round to nearest with ties
  to the even code, keep the sign of the fp32 quotient (so -0 -> 0x80 and a
  negative value that rounds to zero -> 0x80), NaN -> 0x7F | sign;
* INT8: round half to even, clamp to [-127, 127], NaN -> 0; -128 is never
  written;
* FP16 cache: IEEE round-to-nearest-even cast of the fp32 value, no scale;
* dequantise = ``fp32(decoded code) * fp32(scale)``, one fp32 rounding;
* INT8 with runtime scales per token and head ('int8_tok', ReVolta README,
  "Weight and KV formats", INT8 KV): each (token, head) row of D values gets
  its own fp32 scale ``fp32(max_d |x|) / fp32(127)`` and is then quantised
  exactly like per-layer INT8 with that scale; a row of zeros has scale 0
  and codes 0.

Pins (tests/test_oracle_codecs.py): the OCP E4M3 reference values, an
exhaustive 256-code round trip, every midpoint between adjacent codes and
one fp32 ulp either side of it, saturation, a library cross-check against
torch's float8_e4m3fn cast on in-range values, explicit INT8 tie tables and
a nearest-integer property check, FP16 tie and overflow cases; for the
per-token INT8 scales a hand-worked row, the max element at +-127, the
half-step error bound and the zero row.
"""
import numpy as np

E4M3_MAX = 448.0
INT8_MAX = 127

_F32 = np.float32


def e4m3_value(code):
    """Exact real value (float64) of one E4M3 byte, NaN for S.1111.111.

    OCP E4M3: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits
    2..0; exponent field 0 encodes subnormals m * 2^-9.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table():
    """float64[256]: the value of every E4M3 code (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_E4M3 = e4m3_table()
# magnitudes of the non-negative finite codes 0x00..0x7E, ascending in code
_E4M3_POS = _E4M3[:0x7F].copy()


def e4m3_encode(y32):
    """Encode fp32 values (already divided by the scale) to E4M3 bytes.

    Nearest representable magnitude by direct search of the code table, ties
    to the code with mantissa LSB 0; sign from the fp32 sign bit.
    """
    y = np.asarray(y32, dtype=_F32)
    flat = y.reshape(-1)
    nan = np.isnan(flat)
    neg = np.signbit(flat)
    mag = np.abs(flat.astype(np.float64))
    mag = np.where(nan, 0.0, np.minimum(mag, E4M3_MAX))  # saturate, inf -> 448
    hi = np.searchsorted(_E4M3_POS, mag, side="left")       # first value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(mag == _E4M3_POS[hi], hi, code).astype(np.uint8)   # exact hits
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    code = code | np.where(neg, np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    return code.reshape(y.shape)


def e4m3_decode(codes):
    """float64 values of E4M3 bytes (exact)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def int8_encode(y32):
    """Encode fp32 values (already divided by the scale) to int8 codes.

    Round half to even (np.rint), clamp to [-127, 127], NaN -> 0.
    """
    y = np.asarray(y32, dtype=_F32).astype(np.float64)
    y = np.where(np.isnan(y), 0.0, y)
    q = np.clip(np.rint(y), -INT8_MAX, INT8_MAX)
    return q.astype(np.int8)


def f16_encode(x32):
    """FP16 cache element: IEEE round-to-nearest-even cast of fp32."""
    return np.asarray(x32, dtype=_F32).astype(np.float16)


def bf16_bits_to_f32(bits):
    """bfloat16 stored as uint16 bit patterns -> exact float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def source_to_f32(x, src_dtype):
    """New-token K/V or Q as delivered by the caller -> exact float32.

    ``src_dtype`` is 'f16' (numpy float16 array) or 'bf16' (uint16 bits).
    """
    if src_dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(_F32)
    if src_dtype == "bf16":
        return bf16_bits_to_f32(x)
    raise ValueError(src_dtype)


def quantize(x32, kv_dtype, scale):
    """Cache codes for fp32 values.

    kv_dtype 'f16' -> float16 array (scale unused); 'e4m3' -> uint8 codes;
    'int8' -> int8 codes.  The division is numpy float32 '/', i.e. the IEEE
    correctly rounded quotient.
    """
    x32 = np.asarray(x32, dtype=_F32)
    if kv_dtype == "f16":
        return f16_encode(x32)
    s = _F32(scale)
    y = (x32 / s).astype(_F32)
    if kv_dtype == "e4m3":
        return e4m3_encode(y)
    if kv_dtype == "int8":
        return int8_encode(y)
    raise ValueError(kv_dtype)   # 'int8_tok' has per-row scales: quantize_per_token


def dequantize(codes, kv_dtype, scale):
    """Exact fp32 dequantised values: fp32(decode(code)) * fp32(scale)."""
    if kv_dtype == "f16":
        return np.asarray(codes, dtype=np.float16).astype(_F32)
    s = _F32(scale)
    if kv_dtype == "e4m3":
        v = e4m3_decode(codes).astype(_F32)      # every E4M3 value is an fp32
    elif kv_dtype == "int8":
        v = np.asarray(codes, dtype=np.int8).astype(_F32)
    else:
        raise ValueError(kv_dtype)
    return (v * s).astype(_F32)


def token_scales(x32):
    """Per-row INT8 scales over the last axis: fp32(max |x|) / fp32(127)."""
    amax = np.max(np.abs(np.asarray(x32, dtype=_F32)), axis=-1)
    return (amax / _F32(INT8_MAX)).astype(_F32)


def quantize_per_token(x32):
    """('int8_tok') -> (int8 codes, fp32 scales): every row of the last axis
    is quantised with its own scale; a zero row (scale 0) gets codes 0."""
    x32 = np.asarray(x32, dtype=_F32)
    s = token_scales(x32)
    safe = np.where(s > 0, s, _F32(1))
    y = (x32 / safe[..., None]).astype(_F32)
    codes = int8_encode(y)
    codes[s == 0] = 0
    return codes, s


def dequantize_per_token(codes, scales):
    """fp32(code) * fp32(row scale), one fp32 rounding."""
    v = np.asarray(codes, dtype=np.int8).astype(_F32)
    return (v * np.asarray(scales, dtype=_F32)[..., None]).astype(_F32)


def roundtrip(x32, kv_dtype, scale=None):
    """What the cache holds for fp32 values, dequantised exactly (fp32):
    per-layer formats use ``scale``; 'int8_tok' uses per-row scales."""
    if kv_dtype == "int8_tok":
        codes, s = quantize_per_token(x32)
        return dequantize_per_token(codes, s)
    return dequantize(quantize(x32, kv_dtype, scale), kv_dtype, scale)


def code_nbytes(kv_dtype):
    return 2 if kv_dtype == "f16" else 1


def codes_as_bytes(codes, kv_dtype):
    """Little-endian byte image of a code array (uint8, last axis x bytes)."""
    a = np.ascontiguousarray(codes)
    if kv_dtype == "f16":
        return a.view(np.uint8).reshape(a.shape[:-1] + (a.shape[-1] * 2,))
    return a.view(np.uint8)
