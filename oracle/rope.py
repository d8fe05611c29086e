"""Oracle: rotary position embedding with YaRN scaling, and the fused step
that splits packed QKV rows, rotates Q and K and stores K/V in the cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Passages followed
-----------------
* ReVolta README, "Quick start", step 2 ("Download the checkpoint and make
  512K views"): the checkpoint's native context is 262,144 tokens and the
  deployment reaches 524,288 with YaRN, factor 2; the model config gets
  ``rope_type = yarn``, ``factor = 2``, ``original_max_position_embeddings
  = 262144``.
* ReVolta README, DFlash2 settings list (the fused QKV pack option): the
  verifier's Q/K/V rows are packed by one copy kernel, with bit-identical
  output.

The pages print no RoPE formula.  Readings taken where they are silent:

* Rotary embedding (RoFormer): frequencies ``theta_i = base^(-2 i / R)``
  for ``i = 0 .. R/2 - 1`` over the first R = rotary_dim dims of a head;
  dim ``i`` pairs with dim ``i + R/2`` (the half-split pairing the Qwen
  family uses) and the pair turns by ``p * theta_i`` at position p:
  ``y_i = x_i cos - x_{i+R/2} sin``, ``y_{i+R/2} = x_{i+R/2} cos + x_i sin``.
  Dims R .. D-1 pass through.  The base (rope theta) is not in the pages:
  it is a parameter.
* YaRN, as the Hugging Face config format above is applied by the runtimes
  that read it: "NTK-by-parts" interpolation with beta_fast = 32 and
  beta_slow = 1.  The dim whose wavelength fits ``L / beta`` times into
  the original context L is ``R ln(L / (2 pi beta)) / (2 ln base)``; the
  ramp runs linearly over the dim index from floor(that dim for beta_fast)
  to ceil(that dim for beta_slow), both clamped to [0, R - 1].  Dims below
  the ramp keep theta_i (extrapolation), dims above it use theta_i / factor
  (interpolation), and dims on it blend the two linearly.  The attention
  temperature enters as a factor ``0.1 ln(factor) + 1`` on cos and sin
  (so on both q and k).  factor <= 1 means plain RoPE.
* The table handed to the kernel is fp32 ``[max_position][2][R/2]``
  (cos, then sin, each already multiplied by the temperature factor),
  rounded from fp64.
* Packed QKV rows: ``[Hq*D | Hkv*D | Hkv*D]`` per token (Q heads, then K
  heads, then V heads).  The rotation is evaluated in fp32 from the fp32
  table without fused multiply-add: ``y1 = fl(fl(x1 c) - fl(x2 s))``,
  ``y2 = fl(fl(x2 c) + fl(x1 s))``.  Rotated Q is rounded (nearest even)
  to the source dtype; rotated K, and V as given, are quantised exactly as
  the KV store quantises fp32 values (``oracle.codecs``).
* A position outside [0, max_position) gives a NaN Q row and stores no K/V
  for that token; a slot < 0 stores no K/V (Q is still written).

Pins (tests/test_oracle_rope.py): a rotation equals multiplication by
``e^{i p theta}`` in complex arithmetic; pair norms scale by the
temperature factor; position 0 is the identity; q.k after rotation depends
only on the position difference; plain RoPE matches a hand-worked value;
YaRN keeps the highest frequencies, divides the lowest by the factor (so
that the table at position 2p equals plain RoPE at p there), blends
monotonically in between and gives the temperature 1.0693...; YaRN
frequencies and temperature equal, on every dim including both ramp ends,
those of the Hugging Face runtime's own YaRN parameter function for the same
config entry (a library routine that applies the format the pages name), and
a ramp end moved by one dim would differ from it; the fused step at position
0 without scaling reproduces the plain store and Q.
"""
import math

import numpy as np

from oracle import codecs
from oracle import layout


def inv_freq(rotary_dim, base):
    """float64[R/2]: theta_i = base^(-2 i / R)."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return base ** (-2.0 * i / rotary_dim)


def yarn_correction_dim(rotary_dim, base, original_max, beta):
    """Dim index whose wavelength 2 pi / theta fits `beta` times into the
    original context."""
    return rotary_dim * math.log(original_max / (beta * 2.0 * math.pi)) / (2.0 * math.log(base))


def yarn_inv_freq(rotary_dim, base, factor, original_max, beta_fast=32.0, beta_slow=1.0):
    """float64[R/2]: YaRN frequencies (plain RoPE when factor <= 1)."""
    theta = inv_freq(rotary_dim, base)
    if factor <= 1.0:
        return theta
    lo = math.floor(yarn_correction_dim(rotary_dim, base, original_max, beta_fast))
    hi = math.ceil(yarn_correction_dim(rotary_dim, base, original_max, beta_slow))
    lo, hi = max(lo, 0), min(hi, rotary_dim - 1)
    if hi == lo:
        hi = lo + 0.001
    d = np.arange(rotary_dim // 2, dtype=np.float64)
    ramp = np.clip((d - lo) / (hi - lo), 0.0, 1.0)        # 0: keep theta, 1: theta / factor
    return theta * (1.0 - ramp) + (theta / factor) * ramp


def yarn_temperature(factor):
    """Factor on cos and sin: 0.1 ln(factor) + 1 (1 without scaling)."""
    return 0.1 * math.log(factor) + 1.0 if factor > 1.0 else 1.0


def rope_table(max_position, rotary_dim, base, factor=1.0, original_max=None,
               beta_fast=32.0, beta_slow=1.0):
    """float64[max_position][2][R/2]: (cos, sin) of p * theta_i, times the
    temperature factor."""
    th = yarn_inv_freq(rotary_dim, base, factor, original_max if original_max else max_position,
                       beta_fast, beta_slow)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * th[None, :]
    m = yarn_temperature(factor)
    return np.stack([np.cos(ang) * m, np.sin(ang) * m], axis=1)


def rotate_f32(x32, cos32, sin32, rotary_dim):
    """Rotate fp32 rows x [..., D] by fp32 (cos, sin) [..., R/2] broadcast over
    the head axis, in fp32 without fused multiply-add."""
    x32 = np.asarray(x32, dtype=np.float32)
    h = rotary_dim // 2
    x1 = x32[..., :h]
    x2 = x32[..., h:rotary_dim]
    c = np.asarray(cos32, dtype=np.float32)
    s = np.asarray(sin32, dtype=np.float32)
    y = x32.copy()
    y[..., :h] = (x1 * c) - (x2 * s)
    y[..., h:rotary_dim] = (x2 * c) + (x1 * s)
    return y


def _cast_src(x32, src_dtype):
    """fp32 -> the source dtype's storage (fp16 values or bf16 bit patterns), RNE."""
    if src_dtype == "f16":
        return x32.astype(np.float16)
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def qkv_rope_store(qkv, src_dtype, positions, table32, rotary_dim, num_q_heads, num_kv_heads, head_dim,
                   slots, k_cache, v_cache, kv_dtype, k_scale=1.0, v_scale=1.0,
                   k_scales=None, v_scales=None):
    """The fused step on host arrays.

    qkv: [T][(Hq + 2 Hkv) * D] in the source dtype (fp16, or bf16 bits);
    positions int64[T]; table32 fp32 [max_position][2][R/2]; slots int64[T].
    Caches are flat uint8 arrays (scale planes flat fp32 for 'int8_tok').
    Returns (q_out [T][Hq][D] in the source dtype, k_cache, v_cache,
    k_scales, v_scales) as new arrays.
    """
    T = qkv.shape[0]
    hq, hkv, D = num_q_heads, num_kv_heads, head_dim
    x = codecs.source_to_f32(np.asarray(qkv).reshape(T, hq + 2 * hkv, D), src_dtype)
    q, k, v = x[:, :hq], x[:, hq:hq + hkv], x[:, hq + hkv:]
    positions = np.asarray(positions, dtype=np.int64)
    table32 = np.asarray(table32, dtype=np.float32)
    ok = (positions >= 0) & (positions < table32.shape[0])
    p = np.where(ok, positions, 0)
    c = table32[p, 0][:, None, :]
    s = table32[p, 1][:, None, :]
    q_rot = rotate_f32(q, c, s, rotary_dim)
    q_rot[~ok] = np.nan
    k_rot = rotate_f32(k, c, s, rotary_dim)
    store_slots = np.where(ok, np.asarray(slots, dtype=np.int64), -1)
    if kv_dtype == "int8_tok":
        kc, ks = codecs.quantize_per_token(k_rot)
        vc, vs = codecs.quantize_per_token(v)
        k_scales = layout.scatter_scales(k_scales, ks, store_slots, hkv)
        v_scales = layout.scatter_scales(v_scales, vs, store_slots, hkv)
    else:
        kc = codecs.quantize(k_rot, kv_dtype, k_scale)
        vc = codecs.quantize(v, kv_dtype, v_scale)
    k_cache = layout.scatter(k_cache, kc, store_slots, "k", hkv, D, kv_dtype)
    v_cache = layout.scatter(v_cache, vc, store_slots, "v", hkv, D, kv_dtype)
    return _cast_src(q_rot, src_dtype), k_cache, v_cache, k_scales, v_scales
