"""Pins of oracle.rope: RoPE / YaRN tables and the fused QKV + RoPE + store
step, against properties the mathematics fixes (not against a retyped
formula)."""
import math

import numpy as np
import pytest

from oracle import codecs as OC
from oracle import layout as OL
from oracle import rope as R


def _rotate64(x, p, theta, rot):
    """fp64 rotation through complex numbers: (x_i + i x_{i+R/2}) e^{i p theta_i}."""
    h = rot // 2
    z = (x[..., :h] + 1j * x[..., h:rot]) * np.exp(1j * p * theta)
    y = np.array(x, dtype=np.float64, copy=True)
    y[..., :h] = z.real
    y[..., h:rot] = z.imag
    return y


def _rotate_table64(x, tab, p, rot):
    """fp64 rotation with a fp64 table row (cos, sin already scaled)."""
    h = rot // 2
    c, s = tab[p, 0], tab[p, 1]
    y = np.array(x, dtype=np.float64, copy=True)
    y[..., :h] = x[..., :h] * c - x[..., h:rot] * s
    y[..., h:rot] = x[..., h:rot] * c + x[..., :h] * s
    return y


@pytest.mark.parametrize("rot,D", [(128, 128), (64, 128), (64, 64)])
def test_rotation_is_complex_multiplication(rot, D):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, D))
    tab = R.rope_table(3000, rot, 10000.0)
    th = R.inv_freq(rot, 10000.0)
    for p in (0, 1, 17, 2999):
        np.testing.assert_allclose(_rotate_table64(x, tab, p, rot), _rotate64(x, p, th, rot), rtol=0, atol=1e-12)
    # dims past the rotary part pass through untouched
    assert np.array_equal(_rotate_table64(x, tab, 5, rot)[:, rot:], x[:, rot:])


def test_hand_worked_plain_rope_value():
    # R = 4, base 100: theta = (1, 1/10).  At p = 3 the first pair turns by
    # 3 rad and the second by 0.3 rad.
    tab = R.rope_table(4, 4, 100.0)
    assert tab.shape == (4, 2, 2)
    assert abs(tab[3, 0, 0] - math.cos(3.0)) < 1e-15 and abs(tab[3, 1, 0] - math.sin(3.0)) < 1e-15
    assert abs(tab[3, 0, 1] - math.cos(0.3)) < 1e-15 and abs(tab[3, 1, 1] - math.sin(0.3)) < 1e-15
    # x = e_0 (first dim of the first pair) rotates into (cos 3, 0, sin 3, 0)
    y = _rotate_table64(np.array([1.0, 0.0, 0.0, 0.0]), tab, 3, 4)
    np.testing.assert_allclose(y, [math.cos(3.0), 0.0, math.sin(3.0), 0.0], atol=1e-15)


def test_position_zero_is_identity_and_norms_scale_by_temperature():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 128))
    for factor in (1.0, 2.0, 4.0):
        tab = R.rope_table(64, 128, 1e6, factor, original_max=32)
        m = R.yarn_temperature(factor)
        np.testing.assert_allclose(_rotate_table64(x, tab, 0, 128), x * m, atol=1e-14)
        y = _rotate_table64(x, tab, 37, 128)
        n_in = np.hypot(x[:, :64], x[:, 64:])
        n_out = np.hypot(y[:, :64], y[:, 64:])
        np.testing.assert_allclose(n_out, n_in * m, rtol=1e-13)


def test_scores_depend_only_on_position_difference():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    tab = R.rope_table(600, 128, 10000.0, 2.0, original_max=256)
    ref = _rotate_table64(q, tab, 300, 128) @ _rotate_table64(k, tab, 290, 128)
    for a in (10, 55, 123, 589):
        got = _rotate_table64(q, tab, a, 128) @ _rotate_table64(k, tab, a - 10, 128)
        assert abs(got - ref) < 1e-10 * (1 + abs(ref))


def test_yarn_temperature_value():
    assert R.yarn_temperature(1.0) == 1.0
    assert abs(R.yarn_temperature(2.0) - 1.0693147180559945) < 1e-15


def test_yarn_keeps_high_and_divides_low_frequencies():
    rot, base, L, s = 128, 10000.0, 4096, 2.0
    th = R.inv_freq(rot, base)
    ty = R.yarn_inv_freq(rot, base, s, L)
    wavelength = 2 * math.pi / th
    fast = wavelength < L / 32        # turns more than 32 times over the original context
    slow = wavelength > L / 1         # less than one turn
    assert fast.any() and slow.any()
    # the boundary dims may sit on the ramp's rounded ends; the rest are exact
    np.testing.assert_array_equal(ty[fast][:-1], th[fast][:-1])
    np.testing.assert_allclose(ty[slow][1:], th[slow][1:] / s, rtol=1e-15)
    ratio = ty / th
    assert np.all(ratio <= 1 + 1e-15) and np.all(ratio >= 1 / s - 1e-15)
    assert np.all(np.diff(ratio) <= 1e-15)                 # non-increasing along the dims
    assert ((ratio > 1 / s + 1e-12) & (ratio < 1 - 1e-12)).any()   # a real blend on the ramp


def test_yarn_low_dims_are_plain_rope_at_half_the_position():
    rot, base, L = 128, 10000.0, 4096
    th = R.inv_freq(rot, base)
    slow = np.nonzero(2 * math.pi / th > L)[0][1:]
    ty = R.rope_table(1000, rot, base, 2.0, original_max=L)
    tp = R.rope_table(1000, rot, base)
    m = R.yarn_temperature(2.0)
    for p in (2, 400, 998):
        np.testing.assert_allclose(ty[p, :, slow], tp[p // 2, :, slow] * m, rtol=0, atol=1e-12)


def test_factor_one_is_plain_rope():
    a = R.rope_table(50, 64, 5e5, 1.0, original_max=8)
    b = R.rope_table(50, 64, 5e5)
    assert np.array_equal(a, b)


def _fused_inputs(rng, T, hq, hkv, D, src):
    x = rng.standard_normal((T, (hq + 2 * hkv) * D)).astype(np.float32)
    if src == "f16":
        return x.astype(np.float16)
    return R._cast_src(x, "bf16")


@pytest.mark.parametrize("kv", ["f16", "e4m3", "int8", "int8_tok"])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_fused_step_at_position_zero_is_the_plain_store(kv, src):
    """cos = 1, sin = 0: Q comes back unchanged and K/V land as the plain
    store would put them, which pins the Q | K | V split of the row."""
    rng = np.random.default_rng(4)
    T, hq, hkv, D = 7, 4, 2, 64
    qkv = _fused_inputs(rng, T, hq, hkv, D, src)
    table = R.rope_table(8, D, 10000.0).astype(np.float32)
    slots = np.array([3, 17, -1, 40, 5, 63, 20], dtype=np.int64)
    pages = 4
    e = 2 if kv == "f16" else 1
    kc0 = np.zeros(pages * hkv * 16 * D * e, np.uint8)
    planes = (np.zeros(pages * hkv * 16, np.float32), np.zeros(pages * hkv * 16, np.float32))
    q_out, kc, vc, ks, vs = R.qkv_rope_store(qkv, src, np.zeros(T, np.int64), table, D, hq, hkv, D, slots,
                                             kc0, kc0, kv, 0.01, 0.02, *planes)
    x = OC.source_to_f32(qkv.reshape(T, hq + 2 * hkv, D), src)
    assert np.array_equal(np.asarray(q_out).view(np.uint16), np.asarray(qkv[:, :hq * D]).reshape(T, hq, D).view(np.uint16))
    k, v = x[:, hq:hq + hkv], x[:, hq + hkv:]
    if kv == "int8_tok":
        kq, ksc = OC.quantize_per_token(k)
        vq, vsc = OC.quantize_per_token(v)
        assert np.array_equal(ks, OL.scatter_scales(planes[0], ksc, slots, hkv))
        assert np.array_equal(vs, OL.scatter_scales(planes[1], vsc, slots, hkv))
    else:
        kq, vq = OC.quantize(k, kv, 0.01), OC.quantize(v, kv, 0.02)
    assert np.array_equal(kc, OL.scatter(kc0, kq, slots, "k", hkv, D, kv))
    assert np.array_equal(vc, OL.scatter(kc0, vq, slots, "v", hkv, D, kv))


def test_fused_step_rotates_q_and_k_but_not_v():
    rng = np.random.default_rng(5)
    T, hq, hkv, D = 3, 2, 1, 64
    qkv = _fused_inputs(rng, T, hq, hkv, D, "f16")
    tab64 = R.rope_table(100, D, 10000.0, 2.0, original_max=50)
    table = tab64.astype(np.float32)
    pos = np.array([99, 0, 42], dtype=np.int64)
    slots = np.arange(T, dtype=np.int64)
    kc0 = np.zeros(hkv * 16 * D * 2, np.uint8)
    q_out, kc, vc, _, _ = R.qkv_rope_store(qkv, "f16", pos, table, D, hq, hkv, D, slots, kc0, kc0, "f16")
    x = qkv.astype(np.float64).reshape(T, hq + 2 * hkv, D)
    for t in range(T):
        want_q = _rotate_table64(x[t, :hq], tab64, pos[t], D)
        np.testing.assert_allclose(np.asarray(q_out[t], np.float64), want_q, rtol=2e-3, atol=2e-3)
    k = OL.gather(kc, slots, "k", hkv, D, "f16").astype(np.float64)
    v = OL.gather(vc, slots, "v", hkv, D, "f16").astype(np.float64)
    for t in range(T):
        np.testing.assert_allclose(k[t], _rotate_table64(x[t, hq:hq + hkv], tab64, pos[t], D), rtol=2e-3, atol=2e-3)
    assert np.array_equal(v, x[:, hq + hkv:])


def test_fused_step_position_out_of_table():
    rng = np.random.default_rng(6)
    T, hq, hkv, D = 2, 2, 1, 64
    qkv = _fused_inputs(rng, T, hq, hkv, D, "f16")
    table = R.rope_table(10, D, 10000.0).astype(np.float32)
    kc0 = np.full(hkv * 16 * D, 0x7F, np.uint8)
    q_out, kc, vc, _, _ = R.qkv_rope_store(qkv, "f16", np.array([10, 3]), table, D, hq, hkv, D,
                                           np.array([0, 1]), kc0, kc0, "e4m3", 1.0, 1.0)
    assert np.isnan(q_out[0].astype(np.float32)).all() and np.isfinite(q_out[1].astype(np.float32)).all()
    k = OL.gather(kc, np.array([0, 1]), "k", hkv, D, "e4m3")
    assert np.all(k[0] == 0x7F) and not np.all(k[1] == 0x7F)


# ---------------------------------------------------------------------------
# YaRN against a library routine: the Hugging Face runtime's own YaRN
# parameter function (transformers.modeling_rope_utils), which applies the
# config entry the pages give ("Quick start", step 2: rope_type yarn, factor
# 2, original_max_position_embeddings 262144).  Every dim is compared,
# including both ends of the ramp, so a floor / ceil or truncation slip at
# either end fails.  The routine computes in fp32, hence the 2e-6 tolerance;
# moving a ramp end by one dim changes some frequency by far more.

YARN_CASES = [
    # (rotary_dim, head_dim, base, original_max, factor)
    (128, 128, 1e6, 262144, 2.0),     # the pages' deployment (rope base is a parameter)
    (128, 128, 1e4, 262144, 2.0),
    (128, 128, 1e4, 4096, 2.0),
    (64, 64, 1e4, 2048, 4.0),
    (128, 128, 5e5, 8192, 8.0),
    (64, 128, 1e6, 32768, 2.0),       # partial rotary: 64 of 128 dims
    (16, 64, 500.0, 100, 2.0),        # short ramp clamped at both ends
]


def _hf_yarn(rot, head_dim, base, orig, factor):
    transformers = pytest.importorskip("transformers")
    from transformers.modeling_rope_utils import _compute_yarn_parameters
    cfg = transformers.PretrainedConfig()
    cfg.hidden_size = head_dim * 4
    cfg.num_attention_heads = 4
    cfg.head_dim = head_dim
    cfg.max_position_embeddings = int(orig * factor)
    cfg.rope_parameters = {"rope_type": "yarn", "rope_theta": base, "factor": factor,
                           "original_max_position_embeddings": orig,
                           "partial_rotary_factor": rot / head_dim}
    inv, attention_factor = _compute_yarn_parameters(cfg, "cpu")
    return inv.double().numpy(), float(attention_factor)


@pytest.mark.parametrize("rot,head_dim,base,orig,factor", YARN_CASES)
def test_yarn_matches_the_runtime_routine_on_every_dim(rot, head_dim, base, orig, factor):
    want, m = _hf_yarn(rot, head_dim, base, orig, factor)
    got = R.yarn_inv_freq(rot, base, factor, orig)
    assert got.shape == want.shape
    np.testing.assert_allclose(got, want, rtol=2e-6, atol=0)
    assert abs(R.yarn_temperature(factor) - m) < 1e-12


@pytest.mark.parametrize("rot,head_dim,base,orig,factor", YARN_CASES[:5])
def test_yarn_ramp_end_slips_are_caught(rot, head_dim, base, orig, factor):
    """The comparison above has the power to see a ramp end moved by one dim:
    the frequencies with either end shifted differ from the routine's by far
    more than its tolerance."""
    want, _ = _hf_yarn(rot, head_dim, base, orig, factor)
    theta = R.inv_freq(rot, base)
    lo = max(math.floor(R.yarn_correction_dim(rot, base, orig, 32.0)), 0)
    hi = min(math.ceil(R.yarn_correction_dim(rot, base, orig, 1.0)), rot - 1)
    d = np.arange(rot // 2, dtype=np.float64)
    for l2, h2 in ((lo + 1, hi), (lo - 1, hi), (lo, hi + 1), (lo, hi - 1)):
        if l2 < 0 or h2 <= l2:
            continue
        ramp = np.clip((d - l2) / (h2 - l2), 0.0, 1.0)
        slipped = theta * (1.0 - ramp) + theta / factor * ramp
        assert np.max(np.abs(slipped - want) / want) > 1e-3, (l2, h2)
