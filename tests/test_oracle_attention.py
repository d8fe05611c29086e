"""Pins for the oracle's attention, split-KV partials and LSE merge (CPU only).

The pages print no attention values, so the oracle is pinned to a library
routine (torch scaled_dot_product_attention in float64 on the CPU, with an
explicit boolean mask and repeated KV heads), to an independent brute-force
formulation in extended precision, to closed forms worked by hand, and to
invariants that a dropped term, a wrong sign or a transposed operand breaks.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, scale, mask):
    """torch SDPA in float64 with repeated KV heads; q [q_len,Hq,D]."""
    hq, hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    kt = kt.repeat_interleave(hq // hkv, dim=0)[None]
    vt = vt.repeat_interleave(hq // hkv, dim=0)[None]
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("ctx,q_len,hq,hkv,d,w,sinks", [
    (37, 1, 4, 1, 8, -1, 0),
    (100, 5, 16, 2, 16, -1, 0),
    (513, 5, 8, 2, 32, -1, 0),
    (300, 16, 4, 2, 8, 64, 4),
    (4096, 3, 6, 3, 64, 1000, 0),
    (77, 7, 2, 2, 4, 5, 2),
])
def test_matches_torch_sdpa_float64(ctx, q_len, hq, hkv, d, w, sinks):
    rng = np.random.default_rng(ctx + q_len)
    q, k, v = _rand(rng, q_len, hq, d), _rand(rng, ctx, hkv, d), _rand(rng, ctx, hkv, d)
    scale = 1 / math.sqrt(d)
    out, lse = A.attention(q, k, v, scale, w, sinks)
    mask = A.visible_mask(ctx, q_len, w, sinks)
    ref = _sdpa(q, k, v, scale, mask)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_visible_mask_worked_by_hand():
    # ctx 6, block of 2 queries at positions 4 and 5, window 3, 1 sink:
    # pos 4 sees j <= 4 with 4 - j < 3 (j >= 2) or j < 1 -> {0, 2, 3, 4}
    # pos 5 sees j <= 5 with j >= 3 or j == 0          -> {0, 3, 4, 5}
    m = A.visible_mask(6, 2, 3, 1)
    assert m.tolist() == [[True, False, True, True, True, False],
                          [True, False, False, True, True, True]]
    # no window: causal within the verify block only
    m = A.visible_mask(5, 3)
    assert m.tolist() == [[True, True, True, False, False],
                          [True, True, True, True, False],
                          [True, True, True, True, True]]


def test_brute_force_longdouble_tiny():
    rng = np.random.default_rng(5)
    for trial in range(30):
        ctx = int(rng.integers(1, 9))
        q_len = int(rng.integers(1, ctx + 1))
        d = int(rng.integers(1, 5))
        hkv = int(rng.integers(1, 3))
        g = int(rng.integers(1, 3))
        w = int(rng.integers(-1, 5))
        sinks = int(rng.integers(0, 3)) if w > 0 else 0
        q, k, v = _rand(rng, q_len, hkv * g, d), _rand(rng, ctx, hkv, d), _rand(rng, ctx, hkv, d)
        scale = float(rng.uniform(0.2, 1.5))
        out, lse = A.attention(q, k, v, scale, w, sinks)
        for i in range(q_len):
            pos = ctx - q_len + i
            for h in range(hkv * g):
                kh = h // g
                num = np.zeros(d, dtype=np.longdouble)
                den = np.longdouble(0)
                for j in range(ctx):
                    if j > pos:
                        continue
                    if w >= 0 and not (pos - j < w or j < sinks):
                        continue
                    s = np.longdouble(scale) * sum(np.longdouble(q[i, h, t]) * np.longdouble(k[j, kh, t])
                                                   for t in range(d))
                    e = np.exp(s)
                    den += e
                    num += e * v[j, kh].astype(np.longdouble)
                if den == 0:
                    assert lse[i, h] == -np.inf and np.all(out[i, h] == 0)
                else:
                    np.testing.assert_allclose(out[i, h], (num / den).astype(np.float64),
                                               rtol=1e-12, atol=1e-13)
                    assert abs(lse[i, h] - float(np.log(den))) < 1e-12


def test_closed_form_two_keys():
    # scores 0 and ln 3 -> weights 1/4, 3/4; values 4 and 8 -> out 7; lse = ln 4
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3.0)]]])
    v = np.array([[[4.0]], [[8.0]]])
    out, lse = A.attention(q, k, v, 1.0)
    assert abs(out[0, 0, 0] - 7.0) < 1e-14
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14


def test_uniform_values_give_that_value():
    rng = np.random.default_rng(9)
    ctx, d = 200, 16
    q, k = _rand(rng, 5, 8, d), _rand(rng, ctx, 2, d)
    vec = _rand(rng, 2, d)
    v = np.broadcast_to(vec, (ctx, 2, d)).copy()
    out, _ = A.attention(q, k, v, 0.25, 50, 3)
    for h in range(8):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(vec[h // 4], (5, d)), atol=1e-15, rtol=4e-16 * 8)


def test_identical_keys_mean_and_lse_closed_form():
    rng = np.random.default_rng(10)
    ctx, q_len, d, w, sinks = 90, 4, 8, 20, 3
    q = _rand(rng, q_len, 2, d)
    key = _rand(rng, 1, d)
    k = np.broadcast_to(key, (ctx, 1, d)).copy()
    v = _rand(rng, ctx, 1, d)
    out, lse = A.attention(q, k, v, 0.5, w, sinks)
    vis = A.visible_mask(ctx, q_len, w, sinks)
    for i in range(q_len):
        n = vis[i].sum()
        for h in range(2):
            s = 0.5 * float(q[i, h] @ key[0])
            assert abs(lse[i, h] - (s + math.log(n))) < 1e-12
            np.testing.assert_allclose(out[i, h], v[vis[i], 0].mean(axis=0), atol=1e-13)


def test_single_visible_key():
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 3, 8), _rand(rng, 1, 1, 8), _rand(rng, 1, 1, 8)
    out, lse = A.attention(q, k, v, 0.3)
    for h in range(3):
        assert abs(lse[0, h] - 0.3 * float(q[0, h] @ k[0, 0])) < 1e-14
        np.testing.assert_array_equal(out[0, h], v[0, 0])


def test_dominant_key():
    rng = np.random.default_rng(13)
    ctx, d = 64, 4
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 1.0
    k = rng.uniform(-1, 1, (ctx, 1, d)); k[:, 0, 0] = rng.uniform(-1, 1, ctx)
    k[17, 0, 0] = 61.0           # score at least 60 above every other key
    v = _rand(rng, ctx, 1, d)
    out, _ = A.attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[17, 0], atol=1e-20 + 1e-15, rtol=1e-15)


def test_wide_window_equals_causal():
    rng = np.random.default_rng(14)
    ctx, q_len = 150, 6
    q, k, v = _rand(rng, q_len, 4, 8), _rand(rng, ctx, 2, 8), _rand(rng, ctx, 2, 8)
    a = A.attention(q, k, v, 0.4)
    b = A.attention(q, k, v, 0.4, window_left=ctx, num_sinks=0)
    c = A.attention(q, k, v, 0.4, window_left=10 * ctx, num_sinks=5)
    for x, y in [(a, b), (a, c)]:
        np.testing.assert_array_equal(x[0], y[0])
        np.testing.assert_array_equal(x[1], y[1])


def test_permutation_invariance_over_keys():
    rng = np.random.default_rng(15)
    ctx = 333
    q, k, v = _rand(rng, 1, 4, 16), _rand(rng, ctx, 2, 16), _rand(rng, ctx, 2, 16)
    perm = rng.permutation(ctx)
    o1, l1 = A.attention(q, k, v, 0.25)
    o2, l2 = A.attention(q, k[perm], v[perm], 0.25)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_gqa_head_grouping_is_consecutive():
    # query head h reads KV head h // g: a query head whose group's KV are
    # swapped must change, the other group must not
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 2, 4, 8), _rand(rng, 20, 2, 8), _rand(rng, 20, 2, 8)
    o, _ = A.attention(q, k, v, 0.3)
    k2, v2 = k.copy(), v.copy()
    k2[:, 1], v2[:, 1] = _rand(rng, 20, 8), _rand(rng, 20, 8)
    o2, _ = A.attention(q, k2, v2, 0.3)
    np.testing.assert_array_equal(o[:, :2], o2[:, :2])
    assert np.all(np.abs(o[:, 2:] - o2[:, 2:]).max(axis=-1) > 0)


@pytest.mark.parametrize("ctx,q_len,S,w,sinks", [
    (100, 5, 1, -1, 0), (100, 5, 2, -1, 0), (100, 5, 3, -1, 0), (100, 5, 7, -1, 0),
    (40, 3, 7, -1, 0),            # partitions 3..6 are empty
    (160, 1, 10, -1, 0),          # one page per partition
    (1000, 16, 64, 100, 4),       # window + sinks: most partitions see nothing
])
def test_merge_of_split_equals_unsplit(ctx, q_len, S, w, sinks):
    rng = np.random.default_rng(ctx * S)
    q, k, v = _rand(rng, q_len, 4, 8), _rand(rng, ctx, 2, 8), _rand(rng, ctx, 2, 8)
    o, l = A.attention(q, k, v, 0.35, w, sinks)
    po, pl = A.split_attention(q, k, v, 0.35, w, sinks, num_splits=S)
    assert po.shape[0] == S
    mo, ml = A.lse_merge(po, pl)
    np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml, l, rtol=1e-13, atol=1e-13)
    bounds = A.partition_bounds(ctx, num_splits=S)
    for s, (lo, hi) in enumerate(bounds):
        if lo >= hi:
            assert np.all(pl[s] == -np.inf) and np.all(po[s] == 0)


def test_partition_bounds_page_aligned():
    assert A.partition_size(524288, 64) == 8192
    assert A.partition_size(100, 3) == 48
    assert A.partition_size(40, 7) == 16
    assert A.partition_bounds(40, num_splits=7)[2:4] == [(32, 40), (48, 40)]
    assert A.partition_bounds(5000, part_tokens=2048) == [(0, 2048), (2048, 4096), (4096, 5000)]


def test_merge_associative_and_identity():
    rng = np.random.default_rng(17)
    po = _rand(rng, 6, 3, 4, 8)
    pl = rng.uniform(-5, 5, (6, 3, 4))
    pl[2, 0, 0] = -np.inf
    o, l = A.lse_merge(po, pl)
    oa, la = A.lse_merge(po[:2], pl[:2])
    ob, lb = A.lse_merge(po[2:5], pl[2:5])
    o2, l2 = A.lse_merge(np.stack([oa, ob, po[5]]), np.stack([la, lb, pl[5]]))
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=1e-13)
    o1, l1 = A.lse_merge(po[:1], pl[:1])
    np.testing.assert_array_equal(o1, po[0])
    np.testing.assert_array_equal(l1, pl[0])


def test_merge_all_empty():
    po = np.ones((3, 2, 4))
    pl = np.full((3, 2), -np.inf)
    o, l = A.lse_merge(po, pl)
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_merge_closed_form():
    # two partials with lse ln 1 and ln 3: weights 1/4 and 3/4
    po = np.array([[[2.0]], [[6.0]]])
    pl = np.array([[0.0], [math.log(3.0)]])
    o, l = A.lse_merge(po, pl)
    assert abs(o[0, 0] - 5.0) < 1e-14 and abs(l[0] - math.log(4.0)) < 1e-14


def test_explicit_positions_select_rows_of_the_block():
    """Rows are independent: evaluating a subset of a block's queries at their
    own positions gives exactly those rows of the whole block; the default
    positions are the context's last q_len tokens."""
    rng = np.random.default_rng(21)
    ctx, q_len, hq, hkv, d = 90, 40, 4, 2, 8
    q = rng.standard_normal((q_len, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    for w, sinks in [(-1, 0), (13, 3)]:
        full_o, full_l = A.attention(q, k, v, 0.3, w, sinks)
        pos = ctx - q_len + np.arange(q_len)
        o, l = A.attention(q, k, v, 0.3, w, sinks, positions=pos)
        assert np.array_equal(o, full_o) and np.array_equal(l, full_l)
        sub = np.array([0, 7, 8, 31, 39])
        o, l = A.attention(q[sub], k, v, 0.3, w, sinks, positions=pos[sub])
        np.testing.assert_allclose(o, full_o[sub], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l, full_l[sub], rtol=1e-12, atol=1e-14)


def test_explicit_positions_match_brute_force():
    """A query at position p sees keys 0..p (and with a window the last W plus
    the sinks): brute force over explicit positions, including one before
    every key of a window."""
    rng = np.random.default_rng(22)
    ctx, hq, hkv, d = 12, 2, 1, 3
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    positions = np.array([0, 3, 11, 20])
    q = rng.standard_normal((positions.size, hq, d))
    for w, sinks in [(-1, 0), (4, 2)]:
        o, l = A.attention(q, k, v, 0.5, w, sinks, positions=positions)
        for i, p in enumerate(positions):
            keys = [j for j in range(ctx) if j <= p and (w < 0 or p - j < w or j < sinks)]
            for h in range(hq):
                s = np.array([0.5 * float(q[i, h] @ k[j, 0]) for j in keys])
                m = s.max()
                e = np.exp(s - m)
                want = (e[:, None] * v[keys, 0]).sum(axis=0) / e.sum()
                np.testing.assert_allclose(o[i, h], want, rtol=1e-12, atol=1e-14)
                assert abs(l[i, h] - (m + np.log(e.sum()))) < 1e-12


# ---------------------------------------------------------------------------
# NaN inputs: the definition evaluated in IEEE arithmetic.  A NaN score makes
# the row's maximum NaN (IEEE maximum propagates it), so the row's out and lse
# are NaN; a NaN value makes out NaN (lse does not depend on V); rows that do
# not see the NaN key or value are unchanged.

def _nan_case(seed=7):
    rng = np.random.default_rng(seed)
    ctx, ql, hq, hkv, D = 40, 4, 4, 2, 16
    q = rng.standard_normal((ql, hq, D))
    k = rng.standard_normal((ctx, hkv, D))
    v = rng.standard_normal((ctx, hkv, D))
    return q, k, v, 0.25


def test_nan_query_row_is_nan_and_others_unchanged():
    q, k, v, sc = _nan_case()
    ref_o, ref_l = A.attention(q, k, v, sc)
    q2 = q.copy()
    q2[2, 1, 5] = np.nan                      # query 2, head 1
    o, l = A.attention(q2, k, v, sc)
    assert np.isnan(o[2, 1]).all() and np.isnan(l[2, 1])
    keep = np.ones(o.shape[:2], bool)
    keep[2, 1] = False
    assert np.array_equal(o[keep], ref_o[keep]) and np.array_equal(l[keep], ref_l[keep])


def test_nan_key_poisons_exactly_the_queries_that_see_it():
    q, k, v, sc = _nan_case()
    ref_o, ref_l = A.attention(q, k, v, sc)
    ctx, ql = k.shape[0], q.shape[0]
    j = ctx - ql + 2                          # visible to queries 2, 3 only (causal)
    k2 = k.copy()
    k2[j, 0, 3] = np.nan                      # KV head 0 = query heads 0, 1
    o, l = A.attention(q, k2, v, sc)
    for i in range(ql):
        for h in range(q.shape[1]):
            if i >= 2 and h < 2:
                assert np.isnan(o[i, h]).all() and np.isnan(l[i, h])
            else:
                assert np.array_equal(o[i, h], ref_o[i, h]) and l[i, h] == ref_l[i, h]


def test_nan_value_poisons_out_of_the_queries_that_see_it_only():
    q, k, v, sc = _nan_case()
    ref_o, ref_l = A.attention(q, k, v, sc)
    ctx, ql = k.shape[0], q.shape[0]
    j = ctx - 1                               # visible to the last query only
    v2 = v.copy()
    v2[j, 1, 7] = np.nan                      # KV head 1 = query heads 2, 3; dim 7
    o, l = A.attention(q, k, v2, sc)
    assert np.array_equal(l, ref_l)           # lse does not depend on V
    for i in range(ql):
        for h in range(q.shape[1]):
            # (a value that is not finite takes the oracle's row-by-row sum, which
            # may round differently from the matrix product in the last bit)
            if i == ql - 1 and h >= 2:
                assert np.isnan(o[i, h, 7])
                np.testing.assert_allclose(np.delete(o[i, h], 7), np.delete(ref_o[i, h], 7), rtol=1e-13, atol=0)
            else:
                np.testing.assert_allclose(o[i, h], ref_o[i, h], rtol=1e-13, atol=0)


def test_nan_partial_lse_poisons_its_merged_row():
    rng = np.random.default_rng(8)
    po = rng.standard_normal((3, 5, 8))
    pl = rng.standard_normal((3, 5))
    pl[1, 0] = -np.inf                        # an empty partition: contributes nothing
    po[1, 0] = np.nan                         # ... whatever its out holds
    pl[2, 3] = np.nan
    o, l = A.lse_merge(po, pl)
    assert np.isnan(o[3]).all() and np.isnan(l[3])
    ref = A.lse_merge(po[[0, 2]][:, [0]], pl[[0, 2]][:, [0]])
    np.testing.assert_allclose(o[0], ref[0][0], rtol=1e-15)
    assert np.isfinite(o[[0, 1, 2, 4]]).all() and np.isfinite(l[[0, 1, 2, 4]]).all()
