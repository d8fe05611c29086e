"""Pins for the oracle's paged layout, scatter and gather (CPU only)."""
import os

import numpy as np
import pytest

from oracle import codecs, layout
from tests.conftest import GOLDEN


@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("e", [1, 2])
def test_offsets_are_a_bijection_onto_the_block(which, D, e):
    tab = layout.offset_table(which, D, e)
    covered = np.concatenate([tab.reshape(-1) + j for j in range(e)])
    assert np.array_equal(np.sort(covered), np.arange(layout.block_bytes(D, e)))
    assert np.all(tab % e == 0)


def test_hand_worked_offsets():
    n = 0
    with open(os.path.join(GOLDEN, "layout_offsets.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            which, D, e, t, d, off = line.split()
            fn = layout.k_offset if which == "k" else layout.v_offset
            assert fn(int(t), int(d), int(D), int(e)) == int(off), line
            n += 1
    assert n >= 10


def test_k_lane_holds_one_token_contiguous_dim_slice():
    # the defining property of the K layout: the 16-byte pieces at lane L
    # hold token L % 16, dims [(L // 16) * D/4, +D/4) in order
    D, e = 128, 1
    tab = layout.offset_table("k", D, e)
    for t in range(16):
        for k in range(4):
            dims = np.arange(k * 32, (k + 1) * 32)
            offs = tab[t, dims]
            lane = 16 * k + t
            assert np.array_equal(offs, [(i // 16) * 1024 + lane * 16 + i % 16 for i in range(32)])


@pytest.mark.parametrize("kv", ["f16", "e4m3", "int8"])
@pytest.mark.parametrize("D", [64, 128])
def test_scatter_gather_round_trip(kv, D):
    rng = np.random.default_rng(D)
    hkv, pages = 2, 9
    n = pages * 16
    slots = rng.permutation(n).astype(np.int64)
    x = rng.standard_normal((n, hkv, D)).astype(np.float32)
    codes = codecs.quantize(x, kv, np.float32(0.01))
    e = codecs.code_nbytes(kv)
    cache0 = np.zeros(pages * hkv * 16 * D * e, dtype=np.uint8)
    for which in ("k", "v"):
        cache = layout.scatter(cache0, codes, slots, which, hkv, D, kv)
        back = layout.gather(cache, slots, which, hkv, D, kv)
        assert np.array_equal(back.view(np.uint8), np.ascontiguousarray(codes).view(np.uint8))


def test_scatter_skips_negative_slots_and_keeps_other_bytes():
    rng = np.random.default_rng(1)
    hkv, D, pages = 1, 64, 4
    cache0 = rng.integers(0, 256, pages * hkv * 16 * D, dtype=np.uint8)
    slots = np.array([5, -1, 40, -7], dtype=np.int64)
    codes = rng.integers(0, 255, (4, hkv, D), dtype=np.uint8)
    cache = layout.scatter(cache0, codes, slots, "k", hkv, D, "e4m3")
    changed = np.nonzero(cache != cache0)[0]
    allowed = set()
    for s in (5, 40):
        page, t = divmod(s, 16)
        for d in range(D):
            allowed.add(page * 16 * D + layout.k_offset(t, d, D, 1))
    assert set(changed.tolist()) <= allowed
    back = layout.gather(cache, np.array([5, 40]), "k", hkv, D, "e4m3")
    assert np.array_equal(back, codes[[0, 2]])


def test_slots_for_sequence():
    row = np.array([7, 2, 9])
    s = layout.slots_for_sequence(row, 35)
    assert s[0] == 112 and s[15] == 127 and s[16] == 32 and s[34] == 146


def test_scale_plane_offsets_and_round_trip():
    # hand-worked: Hkv = 2, slot 37 = page 2, token 5 -> (2 * 2 + h) * 16 + 5
    assert layout.scale_index([37], 2).tolist() == [[69, 85]]
    rng = np.random.default_rng(5)
    pages, hkv = 12, 2
    slots = rng.permutation(pages * 16)[:100].astype(np.int64)
    slots[::9] = -1
    sc = rng.standard_normal((100, hkv)).astype(np.float32)
    plane0 = np.full(pages * hkv * 16, np.float32(7.0))
    plane = layout.scatter_scales(plane0, sc, slots, hkv)
    keep = slots >= 0
    np.testing.assert_array_equal(layout.gather_scales(plane, slots[keep], hkv), sc[keep])
    touched = np.zeros(plane.size, bool)
    touched[layout.scale_index(slots[keep], hkv).ravel()] = True
    assert np.all(plane[~touched] == 7.0)
