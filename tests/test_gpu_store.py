"""GPU parity of ra_kv_store and ra_kv_gather_dequant against the oracle.

Bit-exact: cache bytes after the store equal the oracle's scatter of its
quantised codes into the same sentinel-filled cache; the gather returns the
oracle's fp32 dequantised values bit for bit.
"""
import numpy as np
import pytest
import torch

import paged_quantized_kv_ra_amd as P
from oracle import codecs as OC
from oracle import layout as OL
from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import DeviceWorkload, log

pytestmark = pytest.mark.gpu


def _oracle_cache(w, which):
    e = 2 if w.kv_dtype == "f16" else 1
    nbytes = w.num_pages * w.num_kv_heads * 16 * w.head_dim * e
    if w.kv_dtype == "f16":
        cache = np.frombuffer(np.full(nbytes // 2, w.cache_sentinel, np.uint16).tobytes(), np.uint8).copy()
    else:
        cache = np.full(nbytes, w.cache_sentinel, np.uint8)
    src = w.tokens_k if which == "k" else w.tokens_v
    scale = w.k_scale if which == "k" else w.v_scale
    codes = OC.quantize(OC.source_to_f32(src, w.src_dtype), w.kv_dtype, scale)
    return OL.scatter(cache, codes, w.token_slots, which, w.num_kv_heads, w.head_dim, w.kv_dtype)


def _gpu_bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


@pytest.mark.parametrize("kv", ["f16", "e4m3", "int8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_store_bit_exact_small(kv, D, src):
    w = W.build(f"store_{kv}_{D}_{src}", 11, ctx=[50, 33, 70, 16, 1], q_len=1, num_q_heads=4, num_kv_heads=2,
                head_dim=D, kv_dtype=kv, src_dtype=src, q_dtype="f16", pool_pages=24)
    dw = DeviceWorkload(w)
    torch.cuda.synchronize()
    for which, cache in (("k", dw.k_cache), ("v", dw.v_cache)):
        got = _gpu_bytes(cache)
        want = _oracle_cache(w, which)
        assert got.shape == want.shape
        diff = np.nonzero(got != want)[0]
        assert diff.size == 0, f"{which}: {diff.size} bytes differ, first at {diff[:8]}"


def _all_16bit_tokens(src, D):
    """Every 16-bit pattern of the source dtype, as [65536 / D][1][D]."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if src == "f16":
        return bits.view(np.float16).reshape(-1, 1, D)
    return bits.reshape(-1, 1, D)


@pytest.mark.parametrize("kv", ["e4m3", "int8", "f16"])
@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.0130004883, 2.0 ** -7, 3.7e-3, 1000.0])
def test_store_every_16bit_input(kv, src, scale):
    """Exhaustive over the store's reachable inputs for a given scale: every
    fp16 / bf16 bit pattern (NaN, inf, subnormals, ties) through the fp32
    divide and the encoder."""
    D = 128
    x = _all_16bit_tokens(src, D)
    T = x.shape[0]
    pages = T // 16
    slots = np.random.default_rng(1).permutation(T).astype(np.int64)
    kc = P.new_cache(pages, 1, D, kv, fill=0)
    vc = P.new_cache(pages, 1, D, kv, fill=0)
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    xt = xt.view(torch.float16) if src == "f16" else xt.view(torch.bfloat16)
    P.kv_store(xt, xt, torch.from_numpy(slots).cuda(), kc, vc, kv, scale, scale)
    torch.cuda.synchronize()
    codes = OC.quantize(OC.source_to_f32(x, src), kv, scale)
    e = 2 if kv == "f16" else 1
    zero = np.zeros(pages * 16 * D * e, np.uint8)
    for which, cache in (("k", kc), ("v", vc)):
        want = OL.scatter(zero, codes, slots, which, 1, D, kv)
        got = _gpu_bytes(cache)
        if kv == "f16":   # NaN payloads may differ only in quiet bits; compare values
            g16, w16 = got.view(np.float16), want.view(np.float16)
            same = (g16.view(np.uint16) == w16.view(np.uint16)) | (np.isnan(g16) & np.isnan(w16))
            assert same.all(), f"{which}: {(~same).sum()} differ"
        else:
            diff = np.nonzero(got != want)[0]
            assert diff.size == 0, f"{which}: {diff.size} bytes differ"


def test_store_skips_negative_and_out_of_range_slots():
    D, hkv, pages = 64, 2, 4
    kc = P.new_cache(pages, hkv, D, "e4m3", fill=0x5A)
    vc = P.new_cache(pages, hkv, D, "e4m3", fill=0x5A)
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((4, hkv, D)).astype(np.float16)).cuda()
    slots = torch.tensor([-1, 5, pages * 16, -100], dtype=torch.int64).cuda()
    P.kv_store(x, x, slots, kc, vc, "e4m3", 0.01, 0.01)
    torch.cuda.synchronize()
    got = _gpu_bytes(kc)
    cache0 = np.full(got.size, 0x5A, np.uint8)
    codes = OC.quantize(x.cpu().numpy().astype(np.float32), "e4m3", 0.01)
    want = OL.scatter(cache0, codes, np.array([-1, 5, -1, -1]), "k", hkv, D, "e4m3")
    assert np.array_equal(got, want)


def test_store_strided_source_view():
    """K and V may be views into a fused [T][3][Hkv][D] QKV buffer."""
    D, hkv, T = 128, 2, 40
    rng = np.random.default_rng(3)
    qkv = torch.from_numpy(rng.standard_normal((T, 3, hkv, D)).astype(np.float16)).cuda()
    k, v = qkv[:, 1], qkv[:, 2]
    assert k.stride(0) == 3 * hkv * D
    slots = torch.from_numpy(rng.permutation(64)[:T].astype(np.int64)).cuda()
    kc = P.new_cache(4, hkv, D, "int8", fill=0)
    vc = P.new_cache(4, hkv, D, "int8", fill=0)
    P.kv_store(k, v, slots, kc, vc, "int8", 0.02, 0.03)
    torch.cuda.synchronize()
    for which, src, sc, cache in (("k", k, 0.02, kc), ("v", v, 0.03, vc)):
        codes = OC.quantize(src.cpu().numpy().astype(np.float32), "int8", sc)
        want = OL.scatter(np.zeros(4 * hkv * 16 * D, np.uint8), codes, slots.cpu().numpy(), which, hkv, D, "int8")
        assert np.array_equal(_gpu_bytes(cache), want)


@pytest.mark.parametrize("kv", ["e4m3", "int8"])
@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
def test_gather_dequant_every_code(kv, which, D):
    """Every byte value decodes exactly: fp32(decode(code)) * scale."""
    hkv, pages = 2, 8
    n = pages * hkv * 16 * D
    raw = np.arange(n, dtype=np.int64) % 256
    raw = np.random.default_rng(D + which).permutation(raw).astype(np.uint8)
    cache = torch.from_numpy(raw.reshape(pages, hkv, 16 * D)).cuda()
    bt = torch.from_numpy(np.random.default_rng(4).permutation(pages).astype(np.int32)).cuda()
    ctx = pages * 16
    scale = 0.0130004883
    got = P.kv_gather_dequant(cache, which, kv, scale, bt, ctx, D).cpu().numpy()
    slots = OL.slots_for_sequence(bt.cpu().numpy(), ctx)
    codes = OL.gather(raw, slots, "k" if which == 0 else "v", hkv, D, kv)
    want = OC.dequantize(codes, kv, scale)
    both_nan = np.isnan(got) & np.isnan(want)
    same = (got.view(np.uint32) == want.view(np.uint32)) | both_nan
    assert same.all(), f"{(~same).sum()} values differ"
    if kv == "e4m3":
        assert both_nan.sum() == 2 * (n // 256)      # codes 0x7F and 0xFF


def test_gather_dequant_f16_and_bad_page():
    D, hkv, pages = 64, 1, 3
    rng = np.random.default_rng(5)
    vals = rng.standard_normal(pages * hkv * 16 * D).astype(np.float16)
    cache = torch.from_numpy(vals.reshape(pages, hkv, 16 * D)).cuda()
    bt = torch.tensor([2, 99, 0], dtype=torch.int32).cuda()     # 99 is not a page
    got = P.kv_gather_dequant(cache, 0, "f16", 1.0, bt, 40, D).cpu().numpy()
    codes = OL.gather(vals.view(np.uint8), OL.slots_for_sequence([2, 0, 0], 40), "k", hkv, D, "f16")
    want = codes.astype(np.float32)
    assert np.array_equal(got[:16], want[:16])
    assert np.isnan(got[16:32]).all()
    assert np.array_equal(got[32:], want[32:])
    log("gather ok")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_store_int8_token_codes_and_scales_bit_exact(D, src):
    """Per-token INT8: the codes in the cache and the fp32 scales in the two
    planes equal the oracle's, bit for bit; unwritten scales stay NaN."""
    w = W.build(f"store_int8tok_{D}_{src}", 12, ctx=[50, 33, 70, 16, 1], q_len=1, num_q_heads=4, num_kv_heads=2,
                head_dim=D, kv_dtype="int8_tok", src_dtype=src, q_dtype="f16", pool_pages=24)
    rng = np.random.default_rng(3)
    # a zero row and rows of very different magnitude
    w.tokens_k[5, 1] = 0
    w.tokens_v[7, 0] = 0
    if src == "f16":
        w.tokens_k[9] = (w.tokens_k[9].astype(np.float32) * 300).astype(np.float16)
        w.tokens_v[11] = (w.tokens_v[11].astype(np.float32) * 1e-3).astype(np.float16)
    dw = DeviceWorkload(w)
    torch.cuda.synchronize()
    e = 1
    nbytes = w.num_pages * w.num_kv_heads * 16 * w.head_dim * e
    for which, cache, plane in (("k", dw.k_cache, dw.k_scales), ("v", dw.v_cache, dw.v_scales)):
        src_x = w.tokens_k if which == "k" else w.tokens_v
        codes, sc = OC.quantize_per_token(OC.source_to_f32(src_x, w.src_dtype))
        want = OL.scatter(np.full(nbytes, w.cache_sentinel, np.uint8), codes, w.token_slots, which,
                          w.num_kv_heads, w.head_dim, "int8_tok")
        got = _gpu_bytes(cache)
        diff = np.nonzero(got != want)[0]
        assert diff.size == 0, f"{which}: {diff.size} code bytes differ, first at {diff[:8]}"
        want_plane = OL.scatter_scales(np.full(w.num_pages * w.num_kv_heads * 16, np.nan, np.float32), sc,
                                       w.token_slots, w.num_kv_heads)
        got_plane = plane.cpu().numpy().reshape(-1)
        assert np.array_equal(got_plane.view(np.uint32), want_plane.view(np.uint32)), f"{which}: scales differ"
    # exact read-back through a block table, scale plane included
    for b in range(w.batch):
        bt = torch.from_numpy(w.block_tables[b]).cuda()
        ctx = int(w.ctx[b])
        rows = w.seq_rows[b]
        for which, cache, plane in ((0, dw.k_cache, dw.k_scales), (1, dw.v_cache, dw.v_scales)):
            got = P.kv_gather_dequant(cache, which, "int8_tok", 1.0, bt, ctx, w.head_dim, scales=plane)
            src_x = w.tokens_k if which == 0 else w.tokens_v
            want = OC.roundtrip(OC.source_to_f32(src_x[rows], w.src_dtype), "int8_tok")
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), (b, which)


def _quad_mix_slots(pages):
    """Slots of 43 source tokens (10 quads and a short tail) that exercise the
    store's whole-quad V path next to every case that must not take it."""
    s = []
    s += [5 * 16 + i for i in range(16)]                  # quads 0-3: one page, in order
    s += [2 * 16 + 4 + i for i in range(4)]               # quad 4: whole group 1 of page 2
    s += [2 * 16 + 9 + i for i in range(4)]               # quad 5: consecutive but misaligned
    s += [3 * 16 + 0, -1, 3 * 16 + 2, 3 * 16 + 3]        # quad 6: a skipped slot inside
    s += [3 * 16 + 11 - i for i in range(4)]              # quad 7: one group, reversed
    s += [4 * 16 + 12, 4 * 16 + 13, 4 * 16 + 14, 6 * 16 + 15]   # quad 8: last token elsewhere
    s += [pages * 16 - 4 + i for i in range(4)]           # quad 9: the pool's last group
    s += [7 * 16 + i for i in range(3)]                   # tail: an aligned but short quad
    assert len(s) == 43 and len({x for x in s if x >= 0}) == 42
    return np.array(s, np.int64)


def _check_store(kv, D, src, slots, pages, seed):
    """Store random K/V rows at `slots` and compare every cache byte (and
    per-token scale) with the oracle's scatter into the same sentinel-filled
    caches."""
    hkv = 2
    T = slots.size
    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((2, T, hkv, D)).astype(np.float32)
    x32[1, 9, 1] *= 1e-3                                  # rows of very different magnitude
    x32[0, 17, 0] = 0.0                                   # and a zero row (per-token scale 0)
    if src == "f16":
        xs = x32.astype(np.float16)
        kt, vt = (torch.from_numpy(xs[i]).cuda() for i in range(2))
    else:
        xs = (x32.view(np.uint32) >> 16).astype(np.uint16)
        kt, vt = (torch.from_numpy(xs[i].view(np.int16)).cuda().view(torch.bfloat16) for i in range(2))
    e = 2 if kv == "f16" else 1
    sentinel = 0x3C01 if kv == "f16" else 0xA5
    kc = P.new_cache(pages, hkv, D, kv, fill=sentinel)
    vc = P.new_cache(pages, hkv, D, kv, fill=sentinel)
    st = torch.from_numpy(slots).cuda()
    if kv == "int8_tok":
        ksp, vsp = P.new_scale_plane(pages, hkv), P.new_scale_plane(pages, hkv)
        P.kv_store(kt, vt, st, kc, vc, kv, k_scales=ksp, v_scales=vsp)
    else:
        P.kv_store(kt, vt, st, kc, vc, kv, 0.0130004883, 0.02)
    torch.cuda.synchronize()
    log(f"store {kv} D={D} {src}: {T} tokens")
    nbytes = pages * hkv * 16 * D * e
    for which, i, cache in (("k", 0, kc), ("v", 1, vc)):
        xf = OC.source_to_f32(xs[i], src)
        if kv == "f16":
            cache0 = np.frombuffer(np.full(nbytes // 2, sentinel, np.uint16).tobytes(), np.uint8).copy()
        else:
            cache0 = np.full(nbytes, sentinel, np.uint8)
        if kv == "int8_tok":
            codes, sc = OC.quantize_per_token(xf)
            plane = (ksp if which == "k" else vsp).cpu().numpy().reshape(-1)
            want_plane = OL.scatter_scales(np.full(pages * hkv * 16, np.nan, np.float32), sc, slots, hkv)
            assert np.array_equal(plane.view(np.uint32), want_plane.view(np.uint32)), f"{which}: scales differ"
        else:
            codes = OC.quantize(xf, kv, 0.0130004883 if which == "k" else 0.02)
        want = OL.scatter(cache0, codes, slots, which, hkv, D, kv)
        got = _gpu_bytes(cache)
        diff = np.nonzero(got != want)[0]
        assert diff.size == 0, f"{which}: {diff.size} bytes differ, first at {diff[:8]}"


@pytest.mark.parametrize("kv", ["f16", "e4m3", "int8", "int8_tok"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_store_token_quads_mixed(kv, D, src):
    """A small store (one token per thread): every slot pattern of the mix,
    bytes equal to the oracle's scatter, unwritten bytes keep their sentinel."""
    _check_store(kv, D, src, _quad_mix_slots(10), 10, D + (kv == "f16") + 7 * (src == "bf16"))


@pytest.mark.parametrize("kv", ["f16", "e4m3", "int8_tok"])
@pytest.mark.parametrize("D", [64, 128])
def test_store_bulk_token_quads(kv, D):
    """A bulk store (four tokens per thread: at least 131,072 (token, head)
    rows).  A group of four source tokens whose slots are one 4-token group
    of a page writes its V codes as whole 16-byte pieces; every other group
    (the mix's cases, and a run that only lines up from its second token on)
    stores element by element.  Every byte equals the oracle's scatter."""
    pages = 4200
    mix = _quad_mix_slots(pages)                          # source tokens 0 .. 42
    # token 43 takes a slot = 3 (mod 4), so the groups from token 44 on are whole
    bulk = 8 * 16 + 3 + np.arange(65536, dtype=np.int64)
    slots = np.concatenate([mix, bulk])
    assert slots.size * 2 >= 131072 and bulk[-1] < (pages - 1) * 16
    _check_store(kv, D, "f16", slots, pages, 40 + D)
