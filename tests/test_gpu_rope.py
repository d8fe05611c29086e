"""GPU parity of ra_qkv_rope_store (packed QKV rows -> rotary embedding of Q
and K -> Q for attention, K/V quantised into the pages) against the oracle,
bit for bit: the rotation runs in fp32 from the same fp32 table on both
sides, and Q rounding and the K/V codes are integer decisions taken in that
precision.  The table fed to the kernel is the oracle's (fp64 rounded to
fp32); the library's own table builder is compared with it on the CPU.

Covers FP16 / E4M3 / INT8 / per-token INT8 caches, fp16 and bf16 sources,
D 64 and 128, partial rotary dims, plain RoPE and YaRN, padded row strides,
skipped slots, positions outside the table, and the verify-step and
8K-prefill token sets at full size.
"""
import numpy as np
import pytest
import torch

import paged_quantized_kv_ra_amd as P
from oracle import rope as R
from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import log, t_src

pytestmark = pytest.mark.gpu

# name, T, Hq, Hkv, D, rot, kv, src, factor, max_pos, row_pad
CASES = [
    ("f16_d128_plain", 37, 16, 2, 128, 128, "f16", "f16", 1.0, 4096, 0),
    ("e4m3_d128_yarn", 40, 16, 2, 128, 128, "e4m3", "f16", 2.0, 8192, 0),
    ("int8_d64_bf16_partial", 29, 8, 2, 64, 32, "int8", "bf16", 2.0, 2048, 0),
    ("int8tok_d128_yarn_pad", 50, 16, 2, 128, 128, "int8_tok", "f16", 2.0, 8192, 64),
    ("int8tok_d64_rot48_bf16", 17, 4, 4, 64, 48, "int8_tok", "bf16", 1.0, 512, 8),
    ("e4m3_g1_d128_rot64", 300, 4, 4, 128, 64, "e4m3", "f16", 4.0, 1024, 0),
]


def _sentinel(kv):
    return {"f16": 0x7E00, "e4m3": 0x7F, "int8": 0x80, "int8_tok": 0x80}[kv]


def _flat_bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def _run_case(T, hq, hkv, D, rot, kv, src, factor, max_pos, row_pad, seed, positions=None, slots=None,
              pages=None):
    rng = np.random.default_rng(seed)
    qkv_np = W.packed_qkv(seed, T, hq, hkv, D, src, row_pad)
    if positions is None:
        positions = rng.integers(0, max_pos, size=T).astype(np.int64)
        positions[::7] = max_pos - 1
        positions[1] = 0
        if T > 5:
            positions[5] = max_pos          # outside the table: NaN Q, nothing stored
    if pages is None:
        pages = -(-T // 16) + 2
    if slots is None:
        slots = rng.permutation(pages * 16)[:T].astype(np.int64)
        slots[3 % T] = -1                   # padding token
    table32 = R.rope_table(max_pos, rot, 1e6 if factor > 1 else 10000.0, factor,
                           original_max=max_pos // 2 if factor > 1 else None).astype(np.float32)
    ks = vs = 0.0
    if kv in ("e4m3", "int8"):
        x = np.abs(np.asarray(qkv_np[:, :(hq + 2 * hkv) * D], np.float32)).max() * 1.3   # room for rotation
        ks = vs = float(x / (448.0 if kv == "e4m3" else 127.0))
    dev = "cuda"
    kc = P.new_cache(pages, hkv, D, kv, dev, fill=_sentinel(kv))
    vc = P.new_cache(pages, hkv, D, kv, dev, fill=_sentinel(kv))
    kp = vp = None
    if kv == "int8_tok":
        kp, vp = P.new_scale_plane(pages, hkv, dev), P.new_scale_plane(pages, hkv, dev)
    kc0, vc0 = _flat_bytes(kc), _flat_bytes(vc)
    kp0 = None if kp is None else kp.cpu().numpy().reshape(-1)
    vp0 = None if vp is None else vp.cpu().numpy().reshape(-1)
    qkv = t_src(qkv_np, src)
    q_out = P.qkv_rope_store(qkv, torch.from_numpy(positions).to(dev), torch.from_numpy(table32).to(dev),
                             torch.from_numpy(slots).to(dev), kc, vc, kv, num_q_heads=hq, rotary_dim=rot,
                             k_scale=ks if ks else 1.0, v_scale=vs if vs else 1.0, k_scales=kp, v_scales=vp)
    torch.cuda.synchronize()
    packed = np.ascontiguousarray(qkv_np[:, :(hq + 2 * hkv) * D])
    want_q, want_k, want_v, want_kp, want_vp = R.qkv_rope_store(
        packed, src, positions, table32, rot, hq, hkv, D, slots, kc0, vc0, kv,
        ks if ks else 1.0, vs if vs else 1.0, kp0, vp0)
    got_q = q_out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want_q = np.asarray(want_q).view(np.uint16).reshape(got_q.shape)
    bad_pos = (positions < 0) | (positions >= max_pos)
    qf = (got_q.astype(np.uint32) << 16).view(np.float32) if src == "bf16" else got_q.view(np.float16)
    assert np.isnan(qf[bad_pos]).all(), "Q rows of positions outside the table must be NaN"
    assert np.array_equal(got_q[~bad_pos], want_q[~bad_pos]), \
        f"Q differs at {np.argwhere(got_q[~bad_pos] != want_q[~bad_pos])[:5]}"
    assert np.array_equal(_flat_bytes(kc), want_k), "K cache bytes differ"
    assert np.array_equal(_flat_bytes(vc), want_v), "V cache bytes differ"
    if kv == "int8_tok":
        assert np.array_equal(kp.cpu().numpy().reshape(-1).view(np.uint32), want_kp.view(np.uint32))
        assert np.array_equal(vp.cpu().numpy().reshape(-1).view(np.uint32), want_vp.view(np.uint32))
    return q_out


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_qkv_rope_store_matches_oracle(case):
    name, T, hq, hkv, D, rot, kv, src, factor, max_pos, pad = case
    _run_case(T, hq, hkv, D, rot, kv, src, factor, max_pos, pad, seed=len(name))
    log(f"{name}: Q, K/V codes{' and scales' if kv == 'int8_tok' else ''} bit-exact")


@pytest.mark.parametrize("make", [W.verify_fp8_32k, W.prefill_fp8_8k], ids=["verify_fp8_32k", "prefill_fp8_8k"])
def test_benchmark_step_tokens(make):
    """The new tokens of a benchmark step (their positions and slots), at
    full size, YaRN factor 2 over a 262,144-position table window."""
    w = make()
    pos, slots = W.step_positions_and_slots(w)
    max_pos = int(pos.max()) + 1
    _run_case(len(pos), w.num_q_heads, w.num_kv_heads, w.head_dim, w.head_dim, w.kv_dtype, "f16", 2.0, max_pos,
              0, seed=w.seed, positions=pos, slots=slots, pages=w.num_pages)
    log(f"{w.name}: {len(pos)} tokens bit-exact")
