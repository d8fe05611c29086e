"""Edge cases of ra_paged_attn against the oracle: sequences with no queries
or no keys inside a batch, the narrowest and widest windows, sinks covering
the whole context, more partitions than pages, the maximum split count, a
long D = 64 context, block tables far wider than the context, one query head
per KV head with a 16-token block, and the fused store next to empty
sequences."""
import numpy as np
import pytest
import torch

import paged_quantized_kv_ra_amd as P
from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import DeviceWorkload, compare, log, oracle_seq, out_to_np

pytestmark = pytest.mark.gpu

# name, ctx, q_len, Hq, Hkv, D, kv, window, sinks, num_splits, extra_stride
CASES = [
    ("empty_seqs_mixed", [300, 0, 77, 500, 16], [5, 0, 0, 3, 16], 16, 2, 128, "e4m3", -1, 0, 0, 1),
    ("window_one_sinks3", [200, 64], 5, 16, 2, 128, "int8", 1, 3, 2, 1),
    ("window_wider_than_ctx", [300, 40], 4, 16, 2, 64, "f16", 10000, 2, 0, 1),
    ("sinks_cover_ctx", [150, 33], 2, 16, 2, 128, "e4m3", 10, 5000, 3, 1),
    ("splits_exceed_pages", [100, 17, 1], 1, 16, 2, 128, "int8_tok", -1, 0, 64, 1),
    ("max_splits_d64", [70000], 1, 16, 2, 64, "e4m3", -1, 0, 4096, 1),
    ("long_d64_int8_q3", [65537, 9], 3, 8, 2, 64, "int8", -1, 0, 0, 1),
    ("wide_block_table", [100, 260], 5, 16, 2, 128, "e4m3", -1, 0, 0, 4900),
    ("g1_q16", [40, 16, 1000], 16, 4, 4, 128, "e4m3", -1, 0, 0, 1),
]


def _build(case, seed=61):
    name, ctx, ql, hq, hkv, D, kv, win, sinks, S, extra = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    return W.build(name, seed, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                   pool_pages=pool, window_left=win, num_sinks=sinks, num_splits=S, extra_stride=extra)


def _check(w, out, lse, what):
    out = out_to_np(out)
    lse = lse.cpu().numpy().astype(np.float64)
    for b in range(w.batch):
        q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
        if q1 == q0:
            continue
        ro, rl = oracle_seq(w, b)
        compare(out[q0:q1], lse[q0:q1], ro, rl, f"{what} seq {b}")
    assert np.isfinite(lse).all() or w.window_left >= 0


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_edge_case_matches_oracle(case):
    w = _build(case)
    dw = DeviceWorkload(w)
    out, lse = dw.attn()
    torch.cuda.synchronize()
    _check(w, out, lse, case[0])
    g = w.num_q_heads // w.num_kv_heads
    if g * w.max_q_len <= 48:     # again with the step's own tokens stored by the attention launch
        dwf = DeviceWorkload(w, fused_new=True)
        out2, lse2 = dwf.attn()
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), out.view(torch.int16)), case[0]
        assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32)), case[0]
        assert torch.equal(dwf.k_cache.view(torch.uint8), dw.k_cache.view(torch.uint8)), case[0]
        assert torch.equal(dwf.v_cache.view(torch.uint8), dw.v_cache.view(torch.uint8)), case[0]
    log(f"{case[0]}: matches the oracle" + (" (and with the fused store)" if g * w.max_q_len <= 48 else ""))


def test_max_splits_partials_of_empty_partitions():
    """4096 partitions over 70,000 keys: the partitions past the context are
    empty and carry (0, -inf); the merge of all of them is the oracle's."""
    w = _build(CASES[5])
    dw = DeviceWorkload(w)
    po, pl = dw.attn(partials_only=True)
    torch.cuda.synchronize()
    P_tok = 16 * -(-(-(-70000 // 4096)) // 16)        # 16 * ceil(ceil(70000 / 4096) / 16) = 32
    live = -(-70000 // P_tok)
    pl_np = pl.cpu().numpy()
    assert np.all(pl_np[live:] == -np.inf) and np.all(po[live:].cpu().numpy() == 0.0)
    assert np.isfinite(pl_np[:live]).all()
    out, lse = P.lse_merge(po, pl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle_seq(w, 0)
    compare(out_to_np(out), lse.cpu().numpy().astype(np.float64), ro, rl, "max_splits merged")
    log(f"max_splits_d64: {live} live partitions of 4096, merged result matches the oracle")
