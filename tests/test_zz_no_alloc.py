"""ra_paged_attn_noalloc (the entry point for callers that cannot allocate)
against ra_paged_attn with a caller workspace: the same kernels over the
same inputs, so out and lse must agree bit for bit.  Two calls in a row on
one GPU, the second with a smaller input (fewer sequences, fewer partition
slots and rows), so that the second call must not read anything the first
left in the shared scratch; both through the C ABI."""
import numpy as np
import pytest
import torch

from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import DeviceWorkload, compare, log, oracle_seq, out_to_np

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


# name, ctx, q_len, Hq, Hkv, D, kv, num_splits: a large split call, then smaller ones
CALLS = [
    ("verify_e4m3_auto", [40000, 9000, 513, 77], 5, 16, 2, 128, "e4m3", 0),
    ("decode_int8tok_split5", [3000, 700], 1, 16, 2, 128, "int8_tok", 5),
    ("verify_f16_direct", [300], 3, 8, 2, 64, "f16", 1),
]


def _run_pair(case):
    name, ctx, ql, hq, hkv, D, kv, S = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    w = W.build(name, 61, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                pool_pages=pool, num_splits=S)
    dw = DeviceWorkload(w)
    ref_o, ref_l = dw.attn()                       # ra_paged_attn with a torch-allocated workspace
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    got_o, got_l = dw.attn(no_alloc=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got_o), _bits(ref_o)), f"{name}: out differs from ra_paged_attn"
    assert torch.equal(_bits(got_l), _bits(ref_l)), f"{name}: lse differs from ra_paged_attn"
    return w, got_o, got_l


def test_noalloc_equals_workspace_entry_point_on_successive_calls():
    for case in CALLS:
        w, o, l = _run_pair(case)
        # and against the oracle, one sequence of each call
        ro, rl = oracle_seq(w, 0)
        q1 = int(w.query_start_loc[1])
        compare(out_to_np(o)[:q1], l.cpu().numpy().astype(np.float64)[:q1], ro, rl, f"{case[0]} seq 0")
        log(f"{case[0]}: ra_paged_attn_noalloc == ra_paged_attn bit for bit")
