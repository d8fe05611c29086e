"""The attention launch's fused store (new_k / new_v / new_slots in
ra_attn_args) against the two-call path (ra_kv_store, then ra_paged_attn),
bit for bit: the caches (and per-token INT8 scale planes) afterwards, the
outputs and the lse.  The two-call path is itself checked against the oracle
in test_gpu_store.py and test_gpu_attn.py.

Cases cover E4M3 / INT8 / per-token INT8 / FP16 caches, fp16 and bf16
sources, decode and verify blocks, automatic and explicit splits (with the
new tokens of one sequence straddling a partition boundary), a window with
sinks, a padding token (slot -1), and the merged (partials) and direct
outputs.
"""
import numpy as np
import pytest
import torch

import paged_quantized_kv_ra_amd as P
from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import log, t_src

pytestmark = pytest.mark.gpu

# name, ctx, q_len, Hq, Hkv, D, kv, src, window, sinks, num_splits
CASES = [
    ("verify_e4m3_auto_straddle", [1000, 77, 513, 5, 4097], 5, 16, 2, 128, "e4m3", "f16", -1, 0, 0),
    ("decode_int8_split3", [1000, 77, 513], 1, 16, 2, 128, "int8", "f16", -1, 0, 3),
    ("verify_int8tok_d64_bf16", [700, 33, 300], 5, 8, 2, 64, "int8_tok", "bf16", -1, 0, 2),
    ("verify_f16_window_sinks_q3", [900, 120], 3, 16, 2, 128, "f16", "f16", 100, 4, 0),
    ("verify_e4m3_direct", [600, 300], 6, 16, 2, 128, "e4m3", "bf16", -1, 0, 1),
]


def _sentinel(kv):
    return {"f16": 0x7E00, "e4m3": 0x7F, "int8": 0x80, "int8_tok": 0x80}[kv]


def _caches(w, rows):
    """Fresh caches holding the given token rows (stored with ra_kv_store)."""
    D, hkv = w.head_dim, w.num_kv_heads
    kc = P.new_cache(w.num_pages, hkv, D, w.kv_dtype, fill=_sentinel(w.kv_dtype))
    vc = P.new_cache(w.num_pages, hkv, D, w.kv_dtype, fill=_sentinel(w.kv_dtype))
    ks = vs = None
    if w.kv_dtype == "int8_tok":
        ks, vs = P.new_scale_plane(w.num_pages, hkv), P.new_scale_plane(w.num_pages, hkv)
    if len(rows):
        P.kv_store(t_src(w.tokens_k[rows], w.src_dtype), t_src(w.tokens_v[rows], w.src_dtype),
                   torch.from_numpy(w.token_slots[rows]).cuda(), kc, vc, w.kv_dtype, w.k_scale, w.v_scale,
                   k_scales=ks, v_scales=vs)
    return kc, vc, ks, vs


def _bits(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_store_equals_separate_store(case):
    name, ctx, ql, hq, hkv, D, kv, src, win, sinks, S = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    w = W.build(name, 51, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                q_dtype="f16", src_dtype=src, pool_pages=pool, window_left=win, num_sinks=sinks, num_splits=S)
    new_rows = w.new_token_rows()
    old_rows = np.setdiff1d(np.arange(w.tokens_k.shape[0]), new_rows)
    slots = w.token_slots[new_rows].copy()
    slots[1] = -1                     # a padding token: stored by neither path
    # path A: every older token stored, the query tokens' own K/V stored by the attention launch
    kA, vA, ksA, vsA = _caches(w, old_rows)
    # path B: the same older tokens, then ra_kv_store of the query tokens, then the attention
    kB, vB, ksB, vsB = _caches(w, old_rows)
    new_k = t_src(w.tokens_k[new_rows], w.src_dtype)
    new_v = t_src(w.tokens_v[new_rows], w.src_dtype)
    new_slots = torch.from_numpy(slots).cuda()
    P.kv_store(new_k, new_v, new_slots, kB, vB, kv, w.k_scale, w.v_scale, k_scales=ksB, v_scales=vsB)
    q = t_src(w.q, w.q_dtype)
    common = dict(kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale,
                  max_q_len=w.max_q_len, min_q_len=int(w.q_len.min()), max_context_len=w.max_context_len,
                  window_left=win, num_sinks=sinks, num_splits=S)
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.ctx).cuda()
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    oA, lA = P.paged_attn(q, kA, vA, bt, cl, qsl, k_scales=ksA, v_scales=vsA, new_k=new_k, new_v=new_v,
                          new_slots=new_slots, **common)
    oB, lB = P.paged_attn(q, kB, vB, bt, cl, qsl, k_scales=ksB, v_scales=vsB, **common)
    torch.cuda.synchronize()
    assert torch.equal(_bits(kA), _bits(kB)) and torch.equal(_bits(vA), _bits(vB)), f"{name}: caches differ"
    if kv == "int8_tok":
        assert torch.equal(_bits(ksA), _bits(ksB)) and torch.equal(_bits(vsA), _bits(vsB)), f"{name}: scales differ"
    assert torch.equal(_bits(oA), _bits(oB)), f"{name}: outputs differ"
    assert torch.equal(_bits(lA), _bits(lB)), f"{name}: lse differs"
    # the padding token was left alone: its position still reads back the unused-memory pattern
    b = int(np.searchsorted(w.query_start_loc, 1, side="right")) - 1
    pos = int(w.ctx[b]) - int(w.q_len[b]) + (1 - int(w.query_start_loc[b]))
    back = P.kv_gather_dequant(kA, 0, kv, w.k_scale, bt[b], int(w.ctx[b]), D, scales=ksA)[pos].cpu().numpy()
    if kv == "int8":
        assert np.all(back == np.float32(-128.0) * np.float32(w.k_scale)), name
    else:
        assert np.isnan(back).all(), name
    log(f"{name}: fused store == ra_kv_store + ra_paged_attn, bit for bit")


def test_fused_store_graph_replay():
    """The fused store inside a captured graph: every replay leaves the same
    caches and outputs as the eager launch."""
    w = W.build("fused_graph", 52, ctx=[800, 333], q_len=5, num_q_heads=16, num_kv_heads=2, head_dim=128,
                kv_dtype="e4m3", pool_pages=100, num_splits=0)
    new_rows = w.new_token_rows()
    old_rows = np.setdiff1d(np.arange(w.tokens_k.shape[0]), new_rows)
    kc, vc, _, _ = _caches(w, old_rows)
    new_k = t_src(w.tokens_k[new_rows], w.src_dtype)
    new_v = t_src(w.tokens_v[new_rows], w.src_dtype)
    new_slots = torch.from_numpy(w.token_slots[new_rows]).cuda()
    q = t_src(w.q, w.q_dtype)
    bt, cl, qsl = (torch.from_numpy(x).cuda() for x in (w.block_tables, w.ctx, w.query_start_loc))
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device="cuda")
    kw = dict(kv_dtype="e4m3", k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale, max_q_len=5,
              min_q_len=5, max_context_len=w.max_context_len, new_k=new_k, new_v=new_v, new_slots=new_slots)
    a = P._lib._attn_args(q, kc, vc, bt, cl, qsl, "e4m3", w.k_scale, w.v_scale, w.softmax_scale, 5, 5,
                          w.max_context_len, -1, 0, 0, 2, None, None, None, None, new_k, new_v, new_slots)
    S, _, _ = P._lib.paged_attn_workspace(a)
    po = torch.empty((S, q.shape[0], q.shape[1], 128), dtype=torch.float32, device="cuda")
    pl = torch.empty((S, q.shape[0], q.shape[1]), dtype=torch.float32, device="cuda")
    pre_k, pre_v = kc.clone(), vc.clone()
    P.paged_attn(q, kc, vc, bt, cl, qsl, out=out, lse=lse, workspace=(po, pl), **kw)
    torch.cuda.synchronize()
    ref_o, ref_l, ref_k, ref_v = out.clone(), lse.clone(), kc.clone(), vc.clone()
    assert not torch.equal(ref_k, pre_k) and not torch.equal(ref_v, pre_v)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        P.paged_attn(q, kc, vc, bt, cl, qsl, out=out, lse=lse, workspace=(po, pl), stream=side, **kw)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        kc.copy_(pre_k)              # back to the caches before the step's tokens
        vc.copy_(pre_v)
        y = torch.arange(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(y) > 0
        assert torch.equal(_bits(out), _bits(ref_o)) and torch.equal(_bits(lse), _bits(ref_l)), rep
        assert torch.equal(kc, ref_k) and torch.equal(vc, ref_v), rep
    log("fused store: 3 graph replays equal to the eager launch")
    del g


# name, ctx, q_len, Hq, Hkv, D, kv, src, rotary_dim, yarn factor, num_splits
ROPE_CASES = [
    ("verify_e4m3_yarn", [1000, 77, 513, 4097], 5, 16, 2, 128, "e4m3", "f16", 128, 2.0, 0),
    ("decode_int8tok_d64_partial_bf16", [700, 33, 300], 1, 8, 2, 64, "int8_tok", "bf16", 32, 1.0, 2),
    ("verify_f16_rot64_q3", [600, 200], 3, 16, 2, 128, "f16", "f16", 64, 4.0, 1),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_fused_rope_equals_qkv_rope_store_then_attention(case):
    """RoPE on the fused path, with q, new_k and new_v as views into packed
    QKV rows, against ra_qkv_rope_store followed by a plain ra_paged_attn:
    caches (and scale planes), outputs and lse bit for bit.  A padding token
    (slot -1) and a token whose position is outside the table are included."""
    from oracle import rope as R
    name, ctx, ql, hq, hkv, D, kv, src, rot, factor, S = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    w = W.build(name, 53, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                q_dtype=src, src_dtype=src, pool_pages=pool, num_splits=S)
    new_rows = w.new_token_rows()
    old_rows = np.setdiff1d(np.arange(w.tokens_k.shape[0]), new_rows)
    pos, slots = W.step_positions_and_slots(w)
    slots = slots.copy()
    slots[1] = -1
    max_pos = int(pos.max()) + 1
    pos = pos.copy()
    if len(pos) > 3:
        pos[3] = max_pos               # outside the table: NaN rows, nothing stored
    T = len(pos)
    qkv = t_src(W.packed_qkv(53, T, hq, hkv, D, src, row_pad=8), src)
    table = torch.from_numpy(R.rope_table(max_pos, rot, 1e6, factor, original_max=max(1, max_pos // 2))
                             .astype(np.float32)).cuda()
    q_view = qkv[:, :hq * D].view(T, hq, D)
    k_view = qkv[:, hq * D:(hq + hkv) * D].view(T, hkv, D)
    v_view = qkv[:, (hq + hkv) * D:(hq + 2 * hkv) * D].view(T, hkv, D)
    pos_t = torch.from_numpy(pos).cuda()
    slots_t = torch.from_numpy(slots).cuda()
    bt = torch.from_numpy(w.block_tables).cuda()
    cl = torch.from_numpy(w.ctx).cuda()
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    common = dict(kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale,
                  max_q_len=w.max_q_len, min_q_len=int(w.q_len.min()), max_context_len=w.max_context_len,
                  num_splits=S)
    # path A: one attention launch with the fused store and RoPE
    kA, vA, ksA, vsA = _caches(w, old_rows)
    oA, lA = P.paged_attn(q_view, kA, vA, bt, cl, qsl, k_scales=ksA, v_scales=vsA, new_k=k_view, new_v=v_view,
                          new_slots=slots_t, rope_table=table, positions=pos_t, rotary_dim=rot, **common)
    # path B: the fused QKV + RoPE + store kernel, then a plain attention
    kB, vB, ksB, vsB = _caches(w, old_rows)
    q_rot = P.qkv_rope_store(qkv, pos_t, table, slots_t, kB, vB, kv, num_q_heads=hq, rotary_dim=rot,
                             k_scale=w.k_scale, v_scale=w.v_scale, k_scales=ksB, v_scales=vsB)
    oB, lB = P.paged_attn(q_rot, kB, vB, bt, cl, qsl, k_scales=ksB, v_scales=vsB, **common)
    torch.cuda.synchronize()
    assert torch.equal(_bits(kA), _bits(kB)) and torch.equal(_bits(vA), _bits(vB)), f"{name}: caches differ"
    if kv == "int8_tok":
        assert torch.equal(_bits(ksA), _bits(ksB)) and torch.equal(_bits(vsA), _bits(vsB)), f"{name}: scales differ"
    assert torch.equal(_bits(oA), _bits(oB)), f"{name}: outputs differ"
    assert torch.equal(_bits(lA), _bits(lB)), f"{name}: lse differs"
    log(f"{name}: RoPE + fused store in the attention launch == ra_qkv_rope_store + ra_paged_attn, bit for bit")
