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


def _oracle_fused_rope_attention(w, qkv_host, src, pos, slots, table32, rot):
    """The oracle's answer for one attention launch with the fused store and
    RoPE: older tokens dequantised from their codes, the block's own tokens
    rotated, quantised and dequantised by oracle.rope.qkv_rope_store (tokens
    it does not store read back the caches' zero fill), and fp64 attention
    with the rotated queries."""
    from oracle import attention as OA
    from oracle import codecs as OC
    from oracle import layout as OL
    from oracle import rope as R
    from tests.gpu_util import dequant_tokens
    hq, hkv, D, kv = w.num_q_heads, w.num_kv_heads, w.head_dim, w.kv_dtype
    T = qkv_host.shape[0]
    packed = (hq + 2 * hkv) * D
    local = np.where(slots >= 0, np.arange(T, dtype=np.int64), -1)     # one scratch slot per token
    e = 2 if kv == "f16" else 1
    npg = -(-T // 16)
    zc = np.zeros(npg * hkv * 16 * D * e, np.uint8)
    zp = np.zeros(npg * hkv * 16, np.float32)
    q_rot, kc, vc, ks, vs = R.qkv_rope_store(np.ascontiguousarray(qkv_host[:, :packed]), src, pos, table32, rot,
                                             hq, hkv, D, local, zc, zc.copy(), kv, w.k_scale, w.v_scale,
                                             zp, zp.copy())
    idx = np.arange(T, dtype=np.int64)
    kq = OL.gather(kc, idx, "k", hkv, D, kv)
    vq = OL.gather(vc, idx, "v", hkv, D, kv)
    if kv == "int8_tok":
        k_new = OC.dequantize_per_token(kq, OL.gather_scales(ks, idx, hkv))
        v_new = OC.dequantize_per_token(vq, OL.gather_scales(vs, idx, hkv))
    else:
        k_new = OC.dequantize(kq, kv, w.k_scale)
        v_new = OC.dequantize(vq, kv, w.v_scale)
    q64 = OC.source_to_f32(q_rot, src).astype(np.float64)
    outs, lses = [], []
    for b in range(w.batch):
        q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
        old = w.seq_rows[b][:int(w.ctx[b]) - (q1 - q0)]
        k = np.concatenate([dequant_tokens(w, old, "k"), k_new[q0:q1]])
        v = np.concatenate([dequant_tokens(w, old, "v"), v_new[q0:q1]])
        o, l = OA.attention(q64[q0:q1], k, v, w.softmax_scale)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


ROPE_ORACLE_CASES = ROPE_CASES + [
    ("verify_e4m3_yarn_direct", [1000, 77, 513, 4097], 5, 16, 2, 128, "e4m3", "f16", 128, 2.0, 1),
]


@pytest.mark.parametrize("case", ROPE_ORACLE_CASES, ids=[c[0] for c in ROPE_ORACLE_CASES])
def test_fused_rope_attention_matches_oracle(case):
    """One attention launch with RoPE and the fused store against the oracle
    directly.  The last token of sequence 0 has a position outside the
    table: its Q rows are NaN, so its out and lse must come back NaN (with
    one partition slot and with several), and nothing is stored for it; the
    last token of sequence 1 is padding (slot -1).  The caches start zeroed,
    so the positions of unstored tokens read back zeros on both sides."""
    from oracle import rope as R
    from tests.gpu_util import compare, out_to_np
    name, ctx, ql, hq, hkv, D, kv, src, rot, factor, S = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    w = W.build(name, 54, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                q_dtype=src, src_dtype=src, pool_pages=pool, num_splits=S)
    new_rows = w.new_token_rows()
    old_rows = np.setdiff1d(np.arange(w.tokens_k.shape[0]), new_rows)
    pos, slots = W.step_positions_and_slots(w)
    pos, slots = pos.copy(), slots.copy()
    max_pos = int(pos.max()) + 1
    qsl = w.query_start_loc
    pos[int(qsl[1]) - 1] = max_pos                # outside the table
    slots[int(qsl[2]) - 1] = -1                   # padding
    T = len(pos)
    qkv_host = W.packed_qkv(54, T, hq, hkv, D, src, row_pad=8)
    table32 = R.rope_table(max_pos, rot, 1e6, factor, original_max=max(1, max_pos // 2)).astype(np.float32)
    qkv = t_src(qkv_host, src)
    kc = P.new_cache(w.num_pages, hkv, D, kv, fill=0)
    vc = P.new_cache(w.num_pages, hkv, D, kv, fill=0)
    ks = vs = None
    if kv == "int8_tok":
        ks, vs = P.new_scale_plane(w.num_pages, hkv, fill=0.0), P.new_scale_plane(w.num_pages, hkv, fill=0.0)
    P.kv_store(t_src(w.tokens_k[old_rows], src), t_src(w.tokens_v[old_rows], src),
               torch.from_numpy(w.token_slots[old_rows]).cuda(), kc, vc, kv, w.k_scale, w.v_scale,
               k_scales=ks, v_scales=vs)
    out, lse = P.paged_attn(qkv[:, :hq * D].view(T, hq, D), kc, vc, torch.from_numpy(w.block_tables).cuda(),
                            torch.from_numpy(w.ctx).cuda(), torch.from_numpy(qsl).cuda(),
                            kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale,
                            max_q_len=w.max_q_len, min_q_len=int(w.q_len.min()), max_context_len=w.max_context_len,
                            num_splits=S, k_scales=ks, v_scales=vs,
                            new_k=qkv[:, hq * D:(hq + hkv) * D].view(T, hkv, D),
                            new_v=qkv[:, (hq + hkv) * D:(hq + 2 * hkv) * D].view(T, hkv, D),
                            new_slots=torch.from_numpy(slots).cuda(), rope_table=torch.from_numpy(table32).cuda(),
                            positions=torch.from_numpy(pos).cuda(), rotary_dim=rot)
    torch.cuda.synchronize()
    ro, rl = _oracle_fused_rope_attention(w, qkv_host, src, pos, slots, table32, rot)
    got_o = out_to_np(out)
    got_l = lse.cpu().numpy().astype(np.float64)
    nan_tok = int(qsl[1]) - 1
    assert np.isnan(ro[nan_tok]).all() and np.isnan(rl[nan_tok]).all()
    assert np.isnan(got_o[nan_tok]).all(), f"{name}: out of the out-of-table token is not NaN"
    assert np.isnan(got_l[nan_tok]).all(), f"{name}: lse of the out-of-table token is not NaN"
    keep = np.ones(T, bool)
    keep[nan_tok] = False
    e = compare(got_o[keep], got_l[keep], ro[keep], rl[keep], name)
    log(f"{name}: fused RoPE attention vs oracle: max abs {e[0]:.2e} normwise {e[1]:.2e} lse {e[2]:.2e}")
