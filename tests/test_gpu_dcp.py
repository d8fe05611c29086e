"""Context-parallel shards (ReVolta README, "Quick start", DCP2): every
sequence's keys are cut into G ranges held by G separate caches, as G GPUs
would hold them.  Each shard runs ra_paged_attn with kv_pos0 (global position
of its first key) and q_pos0 (global position of the first query).

* each shard's (out, lse) equals the oracle's attention restricted to the
  shard's key range (global positions for causality, window and sinks);
* the shards' partials, concatenated along the partition axis and merged by
  ra_lse_merge, equal the oracle's attention over the whole context.

The shards run one after another on one GPU; their boundaries are not page
aligned, and one shard of one sequence is empty.
"""
import numpy as np
import pytest
import torch

import paged_quantized_kv_ra_amd as P
from oracle import attention as OA
from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import compare, dequant_tokens, log, out_to_np, q_f64, t_src

pytestmark = pytest.mark.gpu

# name, ctx, q_len, Hq, Hkv, D, kv, window, sinks, shard boundaries (fractions), num_splits
CASES = [
    ("g2_e4m3_q5", [3000, 1200, 700], 5, 16, 2, 128, "e4m3", -1, 0, [0.37], 0),
    ("g3_int8_q1_split2", [2500, 999, 130], 1, 16, 2, 128, "int8", -1, 0, [0.2, 0.71], 2),
    ("g3_e4m3_q16_window_sinks", [3000, 1700], 16, 16, 2, 128, "e4m3", 300, 4, [0.001, 0.9], 0),
    ("g2_int8tok_q5_d64", [1500, 600, 17], 5, 8, 2, 64, "int8_tok", -1, 0, [0.5], 3),
    # a 300-token prefill chunk per sequence (the prefill kernel's rows)
    ("g2_e4m3_prefill_q300", [1500, 700], 300, 16, 2, 128, "e4m3", -1, 0, [0.4], 0),
]


def _shard_bounds(ctx, fracs):
    cuts = [0] + [int(round(f * ctx)) for f in fracs] + [ctx]
    return [(cuts[g], cuts[g + 1]) for g in range(len(cuts) - 1)]


def _build_shard(w, g, fracs, rng):
    """Cache holding shard g of every sequence: local key j = global key lo_b + j."""
    D, hkv = w.head_dim, w.num_kv_heads
    ranges = [_shard_bounds(int(c), fracs)[g] for c in w.ctx]
    lens = [hi - lo for lo, hi in ranges]
    pages_per = [max(1, -(-n // 16)) for n in lens]
    total = sum(pages_per) + 2
    perm = rng.permutation(total)
    bt = np.full((w.batch, max(pages_per)), W.INT32_MAX, np.int32)
    rows, slots = [], []
    at = 0
    for b, (lo, hi) in enumerate(ranges):
        bt[b, :pages_per[b]] = perm[at:at + pages_per[b]]
        at += pages_per[b]
        j = np.arange(hi - lo)
        slots.append(bt[b, j // 16].astype(np.int64) * 16 + j % 16)
        rows.append(w.seq_rows[b][lo:hi])
    rows = np.concatenate(rows)
    slots = np.concatenate(slots)
    kc = P.new_cache(total, hkv, D, w.kv_dtype, fill=w.cache_sentinel)
    vc = P.new_cache(total, hkv, D, w.kv_dtype, fill=w.cache_sentinel)
    ks = vs = None
    if w.kv_dtype == "int8_tok":
        ks, vs = P.new_scale_plane(total, hkv), P.new_scale_plane(total, hkv)
    if rows.size:
        P.kv_store(t_src(w.tokens_k[rows], w.src_dtype), t_src(w.tokens_v[rows], w.src_dtype),
                   torch.from_numpy(slots).cuda(), kc, vc, w.kv_dtype, w.k_scale, w.v_scale,
                   k_scales=ks, v_scales=vs)
    return dict(kc=kc, vc=vc, ks=ks, vs=vs, bt=torch.from_numpy(bt).cuda(), ranges=ranges,
                ctx=torch.tensor(lens, dtype=torch.int32, device="cuda"),
                kv0=torch.tensor([lo for lo, _ in ranges], dtype=torch.int32, device="cuda"),
                max_ctx=max(lens))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_context_parallel_shards(case):
    name, ctx, ql, hq, hkv, D, kv, win, sinks, fracs, S = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    w = W.build(name, 41, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                q_dtype="f16", pool_pages=pool, window_left=win, num_sinks=sinks, num_splits=S)
    rng = np.random.default_rng(7)
    q = t_src(w.q, w.q_dtype)
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    qpos0 = torch.from_numpy((w.ctx - w.q_len).astype(np.int32)).cuda()
    G = len(fracs) + 1
    parts_o, parts_l = [], []
    for g in range(G):
        sh = _build_shard(w, g, fracs, rng)
        common = dict(kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale,
                      max_q_len=w.max_q_len, min_q_len=int(w.q_len.min()), max_context_len=sh["max_ctx"],
                      window_left=win, num_sinks=sinks, num_splits=S, k_scales=sh["ks"], v_scales=sh["vs"],
                      kv_pos0=sh["kv0"], q_pos0=qpos0)
        out, lse = P.paged_attn(q, sh["kc"], sh["vc"], sh["bt"], sh["ctx"], qsl, **common)
        po, pl = P.paged_attn(q, sh["kc"], sh["vc"], sh["bt"], sh["ctx"], qsl, partials_only=True, **common)
        torch.cuda.synchronize()
        parts_o.append(po)
        parts_l.append(pl)
        out_np = out_to_np(out)
        lse_np = lse.cpu().numpy().astype(np.float64)
        for b in range(w.batch):
            q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
            lo, hi = sh["ranges"][b]
            k = dequant_tokens(w, w.seq_rows[b], "k")
            v = dequant_tokens(w, w.seq_rows[b], "v")
            ro, rl = OA.attention(q_f64(w, b), k, v, w.softmax_scale, win, sinks, key_lo=lo, key_hi=hi)
            compare(out_np[q0:q1], lse_np[q0:q1], ro, rl, f"{name} shard {g} seq {b} keys [{lo}, {hi})")
    # all shards' partials merged in one call = attention over the whole context
    po = torch.cat(parts_o, dim=0).contiguous()
    pl = torch.cat(parts_l, dim=0).contiguous()
    out, lse = P.lse_merge(po, pl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out_np = out_to_np(out)
    lse_np = lse.cpu().numpy().astype(np.float64)
    for b in range(w.batch):
        q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
        k = dequant_tokens(w, w.seq_rows[b], "k")
        v = dequant_tokens(w, w.seq_rows[b], "v")
        ro, rl = OA.attention(q_f64(w, b), k, v, w.softmax_scale, win, sinks)
        compare(out_np[q0:q1], lse_np[q0:q1], ro, rl, f"{name} merged seq {b}")
    log(f"{name}: {G} shards match the oracle per key range and merged")
