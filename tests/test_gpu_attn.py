"""GPU parity of ra_paged_attn / ra_lse_merge against the fp64 oracle, at
small sizes that span several page pairs, partitions and a ragged tail, plus
batch-invariance and determinism checks."""
import numpy as np
import pytest
import torch

import paged_quantized_kv_ra_amd as P
from oracle import attention as OA
from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import (DeviceWorkload, compare, log, oracle_seq, out_to_np, q_f64, dequant_tokens)

pytestmark = pytest.mark.gpu

# name, ctx, q_len, Hq, Hkv, D, kv, q dtype, window, sinks, num_splits
CASES = [
    ("dec_g4_d64_f16", [37, 300, 16, 1, 257], 1, 4, 1, 64, "f16", "f16", -1, 0, 1),
    ("dec_g8_f16_bf16q_auto", [1000, 77, 513, 2100], 1, 16, 2, 128, "f16", "bf16", -1, 0, 0),
    ("dec_g8_e4m3", [1000, 77, 513], 1, 16, 2, 128, "e4m3", "f16", -1, 0, 1),
    ("dec_g8_int8_split3", [1000, 77, 513], 1, 16, 2, 128, "int8", "f16", -1, 0, 3),
    ("dec_g1_q2_d64_e4m3", [200, 31, 2], 2, 2, 2, 64, "e4m3", "f16", -1, 0, 1),
    ("dec_g4_q3_int8_rowgroups", [150, 64], 3, 8, 2, 128, "int8", "bf16", -1, 0, 2),
    ("dec_g8_window_sinks", [900, 120], 1, 16, 2, 128, "e4m3", "f16", 100, 4, 0),
    ("mfma_g8_q5_e4m3", [1000, 77, 513, 5, 4097], 5, 16, 2, 128, "e4m3", "f16", -1, 0, 1),
    ("mfma_g8_q5_e4m3_auto", [1000, 77, 513, 5, 4097], 5, 16, 2, 128, "e4m3", "f16", -1, 0, 0),
    ("mfma_g8_q5_int8_split7", [1000, 77, 513, 40], 5, 16, 2, 128, "int8", "f16", -1, 0, 7),
    ("mfma_g8_q5_f16", [700, 33, 100], 5, 16, 2, 128, "f16", "f16", -1, 0, 1),
    ("mfma_g8_q5_bf16q", [700, 33, 100], 5, 16, 2, 128, "e4m3", "bf16", -1, 0, 2),
    ("mfma_g16_q1_d64_f16", [300, 17], 1, 16, 1, 64, "f16", "f16", -1, 0, 1),
    ("mfma_g8_q3_d64_int8", [300, 47, 1000], 3, 16, 2, 64, "int8", "f16", -1, 0, 0),
    ("mfma_g8_q16_window", [1000, 300, 17], 16, 16, 2, 128, "e4m3", "f16", 100, 4, 4),
    ("mfma_g8_q16_window_nosink", [1000, 600], 16, 16, 2, 128, "e4m3", "f16", 33, 0, 1),
    ("mfma_g6_q4_d128_f16", [129, 400], 4, 12, 2, 128, "f16", "f16", -1, 0, 3),
    ("mixed_paths", [500, 400, 300, 64], [1, 5, 2, 16], 16, 2, 128, "e4m3", "f16", -1, 0, 0),
    # window edges that fall inside pages for the later queries of the block
    ("mfma_g8_q16_window37_direct", [1000, 333, 70], 16, 16, 2, 128, "e4m3", "f16", 37, 0, 1),
    ("mfma_g8_q7_window100_sink20", [1000, 517], 7, 16, 2, 128, "int8", "f16", 100, 20, 1),
    ("mfma_g8_q5_window250_auto", [3000, 260], 5, 16, 2, 128, "f16", "f16", 250, 4, 0),
    ("dec_g4_q3_window45", [700, 90], 3, 8, 2, 128, "e4m3", "f16", 45, 2, 1),
    # decode auto partitions around their rule's bends: 512 tokens up to 16K,
    # ~32 partitions up to 64K, 2048 tokens beyond
    ("dec_g8_e4m3_auto_bends", [16384, 16400, 65536, 65552, 100000, 511], 1, 16, 2, 128, "e4m3", "f16", -1, 0, 0),
    # INT8 with runtime scales per token and head
    ("mfma_g8_q5_int8tok", [1000, 77, 513, 40], 5, 16, 2, 128, "int8_tok", "f16", -1, 0, 3),
    ("dec_g8_int8tok_auto", [3000, 77, 513], 1, 16, 2, 128, "int8_tok", "bf16", -1, 0, 0),
    ("mfma_g8_q16_int8tok_window_d64", [900, 300], 16, 16, 2, 64, "int8_tok", "f16", 100, 4, 2),
    # prefill: long query blocks over many row groups (cold prompts with
    # q_len = ctx, and chunks after a cached prefix), causal page skipping
    ("pre_g8_e4m3_cold", [700, 300, 33], [700, 300, 33], 16, 2, 128, "e4m3", "f16", -1, 0, 0),
    ("pre_g8_int8_chunk_auto_bf16q", [3000, 1500], [600, 250], 16, 2, 128, "int8", "bf16", -1, 0, 0),
    ("pre_g8_e4m3_chunk_split5", [2000, 999], [400, 999], 16, 2, 128, "e4m3", "f16", -1, 0, 5),
    ("pre_g8_e4m3_window_sinks", [1500, 400], [500, 400], 16, 2, 128, "e4m3", "f16", 128, 4, 0),
    ("pre_g4_int8tok_d64", [640, 333], [640, 100], 8, 2, 64, "int8_tok", "f16", -1, 0, 0),
    ("pre_g1_f16_direct", [500, 129], [500, 129], 4, 4, 128, "f16", "f16", -1, 0, 1),
    ("mixed_decode_prefill", [900, 1200, 64], [1, 300, 64], 16, 2, 128, "e4m3", "f16", -1, 0, 0),
]


def _build(case, seed=21):
    name, ctx, ql, hq, hkv, D, kv, qd, win, sinks, S = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    return W.build(name, seed, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                   q_dtype=qd, pool_pages=pool, window_left=win, num_sinks=sinks, num_splits=S)


def _check_all(w, out, lse, what):
    out = out_to_np(out)
    lse = lse.cpu().numpy().astype(np.float64)
    worst = (0.0, 0.0, 0.0)
    for b in range(w.batch):
        q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
        ro, rl = oracle_seq(w, b)
        e = compare(out[q0:q1], lse[q0:q1], ro, rl, f"{what} seq {b}")
        worst = tuple(max(x, y) for x, y in zip(worst, e))
    log(f"{what}: max abs err {worst[0]:.2e}, normwise {worst[1]:.2e}, lse {worst[2]:.2e}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_matches_oracle(case):
    w = _build(case)
    dw = DeviceWorkload(w)
    out, lse = dw.attn()
    torch.cuda.synchronize()
    _check_all(w, out, lse, case[0])


@pytest.mark.parametrize("case", [c for c in CASES if c[-1] > 1], ids=[c[0] for c in CASES if c[-1] > 1])
def test_partials_match_oracle_split(case):
    """With an explicit split count the partials themselves are the oracle's
    per-partition (out, lse); empty partitions are (0, -inf)."""
    w = _build(case)
    dw = DeviceWorkload(w)
    po, pl = dw.attn(partials_only=True)
    torch.cuda.synchronize()
    po = po.cpu().numpy().astype(np.float64)
    pl = pl.cpu().numpy().astype(np.float64)
    g = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
        rows = w.seq_rows[b]
        k = dequant_tokens(w, rows, "k")
        v = dequant_tokens(w, rows, "v")
        ro, rl = OA.split_attention(q_f64(w, b), k, v, w.softmax_scale, w.window_left, w.num_sinks,
                                    num_splits=w.num_splits)
        for s in range(w.num_splits):
            empty = ~np.isfinite(rl[s])
            assert np.all(pl[s, q0:q1][empty] == -np.inf), (b, s)
            assert np.all(po[s, q0:q1][empty] == 0.0), (b, s)
            if (~empty).any():
                compare(po[s, q0:q1][~empty], pl[s, q0:q1][~empty], ro[s][~empty], rl[s][~empty],
                        f"{case[0]} seq {b} part {s}")


def test_merge_matches_oracle():
    rng = np.random.default_rng(8)
    for S, D, rows in [(1, 128, 7), (5, 64, 33), (64, 128, 160), (100, 128, 9)]:
        po = rng.standard_normal((S, rows, D)).astype(np.float32)
        pl = (rng.standard_normal((S, rows)) * 3).astype(np.float32)
        pl[rng.random((S, rows)) < 0.2] = -np.inf
        pl[:, 0] = -np.inf                            # an all-empty row
        po_t = torch.from_numpy(po).cuda()
        pl_t = torch.from_numpy(pl).cuda()
        for dt in (torch.float32, torch.float16, torch.bfloat16):
            out, lse = P.lse_merge(po_t, pl_t, out_dtype=dt)
            torch.cuda.synchronize()
            ro, rl = OA.lse_merge(po, pl)
            o = out.float().cpu().numpy().astype(np.float64)
            tol = 1e-6 if dt == torch.float32 else (2e-3 if dt == torch.float16 else 1e-2)
            assert np.all(np.abs(o - ro) <= tol * (1 + np.abs(ro))), (S, D, dt)
            l = lse.cpu().numpy()
            assert np.array_equal(np.isfinite(l), np.isfinite(rl))
            f = np.isfinite(rl)
            assert np.all(np.abs(l[f] - rl[f]) <= 1e-5 * (1 + np.abs(rl[f])))
            assert np.all(o[0] == 0)


def test_merge_nan_partial_poisons_row():
    po = torch.zeros((3, 2, 64), dtype=torch.float32).cuda()
    pl = torch.tensor([[0.0, 0.0], [float("nan"), 1.0], [2.0, -float("inf")]]).cuda()
    out, lse = P.lse_merge(po, pl)
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.isnan(lse[0])
    assert torch.isfinite(out[1]).all() and torch.isfinite(lse[1])


def _single(w, b):
    """Sequence b of w as a one-sequence workload over the same device caches."""
    q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
    return q0, q1


@pytest.mark.parametrize("case", [CASES[1], CASES[8], CASES[14], CASES[17], CASES[22], CASES[24], CASES[27],
                                  CASES[32]], ids=lambda c: c[0])
def test_batch_invariance_bitwise(case):
    """A sequence's result does not depend on the rest of the batch (other
    lengths change the automatic split count, and mixing decode with verify
    blocks changes the row tiles of the launch)."""
    w = _build(case)
    dw = DeviceWorkload(w)
    out, lse = dw.attn()
    for b in range(w.batch):
        q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
        ql = q1 - q0
        o1, l1 = P.paged_attn(dw.q[q0:q1].contiguous(), dw.k_cache, dw.v_cache, dw.block_tables[b:b + 1].contiguous(),
                              dw.context_lens[b:b + 1].contiguous(),
                              torch.tensor([0, ql], dtype=torch.int32, device="cuda"),
                              kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale,
                              softmax_scale=w.softmax_scale, max_q_len=ql, min_q_len=ql,
                              max_context_len=int(w.ctx[b]), window_left=w.window_left,
                              num_sinks=w.num_sinks, num_splits=w.num_splits,
                              k_scales=dw.k_scales, v_scales=dw.v_scales)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), out[q0:q1].view(torch.int16)), (case[0], b)
        assert torch.equal(l1.view(torch.int32), lse[q0:q1].view(torch.int32)), (case[0], b)


@pytest.mark.parametrize("case", [CASES[2], CASES[7], CASES[15]], ids=lambda c: c[0])
def test_physical_page_placement_is_invisible(case):
    """Same logical KV at different physical pages (another page permutation
    and a larger pool): bitwise equal results."""
    w = _build(case)
    dw = DeviceWorkload(w)
    out, lse = dw.attn()
    w2 = _build(case)
    rng = np.random.default_rng(99)
    n2 = w.num_pages * 2
    remap = rng.permutation(n2)[:w.num_pages]
    bt = w.block_tables.astype(np.int64)
    live = bt != W.INT32_MAX
    bt[live] = remap[bt[live]]
    w2.block_tables = bt.astype(np.int32)
    w2.token_slots = remap[w.token_slots // 16] * 16 + w.token_slots % 16
    w2.num_pages = n2
    dw2 = DeviceWorkload(w2)
    out2, lse2 = dw2.attn()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


def test_self_repeat_bitwise():
    w = _build(CASES[8])
    dw = DeviceWorkload(w)
    ref = [t.clone() for t in dw.attn()]
    for _ in range(5):
        out, lse = dw.attn()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32))


def test_split_counts_agree():
    """Direct (one slot) vs 2, 5, 64 and automatic partitions: all within the
    oracle tolerance of each other."""
    w = _build(("split_sweep", [3000, 1200], 5, 16, 2, 128, "e4m3", "f16", -1, 0, 1))
    dw = DeviceWorkload(w)
    base, base_lse = dw.attn(num_splits=1)
    for S in (2, 5, 64, 0):
        o, l = dw.attn(num_splits=S)
        torch.cuda.synchronize()
        d = (o.float() - base.float()).abs().max().item()
        assert d < 2e-3, (S, d)
        assert (l - base_lse).abs().max().item() < 1e-4


def test_bad_block_table_entry_gives_nan_rows_only():
    w = _build(CASES[7])
    dw = DeviceWorkload(w)
    bt = dw.block_tables.clone()
    bt[1, 2] = w.num_pages + 5            # sequence 1 (ctx 77) reads page 2
    dw.block_tables = bt
    out, lse = dw.attn()
    torch.cuda.synchronize()
    q0, q1 = int(w.query_start_loc[1]), int(w.query_start_loc[2])
    assert torch.isnan(out[q0:q1]).all() and torch.isnan(lse[q0:q1]).all()
    others = torch.ones(out.shape[0], dtype=torch.bool)
    others[q0:q1] = False
    assert torch.isfinite(out[others.cuda()]).all()


def test_context_shorter_than_block_is_nan_not_fault():
    w = _build(CASES[7])
    dw = DeviceWorkload(w)
    ctx = dw.context_lens.clone()
    ctx[3] = 2                              # q_len 5 > ctx 2 breaks the precondition
    dw.context_lens = ctx
    out, lse = dw.attn()
    torch.cuda.synchronize()
    q0, q1 = int(w.query_start_loc[3]), int(w.query_start_loc[4])
    assert torch.isnan(out[q0:q1]).all()
    assert torch.isfinite(out[:q0]).all()


# Per-token INT8 keeps its precision whatever the magnitude of V: the V
# scales ride on the fp16 probabilities relative to a power-of-two reference,
# so p * vs stays in fp16's normal range for small V, and a reference that
# moves up as larger scales arrive rescales what was accumulated exactly.
# The elementwise bound is dominated by its absolute term at these output
# magnitudes; the per-row normwise bound (1e-2) is what these cases test.  The
# queries, and so the outputs, are bf16: outputs near 1e-7 are subnormal in
# fp16 and would carry the output format's rounding, not the kernel's.
def _int8tok_vstd(kind, U):
    if kind == "growing":      # 2^-20 .. 1 along the unique token rows: the reference moves many times
        return np.exp2(np.linspace(-20.0, 0.0, U)).astype(np.float32)
    if kind == "shrinking":    # 1 .. 2^-20: later tokens far below the reference
        return np.exp2(np.linspace(0.0, -20.0, U)).astype(np.float32)
    return float(kind)


@pytest.mark.parametrize("kind", ["1e-2", "1e-3", "1e-4", "growing", "shrinking"])
@pytest.mark.parametrize("ql,S", [(5, 0), (1, 3), (16, 1)], ids=["verify_auto", "decode_split3", "q16_direct"])
def test_int8tok_precision_independent_of_v_magnitude(kind, ql, S):
    ctx = [3000, 700, 77]
    U = sum(ctx)
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    w = W.build(f"int8tok_v{kind}", 23, ctx=ctx, q_len=ql, num_q_heads=16, num_kv_heads=2, head_dim=128,
                kv_dtype="int8_tok", q_dtype="bf16", pool_pages=pool, num_splits=S,
                v_std=_int8tok_vstd(kind, U))
    dw = DeviceWorkload(w)
    out, lse = dw.attn()
    torch.cuda.synchronize()
    _check_all(w, out, lse, f"int8tok V {kind} q_len {ql} S {S}")


# Every shape of the cross-wave merge: per KV format and head_dim, one, two and
# three row tiles (8, 24 and 40 rows per KV head), written directly (one
# partition: out and lse in the query dtype) or as partials merged afterwards.
# The merge passes differ between these shapes (one pass in the rings, one pass
# with slabs past the rings, two passes), and so do the chunk layouts.
MERGE_CASES = [
    (f"merge_{kv}_d{D}_q{ql}_S{S}_{qd}", [700, 333], [ql, ql], 16, 2, D, kv, qd, -1, 0, S)
    for kv in ["f16", "e4m3", "int8", "int8_tok"]
    for D in [64, 128]
    for ql in [1, 3, 5]
    for S, qd in [(1, "bf16"), (3, "f16")]
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_merge_shapes_match_oracle(case):
    w = _build(case, seed=31)
    dw = DeviceWorkload(w)
    out, lse = dw.attn()
    torch.cuda.synchronize()
    _check_all(w, out, lse, case[0])
