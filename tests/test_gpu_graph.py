"""The whole step (store of the new K/V rows, attention partials, LSE merge)
captured into a HIP graph replays to the eager result.

Every replay is preceded by eager work of the program's own (clearing the
outputs, an unrelated kernel) and a synchronisation, and each replay's outputs
are compared bit for bit with the eager launch of the same step.
"""
import pytest
import torch

import paged_quantized_kv_ra_amd as P
from paged_quantized_kv_ra_amd import workloads as W

from gpu_util import DeviceWorkload, log, t_src

pytestmark = pytest.mark.gpu

CASES = [
    ("dec_g8_e4m3_split3", [1000, 77, 513], 1, 16, 2, 128, "e4m3", "f16", -1, 0, 3),
    ("mfma_g8_q5_int8_auto_bf16", [1000, 77, 5000], 5, 16, 2, 128, "int8", "bf16", -1, 0, 0),
    ("mixed_window_sinks", [500, 400, 300], [1, 5, 16], 16, 2, 128, "e4m3", "f16", 100, 4, 2),
]


def _build(case, seed=33):
    name, ctx, ql, hq, hkv, D, kv, qd, win, sinks, S = case
    pool = int(sum(-(-c // 16) for c in ctx) * 1.25) + 3
    return W.build(name, seed, ctx=ctx, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                   q_dtype=qd, pool_pages=pool, window_left=win, num_sinks=sinks, num_splits=S)


class StepBuffers:
    def __init__(self, w, dw):
        self.w, self.dw = w, dw
        rows = w.new_token_rows()
        self.k_new = t_src(w.tokens_k[rows], w.src_dtype)
        self.v_new = t_src(w.tokens_v[rows], w.src_dtype)
        self.slots = torch.from_numpy(w.token_slots[rows]).cuda()
        T, hq, D = dw.q.shape
        a = P._lib._attn_args(dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, dw.qsl,
                              w.kv_dtype, w.k_scale, w.v_scale, w.softmax_scale, w.max_q_len,
                              int(w.q_len.min()), w.max_context_len, w.window_left, w.num_sinks, w.num_splits,
                              w.num_kv_heads)
        S, _, _ = P._lib.paged_attn_workspace(a)
        self.po = torch.empty((S, T, hq, D), dtype=torch.float32, device="cuda")
        self.pl = torch.empty((S, T, hq), dtype=torch.float32, device="cuda")
        self.out = torch.empty_like(dw.q)
        self.lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")

    def run(self, stream):
        w, dw = self.w, self.dw
        P.kv_store(self.k_new, self.v_new, self.slots, dw.k_cache, dw.v_cache, w.kv_dtype, w.k_scale, w.v_scale,
                   stream=stream)
        dw.attn(partials_only=True, workspace=(self.po, self.pl), stream=stream)
        P.lse_merge(self.po, self.pl, out_dtype=dw.q.dtype, out=self.out, lse=self.lse, stream=stream)


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.float16, torch.bfloat16) else t.view(torch.int32)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(case):
    w = _build(case)
    dw = DeviceWorkload(w)
    sb = StepBuffers(w, dw)
    sb.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_out, ref_lse = sb.out.clone(), sb.lse.clone()
    ref_k, ref_v = dw.k_cache.clone(), dw.v_cache.clone()
    assert torch.isfinite(ref_lse).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sb.run(side)                 # one eager launch on the capture stream before capturing
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        sb.run(torch.cuda.current_stream())
    torch.cuda.synchronize()

    x = torch.arange(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(4):
        sb.out.fill_(float("nan"))
        sb.lse.fill_(float("nan"))
        sb.po.zero_()
        y = (x * (rep + 1)).sum()       # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(y) > 0
        assert torch.equal(_bits(sb.out), _bits(ref_out)), f"replay {rep}: output differs"
        assert torch.equal(_bits(sb.lse), _bits(ref_lse)), f"replay {rep}: lse differs"
        assert torch.equal(dw.k_cache, ref_k) and torch.equal(dw.v_cache, ref_v), f"replay {rep}: cache changed"
    log(f"{case[0]}: 4 graph replays bitwise equal to the eager step")
    del g
