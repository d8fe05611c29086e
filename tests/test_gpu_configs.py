"""GPU parity on the benchmark workloads at full size, in the launch
configuration bench.py times.

Store: bit-exact on 4096 random tokens plus every token the step itself
stores (their bytes in the GPU caches against the oracle's codes at the
layout's offsets) and the untouched sentinel of an unused page.  Attention:
every output of every (sequence, KV head) unit against the fp64 oracle,
computed one unit at a time; the prefill workloads, whose blocks hold
thousands of queries, compare sampled query rows of every unit.  As in
bench.py, decode and verify workloads (at most 48 rows per KV head) store
the step's own tokens inside the attention launch.
"""
import numpy as np
import pytest
import torch

from oracle import codecs as OC
from oracle import layout as OL
from paged_quantized_kv_ra_amd import workloads as W
from tests.gpu_util import DeviceWorkload, Timer, compare, log, oracle_seq, out_to_np, qhead_cols

pytestmark = pytest.mark.gpu

# workload factory; "all": every (sequence, KV head) unit with all its
# queries; "sample": every unit with sampled query rows (row-group edges, the
# first and last queries, random ones)
CONFIGS = [
    ("tiny_decode", W.tiny_decode, "all"),
    ("batch8_decode", W.batch8_decode, "all"),
    ("verify_fp8_32k", W.verify_fp8_32k, "all"),
    ("prefix_int8_256k", W.prefix_int8_256k, "all"),
    ("split_fp8_512k", W.split_fp8_512k, "all"),
    # beyond the five: plain decode at 32K, and per-token INT8 at the verify shape
    ("decode_fp8_32k", W.decode_fp8_32k, "all"),
    ("verify_int8tok_32k", W.verify_int8tok_32k, "all"),
    ("prefill_fp8_8k", W.prefill_fp8_8k, "sample"),
    ("chunk_prefill_fp8_128k", W.chunk_prefill_fp8_128k, "sample"),
]
STORE_SAMPLE = 4096


def _query_sample(w, b, seed):
    """Query rows of sequence b: the first and last, both sides of several
    48-row group edges (6 queries of 8 heads each), and random ones."""
    ql = int(w.q_len[b])
    g = w.num_q_heads // w.num_kv_heads
    per_group = 48 // g if 48 % g == 0 else 1
    edges = [e for k in (1, 2, ql // per_group // 2, ql // per_group - 1) for e in (k * per_group - 1, k * per_group)]
    rng = np.random.default_rng(seed)
    rows = np.concatenate([[0, ql - 1], edges, rng.integers(0, ql, size=24)])
    return np.unique(np.clip(rows, 0, ql - 1))


def _check_store_sample(w, dw, n=STORE_SAMPLE, seed=0, extra_rows=None):
    rng = np.random.default_rng(seed)
    rows = rng.choice(w.tokens_k.shape[0], size=min(n, w.tokens_k.shape[0]), replace=False)
    if extra_rows is not None:
        rows = np.unique(np.concatenate([rows, extra_rows]))
    slots = w.token_slots[rows]
    pages = np.unique(slots // 16)
    e = 2 if w.kv_dtype == "f16" else 1
    for which, cache, scale in (("k", dw.k_cache, w.k_scale), ("v", dw.v_cache, w.v_scale)):
        sel = cache[torch.from_numpy(pages).cuda()].contiguous().view(torch.uint8).cpu().numpy().reshape(-1)
        local = np.searchsorted(pages, slots // 16) * 16 + slots % 16
        got = OL.gather(sel, local, which, w.num_kv_heads, w.head_dim, w.kv_dtype)
        src = w.tokens_k[rows] if which == "k" else w.tokens_v[rows]
        if w.kv_dtype == "int8_tok":
            want, want_sc = OC.quantize_per_token(OC.source_to_f32(src, w.src_dtype))
            plane = (dw.k_scales if which == "k" else dw.v_scales).cpu().numpy().reshape(-1)
            got_sc = OL.gather_scales(plane, slots, w.num_kv_heads)
            assert np.array_equal(got_sc.view(np.uint32), want_sc.view(np.uint32)), f"{w.name} {which} scales differ"
        else:
            want = OC.quantize(OC.source_to_f32(src, w.src_dtype), w.kv_dtype, scale)
        assert np.array_equal(np.ascontiguousarray(got).view(np.uint8),
                              np.ascontiguousarray(want).view(np.uint8)), f"{w.name} {which} store differs"
    used = set(np.unique(w.token_slots // 16).tolist())
    unused = [p for p in range(w.num_pages) if p not in used][:1]
    for p in unused:
        blk = dw.k_cache[p].contiguous().view(torch.uint8).cpu().numpy().reshape(-1)
        if w.kv_dtype == "f16":
            assert np.all(blk.view(np.uint16) == w.cache_sentinel)
        else:
            assert np.all(blk == w.cache_sentinel)


def _run(name, make, mode, base=None):
    with Timer(f"{name}: build"):
        w = make() if base is None else make(base)
    fused = (w.num_q_heads // w.num_kv_heads) * w.max_q_len <= 48
    with Timer(f"{name}: upload + store"):
        dw = DeviceWorkload(w, fused_new=fused)
        torch.cuda.synchronize()
    with Timer(f"{name}: attention{' with the fused store' if fused else ''}"):
        out, lse = dw.attn()
        torch.cuda.synchronize()
    with Timer(f"{name}: store check ({STORE_SAMPLE} random tokens + the step's own)"):
        _check_store_sample(w, dw, extra_rows=w.new_token_rows())
    out = out_to_np(out)
    lse = lse.cpu().numpy().astype(np.float64)
    worst = (0.0, 0.0, 0.0)
    with Timer(f"{name}: oracle over {w.batch} x {w.num_kv_heads} units"):
        for b in range(w.batch):
            q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
            for h in range(w.num_kv_heads):
                cols = qhead_cols(w, [h])
                sample = mode == "sample"
                q_rows = _query_sample(w, b, seed=h) if sample else np.arange(q1 - q0)
                ro, rl = oracle_seq(w, b, kv_heads=[h], q_rows=q_rows if sample else None)
                e = compare(out[q0:q1][q_rows][:, cols], lse[q0:q1][q_rows][:, cols], ro, rl,
                            f"{name} seq {b} head {h}")
                worst = tuple(max(x, y) for x, y in zip(worst, e))
    log(f"{name}: every unit within tolerance; worst max abs {worst[0]:.2e} normwise {worst[1]:.2e} "
        f"lse {worst[2]:.2e}")
    assert np.isfinite(out).all()
    return w


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_benchmark_workload(cfg):
    name, make, mode = cfg
    _run(name, make, mode)


@pytest.mark.timeout(900)
def test_sliding_window_workload():
    base = W.split_fp8_512k()
    _run("split_fp8_512k_sliding", W.split_fp8_512k_sliding, "all", base=base)
    _run("split_fp8_512k_sliding_auto", W.split_fp8_512k_sliding_auto, "all", base=base)
