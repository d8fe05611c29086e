"""Helpers for the GPU parity tests: move a workload onto the device through
the library's store, and compute the oracle's answer for chosen rows."""
import sys
import time

import numpy as np
import torch

from oracle import attention as OA
from oracle import codecs as OC
from oracle import layout as OL

PAGE = 16
# tolerance for attention outputs (fp32 accumulation, fp16/bf16 outputs)
ATOL, RTOL = 2e-3, 1e-2
NORM_RTOL = 1e-2
LSE_ATOL = 1e-3


def log(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def t_src(x, dtype, device="cuda"):
    """host fp16 array or uint16 bf16 bits -> device tensor."""
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)


class DeviceWorkload:
    """A workload's caches filled through ra_kv_store, plus device metadata.

    fused_new=True leaves the step's query tokens out of the stores: attn()
    then stores them itself (the attention launch's fused store)."""

    def __init__(self, w, device="cuda", chunk_tokens=1 << 18, store=True, fused_new=False):
        import paged_quantized_kv_ra_amd as P
        self.w = w
        D, hkv = w.head_dim, w.num_kv_heads
        self.k_cache = P.new_cache(w.num_pages, hkv, D, w.kv_dtype, device, fill=w.cache_sentinel)
        self.v_cache = P.new_cache(w.num_pages, hkv, D, w.kv_dtype, device, fill=w.cache_sentinel)
        self.k_scales = self.v_scales = None
        if w.kv_dtype == "int8_tok":          # unwritten scales read as NaN
            self.k_scales = P.new_scale_plane(w.num_pages, hkv, device)
            self.v_scales = P.new_scale_plane(w.num_pages, hkv, device)
        self.fused = None
        rows = np.arange(w.tokens_k.shape[0])
        if fused_new:
            new_rows = w.new_token_rows()
            rows = np.setdiff1d(rows, new_rows)
            self.fused = dict(new_k=t_src(w.tokens_k[new_rows], w.src_dtype, device),
                              new_v=t_src(w.tokens_v[new_rows], w.src_dtype, device),
                              new_slots=torch.from_numpy(w.token_slots[new_rows]).to(device))
        if store:
            U = rows.size
            for lo in range(0, U, chunk_tokens):
                r = rows[lo:min(U, lo + chunk_tokens)]
                k = t_src(w.tokens_k[r], w.src_dtype, device)
                v = t_src(w.tokens_v[r], w.src_dtype, device)
                s = torch.from_numpy(w.token_slots[r]).to(device)
                P.kv_store(k, v, s, self.k_cache, self.v_cache, w.kv_dtype, w.k_scale, w.v_scale,
                           k_scales=self.k_scales, v_scales=self.v_scales)
        self.q = t_src(w.q, w.q_dtype, device)
        self.block_tables = torch.from_numpy(w.block_tables).to(device)
        self.context_lens = torch.from_numpy(w.ctx).to(device)
        self.qsl = torch.from_numpy(w.query_start_loc).to(device)

    def attn(self, num_splits=None, partials_only=False, **kw):
        import paged_quantized_kv_ra_amd as P
        w = self.w
        return P.paged_attn(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens, self.qsl,
                            kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale,
                            softmax_scale=w.softmax_scale, max_q_len=w.max_q_len,
                            min_q_len=int(w.q_len.min()), max_context_len=w.max_context_len,
                            window_left=w.window_left, num_sinks=w.num_sinks,
                            num_splits=w.num_splits if num_splits is None else num_splits,
                            partials_only=partials_only, k_scales=self.k_scales, v_scales=self.v_scales,
                            **(self.fused or {}), **kw)


def dequant_tokens(w, rows, which, heads=None):
    """Oracle: contiguous dequantised K or V (fp32) of the given token rows."""
    src = w.tokens_k if which == "k" else w.tokens_v
    scale = w.k_scale if which == "k" else w.v_scale
    x = src[rows] if heads is None else src[rows][:, heads]
    x32 = OC.source_to_f32(x, w.src_dtype)
    return OC.roundtrip(x32, w.kv_dtype, scale)


def q_f64(w, b):
    q0, q1 = int(w.query_start_loc[b]), int(w.query_start_loc[b + 1])
    return OC.source_to_f32(w.q[q0:q1], w.q_dtype).astype(np.float64)


def oracle_seq(w, b, kv_heads=None, q_rows=None):
    """Oracle (out, lse) of sequence b for the query heads of the given KV heads
    (and only the block's queries q_rows, each at its own position)."""
    hkv = w.num_kv_heads
    g = w.num_q_heads // hkv
    heads = list(range(hkv)) if kv_heads is None else list(kv_heads)
    rows = w.seq_rows[b]
    k = dequant_tokens(w, rows, "k", heads)
    v = dequant_tokens(w, rows, "v", heads)
    q = q_f64(w, b)
    pos = None
    if q_rows is not None:
        q_rows = np.asarray(q_rows, dtype=np.int64)
        q = q[q_rows]
        pos = int(w.ctx[b]) - int(w.q_len[b]) + q_rows
    qh = np.concatenate([q[:, h * g:(h + 1) * g] for h in heads], axis=1)
    return OA.attention(qh, k, v, w.softmax_scale, w.window_left, w.num_sinks, positions=pos)


def qhead_cols(w, kv_heads):
    g = w.num_q_heads // w.num_kv_heads
    return [h * g + j for h in kv_heads for j in range(g)]


def compare(out, lse, ref_out, ref_lse, what=""):
    """Elementwise atol + rtol*|r|, per-row normwise, and lse checks."""
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    err = np.abs(out - ref_out)
    tol = ATOL + RTOL * np.abs(ref_out)
    bad = err > tol
    assert not np.isnan(out).any(), f"{what}: NaN in output"
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance; max err {err.max():.3e}, "
                           f"worst at {np.unravel_index(np.argmax(err - tol), err.shape)}")
    num = np.linalg.norm((out - ref_out).reshape(-1, out.shape[-1]), axis=1)
    den = np.linalg.norm(ref_out.reshape(-1, out.shape[-1]), axis=1)
    live = den > 0
    rel = num[live] / den[live]
    assert (rel <= NORM_RTOL).all(), f"{what}: normwise rel err {rel.max():.3e}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
    lerr = np.abs(lse[fin] - ref_lse[fin]) if fin.any() else np.zeros(1)
    assert (lerr <= LSE_ATOL).all(), f"{what}: lse max err {lerr.max():.3e}"
    return float(err.max()), float(rel.max()) if rel.size else 0.0, float(lerr.max())


def out_to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log(f"{self.what}: {time.time() - self.t:.1f}s")
