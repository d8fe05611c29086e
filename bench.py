#!/usr/bin/env python3
"""Benchmark of one decode/verify step of paged, quantized-KV attention on one MI355X.

A step is the whole hot path over one batch: the store of the step's new K/V
rows (the 1 + 4 verify tokens of every sequence), ra_paged_attn over the
paged cache (partials per KV partition) and ra_lse_merge.  Decode and verify
blocks store their new tokens inside the attention launch (the fused store of
ra_attn_args); prefill blocks, and --separate-store, use a ra_kv_store launch
first.  Inputs are seeded
synthetic data already resident in HBM.  Each step uses the next of L
identical copies of the KV pool (at least 1 GiB in total), the way successive
layers of a model read distinct caches, so the 256 MB Infinity Cache cannot
serve repeated reads.

Output: one JSON line.  `value` is KV tokens attended per second over the
timed steps; `roofline` is the attention kernel's algorithmic HBM bytes per
launch over its average duration (HIP events on the launch stream);
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same step.
Prefill workloads (whole prompts or prompt chunks as the query block) report
query tokens per second instead, and an MFMA roofline in TFLOP/s (4 * D
flops per visible (query head, key) pair); with one partition slot the
attention writes its output directly and there is no merge.
``--fused-qkv`` takes the new tokens from packed QKV rows with RoPE: for
decode and verify blocks the attention launch rotates Q and K and stores K/V
itself; prefill blocks use ra_qkv_rope_store (which also writes the rotated
Q) first.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--fused-qkv] [--gpus 1]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0      # dense fp16 matrix-core peak (the path's MFMA dtype)
POOL_ROTATION_BYTES = 1 << 30
KERNEL_SOURCES = ["paged_quantized_kv_ra_amd/csrc/attn_mfma.hip", "paged_quantized_kv_ra_amd/csrc/attn_prefill.hip",
                  "paged_quantized_kv_ra_amd/csrc/attn_common.h", "paged_quantized_kv_ra_amd/csrc/ra_device.h",
                  "paged_quantized_kv_ra_amd/csrc/ra_internal.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="verify_fp8_32k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-qkv", action="store_true",
                    help="store the new tokens with ra_qkv_rope_store (packed QKV rows, RoPE with YaRN "
                         "factor 2, Q written for attention) instead of ra_kv_store")
    ap.add_argument("--separate-store", action="store_true",
                    help="store the new tokens with a ra_kv_store launch before the attention instead of the "
                         "attention launch's fused store")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from the host instead of replaying captured HIP graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (for counter scaling)")
    return ap.parse_args()


def copy_calibration():
    """A plain 1 GiB device-to-device copy, for scaling HBM byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {n} bytes x3")


class Step:
    """Device state and prebuilt C-ABI argument blocks for one workload."""

    def __init__(self, w, fused_qkv=False, separate_store=False):
        import torch
        import paged_quantized_kv_ra_amd as P
        from paged_quantized_kv_ra_amd import _lib as L
        self.w, self.L, self.P = w, L, P
        self.lib = L.load_library()
        dev = "cuda"
        D, hkv = w.head_dim, w.num_kv_heads
        # one pool filled through the store, then cloned
        k0 = P.new_cache(w.num_pages, hkv, D, w.kv_dtype, dev, fill=w.cache_sentinel)
        v0 = P.new_cache(w.num_pages, hkv, D, w.kv_dtype, dev, fill=w.cache_sentinel)
        ks0 = vs0 = None
        if w.kv_dtype == "int8_tok":      # per-token scale planes beside the caches
            ks0 = P.new_scale_plane(w.num_pages, hkv, dev)
            vs0 = P.new_scale_plane(w.num_pages, hkv, dev)
        U = w.tokens_k.shape[0]
        chunk = 1 << 18
        for lo in range(0, U, chunk):
            hi = min(U, lo + chunk)
            P.kv_store(self._src(w.tokens_k[lo:hi]), self._src(w.tokens_v[lo:hi]),
                       torch.from_numpy(w.token_slots[lo:hi]).to(dev), k0, v0, w.kv_dtype, w.k_scale, w.v_scale,
                       k_scales=ks0, v_scales=vs0)
        pool_bytes = 2 * k0.numel() * k0.element_size() + (2 * ks0.numel() * 4 if ks0 is not None else 0)
        self.copies = max(1, -(-POOL_ROTATION_BYTES // pool_bytes))
        clone = (lambda t: None if t is None else t.clone())
        self.pools = [(k0, v0, ks0, vs0)] + [(k0.clone(), v0.clone(), clone(ks0), clone(vs0))
                                             for _ in range(self.copies - 1)]
        torch.cuda.synchronize()
        # this step's new tokens: the last q_len positions of every sequence
        rows = w.new_token_rows()
        self.k_new = self._src(w.tokens_k[rows])
        self.v_new = self._src(w.tokens_v[rows])
        self.slots_new = torch.from_numpy(w.token_slots[rows]).to(dev)
        self.q = self._src(w.q) if w.q_dtype == "f16" else self._src_bf16(w.q)
        self.bt = torch.from_numpy(w.block_tables).to(dev)
        self.ctx = torch.from_numpy(w.ctx).to(dev)
        self.qsl = torch.from_numpy(w.query_start_loc).to(dev)
        T, hq = self.q.shape[0], self.q.shape[1]
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((T, hq), dtype=torch.float32, device=dev)
        # decode and verify blocks (at most 48 rows per KV head) store their new
        # tokens inside the attention launch (with --fused-qkv also rotating Q
        # and K by RoPE there); prefill blocks and --separate-store store them
        # with a launch of their own first
        g = w.num_q_heads // hkv
        in_launch = not separate_store and g * w.max_q_len <= 48
        if fused_qkv:
            self.store_mode = "fused_rope" if in_launch else "qkv_rope_store"
        else:
            self.store_mode = "fused" if in_launch else "kv_store"
        if fused_qkv:
            # packed QKV rows of the new tokens (fp16), their positions, and
            # the library's YaRN table (factor 2 over half the positions used)
            from paged_quantized_kv_ra_amd import workloads as W
            assert w.q_dtype == "f16" and self.k_new.shape[0] == T
            pos, _ = W.step_positions_and_slots(w)
            self.qkv = self._src(W.packed_qkv(w.seed, T, hq, hkv, D, "f16"))
            self.positions = torch.from_numpy(pos).to(dev)
            max_pos = int(pos.max()) + 1
            self.table = P.rope_table(max_pos, D, 1e6, 2.0, max(1, max_pos // 2), device=dev)
        q_in, k_in, v_in, rope = self.q, self.k_new, self.v_new, {}
        if self.store_mode == "fused_rope":   # Q, K and V straight from the packed rows
            q_in = self.qkv[:, :hq * D].view(T, hq, D)
            k_in = self.qkv[:, hq * D:(hq + hkv) * D].view(T, hkv, D)
            v_in = self.qkv[:, (hq + hkv) * D:].view(T, hkv, D)
            rope = dict(rope_table=self.table, positions=self.positions, rotary_dim=D)
        fused = self.store_mode in ("fused", "fused_rope")
        self.args = []
        for k, v, ks, vs in self.pools:
            a = L._attn_args(q_in, k, v, self.bt, self.ctx, self.qsl, w.kv_dtype, w.k_scale, w.v_scale,
                             w.softmax_scale, w.max_q_len, int(w.q_len.min()), w.max_context_len,
                             w.window_left, w.num_sinks, w.num_splits, hkv, ks, vs,
                             new_k=k_in if fused else None, new_v=v_in if fused else None,
                             new_slots=self.slots_new if fused else None, **rope)
            self.args.append(a)
        self.slots, po_n, _ = L.paged_attn_workspace(self.args[0])
        # one partition slot (a long prefill chunk): the kernel writes out and
        # lse itself and there is nothing to merge; otherwise partials only,
        # and the merge is launched separately
        self.direct = self.slots == 1
        self.po = torch.empty((self.slots, T, hq, D), dtype=torch.float32, device=dev)
        self.pl = torch.empty((self.slots, T, hq), dtype=torch.float32, device=dev)
        for a in self.args:
            if self.direct:
                a.out = self.out.data_ptr()
                a.lse = self.lse.data_ptr()
            else:
                a.partial_out = self.po.data_ptr()
                a.partial_lse = self.pl.data_ptr()
                a.partial_slots = self.slots
        self.rows = T * hq
        self.q_code = L.RA_F16 if w.q_dtype == "f16" else L.RA_BF16
        self.kv_code = L.KV_CODES[w.kv_dtype]
        self.rope_args = None
        if self.store_mode == "qkv_rope_store":
            self.rope_args = [L._rope_args(self.qkv, self.positions, self.table, D, hq, hkv, D, self.q,
                                           self.slots_new, k, v, w.kv_dtype, w.k_scale, w.v_scale, ks, vs)
                              for k, v, ks, vs in self.pools]

    @staticmethod
    def _src(x):
        import numpy as np
        import torch
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")

    @staticmethod
    def _src_bf16(x):
        import numpy as np
        import torch
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)

    def run_attention(self, i, stream):
        """Enqueue only the attention launch of step i."""
        st = self.lib.ra_paged_attn(ctypes.byref(self.args[i % self.copies]), ctypes.c_void_p(stream))
        if st != 0:
            raise RuntimeError(self.lib.ra_last_error().decode())

    def run(self, i, stream, ev=None):
        """Enqueue step i: store, attention (between the two events), merge."""
        w, lib, L = self.w, self.lib, self.L
        k, v, ks, vs = self.pools[i % self.copies]
        s = ctypes.c_void_p(stream)
        if self.store_mode in ("fused", "fused_rope"):
            st = 0                   # the attention launch stores the new tokens itself
        elif self.rope_args is not None:
            st = lib.ra_qkv_rope_store(ctypes.byref(self.rope_args[i % self.copies]), s)
        elif ks is not None:
            st = lib.ra_kv_store_int8_token(self.k_new.data_ptr(), self.v_new.data_ptr(), L.RA_F16,
                                            self.k_new.stride(0), self.v_new.stride(0), self.slots_new.data_ptr(),
                                            self.k_new.shape[0], k.data_ptr(), v.data_ptr(), ks.data_ptr(),
                                            vs.data_ptr(), w.num_pages, w.num_kv_heads, w.head_dim, 16, s)
        else:
            st = lib.ra_kv_store(self.k_new.data_ptr(), self.v_new.data_ptr(), L.RA_F16, self.k_new.stride(0),
                                 self.v_new.stride(0), self.slots_new.data_ptr(), self.k_new.shape[0],
                                 k.data_ptr(), v.data_ptr(), self.kv_code, w.num_pages, w.num_kv_heads,
                                 w.head_dim, 16, w.k_scale, w.v_scale, s)
        if ev is not None:
            ev[0].record()
        st |= lib.ra_paged_attn(ctypes.byref(self.args[i % self.copies]), s)
        if ev is not None:
            ev[1].record()
        if not self.direct:
            st |= lib.ra_lse_merge(self.po.data_ptr(), self.pl.data_ptr(), self.slots, self.rows, w.head_dim,
                                   self.out.data_ptr(), self.q_code, self.lse.data_ptr(), s)
        if st != 0:
            raise RuntimeError(lib.ra_last_error().decode())


def algorithmic_bytes(w):
    """HBM bytes one attention launch must move: the visible KV tokens' codes
    (2 * Hkv * D * e per token, plus 2 * Hkv * 4 B of scales for per-token
    INT8), the block-table entries of the visited pages
    (4 B per 16 tokens per sequence), the queries read and the output and
    its lse written (partials are the implementation's own traffic)."""
    kv = w.kv_bytes_attended()
    bt = 4 * sum(-(-int(c) // 16) for c in w.ctx)
    q = w.q.nbytes
    out = w.q.nbytes + 4 * w.total_q * w.num_q_heads
    return kv + bt + q + out


def cpu_baseline(w, seconds):
    """The oracle (numpy, fp64) on whole sequences of the same step, until
    about `seconds` of CPU time: dequantise the cached codes, then attend."""
    sys.path.insert(0, ROOT)
    from oracle import attention as OA
    from oracle import codecs as OC
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    g = w.num_q_heads // w.num_kv_heads
    if w.meta.get("kind") == "prefill":
        return cpu_baseline_prefill(w, seconds, threads, OA, OC)
    done_tokens, elapsed, seqs = 0, 0.0, 0
    b = 0
    codes = {}
    while elapsed < seconds and seqs < 64 * w.batch:
        if b % w.batch not in codes:       # the cache contents: made once, not timed
            rows = w.seq_rows[b % w.batch]
            codes[b % w.batch] = (
                OC.quantize(OC.source_to_f32(w.tokens_k[rows], w.src_dtype), w.kv_dtype, w.k_scale),
                OC.quantize(OC.source_to_f32(w.tokens_v[rows], w.src_dtype), w.kv_dtype, w.v_scale))
        kc, vc = codes[b % w.batch]
        q0, q1 = int(w.query_start_loc[b % w.batch]), int(w.query_start_loc[b % w.batch + 1])
        q = OC.source_to_f32(w.q[q0:q1], w.q_dtype).astype("float64")
        t = time.perf_counter()
        k = OC.dequantize(kc, w.kv_dtype, w.k_scale)
        v = OC.dequantize(vc, w.kv_dtype, w.v_scale)
        OA.attention(q, k, v, w.softmax_scale, w.window_left, w.num_sinks)
        elapsed += time.perf_counter() - t
        done_tokens += OA.attended_keys(int(w.ctx[b % w.batch]), q1 - q0, w.window_left, w.num_sinks)
        seqs += 1
        b += 1
    return {"value": done_tokens / elapsed, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{seqs} whole sequences (all {w.num_kv_heads} KV heads x {g} query heads) of "
                      f"{w.name}: dequantise + fp64 attention, {elapsed:.1f} s"}


def cpu_baseline_prefill(w, seconds, threads, OA, OC):
    """Prefill: the oracle on evenly spread chunks of sequence 0's queries
    (each at its own position) until about `seconds` of CPU time, after
    dequantising the sequence's K and V once (timed).  Reported as query
    tokens per second of the whole step's mix."""
    import numpy as np
    rows = w.seq_rows[0]
    ctx, ql = int(w.ctx[0]), int(w.q_len[0])
    q_all = OC.source_to_f32(w.q[:ql], w.q_dtype).astype("float64")
    kc = OC.quantize(OC.source_to_f32(w.tokens_k[rows], w.src_dtype), w.kv_dtype, w.k_scale)
    vc = OC.quantize(OC.source_to_f32(w.tokens_v[rows], w.src_dtype), w.kv_dtype, w.v_scale)
    t = time.perf_counter()
    k = OC.dequantize(kc, w.kv_dtype, w.k_scale)
    v = OC.dequantize(vc, w.kv_dtype, w.v_scale)
    elapsed = time.perf_counter() - t
    chunk = max(1, (1 << 24) // (w.num_q_heads * ctx))      # scores of one chunk: <= 2^24 fp64
    order = np.random.default_rng(0).permutation(ql)
    done, flops = 0, 0
    vis = w.visible_per_query()[:ql]
    while elapsed < seconds and done < ql:
        sel = np.sort(order[done:done + chunk])
        t = time.perf_counter()
        OA.attention(q_all[sel], k, v, w.softmax_scale, w.window_left, w.num_sinks, positions=ctx - ql + sel)
        elapsed += time.perf_counter() - t
        done += sel.size
        flops += int(vis[sel].sum()) * w.num_q_heads * 4 * w.head_dim
    # scale the sampled queries' share of the work to the whole step
    frac = flops / w.attention_flops()
    return {"value": w.total_q * frac / elapsed, "unit": "query tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {ql} queries (random positions, all {w.num_q_heads} heads) of {w.name}: "
                      f"dequantise + fp64 attention, {elapsed:.1f} s = {frac:.2%} of the step's flops"}


def traffic_from_profile(wname, src_hash):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's reading), if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"attn_traffic_{wname}.txt")
    if not os.path.exists(p):
        return None
    fields = {}
    with open(p) as f:
        for line in f:
            k, sep, v = line.partition(":")
            if sep and k.strip() in ("kernel_source_hash", "hbm_bytes_per_launch"):
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_hash") != src_hash or "hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["hbm_bytes_per_launch"])


def time_graphs(step, args, torch):
    """Steps replayed from HIP graphs (one per pool copy: store, attention,
    merge), the way a serving loop launches its decode step.  The attention
    kernel's average duration is timed separately over back-to-back replays of
    a graph holding one attention launch per pool copy."""
    cap = torch.cuda.Stream()
    step_graphs, attn_graph = [], torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(cap):
        for c in range(step.copies):          # run once eagerly on the capture stream first
            step.run(c, cap.cuda_stream)
    torch.cuda.synchronize()
    for c in range(step.copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step.run(c, torch.cuda.current_stream().cuda_stream)
        step_graphs.append(g)
    with torch.cuda.graph(attn_graph, stream=cap):
        for c in range(step.copies):
            step.run_attention(c, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step_graphs[i % step.copies].replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step_graphs[(args.warmup + i) % step.copies].replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(stop) / args.steps
    reps = max(1, args.steps // step.copies)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(reps):
        attn_graph.replay()
    a1.record()
    torch.cuda.synchronize()
    attn_avg_ms = a0.elapsed_time(a1) / (reps * step.copies)
    return ms_per_step, attn_avg_ms, wall


def time_eager(step, args, torch):
    """Steps launched one by one from the host; the attention launch of every
    step is bracketed by its own pair of events."""
    sp = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        step.run(i, sp)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step.run(args.warmup + i, sp, evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    return start.elapsed_time(stop) / args.steps, sum(attn_ms) / len(attn_ms), wall


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this path is single-GPU "
              "by design and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    from paged_quantized_kv_ra_amd import workloads as W
    make = W.BENCH_WORKLOADS[args.workload]
    t0 = time.time()
    w = make()
    log(f"built {w.name} in {time.time() - t0:.1f}s")
    step = Step(w, fused_qkv=args.fused_qkv, separate_store=args.separate_store)
    log(f"pool copies: {step.copies}, partition slots: {step.slots}")
    if args.eager:
        ms_per_step, attn_avg_ms, wall = time_eager(step, args, torch)
    else:
        ms_per_step, attn_avg_ms, wall = time_graphs(step, args, torch)
    prefill = w.meta.get("kind") == "prefill"
    tokens = w.attended_keys()
    value = (w.total_q if prefill else tokens) / (ms_per_step / 1e3)
    alg = algorithmic_bytes(w)
    flops = w.attention_flops()
    achieved = alg / (attn_avg_ms / 1e3) / 1e9
    tflops = flops / (attn_avg_ms / 1e3) / 1e12
    src_hash = kernel_source_hash()
    traffic = traffic_from_profile(w.name, src_hash)
    log(f"{args.steps} steps ({'eager' if args.eager else 'graph replay'}): {ms_per_step * 1e3:.1f} us/step "
        f"(wall {wall / args.steps * 1e6:.1f} us/step), "
        f"attention {attn_avg_ms * 1e3:.1f} us avg, {achieved:.0f} GB/s algorithmic, {tflops:.1f} TFLOP/s")
    if prefill:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                "kernel": "attn_prefill_kernel" if w.kv_dtype in ("e4m3", "int8") and w.head_dim == 128
                and w.window_left < 0 and w.max_context_len <= 2 * int(w.q_len.min()) else "attn_mfma_kernel",
                "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": alg,
                "attn_us": round(attn_avg_ms * 1e3, 2), "kernel_source_hash": src_hash}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic, "kernel": "attn_mfma_kernel",
                "algorithmic_bytes_per_launch": alg, "attn_us": round(attn_avg_ms * 1e3, 2),
                "kernel_source_hash": src_hash}
    line = {
        "metric": ("prefill query tokens/sec (paged attention, one layer), FP8 KV" if prefill else
                   "KV tokens attended/sec and achieved HBM GB/s (% of MI355X peak), FP8 KV @32K"),
        "value": round(value, 1),
        "unit": "query tokens/s" if prefill else "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": int(w.ctx.max()), "q_len": w.max_q_len,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "kv_dtype": w.kv_dtype, "page_size": 16, "partition_slots": step.slots,
                   "kv_pool_copies": step.copies, "launch": "eager" if args.eager else "hip_graph",
                   "store": step.store_mode,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "attended_tokens_per_step": tokens,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
