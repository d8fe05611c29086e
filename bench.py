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
                  "paged_quantized_kv_ra_amd/csrc/ra_internal.h", "paged_quantized_kv_ra_amd/csrc/fastdiv.h"]


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
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup phase timings of the attention kernel, from the timing build "
                         "libra_kv_timeline.so (python -m paged_quantized_kv_ra_amd.build --timeline)")
    ap.add_argument("--timeline-launches", type=int, default=20)
    ap.add_argument("--timeline-dump", default=None,
                    help="with --timeline: also save every launch's raw per-workgroup slots (numpy .npy, int64 ticks)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="HBM read rate of random 2/4/8 KiB blocks read the way the attention reads pages "
                         "(libra_probe.so), against a streaming read")
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


def algorithmic_bytes(w, unique=False):
    """HBM bytes one attention launch must move: the visible KV tokens' codes
    (2 * Hkv * D * e per token, plus 2 * Hkv * 4 B of scales for per-token
    INT8), the block-table entries of the visited pages
    (4 B per 16 tokens per sequence), the queries read and the output and
    its lse written (partials are the implementation's own traffic).  With
    unique=True the KV bytes count every physical page once (pages shared by
    several sequences' block tables are read from HBM once at best)."""
    kv = w.kv_bytes_attended()
    if unique and w.window_left < 0:
        per_tok = w.kv_bytes_attended() / max(1, w.attended_keys())
        kv = int(round(per_tok * 16 * w.unique_pages_attended()))
    bt = 4 * sum(-(-int(c) // 16) for c in w.ctx)
    q = w.q.nbytes
    out = w.q.nbytes + 4 * w.total_q * w.num_q_heads
    return kv + bt + q + out


def host_cores():
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS
    when that is set (the host's share of cores for one GPU)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_baseline(w, seconds):
    """The oracle (numpy, fp64, BLAS for the products) on whole sequences of
    the same step: dequantise the cached codes, then attend.  Timed at one
    BLAS thread and at all of the host's cores, each the median of 3 runs of
    about seconds / 6 of CPU work; `value` is the all-cores median."""
    from threadpoolctl import threadpool_limits
    sys.path.insert(0, ROOT)
    from oracle import attention as OA
    from oracle import codecs as OC
    cores = host_cores()
    per_run = max(0.5, seconds / 6.0)
    codes = {}          # the cache contents per sequence: made once, not timed
    res = {}
    for threads in (1, cores):
        runs = []
        with threadpool_limits(limits=threads):
            for _ in range(3):
                if w.meta.get("kind") == "prefill":
                    runs.append(cpu_baseline_prefill(w, per_run, threads, OA, OC))
                else:
                    runs.append(_cpu_decode_run(w, per_run, threads, OA, OC, codes))
        runs.sort(key=lambda r: r["value"])
        res[threads] = runs
    med = res[cores][1]
    one = res[1][1]
    return {"value": med["value"], "unit": med["unit"], "cores": cores, "kind": "oracle",
            "sample": med["sample"] + f"; median of 3 runs at {cores} BLAS threads",
            "runs_value": [round(r["value"], 1) for r in res[cores]],
            "single_thread": {"value": one["value"], "unit": one["unit"], "cores": 1,
                              "runs_value": [round(r["value"], 1) for r in res[1]], "sample": one["sample"]}}


def _cpu_decode_run(w, seconds, threads, OA, OC, codes):
    """One timed run of the oracle on whole sequences until about `seconds`
    (`codes`: the sequences' cached codes, shared between runs)."""
    g = w.num_q_heads // w.num_kv_heads
    done_tokens, elapsed, seqs = 0, 0.0, 0
    b = 0
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
    step.graphs = step_graphs
    return ms_per_step, attn_avg_ms, wall


def launch_percentiles(step, args, torch, n=200):
    """Per-launch times: n attention launches, each bracketed by its own pair
    of HIP events on the launch stream (eager, one pool copy after another),
    and n graph-replayed steps, each bracketed the same way.  us."""
    import numpy as np
    sp = torch.cuda.current_stream().cuda_stream
    mk = (lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
    ev = [mk() for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record()
        step.run_attention(i, sp)
        ev[i][1].record()
    torch.cuda.synchronize()
    attn = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    out = {"attn_us": {k: round(float(np.percentile(attn, q)), 2) for k, q in (("p10", 10), ("median", 50),
                                                                               ("p90", 90))}}
    if getattr(step, "graphs", None):
        ev = [mk() for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            step.graphs[i % len(step.graphs)].replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        st = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        out["step_us"] = {k: round(float(np.percentile(st, q)), 2) for k, q in (("p10", 10), ("median", 50),
                                                                              ("p90", 90))}
    return out


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


def read_ceiling(torch):
    """Read rates of a 2 GiB buffer by libra_probe.so (block reads at a random
    permutation of block ids, 8-wave workgroups, two blocks in flight per
    wave; see probe/read_ceiling.hip), best and median of 5 timed launches
    after one untimed."""
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_quantized_kv_ra_amd", "libra_probe.so"))
    fn = lib.ra_probe_read_blocks
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    n = 2 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    out = torch.empty(1024 * 512, dtype=torch.int32, device="cuda")
    gen = torch.Generator().manual_seed(1)
    perms = {bb: torch.randperm(n // bb, generator=gen).to(torch.int32).cuda() for bb in (2048, 4096, 8192)}
    modes = {0: "LDS DMA ring, default policy", 1: "LDS DMA ring, nontemporal", 2: "plain loads, default policy",
             3: "plain loads, nontemporal", 4: "plain loads, nontemporal, in buffer order (streaming)"}
    # (mode, block bytes, workgroups, workgroups per CU): extra LDS pins the count per CU
    cases = [(4, 2048, 256, 1), (2, 2048, 256, 1), (3, 2048, 256, 1), (0, 2048, 256, 1), (1, 2048, 256, 1),
             (2, 4096, 256, 1), (3, 4096, 256, 1), (2, 8192, 256, 1), (3, 8192, 256, 1),
             (1, 2048, 512, 2), (3, 2048, 512, 2), (1, 2048, 1024, 4)]
    sp = torch.cuda.current_stream().cuda_stream
    results = []
    for mode, bb, grid, per_cu in cases:
        static = {0: 16 * bb, 1: 16 * bb}.get(mode, 0)
        dyn = max(0, (160 * 1024) // per_cu - static - 1024) if per_cu == 1 else \
            max(0, (160 * 1024) // (per_cu + 1) + 1024 - static)
        dyn = min(dyn, 96 * 1024)
        ts = []
        for r in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            st = fn(buf.data_ptr(), perms[bb].data_ptr(), n // bb, bb, mode, grid, dyn, out.data_ptr(), sp)
            b.record()
            if st != 0:
                raise RuntimeError(f"ra_probe_read_blocks refused mode {mode} block {bb} grid {grid}")
            torch.cuda.synchronize()
            if r:
                ts.append(a.elapsed_time(b))
        ts.sort()
        best, med = n / (ts[0] * 1e-3) / 1e9, n / (ts[len(ts) // 2] * 1e-3) / 1e9
        results.append({"mode": modes[mode], "block_bytes": bb, "workgroups": grid, "per_cu": per_cu,
                        "best_gbs": round(best, 1), "median_gbs": round(med, 1)})
        log(f"{modes[mode]:55s} {bb:5d} B blocks, {grid:4d} workgroups ({per_cu}/CU): best {best:7.1f} GB/s, "
            f"median {med:7.1f} GB/s")
    print(json.dumps({"read_ceiling": results}), flush=True)


def _pct(x):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return None
    return {"p10": round(float(np.percentile(x, 10)), 2), "median": round(float(np.median(x)), 2),
            "p90": round(float(np.percentile(x, 90)), 2), "max": round(float(x.max()), 2)}


def timeline(step, args, torch):
    """Per-workgroup phases of the attention kernel from the timing build.
    Every launch is the step's attention launch alone (with its fused store),
    after warm-up steps; the kernel records the 100 MHz real-time counter at
    fixed points (see the RA_TIMELINE slots in attn_mfma.hip).  Times in us,
    over all workgroups of all launches; spans per launch."""
    import numpy as np
    lib = step.lib
    for name in ("ra_timeline_read", "ra_timeline_clear", "ra_timeline_layout"):
        if not hasattr(lib, name):
            raise RuntimeError("--timeline needs the timing build: python -m paged_quantized_kv_ra_amd.build --timeline")
    lib.ra_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    nb, ns = ctypes.c_int32(), ctypes.c_int32()
    lib.ra_timeline_layout(ctypes.byref(nb), ctypes.byref(ns))
    nb, ns = nb.value, ns.value
    TL = dict(entry=0, hwid=1, xcc=2, meta=3, idsq=4, first=5, pages=6, loop=8, comb=16, ml=17, p0w=18, p1w=19,
              p0r=20, p1r=21, end=24, plan=32, idiss=33, idland=34, pgiss=35)
    sp = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        step.run(i, sp)
    torch.cuda.synchronize()
    buf = np.zeros(nb * ns, dtype=np.uint64)
    acc = {k: [] for k in ("start", "meta", "plan", "ids_issued", "ids_landed", "pages_issued", "idsq", "first", "stream_wave_median", "wave_skew", "combine",
                           "comb_barrier1", "comb_row_stats", "comb_pass0_write", "comb_pass0_reduce",
                           "comb_pass1_write", "comb_pass1_reduce", "comb_tail", "block", "end_after_median")}
    spans, blocks_per_cu, raw = [], [], []
    for i in range(args.timeline_launches):
        if lib.ra_timeline_clear() != 0:
            raise RuntimeError("ra_timeline_clear failed")
        step.run_attention(i, sp)
        torch.cuda.synchronize()
        if lib.ra_timeline_read(buf.ctypes.data, buf.nbytes) != 0:
            raise RuntimeError("ra_timeline_read failed")
        t = buf.reshape(nb, ns).astype(np.int64)
        live = (t[:, TL["entry"]] > 0) & (t[:, TL["end"]:TL["end"] + 8].max(axis=1) > 0) & (t[:, TL["first"]] > 0)
        t = t[live]
        if t.shape[0] == 0:
            continue
        if args.timeline_dump:
            raw.append(np.concatenate([np.full((t.shape[0], 1), i, dtype=np.int64), t], axis=1))
        us = 1e-2                                     # 100 MHz ticks
        entry = t[:, TL["entry"]]
        t0 = entry.min()
        nw = int((t[:, TL["loop"]:TL["loop"] + 8] > 0).sum(axis=1).max())   # waves per workgroup
        loops = t[:, TL["loop"]:TL["loop"] + nw]
        ends = t[:, TL["end"]:TL["end"] + nw]
        end = ends.max(axis=1)
        acc["start"] += list((entry - t0) * us)
        acc["meta"] += list((t[:, TL["meta"]] - entry) * us)
        for k, slot in (("plan", "plan"), ("ids_issued", "idiss"), ("ids_landed", "idland"), ("pages_issued", "pgiss")):
            ok = t[:, TL[slot]] > 0
            acc[k] += list((t[ok, TL[slot]] - entry[ok]) * us)
        acc["idsq"] += list((t[:, TL["idsq"]] - entry) * us)
        acc["first"] += list((t[:, TL["first"]] - entry) * us)
        acc["stream_wave_median"] += list((np.median(loops, axis=1) - t[:, TL["first"]]) * us)
        acc["wave_skew"] += list((loops.max(axis=1) - loops.min(axis=1)) * us)
        acc["combine"] += list((end - loops.max(axis=1)) * us)
        steps = [("comb_barrier1", loops.max(axis=1), t[:, TL["comb"]]), ("comb_row_stats", t[:, TL["comb"]], t[:, TL["ml"]]),
                 ("comb_pass0_write", t[:, TL["ml"]], t[:, TL["p0w"]]), ("comb_pass0_reduce", t[:, TL["p0w"]], t[:, TL["p0r"]]),
                 ("comb_pass1_write", t[:, TL["p0r"]], t[:, TL["p1w"]]), ("comb_pass1_reduce", t[:, TL["p1w"]], t[:, TL["p1r"]]),
                 ("comb_tail", t[:, TL["p1r"]], end)]
        for k, a0, a1 in steps:
            ok = (a0 > 0) & (a1 > 0)
            acc[k] += list((a1[ok] - a0[ok]) * us)
        acc["block"] += list((end - entry) * us)
        acc["end_after_median"] += list((end - np.median(end)) * us)
        spans.append((end.max() - t0) * us)
        hw = t[:, TL["hwid"]]
        cu = (t[:, TL["xcc"]] & 0xF) * 4096 + ((hw >> 13) & 0x7) * 512 + ((hw >> 12) & 1) * 256 + ((hw >> 8) & 0xF)
        _, counts = np.unique(cu, return_counts=True)
        blocks_per_cu.append((len(counts), float(counts.mean()), int(counts.max())))
    if args.timeline_dump and raw:
        np.save(args.timeline_dump, np.concatenate(raw, axis=0))   # columns: launch, then the slots
    res = {"workload": step.w.name, "launches": len(spans), "kernel_span_us": _pct(spans),
           "cus_used": blocks_per_cu[-1][0] if blocks_per_cu else None,
           "blocks_per_cu_max": max(b[2] for b in blocks_per_cu) if blocks_per_cu else None,
           "phases_us": {k: _pct(v) for k, v in acc.items()}}
    log(f"timeline of {step.w.name}: {len(spans)} launches, kernel span (first workgroup start to last end) "
        f"{res['kernel_span_us']}")
    log(f"  workgroups on {res['cus_used']} distinct CUs, at most {res['blocks_per_cu_max']} per CU")
    for k, v in res["phases_us"].items():
        log(f"  {k:20s} {v}")
    print(json.dumps({"timeline": res}), flush=True)


def main():
    args = parse()
    if args.timeline:   # the timing build of the library (same ABI), unless another one is named
        os.environ.setdefault("RA_KV_LIB", os.path.join(ROOT, "paged_quantized_kv_ra_amd", "libra_kv_timeline.so"))
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this path is single-GPU "
              "by design and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    if args.read_ceiling:
        read_ceiling(torch)
        return
    from paged_quantized_kv_ra_amd import workloads as W
    make = W.BENCH_WORKLOADS[args.workload]
    t0 = time.time()
    w = make()
    log(f"built {w.name} in {time.time() - t0:.1f}s")
    step = Step(w, fused_qkv=args.fused_qkv, separate_store=args.separate_store)
    log(f"pool copies: {step.copies}, partition slots: {step.slots}")
    if args.timeline:
        timeline(step, args, torch)
        return
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
    pct = launch_percentiles(step, args, torch)
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
        # HBM bytes the counters saw per launch over the same average time
        roof["hbm_gbs"] = round(traffic / (attn_avg_ms / 1e3) / 1e9, 1) if traffic else None
        uniq = algorithmic_bytes(w, unique=True)
        if uniq != alg:   # pages shared between sequences (prefix caching): the bytes counted once
            roof["algorithmic_bytes_unique_per_launch"] = uniq
            roof["achieved_unique"] = round(uniq / (attn_avg_ms / 1e3) / 1e9, 1)
            roof["frac_unique"] = round(uniq / (attn_avg_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
    roof.update({"attn_us_" + k: v for k, v in pct["attn_us"].items()})
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
    if "step_us" in pct:
        line["step_us_percentiles"] = pct["step_us"]
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
