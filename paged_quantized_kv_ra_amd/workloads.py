"""Seeded synthetic inputs for paged decode/verify attention.

This module is the one place that both the HIP path (tests, bench) and the
CPU oracle take their inputs from.  It holds none of the method's
arithmetic: it draws numbers, casts them to the caller's input dtypes,
lays out block tables and slot mappings, and picks per-layer scales the way
a calibration pass would (``max|x| / 448`` for E4M3, ``max|x| / 127`` for
INT8).  Quantisation, paging and attention live elsewhere.

The workload shapes follow the pages' deployment: up to 8 sequences, a
1 + 4 token verify block (MTP4), 16-token pages, E4M3 / INT8 / FP16 KV,
"two 512K or four 256K contexts" in one GPU pool (ReVolta README, intro
list and "Quick start").  Head counts and head_dim are the library's
benchmark shapes (16 query heads, 2 KV heads, head_dim 128), as the pages
never state them.

Recipe: ``numpy.random.default_rng(seed)``; draw order is contexts (if
random), page permutation, K, V, Q; values are fp32 N(0, 1), then cast
with round-to-nearest-even to the input dtype (fp16, or bf16 kept as
uint16 bit patterns).
"""
from dataclasses import dataclass, field

import numpy as np

PAGE = 16
INT32_MAX = 0x7FFFFFFF
K = 1024  # the pages count contexts in K = 1024 tokens (512K = 524,288)

_CHUNK = 1 << 24  # values per RNG draw; draws concatenate to one stream


def f32_to_bf16_bits(x):
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def _normal(rng, shape, out_dtype, std=1.0):
    """Draw fp32 N(0, std^2) of ``shape`` in chunks (N(0,1) draws times std in
    fp32) and cast to ``out_dtype``.  ``std`` is a scalar, or one value per
    index of the first axis (a per-token magnitude)."""
    n = int(np.prod(shape))
    flat = np.empty(n, dtype=np.float16 if out_dtype == "f16" else np.uint16)
    std = np.asarray(std, dtype=np.float32)
    per_row = std.ndim > 0
    if per_row:
        assert std.shape == (shape[0],)
        inner = n // shape[0] if shape[0] else 1
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if per_row:
            x = x * std[np.arange(lo, hi) // inner]
        elif std != 1.0:
            x = x * std
        flat[lo:hi] = x.astype(np.float16) if out_dtype == "f16" else f32_to_bf16_bits(x)
    return flat.reshape(shape)


def _absmax_f32(x, src_dtype):
    if src_dtype == "f16":
        return np.float32(np.abs(x).max()) if x.size else np.float32(0)
    bits = (np.asarray(x, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.float32(np.abs(bits).max()) if x.size else np.float32(0)


@dataclass
class Workload:
    """One batch of paged decode/verify attention inputs (host arrays)."""
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str                 # 'f16' | 'e4m3' | 'int8' | 'int8_tok' (INT8, scale per token and head)
    q_dtype: str                  # 'f16' | 'bf16' (bf16 as uint16 bits)
    src_dtype: str                # dtype of new K/V handed to the store
    ctx: np.ndarray               # int32[B], includes this step's q_len
    q_len: np.ndarray             # int32[B]
    query_start_loc: np.ndarray   # int32[B+1]
    block_tables: np.ndarray      # int32[B][stride], tail = INT32_MAX
    num_pages: int
    tokens_k: np.ndarray          # [U][Hkv][D] unique logical tokens (src dtype)
    tokens_v: np.ndarray
    token_slots: np.ndarray       # int64[U] physical slot of each unique token
    seq_rows: list                # per sequence: int64[ctx_b] rows into tokens_*
    q: np.ndarray                 # [T][Hq][D] (f16 or uint16 bf16 bits)
    k_scale: float
    v_scale: float
    softmax_scale: float
    window_left: int = -1
    num_sinks: int = 0
    num_splits: int = 0           # 0 = library's automatic split
    cache_sentinel: int = 0       # byte pattern (uint16 for f16) of unused cache memory
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.ctx.shape[0])

    @property
    def total_q(self):
        return int(self.query_start_loc[-1])

    @property
    def max_q_len(self):
        return int(self.q_len.max()) if self.batch else 0

    @property
    def max_context_len(self):
        return int(self.ctx.max()) if self.batch else 0

    @property
    def elem_bytes(self):
        return 2 if self.kv_dtype == "f16" else 1

    def cache_bytes(self):
        """Bytes of one K (or V) cache: num_pages * Hkv * 16 * D * e."""
        return self.num_pages * self.num_kv_heads * PAGE * self.head_dim * self.elem_bytes

    def new_token_rows(self):
        """Rows (into tokens_*) of this step's q_len_b newest tokens, in Q order."""
        return np.concatenate([self.seq_rows[b][self.ctx[b] - self.q_len[b]:]
                               for b in range(self.batch)]).astype(np.int64)

    def attended_keys(self):
        """sum over sequences of |union of keys visible to the block's queries|."""
        tot = 0
        for b in range(self.batch):
            c, ql = int(self.ctx[b]), int(self.q_len[b])
            if ql == 0:
                continue
            if self.window_left < 0:
                tot += c
                continue
            lo = max(0, c - ql - self.window_left + 1)     # oldest key in any window
            tot += (c - lo) + min(self.num_sinks, c, lo)    # window span + sinks below it
        return tot

    def kv_bytes_attended(self):
        """K and V bytes of the visible tokens (codes, plus the fp32 K and V
        scales of every token and head for per-token INT8)."""
        per_head = self.head_dim * self.elem_bytes + (4 if self.kv_dtype == "int8_tok" else 0)
        return self.attended_keys() * 2 * self.num_kv_heads * per_head

    def visible_per_query(self):
        """int64[T]: number of keys each query row sees (causal within the
        block, window plus the sinks below it)."""
        out = []
        for b in range(self.batch):
            c, ql = int(self.ctx[b]), int(self.q_len[b])
            p = np.arange(c - ql, c, dtype=np.int64)          # query positions
            if self.window_left < 0:
                out.append(p + 1)
            else:
                w = self.window_left
                out.append(np.minimum(p + 1, w) + np.minimum(self.num_sinks, np.maximum(0, p + 1 - w)))
        return np.concatenate(out) if out else np.zeros(0, np.int64)

    def attention_flops(self):
        """Multiply-adds of QK^T and PV counted as 2 flops each: 4 * D per
        (query head, visible key) pair."""
        return int(self.visible_per_query().sum()) * self.num_q_heads * 4 * self.head_dim

    def unique_pages_attended(self):
        """Distinct physical pages touched (shared prefix pages counted once)."""
        pages = set()
        for b in range(self.batch):
            c = int(self.ctx[b])
            pages.update(self.block_tables[b, :-(-c // PAGE)].tolist())
        return len(pages)


def build(name, seed, *, ctx, q_len, num_q_heads, num_kv_heads, head_dim,
          kv_dtype, q_dtype="f16", src_dtype="f16", pool_pages=None,
          shared_prefix_tokens=0, window_left=-1, num_sinks=0, num_splits=0,
          softmax_scale=None, ctx_range=None, batch=None, extra_stride=1,
          kv_source=None, v_std=1.0):
    """Build a workload.

    ``ctx``: list of context lengths, or None with ``ctx_range=(lo, hi)`` and
    ``batch`` to draw them uniformly (inclusive) from the RNG first.
    ``q_len``: int or list.  ``shared_prefix_tokens`` (multiple of 16): the
    first positions of every sequence map to the same physical pages and
    hold the same K/V.  ``kv_source``: reuse K/V/pages of another workload
    (same seed stream position), used by the sliding-window variant.
    ``v_std``: standard deviation of the V values, a scalar or one value per
    unique token row (small or widely varying V magnitudes probe the
    precision of per-token scales).
    """
    rng = np.random.default_rng(seed)
    if ctx is None:
        lo, hi = ctx_range
        ctx = rng.integers(lo, hi + 1, size=batch)
    ctx = np.asarray(ctx, dtype=np.int64)
    B = ctx.shape[0]
    q_len = np.broadcast_to(np.asarray(q_len, dtype=np.int64), (B,)).copy()
    assert np.all(q_len <= ctx) and np.all(q_len >= 0)
    assert shared_prefix_tokens % PAGE == 0
    assert np.all(ctx >= shared_prefix_tokens)

    shared_pages = shared_prefix_tokens // PAGE
    pages_per_seq = -(-ctx // PAGE)
    private_pages = pages_per_seq - shared_pages
    need = shared_pages + int(private_pages.sum())
    if pool_pages is None:
        pool_pages = need
    assert pool_pages >= need
    perm = rng.permutation(pool_pages).astype(np.int64)

    stride = int(pages_per_seq.max()) + extra_stride
    bt = np.full((B, stride), INT32_MAX, dtype=np.int64)
    shared = perm[:shared_pages]
    off = shared_pages
    for b in range(B):
        n = int(private_pages[b])
        bt[b, :shared_pages] = shared
        bt[b, shared_pages:shared_pages + n] = perm[off:off + n]
        off += n

    # unique logical tokens: the shared prefix once, then each sequence's rest
    U = shared_prefix_tokens + int((ctx - shared_prefix_tokens).sum())
    rows, slots = [], np.empty(U, dtype=np.int64)
    j = np.arange(shared_prefix_tokens, dtype=np.int64)
    slots[:shared_prefix_tokens] = bt[0, j // PAGE] * PAGE + j % PAGE
    off = shared_prefix_tokens
    for b in range(B):
        n = int(ctx[b]) - shared_prefix_tokens
        r = np.concatenate([np.arange(shared_prefix_tokens, dtype=np.int64),
                            np.arange(off, off + n, dtype=np.int64)])
        jj = np.arange(shared_prefix_tokens, int(ctx[b]), dtype=np.int64)
        slots[off:off + n] = bt[b, jj // PAGE] * PAGE + jj % PAGE
        rows.append(r)
        off += n

    shape = (U, num_kv_heads, head_dim)
    if kv_source is not None:
        assert kv_source.tokens_k.shape == shape
        tokens_k, tokens_v = kv_source.tokens_k, kv_source.tokens_v
        # advance the stream exactly as the source's K and V draws did
        for _ in range(2):
            n = int(np.prod(shape))
            for lo_ in range(0, n, _CHUNK):
                rng.standard_normal(min(n, lo_ + _CHUNK) - lo_, dtype=np.float32)
    else:
        tokens_k = _normal(rng, shape, src_dtype)
        tokens_v = _normal(rng, shape, src_dtype, v_std)
    T = int(q_len.sum())
    q = _normal(rng, (T, num_q_heads, head_dim), q_dtype)

    if kv_dtype == "e4m3":
        k_scale = float(_absmax_f32(tokens_k, src_dtype) / np.float32(448.0))
        v_scale = float(_absmax_f32(tokens_v, src_dtype) / np.float32(448.0))
    elif kv_dtype == "int8":
        k_scale = float(_absmax_f32(tokens_k, src_dtype) / np.float32(127.0))
        v_scale = float(_absmax_f32(tokens_v, src_dtype) / np.float32(127.0))
    else:                         # FP16 (no scale) or per-token INT8 (scales made by the store)
        k_scale = v_scale = 1.0
    sentinel = {"f16": 0x7E00, "e4m3": 0x7F, "int8": 0x80, "int8_tok": 0x80}[kv_dtype]
    qsl = np.zeros(B + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(q_len)
    return Workload(
        name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, kv_dtype=kv_dtype, q_dtype=q_dtype, src_dtype=src_dtype,
        ctx=ctx.astype(np.int32), q_len=q_len.astype(np.int32),
        query_start_loc=qsl.astype(np.int32), block_tables=bt.astype(np.int32),
        num_pages=int(pool_pages), tokens_k=tokens_k, tokens_v=tokens_v,
        token_slots=slots, seq_rows=rows, q=q, k_scale=k_scale, v_scale=v_scale,
        softmax_scale=(1.0 / np.sqrt(head_dim)) if softmax_scale is None else softmax_scale,
        window_left=window_left, num_sinks=num_sinks, num_splits=num_splits,
        cache_sentinel=sentinel)


def packed_qkv(seed, num_tokens, num_q_heads, num_kv_heads, head_dim, src_dtype="f16", row_pad=0):
    """Rows of a fused QKV projection output: [T][(Hq + 2 Hkv) * D + row_pad]
    N(0, 1) values in the source dtype (fp16, or bf16 bit patterns); the pad
    columns make the row stride larger than the packed row."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (num_tokens, (num_q_heads + 2 * num_kv_heads) * head_dim + row_pad), src_dtype)


def step_positions_and_slots(w):
    """Positions (ctx_b - q_len_b + i) and cache slots of a workload's new
    tokens, in Q order."""
    pos = np.concatenate([np.arange(int(w.ctx[b]) - int(w.q_len[b]), int(w.ctx[b]), dtype=np.int64)
                          for b in range(w.batch)])
    return pos, w.token_slots[w.new_token_rows()]


# ---------------------------------------------------------------------------
# The five benchmark workloads (seed = index - 1) and the sliding-window one.

def tiny_decode():
    """1 x 256 ctx, 4/1 heads, D 64, q_len 1, FP16 KV, fp16 Q; pool of 32
    pages of which a random 16 form the permuted block table."""
    return build("tiny_decode_ctx256_f16", 0, ctx=[256], q_len=1, num_q_heads=4,
                 num_kv_heads=1, head_dim=64, kv_dtype="f16", q_dtype="f16",
                 pool_pages=32)


def batch8_decode():
    """8 sequences, ctx uniform in [1K, 8K], 16/2 heads, D 128, q_len 1,
    bf16 Q, FP16 KV, pages shuffled in a pool of 8192."""
    return build("batch8_decode_1k_8k_f16", 1, ctx=None, ctx_range=(1 * K, 8 * K),
                 batch=8, q_len=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
                 kv_dtype="f16", q_dtype="bf16", pool_pages=8192)


def verify_fp8_32k():
    """8 x 32K, 16/2 heads, D 128, q_len 5 (1 + 4 drafts), E4M3 KV."""
    return build("verify_e4m3_8x32k_q5", 2, ctx=[32 * K] * 8, q_len=5, num_q_heads=16,
                 num_kv_heads=2, head_dim=128, kv_dtype="e4m3", q_dtype="f16",
                 pool_pages=16384)


def decode_fp8_32k():
    """Plain decode (q_len 1) over the 8 x 32K E4M3 shape: an extra measurement
    of the decode rows (g = 8 < 16) on long contexts."""
    return build("decode_e4m3_8x32k_q1", 5, ctx=[32 * K] * 8, q_len=1, num_q_heads=16,
                 num_kv_heads=2, head_dim=128, kv_dtype="e4m3", q_dtype="f16",
                 pool_pages=16384)


def verify_int8tok_32k():
    """The 8 x 32K verify shape with INT8 KV scaled per token and head at
    runtime (ReVolta README, "Weight and KV formats", INT8 KV)."""
    return build("verify_int8tok_8x32k_q5", 6, ctx=[32 * K] * 8, q_len=5, num_q_heads=16,
                 num_kv_heads=2, head_dim=128, kv_dtype="int8_tok", q_dtype="f16",
                 pool_pages=16384)


def prefix_int8_256k():
    """4 x 256K sharing the first 192K tokens' pages, INT8 KV, q_len 5."""
    return build("prefix_int8_4x256k_shared192k_q5", 3, ctx=[256 * K] * 4, q_len=5,
                 num_q_heads=16, num_kv_heads=2, head_dim=128, kv_dtype="int8",
                 q_dtype="f16", pool_pages=28672, shared_prefix_tokens=192 * K)


def split_fp8_512k():
    """2 x 512K, E4M3 KV, q_len 5, 64 partitions merged by LSE."""
    return build("split_e4m3_2x512k_q5_s64", 4, ctx=[512 * K] * 2, q_len=5,
                 num_q_heads=16, num_kv_heads=2, head_dim=128, kv_dtype="e4m3",
                 q_dtype="f16", pool_pages=65536, num_splits=64)


def split_fp8_512k_sliding(base=None):
    """The 512K workload's KV with a 16-token query block, window 4096 and
    4 sink tokens, 64 partitions."""
    return build("split_e4m3_2x512k_q16_w4096_sink4", 4, ctx=[512 * K] * 2, q_len=16,
                 num_q_heads=16, num_kv_heads=2, head_dim=128, kv_dtype="e4m3",
                 q_dtype="f16", pool_pages=65536, num_splits=64, window_left=4096,
                 num_sinks=4, kv_source=base)


def split_fp8_512k_sliding_auto(base=None):
    """The sliding-window variant with automatic partitions (num_splits = 0),
    which cut the window span instead of the whole 512K context."""
    return build("split_e4m3_2x512k_q16_w4096_sink4_auto", 4, ctx=[512 * K] * 2, q_len=16,
                 num_q_heads=16, num_kv_heads=2, head_dim=128, kv_dtype="e4m3",
                 q_dtype="f16", pool_pages=65536, num_splits=0, window_left=4096,
                 num_sinks=4, kv_source=base)


def prefill_fp8_8k():
    """Cold prefill of an 8K prompt: one sequence whose 8,192 tokens are all
    queries, causal, E4M3 KV (ReVolta README, intro table, "Cold prompt 8K
    tokens" prefill throughput)."""
    w = build("prefill_e4m3_1x8k", 7, ctx=[8 * K], q_len=8 * K, num_q_heads=16, num_kv_heads=2,
              head_dim=128, kv_dtype="e4m3", q_dtype="f16", pool_pages=1024)
    w.meta["kind"] = "prefill"
    return w


def chunk_prefill_fp8_128k():
    """One chunk of a 131,072-token cold prompt: the last 4,896 tokens (the
    long-prefill token threshold of the recommended launch flags) attending
    to the whole prompt, E4M3 KV (ReVolta README, intro table, "Cold prompt
    131K tokens"; "Quick start" launch flags)."""
    w = build("chunk_prefill_e4m3_1x128k_q4896", 8, ctx=[128 * K], q_len=4896, num_q_heads=16,
              num_kv_heads=2, head_dim=128, kv_dtype="e4m3", q_dtype="f16", pool_pages=8704)
    w.meta["kind"] = "prefill"
    return w


BENCH_WORKLOADS = {
    "tiny_decode": tiny_decode,
    "batch8_decode": batch8_decode,
    "verify_fp8_32k": verify_fp8_32k,
    "decode_fp8_32k": decode_fp8_32k,
    "verify_int8tok_32k": verify_int8tok_32k,
    "prefix_int8_256k": prefix_int8_256k,
    "split_fp8_512k": split_fp8_512k,
    "split_fp8_512k_sliding": split_fp8_512k_sliding,
    "split_fp8_512k_sliding_auto": split_fp8_512k_sliding_auto,
    "prefill_fp8_8k": prefill_fp8_8k,
    "chunk_prefill_fp8_128k": chunk_prefill_fp8_128k,
}
