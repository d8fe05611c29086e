"""Oracle: decode/verify attention over dequantised KV, split-KV and LSE merge.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Passages followed
-----------------
* ReVolta README, intro and "Weight and KV formats": attention runs over
  KV that is stored compressed and converted to FP16 for the arithmetic,
  i.e. plain softmax attention over the dequantised values.
* ReVolta README, intro list and "Quick start" (speculative config with
  4 speculative tokens): MTP4 verifies a block of 1 + 4 query tokens per
  sequence per step.
* ReVolta README, "Quick start" (decode context parallel size 2) and
  "Hardware" (TP4 + DCP2): one sequence's context is split into parts whose
  partial results are combined.
* ReVolta README, "DFlash2 speculative decoding" (sliding-window layers,
  2048-token window) and "ReVolta 0.1.3", "Behaviour changes" (sliding
  windows or attention sinks): some layers attend to a window plus sinks.

The pages give none of the formulas; what is computed here is the textbook
definition, in float64, over contiguous (unpaged) dequantised KV:

For sequence b with context length ctx (which includes this step's q_len
tokens), query i < q_len sits at position pos_i = ctx - q_len + i.  Query
head h reads KV head h // (Hq / Hkv).  Key j is visible to query i iff
j <= pos_i and (W < 0 or pos_i - j < W or j < n_sink).  Then
    s_j = softmax_scale * q_i . k_j,   m = max s_j,   l = sum exp(s_j - m),
    out = sum exp(s_j - m) v_j / l,    lse = m + ln l      (natural log).
A query with no visible key gets out = 0 and lse = -inf.  The arithmetic is
IEEE's: a NaN score (a NaN in q or in a visible key) makes m, and with it
out and lse, NaN for that query; a NaN in a visible value makes out NaN.

Split-KV: partition s of a sequence covers keys [s*P, min((s+1)*P, ctx));
with an explicit count S, P = 16 * ceil(ceil(ctx / S) / 16).  Each
partition yields (out_s, lse_s) as above restricted to its keys.  Merge:
M = max lse_s; if M = -inf the result is (0, -inf); else
a_s = exp(lse_s - M), out = sum a_s out_s / sum a_s, lse = M + ln sum a_s
(a NaN lse_s makes the row NaN; an empty partition, lse_s = -inf, adds
nothing whatever its out holds).

Pins (tests/test_oracle_attention.py): torch scaled_dot_product_attention
in float64 on the CPU with an explicit boolean mask and repeated KV heads;
a brute-force np.longdouble formulation without max subtraction on tiny
cases; a hand-computed closed-form case; uniform-V, identical-key,
single-key and dominant-key invariants; window >= ctx equals plain causal;
token permutation invariance; merge(split(S)) equals unsplit for several S
including empty partitions; merge associativity; S = 1 identity; NaN in a
query row, a visible key or a visible value propagates under IEEE
arithmetic to exactly the rows that see it, and a NaN partial lse poisons
its merged row.
"""
import math

import numpy as np

PAGE = 16


def visible_mask(ctx, q_len, window_left=-1, num_sinks=0, key_lo=0, key_hi=None, positions=None):
    """bool[q_len, ctx]: key j visible to query i (optionally inside [lo, hi)).

    Query i sits at position ``positions[i]``, by default ctx - q_len + i (the
    block is the context's last q_len tokens)."""
    if key_hi is None:
        key_hi = ctx
    j = np.arange(ctx, dtype=np.int64)[None, :]
    if positions is None:
        positions = ctx - q_len + np.arange(q_len, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)[:, None]
    vis = j <= pos
    if window_left is not None and window_left >= 0:
        vis &= ((pos - j) < window_left) | (j < num_sinks)
    vis &= (j >= key_lo) & (j < key_hi)
    return vis


def attention(q, k, v, softmax_scale, window_left=-1, num_sinks=0,
              key_lo=0, key_hi=None, positions=None):
    """Attention of one sequence's query block.

    q: [q_len, Hq, D]; k, v: [ctx, Hkv, D] (dequantised values, any float
    type).  ``positions``: the queries' positions (default: the context's
    last q_len tokens), so that any subset of a block's queries can be
    evaluated on its own.  Returns (out [q_len, Hq, D] float64, lse
    [q_len, Hq] float64).
    """
    q = np.asarray(q)
    q_len, hq, dim = q.shape
    ctx, hkv, _ = k.shape
    assert hq % hkv == 0 and (positions is not None or q_len <= ctx)
    g = hq // hkv
    vis = visible_mask(ctx, q_len, window_left, num_sinks, key_lo, key_hi, positions)
    cols = np.nonzero(vis.any(axis=0))[0]          # keys any query can see
    out = np.zeros((q_len, hq, dim), dtype=np.float64)
    lse = np.full((q_len, hq), -np.inf, dtype=np.float64)
    if cols.size == 0:
        return out, lse
    vis_c = vis[:, cols]                            # [q_len, n]
    for h in range(hkv):
        kh = np.asarray(k[cols, h, :], dtype=np.float64)     # [n, D]
        vh = np.asarray(v[cols, h, :], dtype=np.float64)
        qh = np.asarray(q[:, h * g:(h + 1) * g, :], dtype=np.float64)
        qh = qh.reshape(q_len * g, dim)                       # row = i*g + head
        s = softmax_scale * (qh @ kh.T)                       # [q_len*g, n]
        mask = np.repeat(vis_c, g, axis=0)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1)                                     # NaN if any visible score is NaN
        has = m != -np.inf                                    # no visible key: m = -inf
        w = np.where(mask, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
        l = w.sum(axis=1)
        o = np.zeros((q_len * g, dim))
        if np.isfinite(vh).all():
            o[has] = (w[has] @ vh) / l[has][:, None]
        else:   # sum over each row's visible keys only, so that 0 * NaN never enters
            for r in np.nonzero(has)[0]:
                o[r] = (w[r, mask[r]] @ vh[mask[r]]) / l[r]
        ls = np.full(q_len * g, -np.inf)
        ls[has] = m[has] + np.log(l[has])
        out[:, h * g:(h + 1) * g, :] = o.reshape(q_len, g, dim)
        lse[:, h * g:(h + 1) * g] = ls.reshape(q_len, g)
    return out, lse


def partition_size(ctx, num_splits):
    """Tokens per partition for an explicit split count (page aligned)."""
    per = -(-ctx // num_splits)
    return PAGE * (-(-per // PAGE))


def partition_bounds(ctx, num_splits=None, part_tokens=None):
    """[(lo, hi)] for every partition slot (empty slots have lo >= hi)."""
    if part_tokens is None:
        part_tokens = partition_size(ctx, num_splits)
    n = num_splits if num_splits is not None else -(-ctx // part_tokens)
    return [(s * part_tokens, min((s + 1) * part_tokens, ctx)) for s in range(n)]


def split_attention(q, k, v, softmax_scale, window_left=-1, num_sinks=0,
                    num_splits=None, part_tokens=None):
    """Per-partition partials: (out [S, q_len, Hq, D], lse [S, q_len, Hq])."""
    ctx = k.shape[0]
    outs, lses = [], []
    for lo, hi in partition_bounds(ctx, num_splits, part_tokens):
        o, l = attention(q, k, v, softmax_scale, window_left, num_sinks,
                         key_lo=lo, key_hi=max(lo, hi))
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def lse_merge(partial_out, partial_lse):
    """Merge partials along axis 0: returns (out, lse) in float64."""
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    m = pl.max(axis=0)                                        # NaN if any lse_s is NaN
    has = m != -np.inf                                        # every partition empty: m = -inf
    live = pl != -np.inf                                      # empty partitions add nothing
    a = np.where(live, np.exp(pl - np.where(has, m, 0.0)), 0.0)
    den = a.sum(axis=0)
    num = (a[..., None] * np.where(live[..., None], po, 0.0)).sum(axis=0)
    out = np.where(has[..., None], num / np.where(has, den, 1.0)[..., None], 0.0)
    lse = np.where(has, m + np.log(np.where(has, den, 1.0)), -np.inf)
    return out, lse


def attended_keys(ctx, q_len, window_left=-1, num_sinks=0):
    """Number of distinct keys visible to at least one query of the block."""
    return int(visible_mask(ctx, q_len, window_left, num_sinks).any(axis=0).sum())


def default_softmax_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)
