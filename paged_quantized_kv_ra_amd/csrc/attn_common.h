// attn_common.h -- work decomposition of the attention kernel.
//
// One workgroup handles one (sequence b, KV head h, partition slot s, row group)
// unit.  Rows of a unit are the query-block rows r = i * g + j (query token i of
// the block, query head h * g + j), g = Hq / Hkv (ReVolta README, "Quick start":
// MTP4 verifies 1 + 4 tokens per sequence; the graded shapes use grouped query
// heads).  Partition s covers the sequence's keys [s * P_b, min((s + 1) * P_b,
// ctx_b)); only the pages holding a key visible to some row of the block are
// visited: keys up to the last query's position, restricted with a window to
// the sink keys and to keys within W of the first query (ReVolta README,
// "DFlash2 speculative decoding"; "ReVolta 0.1.3", "Behaviour changes").
//
// Positions.  The cache holds the sequence's keys 0 .. ctx_b - 1.  With
// context parallelism (ReVolta README, "Quick start", DCP2) a GPU holds only a
// range of a sequence's keys, starting at global position kv_pos0[b], and the
// block's queries sit at global positions q_pos0[b] + i.  All masks work in
// the cache's local key index: a query's local position is its global one
// minus kv_pos0[b], and a sink bound num_sinks becomes num_sinks - kv_pos0[b].
// Without the two arrays kv_pos0 = 0 and the queries are the last q_len
// positions of the context, q_pos0 = ctx_b - q_len.
#pragma once

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

// floor(n / f.d) for 0 <= n < 2^31 (fastdiv.h)
__device__ __forceinline__ uint32_t fdiv(const FastDiv& f, uint32_t n) { return (__umulhi(n, f.m) + n) >> f.l; }

struct UnitPages {
  int32_t p0a, na;   // first page and count of the first page range
  int32_t p0b, nb;   // second range (window pages when a sink range exists)
  __device__ __forceinline__ int32_t count() const { return na + nb; }
  __device__ __forceinline__ int32_t page(int32_t n) const { return n < na ? p0a + n : p0b + (n - na); }
};

// Partition size (tokens, a multiple of 16) of a sequence with the given
// context and row count.
__device__ __forceinline__ int32_t partition_tokens(const AttnLaunch& a, int32_t ctx, int32_t rows) {
  if (a.num_splits > 0) {
    const int32_t per = (ctx + a.num_splits - 1) / a.num_splits;
    return ((per + kPage - 1) / kPage) * kPage;
  }
  if (rows >= kSmallUnitRows) {
    const int32_t units = a.hkv * ((rows + kMfmaRowsPerBlock - 1) / kMfmaRowsPerBlock);
    const int32_t want = units >= kFillUnits ? 1 : (kFillUnits + units - 1) / units;
    const int32_t per = ((ctx + want - 1) / want + kPage - 1) / kPage * kPage;
    return max(per, a.part_tokens);
  }
  const int32_t per = (ctx + kSmallSplits - 1) / kSmallSplits;
  const int32_t p = ((per + kPage - 1) / kPage) * kPage;
  return min(max(p, a.part_small), a.part_tokens);
}

// A unit's queries in the cache's local key index: query i of the block sits
// at local position pmin + i (pmax for the last one); keys below `sinks` are
// sink keys.
struct SeqFrame {
  int32_t pmin, pmax, sinks;
};

// Visible page ranges of partition [lo, hi).
__device__ __forceinline__ UnitPages unit_pages(const AttnLaunch& a, const SeqFrame& f, int32_t lo, int32_t hi) {
  UnitPages u{0, 0, 0, 0};
  hi = min(hi, f.pmax + 1);       // keys after the last query are seen by none
  if (lo >= hi) return u;
  if (a.window < 0) {
    u.p0a = lo / kPage;
    u.na = (hi + kPage - 1) / kPage - u.p0a;
    return u;
  }
  // keys any query sees: [0, sinks) U [pmin - W + 1, pmax]
  const int32_t wlo = max(f.pmin - a.window + 1, 0);
  const int32_t sa0 = lo, sa1 = min(hi, f.sinks);
  const int32_t sb0 = max(lo, wlo), sb1 = hi;
  int32_t pa0 = 0, pa1 = 0, pb0 = 0, pb1 = 0;
  if (sa1 > sa0) { pa0 = sa0 / kPage; pa1 = (sa1 + kPage - 1) / kPage; }
  if (sb1 > sb0) { pb0 = sb0 / kPage; pb1 = (sb1 + kPage - 1) / kPage; }
  if (pa1 > pa0 && pb1 > pb0 && pa1 >= pb0) {       // ranges touch: one range
    u.p0a = min(pa0, pb0);
    u.na = max(pa1, pb1) - u.p0a;
  } else {
    u.p0a = pa0; u.na = pa1 - pa0;
    u.p0b = pb0; u.nb = pb1 - pb0;
    if (u.na == 0) { u.p0a = u.p0b; u.na = u.nb; u.p0b = 0; u.nb = 0; }
  }
  return u;
}

// Key j visible to the query at (local) position pos.
__device__ __forceinline__ bool key_visible(const AttnLaunch& a, const SeqFrame& f, int32_t j, int32_t pos) {
  return j <= pos && (a.window < 0 || pos - j < a.window || j < f.sinks);
}

// Block index -> logical unit id.  Consecutive workgroups are dispatched to the
// 8 XCDs round-robin.  With one row group the remap places consecutive logical
// ids on one XCD so units that read the same pages (the sequences of a shared
// prefix) share that XCD's L2.  With several row groups (long query blocks,
// whose causal row groups differ in work) the ids stay in dispatch order, so
// that the heaviest-first order below is spread evenly over the XCDs.
// The grid is padded_grid(units): a multiple of 8 below 2^31 (the host
// rejects larger problems), so 32-bit arithmetic holds, and the per-XCD count
// comes from the launch fields rather than from gridDim (which would cost a
// dependent load of the dispatch packet before any other work).
__device__ __forceinline__ uint32_t logical_block(uint32_t units, int32_t row_groups) {
  const uint32_t bid = blockIdx.x;
  if (row_groups > 1) return bid;
  const uint32_t per_xcd = (units + 7u) / 8u;
  return (bid % 8u) * per_xcd + bid / 8u;
}

struct UnitId {
  int32_t b, h, s, rg;
};

// logical id = ((s * row_groups + (row_groups - 1 - rg)) * Hkv + h) * batch + b:
// within a partition slot the last row group (the latest queries, which see
// the most keys under the causal mask) comes first
__device__ __forceinline__ bool decode_unit(const AttnLaunch& a, int32_t row_groups, UnitId& u) {
  const uint32_t total = (uint32_t)a.slots * (uint32_t)a.hkv * (uint32_t)row_groups * (uint32_t)a.batch;
  uint32_t id = logical_block(total, row_groups);
  if (id >= total) return false;
  uint32_t q = fdiv(a.fd_batch, id);
  u.b = (int32_t)(id - q * (uint32_t)a.batch);
  id = q;
  q = fdiv(a.fd_hkv, id);
  u.h = (int32_t)(id - q * (uint32_t)a.hkv);
  id = q;
  q = fdiv(a.fd_rg, id);
  u.rg = row_groups - 1 - (int32_t)(id - q * (uint32_t)row_groups);
  u.s = (int32_t)q;
  return true;
}

inline unsigned padded_grid(int64_t units) {
  return (unsigned)(((units + 7) / 8) * 8);
}

// Sequence preconditions that the host cannot check.  A violating sequence
// gets NaN rows instead of an out-of-bounds access.  Without explicit
// positions the block's queries must be the context's last q_len tokens.
__device__ __forceinline__ bool seq_ok(const AttnLaunch& a, int32_t ctx, int32_t q0, int32_t q1, int32_t kv0,
                                       int32_t qp0) {
  return ctx >= 0 && ctx <= a.max_ctx && q0 >= 0 && q1 >= q0 && q1 <= a.total_q && q1 - q0 <= a.max_q_len &&
         q1 - q0 >= a.min_q_len &&
         (a.q_pos0 ? qp0 >= 0 : q1 - q0 <= ctx) && kv0 >= 0;
}

// The unit's frame (see "Positions" above).
__device__ __forceinline__ SeqFrame seq_frame(const AttnLaunch& a, int32_t ctx, int32_t q_len, int32_t kv0,
                                              int32_t qp0) {
  SeqFrame f;
  f.pmin = (a.q_pos0 ? qp0 : ctx - q_len + kv0) - kv0;
  f.pmax = f.pmin + q_len - 1;
  f.sinks = a.window < 0 ? 0 : a.sinks - kv0;
  return f;
}

}  // namespace ra
