// attn_common.h -- work decomposition shared by the two attention kernels.
//
// One workgroup handles one (sequence b, KV head h, partition slot s, row group)
// unit.  Rows of a unit are the query-block rows r = i * g + j (query token i of
// the block, query head h * g + j), g = Hq / Hkv (ReVolta README, "Quick start":
// MTP4 verifies 1 + 4 tokens per sequence; the graded shapes use grouped query
// heads).  Partition s covers keys [s * P_b, min((s + 1) * P_b, ctx_b)); only
// the pages holding a key visible to some row of the block are visited: the
// sink pages [0, num_sinks) and the window pages [ctx - q_len - W + 1, ctx)
// when a window is set (ReVolta README, "DFlash2 speculative decoding"; "ReVolta
// 0.1.3", "Behaviour changes"), every page of the partition otherwise.
#pragma once

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

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
  if (rows >= kSmallUnitRows) return a.part_tokens;
  const int32_t per = (ctx + kSmallSplits - 1) / kSmallSplits;
  const int32_t p = ((per + kPage - 1) / kPage) * kPage;
  return min(max(p, a.part_small), a.part_tokens);
}

// Visible page ranges of partition [lo, hi) for a block of q_len queries.
__device__ __forceinline__ UnitPages unit_pages(const AttnLaunch& a, int32_t ctx, int32_t q_len,
                                                int32_t lo, int32_t hi) {
  UnitPages u{0, 0, 0, 0};
  if (lo >= hi) return u;
  if (a.window < 0) {
    u.p0a = lo / kPage;
    u.na = (hi + kPage - 1) / kPage - u.p0a;
    return u;
  }
  // keys any query sees: [0, sinks) U [ctx - q_len - W + 1, ctx)
  const int32_t wlo = max(ctx - q_len - a.window + 1, 0);
  const int32_t sa0 = lo, sa1 = min(hi, a.sinks);
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

// Key j visible to the query at position pos.
__device__ __forceinline__ bool key_visible(const AttnLaunch& a, int32_t j, int32_t pos) {
  return j <= pos && (a.window < 0 || pos - j < a.window || j < a.sinks);
}

// Block index -> logical unit id.  Consecutive workgroups are dispatched to the
// 8 XCDs round-robin; the remap places consecutive logical ids on one XCD so
// units that read the same pages (the sequences of a shared prefix, the row
// groups of one sequence) share that XCD's L2.  gridDim.x is a multiple of 8.
__device__ __forceinline__ int64_t logical_block() {
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t bid = blockIdx.x;
  return (bid % 8) * per_xcd + bid / 8;
}

struct UnitId {
  int32_t b, h, s, rg;
};

// logical id = ((s * Hkv + h) * row_groups + rg) * batch + b
__device__ __forceinline__ bool decode_unit(const AttnLaunch& a, int32_t row_groups, UnitId& u) {
  int64_t id = logical_block();
  const int64_t total = (int64_t)a.slots * a.hkv * row_groups * a.batch;
  if (id >= total) return false;
  u.b = (int32_t)(id % a.batch); id /= a.batch;
  u.rg = (int32_t)(id % row_groups); id /= row_groups;
  u.h = (int32_t)(id % a.hkv); id /= a.hkv;
  u.s = (int32_t)id;
  return true;
}

inline unsigned padded_grid(int64_t units) {
  return (unsigned)(((units + 7) / 8) * 8);
}

// Sequence preconditions that the host cannot check.  A violating sequence
// gets NaN rows instead of an out-of-bounds access.
__device__ __forceinline__ bool seq_ok(const AttnLaunch& a, int32_t ctx, int32_t q0, int32_t q1) {
  return ctx >= 0 && ctx <= a.max_ctx && q0 >= 0 && q1 >= q0 && q1 <= a.total_q &&
         q1 - q0 <= a.max_q_len && q1 - q0 <= ctx;
}

}  // namespace ra
