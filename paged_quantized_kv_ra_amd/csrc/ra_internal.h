// ra_internal.h -- host-side launch interface between the C ABI layer
// (ra_api.hip, which validates arguments) and the kernel translation units.
// Launchers assume validated arguments and return the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"

namespace ra {

// KV_I8T: INT8 codes with fp32 scales per (token, head) in separate planes.
enum KvKind { KV_F16 = 0, KV_E4M3 = 1, KV_I8 = 2, KV_I8T = 3 };

struct StoreLaunch {
  const void* k;
  const void* v;
  bool src_bf16;
  int64_t k_stride;      // elements
  int64_t v_stride;
  const int64_t* slots;
  int64_t num_tokens;
  void* k_cache;
  void* v_cache;
  int kv;                // KvKind
  int64_t num_pages;
  int hkv;
  int head_dim;
  float k_scale;
  float v_scale;
  float* k_scales;       // KV_I8T scale planes [num_pages][hkv][16]
  float* v_scales;
};
hipError_t launch_kv_store(const StoreLaunch& a, hipStream_t s);

// Packed QKV rows -> rotated Q, and rotated K + V quantised into the caches.
struct RopeLaunch {
  const void* qkv;       // [T][(hq + 2 hkv) * head_dim] fp16 / bf16
  bool src_bf16;
  int64_t qkv_stride;    // elements per token
  int64_t num_tokens;
  const int64_t* positions;
  const float* table;    // [max_pos][2][rot / 2] fp32: cos, then sin
  int64_t max_pos;
  int rot;               // rotary dims, a multiple of 16, <= head_dim
  void* q_out;           // [T][hq][head_dim], source dtype
  int64_t q_stride;      // elements per token
  const int64_t* slots;
  void* k_cache;
  void* v_cache;
  int kv;                // KvKind
  int64_t num_pages;
  int hq;
  int hkv;
  int head_dim;
  float k_scale;         // 1 unless per-layer E4M3 / INT8
  float v_scale;
  float* k_scales;       // KV_I8T scale planes
  float* v_scales;
};
hipError_t launch_qkv_rope(const RopeLaunch& a, hipStream_t s);

struct GatherLaunch {
  const void* cache;
  int which;             // 0 K, 1 V
  int kv;
  float scale;
  const int32_t* bt_row;
  int32_t ctx;
  int64_t num_pages;
  int hkv;
  int head_dim;
  float* out;
  const float* scales;   // KV_I8T scale plane
};
hipError_t launch_kv_gather(const GatherLaunch& a, hipStream_t s);

// Attention work description shared by both attention kernels.
struct AttnLaunch {
  const void* q;
  bool q_bf16;
  void* out;             // final output (direct write) or nullptr
  float* lse;            // final lse (direct write) or nullptr
  float* part_out;       // [slots][total_q][Hq][D] when slots > 1 or out == nullptr
  float* part_lse;       // [slots][total_q][Hq]
  uint8_t* k_cache;      // read; written by the fused store
  uint8_t* v_cache;
  int kv;                // KvKind
  float k_scale;         // 1 for FP16 caches
  float v_scale;
  const int32_t* block_tables;
  int32_t bt_stride;
  const int32_t* context_lens;
  const int32_t* qsl;
  int32_t batch;
  int32_t total_q;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  int64_t num_pages;
  int32_t max_q_len;
  int32_t min_q_len;     // host lower bound of every q_len (0: unknown); the grid's slot count relies on it
  int32_t max_ctx;
  float softmax_scale;
  int32_t window;        // < 0: none
  int32_t sinks;
  int32_t num_splits;    // > 0 explicit, 0 auto
  int32_t slots;         // partition slots per sequence in the grid
  int32_t part_tokens;   // auto mode: partition size (tokens) of units with >= kSmallUnitRows rows
  int32_t part_small;    // auto mode: partition size of units with fewer rows
  int32_t part_window;   // auto mode with a window: partition size over the window span
  bool direct;           // write out/lse directly (one slot)
  float* k_scales;       // KV_I8T scale planes [num_pages][hkv][16] (written by the fused store)
  float* v_scales;
  const int32_t* kv_pos0;  // [batch] global position of cache key 0, or nullptr (0)
  const int32_t* q_pos0;   // [batch] global position of the block's first query, or nullptr
  // fused store of the query tokens' own K/V rows (nullptr: none)
  const void* new_k;       // [total_q][hkv][head_dim] fp16 / bf16, new_k_stride elements per token
  const void* new_v;
  bool new_bf16;
  int64_t new_k_stride;
  int64_t new_v_stride;
  const int64_t* new_slots;  // [total_q] cache slot of each query token
  bool prefill;            // the prefill kernel takes the sequences prefill_sequence() selects
  int64_t q_stride;        // elements between query tokens
  const float* rope;       // RoPE table on the fused path, or nullptr
  int32_t rope_max_pos;
  int32_t rot;
  const int64_t* positions;
  // divisions by launch constants (filled by the decode/verify launcher):
  // g = hq / hkv, batch, hkv and the row groups per unit
  FastDiv fd_g, fd_batch, fd_hkv, fd_rg;
};

// Rows of a (sequence, KV head) unit: g * q_len, in 16-row matrix-core tiles
// (a decode unit with fewer rows uses one padded tile), at most
// kMfmaRowsPerBlock rows per workgroup.
constexpr int kMfmaRowsPerBlock = 48;   // rows beyond this split over row groups

// Automatic partitions (num_splits = 0).  Units with at least kSmallUnitRows
// rows use kAutoPartLarge tokens, or more when the sequence's own row groups
// already give kFillUnits workgroups or more across the KV heads (a long
// prefill chunk): its keys are then cut into only as many partitions as it
// takes to reach kFillUnits, down to one.  Smaller (decode) units take about
// kSmallSplits partitions of their own sequence's context, clamped to
// [kAutoPartSmall, kAutoPartLarge] tokens, so that a decode batch still fills
// the chip while long contexts keep few partials.  Either rule depends only on
// the sequence itself, never on the rest of the batch.
#ifndef RA_AUTO_PART_LARGE
#define RA_AUTO_PART_LARGE 2048
#endif
constexpr int kSmallUnitRows = 16;
constexpr int kAutoPartLarge = RA_AUTO_PART_LARGE;
constexpr int kAutoPartSmall = 512;
constexpr int kSmallSplits = 32;
constexpr int kFillUnits = 2048;
// Automatic partitions of a windowed block (window_left >= 0): only the sinks
// and the window span [pmin - W + 1, pmax] of the block hold visible keys, so
// the partitions cut that span, from its first page on, instead of [0, ctx):
// partition s covers [base + s P, base + (s + 1) P), base the first page of
// the span, and partition 0 also takes the sink keys below base.  P depends
// only on the window: about kWindowSplits partitions of a window, at least
// kAutoPartWindow tokens each.
constexpr int kAutoPartWindow = 256;
constexpr int kWindowSplits = 32;
__host__ __device__ inline int32_t window_partition_tokens(int32_t window) {
  const int32_t per = (window + kWindowSplits - 1) / kWindowSplits;
  const int32_t p = ((per + 15) / 16) * 16;
  return p > kAutoPartWindow ? p : kAutoPartWindow;
}

hipError_t launch_attn_mfma(const AttnLaunch& a, hipStream_t s);

// Long query blocks (prefill): a sequence with more than kPrefillMinRows rows
// per KV head is attended by the prefill kernel (rows split over waves, each
// 64-key tile decoded once per workgroup) when the call's constants allow it
// (FP8 E4M3 or INT8 with per-layer scales, head_dim 128, no window) ...
constexpr int kPrefillMinRows = 256;
// ... and whose block is at least half of its context (cold prompts and early
// chunks, whose causal row groups see few keys each; a short chunk after a
// long cached context streams better through the decode kernel, whose waves
// split the keys)
__host__ __device__ inline bool prefill_sequence(const AttnLaunch& a, int32_t rows, int32_t ctx, int32_t q_len) {
  return a.prefill && rows > kPrefillMinRows && (int64_t)ctx <= 2 * (int64_t)q_len;
}
bool prefill_kernel_serves(const AttnLaunch& a);
hipError_t launch_attn_prefill(const AttnLaunch& a, hipStream_t s);

struct MergeLaunch {
  const float* part_out;
  const float* part_lse;
  int32_t parts;
  int64_t rows;
  int32_t head_dim;
  void* out;
  int out_dtype;         // 1 f16, 2 bf16, 3 f32
  float* lse;
};
hipError_t launch_lse_merge(const MergeLaunch& a, hipStream_t s);

}  // namespace ra
