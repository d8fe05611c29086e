// ra_api.hip -- the C ABI of libra_kv.so: host-side validation and dispatch.
//
// Every host-checkable precondition is checked before anything is enqueued
// (the pages' engine rejects unsupported configurations before it loads
// anything and refuses E4M3 KV without calibrated scales in strict mode:
// ReVolta README, "Weight and KV formats"; "ReVolta 0.1.3", "Behaviour
// changes").  On failure the call returns a status, records a message for
// ra_last_error() and touches no output.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "ra_internal.h"
#include "ra_kv.h"

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }

int kv_kind(int32_t kv) {
  switch (kv) {
    case RA_KV_F16: return ra::KV_F16;
    case RA_KV_FP8_E4M3: return ra::KV_E4M3;
    case RA_KV_INT8: return ra::KV_I8;
    case RA_KV_INT8_TOKEN: return ra::KV_I8T;
    default: return -1;
  }
}

const char* kv_name(int32_t kv) {
  return kv == RA_KV_F16 ? "FP16" : kv == RA_KV_FP8_E4M3 ? "FP8 E4M3" : kv == RA_KV_INT8 ? "INT8" : "per-token INT8";
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool per_layer_scales(int32_t kv) { return kv == RA_KV_FP8_E4M3 || kv == RA_KV_INT8; }

// Split plan of an attention call: partition slots per sequence and, in the
// automatic mode, each kernel's fixed partition size.
struct Plan {
  int32_t slots;
  int32_t part_large, part_small;
  bool direct;
};

int32_t check_attn(const ra_attn_args* a, Plan* plan) {
  if (!a) return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: args is NULL");
  if (a->struct_size < sizeof(ra_attn_args))
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: struct_size %u < %zu (ABI %d)", a->struct_size,
                sizeof(ra_attn_args), RA_KV_ABI_VERSION);
  if (a->batch < 0 || a->total_q < 0)
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: batch (%d) and total_q (%d) must be >= 0", a->batch,
                a->total_q);
  if (a->q_dtype != RA_F16 && a->q_dtype != RA_BF16)
    return fail(RA_ERR_UNSUPPORTED, "ra_paged_attn: q_dtype %d is not RA_F16 or RA_BF16", a->q_dtype);
  if (kv_kind(a->kv_dtype) < 0)
    return fail(RA_ERR_UNSUPPORTED, "ra_paged_attn: unknown kv_dtype %d", a->kv_dtype);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "ra_paged_attn: head_dim %d is not 64 or 128", a->head_dim);
  if (a->page_size != RA_KV_PAGE_SIZE)
    return fail(RA_ERR_UNSUPPORTED, "ra_paged_attn: page_size %d is not 16", a->page_size);
  if (a->num_q_heads < 1 || a->num_kv_heads < 1 || a->num_q_heads % a->num_kv_heads != 0)
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: num_q_heads %d must be a positive multiple of num_kv_heads %d",
                a->num_q_heads, a->num_kv_heads);
  if (a->num_pages < 1) return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: num_pages must be >= 1");
  if (a->block_table_stride < 1) return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: block_table_stride must be >= 1");
  if (a->max_q_len < 1) return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: max_q_len must be >= 1");
  if (a->min_q_len < 0 || a->min_q_len > a->max_q_len)
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: min_q_len %d outside [0, max_q_len %d]", a->min_q_len,
                a->max_q_len);
  if (a->max_context_len < 0 || (int64_t)a->max_context_len > (int64_t)a->block_table_stride * RA_KV_PAGE_SIZE)
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: max_context_len %d outside [0, block_table_stride * 16 = %lld]",
                a->max_context_len, (long long)a->block_table_stride * RA_KV_PAGE_SIZE);
  if (!(std::isfinite(a->softmax_scale) && a->softmax_scale > 0.0f))
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: softmax_scale must be finite and > 0");
  if (per_layer_scales(a->kv_dtype) && !(good_scale(a->k_scale) && good_scale(a->v_scale)))
    return fail(RA_ERR_INVALID_ARG,
                "ra_paged_attn: %s KV needs finite positive per-layer k_scale and v_scale (got %g, %g); "
                "there is no fallback scale", kv_name(a->kv_dtype), (double)a->k_scale, (double)a->v_scale);
  if (a->num_sinks < 0) return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: num_sinks must be >= 0");
  if (a->num_splits < 0 || a->num_splits > RA_KV_MAX_SPLITS)
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: num_splits %d outside [0, %d]", a->num_splits,
                RA_KV_MAX_SPLITS);

  const int64_t g = a->num_q_heads / a->num_kv_heads;
  const int64_t rows_max = g * a->max_q_len;
  const int64_t rows_min = g * (a->min_q_len > 0 ? a->min_q_len : 1);
  plan->part_large = ra::kAutoPartLarge;
  plan->part_small = ra::kAutoPartSmall;
  if (a->num_splits > 0) {
    plan->slots = a->num_splits;
  } else {
    // the partition size is chosen per sequence by its row count; the grid
    // holds enough slots for either kind the bounds admit
    int64_t s = 1;
    if (rows_max >= ra::kSmallUnitRows) {
      // a sequence with rows >= kSmallUnitRows takes at most
      // ceil(kFillUnits / (Hkv * its row groups)) partitions; the fewest row
      // groups such a sequence can have bound them all
      const int64_t rg_lo = ceil_div(std::max<int64_t>(rows_min, ra::kSmallUnitRows), ra::kMfmaRowsPerBlock);
      const int64_t fill = ceil_div(ra::kFillUnits, a->num_kv_heads * rg_lo);
      s = std::max<int64_t>(s, std::min<int64_t>(ceil_div(a->max_context_len, plan->part_large), fill));
    }
    if (rows_min < ra::kSmallUnitRows) {
      // decode units: at most kSmallSplits partitions up to kSmallSplits * kAutoPartLarge
      // tokens, kAutoPartLarge-token partitions beyond
      const int64_t c = a->max_context_len;
      const int64_t sm = c <= (int64_t)ra::kSmallSplits * plan->part_large
                             ? std::min<int64_t>(ra::kSmallSplits, ceil_div(c, plan->part_small))
                             : ceil_div(c, plan->part_large);
      s = std::max<int64_t>(s, sm);
    }
    if (a->window_left >= 0) {
      // windowed blocks: partitions over the window span (from its first
      // page: up to 15 keys before it) plus, in partition 0, the sinks
      const int64_t span = std::min<int64_t>(a->max_context_len, (int64_t)a->window_left + a->max_q_len + 14);
      s = std::max<int64_t>(1, ceil_div(span, ra::window_partition_tokens(a->window_left)));
    }
    if (s > RA_KV_MAX_SPLITS * 64)
      return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: max_context_len %d needs too many partitions",
                  a->max_context_len);
    plan->slots = (int32_t)s;
  }
  plan->direct = plan->slots == 1 && a->out != nullptr;

  // the merge launches one workgroup per query row
  if ((int64_t)a->total_q * a->num_q_heads > (int64_t)0x7FFFFFF0)
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: total_q * num_q_heads above 2^31 - 16");
  // grid size: slots * Hkv * row groups * batch blocks
  const int64_t rg = ceil_div(rows_max, ra::kMfmaRowsPerBlock);
  if ((int64_t)plan->slots * a->num_kv_heads * rg * a->batch > (int64_t)0x7FFFFFF0)
    return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: problem needs more than 2^31 workgroups");
  return RA_OK;
}

int32_t check_attn_pointers(const ra_attn_args* a, const Plan& p) {
  if (!a->q || !a->k_cache || !a->v_cache || !a->block_tables || !a->context_lens || !a->query_start_loc)
    return fail(RA_ERR_INVALID_ARG,
                "ra_paged_attn: q, k_cache, v_cache, block_tables, context_lens and query_start_loc must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) || (a->out && !aligned16(a->out)))
    return fail(RA_ERR_MISALIGNED, "ra_paged_attn: q, out, k_cache and v_cache must be 16-byte aligned");
  if (a->q_token_stride != 0) {
    if (a->q_token_stride < (int64_t)a->num_q_heads * a->head_dim)
      return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: q_token_stride %lld smaller than num_q_heads * head_dim",
                  (long long)a->q_token_stride);
    if (a->q_token_stride % 8) return fail(RA_ERR_MISALIGNED, "ra_paged_attn: q_token_stride must be a multiple of 8");
  }
  if (a->rope_table) {
    if (!a->new_k)
      return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: rope_table needs the fused store (new_k, new_v, new_slots)");
    if (!a->positions) return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: rope_table needs positions");
    if (a->rotary_dim < 16 || a->rotary_dim % 16 || a->rotary_dim > a->head_dim)
      return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: rotary_dim %d must be a multiple of 16 in [16, head_dim]",
                  a->rotary_dim);
    if (a->rope_max_position < 1) return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: rope_max_position must be >= 1");
    if (!aligned16(a->rope_table)) return fail(RA_ERR_MISALIGNED, "ra_paged_attn: rope_table must be 16-byte aligned");
  }
  if (a->kv_dtype == RA_KV_INT8_TOKEN) {
    if (!a->k_scales || !a->v_scales)
      return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: per-token INT8 KV needs the k_scales and v_scales planes");
    if (!aligned16(a->k_scales) || !aligned16(a->v_scales))
      return fail(RA_ERR_MISALIGNED, "ra_paged_attn: k_scales and v_scales must be 16-byte aligned");
  }
  if (!p.direct) {
    if (!a->partial_out || !a->partial_lse)
      return fail(RA_ERR_WORKSPACE, "ra_paged_attn: %d partition slot(s) need partial_out and partial_lse%s",
                  p.slots, a->out ? "" : " (out is NULL)");
    if (a->partial_slots < p.slots)
      return fail(RA_ERR_WORKSPACE, "ra_paged_attn: partial buffers hold %d slots, %d needed", a->partial_slots,
                  p.slots);
    if (!aligned16(a->partial_out))
      return fail(RA_ERR_MISALIGNED, "ra_paged_attn: partial_out must be 16-byte aligned");
  }
  if (a->new_k) {   // fused store of the query tokens' K/V
    const int64_t g = a->num_q_heads / a->num_kv_heads;
    if (g * a->max_q_len > ra::kMfmaRowsPerBlock)
      return fail(RA_ERR_UNSUPPORTED,
                  "ra_paged_attn: the fused store needs (Hq / Hkv) * max_q_len <= %d (got %lld); store longer "
                  "blocks with ra_kv_store first", ra::kMfmaRowsPerBlock, (long long)(g * a->max_q_len));
    if (!a->new_v || !a->new_slots)
      return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: the fused store needs new_v and new_slots with new_k");
    if (a->new_dtype != RA_F16 && a->new_dtype != RA_BF16)
      return fail(RA_ERR_UNSUPPORTED, "ra_paged_attn: new_dtype %d is not RA_F16 or RA_BF16", a->new_dtype);
    const int64_t row = (int64_t)a->num_kv_heads * a->head_dim;
    if (a->new_k_stride < row || a->new_v_stride < row)
      return fail(RA_ERR_INVALID_ARG, "ra_paged_attn: new_k_stride / new_v_stride (%lld, %lld) smaller than "
                  "num_kv_heads * head_dim", (long long)a->new_k_stride, (long long)a->new_v_stride);
    if (!aligned16(a->new_k) || !aligned16(a->new_v) || (a->new_k_stride % 8) || (a->new_v_stride % 8))
      return fail(RA_ERR_MISALIGNED, "ra_paged_attn: new_k and new_v must be 16-byte aligned and their strides "
                  "multiples of 8");
  }
  return RA_OK;
}

ra::AttnLaunch make_launch(const ra_attn_args* a, const Plan& p) {
  ra::AttnLaunch L{};
  L.new_k = a->new_k;
  L.new_v = a->new_v;
  L.new_bf16 = a->new_dtype == RA_BF16;
  L.new_k_stride = a->new_k_stride;
  L.new_v_stride = a->new_v_stride;
  L.new_slots = a->new_slots;
  L.q_stride = a->q_token_stride > 0 ? a->q_token_stride : (int64_t)a->num_q_heads * a->head_dim;
  L.rope = a->rope_table;
  L.rope_max_pos = a->rope_max_position;
  L.rot = a->rotary_dim;
  L.positions = a->positions;
  L.q = a->q;
  L.q_bf16 = a->q_dtype == RA_BF16;
  L.out = p.direct ? a->out : nullptr;
  L.lse = p.direct ? a->lse : nullptr;
  L.part_out = a->partial_out;
  L.part_lse = a->partial_lse;
  L.k_cache = static_cast<uint8_t*>(a->k_cache);
  L.v_cache = static_cast<uint8_t*>(a->v_cache);
  L.kv = kv_kind(a->kv_dtype);
  const bool quant = per_layer_scales(a->kv_dtype);
  L.k_scale = quant ? a->k_scale : 1.0f;
  L.v_scale = quant ? a->v_scale : 1.0f;
  L.k_scales = a->kv_dtype == RA_KV_INT8_TOKEN ? a->k_scales : nullptr;
  L.v_scales = a->kv_dtype == RA_KV_INT8_TOKEN ? a->v_scales : nullptr;
  L.kv_pos0 = a->kv_pos0;
  L.q_pos0 = a->q_pos0;
  L.block_tables = a->block_tables;
  L.bt_stride = a->block_table_stride;
  L.context_lens = a->context_lens;
  L.qsl = a->query_start_loc;
  L.batch = a->batch;
  L.total_q = a->total_q;
  L.hq = a->num_q_heads;
  L.hkv = a->num_kv_heads;
  L.head_dim = a->head_dim;
  L.num_pages = a->num_pages;
  L.max_q_len = a->max_q_len;
  L.min_q_len = a->min_q_len;
  L.max_ctx = a->max_context_len;
  L.softmax_scale = a->softmax_scale;
  L.window = a->window_left < 0 ? -1 : a->window_left;
  L.sinks = a->window_left < 0 ? 0 : a->num_sinks;
  L.num_splits = a->num_splits;
  L.slots = p.slots;
  L.direct = p.direct;
  return L;
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry point: the fp32 partials of the split
// KV partitions live in this array instead of a caller's workspace.  Each GPU
// the library runs on holds its own copy for the life of the process.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on first use.
constexpr size_t kScratchBytes = (size_t)RA_KV_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int32_t scratch_address(const char* fn, float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_ERR_UNSUPPORTED, "%s: device index %d >= %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(RA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return RA_OK;
}

int32_t store_common(const char* fn, const void* k, const void* v, int32_t src_dtype, int64_t k_token_stride,
                     int64_t v_token_stride, const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                     void* v_cache, int32_t kv_dtype, float* k_scales, float* v_scales, int64_t num_pages,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size, float k_scale, float v_scale,
                     void* stream) {
  if (num_tokens < 0) return fail(RA_ERR_INVALID_ARG, "%s: num_tokens must be >= 0", fn);
  if (src_dtype != RA_F16 && src_dtype != RA_BF16)
    return fail(RA_ERR_UNSUPPORTED, "%s: src_dtype %d is not RA_F16 or RA_BF16", fn, src_dtype);
  if (kv_kind(kv_dtype) < 0) return fail(RA_ERR_UNSUPPORTED, "%s: unknown kv_dtype %d", fn, kv_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "%s: head_dim %d is not 64 or 128", fn, head_dim);
  if (page_size != RA_KV_PAGE_SIZE) return fail(RA_ERR_UNSUPPORTED, "%s: page_size %d is not 16", fn, page_size);
  if (num_kv_heads < 1) return fail(RA_ERR_INVALID_ARG, "%s: num_kv_heads must be >= 1", fn);
  if (num_pages < 1) return fail(RA_ERR_INVALID_ARG, "%s: num_pages must be >= 1", fn);
  if (per_layer_scales(kv_dtype) && !(good_scale(k_scale) && good_scale(v_scale)))
    return fail(RA_ERR_INVALID_ARG,
                "%s: %s KV needs finite positive per-layer k_scale and v_scale (got %g, %g); "
                "there is no fallback scale", fn, kv_name(kv_dtype), (double)k_scale, (double)v_scale);
  if (k_token_stride < (int64_t)num_kv_heads * head_dim || v_token_stride < (int64_t)num_kv_heads * head_dim)
    return fail(RA_ERR_INVALID_ARG, "%s: token strides (%lld, %lld) smaller than num_kv_heads * head_dim", fn,
                (long long)k_token_stride, (long long)v_token_stride);
  if (num_tokens > (int64_t)(1 << 30) / ((int64_t)num_kv_heads * (head_dim / 8)))
    return fail(RA_ERR_INVALID_ARG,
                "%s: num_tokens * num_kv_heads * head_dim / 8 must not exceed 2^30; store in chunks", fn);
  if (num_tokens == 0) return RA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(RA_ERR_INVALID_ARG, "%s: k, v, slot_mapping, k_cache and v_cache must be non-NULL", fn);
  if (kv_dtype == RA_KV_INT8_TOKEN && (!k_scales || !v_scales))
    return fail(RA_ERR_INVALID_ARG, "%s: k_scales and v_scales must be non-NULL", fn);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) || (k_token_stride % 8) ||
      (v_token_stride % 8) || (kv_dtype == RA_KV_INT8_TOKEN && (!aligned16(k_scales) || !aligned16(v_scales))))
    return fail(RA_ERR_MISALIGNED,
                "%s: k, v, k_cache, v_cache (and scale planes) must be 16-byte aligned and token strides "
                "multiples of 8", fn);
  const bool quant = per_layer_scales(kv_dtype);
  ra::StoreLaunch L{k, v, src_dtype == RA_BF16, k_token_stride, v_token_stride, slot_mapping, num_tokens,
                    k_cache, v_cache, kv_kind(kv_dtype), num_pages, num_kv_heads, head_dim,
                    quant ? k_scale : 1.0f, quant ? v_scale : 1.0f, k_scales, v_scales};
  const hipError_t e = ra::launch_kv_store(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return RA_OK;
}

}  // namespace

extern "C" {

int32_t ra_kv_store(const void* k, const void* v, int32_t src_dtype, int64_t k_token_stride,
                    int64_t v_token_stride, const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                    void* v_cache, int32_t kv_dtype, int64_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                    int32_t page_size, float k_scale, float v_scale, void* stream) {
  if (kv_dtype == RA_KV_INT8_TOKEN)
    return fail(RA_ERR_UNSUPPORTED, "ra_kv_store: per-token INT8 KV is stored with ra_kv_store_int8_token");
  return store_common("ra_kv_store", k, v, src_dtype, k_token_stride, v_token_stride, slot_mapping, num_tokens,
                      k_cache, v_cache, kv_dtype, nullptr, nullptr, num_pages, num_kv_heads, head_dim, page_size,
                      k_scale, v_scale, stream);
}

int32_t ra_kv_store_int8_token(const void* k, const void* v, int32_t src_dtype, int64_t k_token_stride,
                               int64_t v_token_stride, const int64_t* slot_mapping, int64_t num_tokens,
                               void* k_cache, void* v_cache, float* k_scales, float* v_scales, int64_t num_pages,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size, void* stream) {
  return store_common("ra_kv_store_int8_token", k, v, src_dtype, k_token_stride, v_token_stride, slot_mapping,
                      num_tokens, k_cache, v_cache, RA_KV_INT8_TOKEN, k_scales, v_scales, num_pages, num_kv_heads,
                      head_dim, page_size, 1.0f, 1.0f, stream);
}

int32_t ra_paged_attn_workspace(const ra_attn_args* args, int32_t* slots, int64_t* partial_out_floats,
                                int64_t* partial_lse_floats) {
  Plan p{};
  const int32_t st = check_attn(args, &p);
  if (st != RA_OK) return st;
  const int64_t rows = (int64_t)args->total_q * args->num_q_heads;
  if (slots) *slots = p.slots;
  if (partial_out_floats) *partial_out_floats = p.direct ? 0 : (int64_t)p.slots * rows * args->head_dim;
  if (partial_lse_floats) *partial_lse_floats = p.direct ? 0 : (int64_t)p.slots * rows;
  return RA_OK;
}

int32_t ra_paged_attn(const ra_attn_args* args, void* stream) {
  Plan p{};
  int32_t st = check_attn(args, &p);
  if (st != RA_OK) return st;
  if (args->batch == 0 || args->total_q == 0) return RA_OK;
  st = check_attn_pointers(args, p);
  if (st != RA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  ra::AttnLaunch L = make_launch(args, p);
  hipError_t e = hipSuccess;
  L.part_tokens = p.part_large;
  L.part_small = p.part_small;
  L.part_window = args->window_left >= 0 ? ra::window_partition_tokens(args->window_left) : 0;
  // long query blocks (more than kPrefillMinRows rows per KV head) go to the
  // prefill kernel when the call's constants allow; the decode kernel's grid
  // then covers only the shorter blocks
  const int32_t g = args->num_q_heads / args->num_kv_heads;
  L.prefill = ra::prefill_kernel_serves(L) && (int64_t)g * args->max_q_len > ra::kPrefillMinRows;
  // the decode kernel is skipped only when the host bounds prove every
  // sequence is the prefill kernel's (a batch of cold prompts)
  const bool all_prefill = L.prefill && (int64_t)g * args->min_q_len > ra::kPrefillMinRows &&
                           (int64_t)args->max_context_len <= 2 * (int64_t)args->min_q_len;
  if (!all_prefill) {
    e = ra::launch_attn_mfma(L, s);
    if (e != hipSuccess)
      return fail(RA_ERR_HIP, "ra_paged_attn: attention kernel launch failed: %s", hipGetErrorString(e));
  }
  if (L.prefill) {
    e = ra::launch_attn_prefill(L, s);
    if (e != hipSuccess)
      return fail(RA_ERR_HIP, "ra_paged_attn: prefill kernel launch failed: %s", hipGetErrorString(e));
  }
  if (!p.direct && args->out) {
    ra::MergeLaunch M{args->partial_out, args->partial_lse, p.slots, (int64_t)args->total_q * args->num_q_heads,
                      args->head_dim, args->out, args->q_dtype, args->lse};
    e = ra::launch_lse_merge(M, s);
    if (e != hipSuccess) return fail(RA_ERR_HIP, "ra_paged_attn: merge launch failed: %s", hipGetErrorString(e));
  }
  return RA_OK;
}

int32_t ra_paged_attn_noalloc(const ra_attn_args* args, void* stream) {
  static const char* fn = "ra_paged_attn_noalloc";
  Plan p{};
  int32_t st = check_attn(args, &p);
  if (st != RA_OK) return st;
  if (args->batch == 0 || args->total_q == 0) return RA_OK;
  if (!args->out)
    return fail(RA_ERR_INVALID_ARG, "%s: out must be non-NULL (the partials stay in the library's scratch)", fn);
  ra_attn_args a = *args;
  if (!p.direct) {
    // partial_out [slots][rows][D] then partial_lse [slots][rows]; rows * D is
    // a multiple of 64 floats, so the lse part stays 16-byte aligned
    const int64_t rows = (int64_t)args->total_q * args->num_q_heads;
    const int64_t out_floats = (int64_t)p.slots * rows * args->head_dim;
    const int64_t bytes = (out_floats + (int64_t)p.slots * rows) * (int64_t)sizeof(float);
    if (bytes > (int64_t)kScratchBytes)
      return fail(RA_ERR_WORKSPACE,
                  "%s: %d partition slot(s) x %lld rows need %lld bytes of partials, more than the %zu-byte "
                  "static scratch; call ra_paged_attn with a workspace", fn, p.slots, (long long)rows,
                  (long long)bytes, kScratchBytes);
    float* base = nullptr;
    st = scratch_address(fn, &base);
    if (st != RA_OK) return st;
    a.partial_out = base;
    a.partial_lse = base + out_floats;
    a.partial_slots = p.slots;
  }
  return ra_paged_attn(&a, stream);
}

int32_t ra_lse_merge(const float* partial_out, const float* partial_lse, int32_t num_partitions, int64_t rows,
                     int32_t head_dim, void* out, int32_t out_dtype, float* lse_out, void* stream) {
  if (num_partitions < 1 || num_partitions > RA_KV_MAX_SPLITS)
    return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: num_partitions %d outside [1, %d]", num_partitions,
                RA_KV_MAX_SPLITS);
  if (rows < 0) return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: rows must be >= 0");
  if (head_dim != 64 && head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "ra_lse_merge: head_dim %d is not 64 or 128", head_dim);
  if (out_dtype != RA_F16 && out_dtype != RA_BF16 && out_dtype != RA_F32)
    return fail(RA_ERR_UNSUPPORTED, "ra_lse_merge: out_dtype %d unknown", out_dtype);
  if (rows == 0) return RA_OK;
  if (rows > (int64_t)0x7FFFFFF0) return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: too many rows");   // one workgroup per row
  if (!partial_out || !partial_lse || !out)
    return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: partial_out, partial_lse and out must be non-NULL");
  if (!aligned16(partial_out) || !aligned16(out))
    return fail(RA_ERR_MISALIGNED, "ra_lse_merge: partial_out and out must be 16-byte aligned");
  ra::MergeLaunch M{partial_out, partial_lse, num_partitions, rows, head_dim, out, out_dtype, lse_out};
  const hipError_t e = ra::launch_lse_merge(M, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "ra_lse_merge: launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}

int32_t ra_kv_gather_dequant(const void* cache, int32_t which, int32_t kv_dtype, float scale, const float* scales,
                             const int32_t* block_table_row, int32_t ctx, int64_t num_pages, int32_t num_kv_heads,
                             int32_t head_dim, float* out, void* stream) {
  if (which != 0 && which != 1) return fail(RA_ERR_INVALID_ARG, "ra_kv_gather_dequant: which must be 0 (K) or 1 (V)");
  if (kv_kind(kv_dtype) < 0) return fail(RA_ERR_UNSUPPORTED, "ra_kv_gather_dequant: unknown kv_dtype %d", kv_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "ra_kv_gather_dequant: head_dim %d is not 64 or 128", head_dim);
  if (ctx < 0 || num_pages < 1 || num_kv_heads < 1)
    return fail(RA_ERR_INVALID_ARG, "ra_kv_gather_dequant: ctx >= 0, num_pages >= 1 and num_kv_heads >= 1 required");
  if (per_layer_scales(kv_dtype) && !good_scale(scale))
    return fail(RA_ERR_INVALID_ARG, "ra_kv_gather_dequant: scale must be finite and > 0");
  if (ctx == 0) return RA_OK;
  if (!cache || !block_table_row || !out)
    return fail(RA_ERR_INVALID_ARG, "ra_kv_gather_dequant: cache, block_table_row and out must be non-NULL");
  if (!aligned16(cache)) return fail(RA_ERR_MISALIGNED, "ra_kv_gather_dequant: cache must be 16-byte aligned");
  if (kv_dtype == RA_KV_INT8_TOKEN && !scales)
    return fail(RA_ERR_INVALID_ARG, "ra_kv_gather_dequant: per-token INT8 KV needs its scale plane");
  ra::GatherLaunch G{cache, which, kv_kind(kv_dtype), per_layer_scales(kv_dtype) ? scale : 1.0f, block_table_row,
                     ctx, num_pages, num_kv_heads, head_dim, out, scales};
  const hipError_t e = ra::launch_kv_gather(G, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "ra_kv_gather_dequant: launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}

int32_t ra_rope_table(float* out, int32_t max_position, int32_t rotary_dim, double base, double factor,
                      int32_t original_max_position, double beta_fast, double beta_slow) {
  if (!out) return fail(RA_ERR_INVALID_ARG, "ra_rope_table: out must be non-NULL");
  if (max_position < 1 || rotary_dim < 2 || rotary_dim % 2)
    return fail(RA_ERR_INVALID_ARG, "ra_rope_table: max_position >= 1 and an even rotary_dim >= 2 required");
  if (!(std::isfinite(base) && base > 1.0) || !std::isfinite(factor))
    return fail(RA_ERR_INVALID_ARG, "ra_rope_table: base must be finite and > 1, factor finite");
  const bool yarn = factor > 1.0;
  if (yarn && !(original_max_position >= 1 && std::isfinite(beta_fast) && std::isfinite(beta_slow) &&
                beta_fast > 0.0 && beta_slow > 0.0))
    return fail(RA_ERR_INVALID_ARG, "ra_rope_table: YaRN needs original_max_position >= 1 and positive betas");
  const int half = rotary_dim / 2;
  double lo = 0.0, hi = 1.0;
  if (yarn) {
    // the dim whose wavelength fits `beta` times into the original context
    const auto dim_for = [&](double beta) {
      return rotary_dim * std::log(original_max_position / (beta * 2.0 * M_PI)) / (2.0 * std::log(base));
    };
    lo = std::max(std::floor(dim_for(beta_fast)), 0.0);
    hi = std::min(std::ceil(dim_for(beta_slow)), (double)(rotary_dim - 1));
    if (hi == lo) hi = lo + 0.001;
  }
  const double temp = yarn ? 0.1 * std::log(factor) + 1.0 : 1.0;
  std::vector<double> freq(half);
  for (int i = 0; i < half; ++i) {
    const double f = std::pow(base, -2.0 * i / rotary_dim);
    const double ramp = yarn ? std::min(std::max((i - lo) / (hi - lo), 0.0), 1.0) : 0.0;
    freq[i] = f * (1.0 - ramp) + (f / (yarn ? factor : 1.0)) * ramp;
  }
  for (int64_t p = 0; p < max_position; ++p) {
    float* row = out + p * rotary_dim;
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * freq[i];
      row[i] = (float)(std::cos(ang) * temp);
      row[half + i] = (float)(std::sin(ang) * temp);
    }
  }
  return RA_OK;
}

int32_t ra_qkv_rope_store(const ra_qkv_rope_args* a, void* stream) {
  const char* fn = "ra_qkv_rope_store";
  if (!a) return fail(RA_ERR_INVALID_ARG, "%s: args is NULL", fn);
  if (a->struct_size < sizeof(ra_qkv_rope_args))
    return fail(RA_ERR_INVALID_ARG, "%s: struct_size %u < %zu (ABI %d)", fn, a->struct_size,
                sizeof(ra_qkv_rope_args), RA_KV_ABI_VERSION);
  if (a->num_tokens < 0) return fail(RA_ERR_INVALID_ARG, "%s: num_tokens must be >= 0", fn);
  if (a->src_dtype != RA_F16 && a->src_dtype != RA_BF16)
    return fail(RA_ERR_UNSUPPORTED, "%s: src_dtype %d is not RA_F16 or RA_BF16", fn, a->src_dtype);
  if (kv_kind(a->kv_dtype) < 0) return fail(RA_ERR_UNSUPPORTED, "%s: unknown kv_dtype %d", fn, a->kv_dtype);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "%s: head_dim %d is not 64 or 128", fn, a->head_dim);
  if (a->page_size != RA_KV_PAGE_SIZE)
    return fail(RA_ERR_UNSUPPORTED, "%s: page_size %d is not 16", fn, a->page_size);
  if (a->num_q_heads < 1 || a->num_kv_heads < 1)
    return fail(RA_ERR_INVALID_ARG, "%s: num_q_heads and num_kv_heads must be >= 1", fn);
  if (a->num_pages < 1) return fail(RA_ERR_INVALID_ARG, "%s: num_pages must be >= 1", fn);
  if (a->rotary_dim < 16 || a->rotary_dim % 16 || a->rotary_dim > a->head_dim)
    return fail(RA_ERR_INVALID_ARG, "%s: rotary_dim %d must be a multiple of 16 in [16, head_dim]", fn,
                a->rotary_dim);
  if (a->max_position < 1) return fail(RA_ERR_INVALID_ARG, "%s: max_position must be >= 1", fn);
  if (per_layer_scales(a->kv_dtype) && !(good_scale(a->k_scale) && good_scale(a->v_scale)))
    return fail(RA_ERR_INVALID_ARG,
                "%s: %s KV needs finite positive per-layer k_scale and v_scale (got %g, %g); "
                "there is no fallback scale", fn, kv_name(a->kv_dtype), (double)a->k_scale, (double)a->v_scale);
  const int64_t h3 = (int64_t)a->num_q_heads + 2 * (int64_t)a->num_kv_heads;
  if (a->qkv_token_stride < h3 * a->head_dim)
    return fail(RA_ERR_INVALID_ARG, "%s: qkv_token_stride %lld smaller than (Hq + 2 Hkv) * head_dim", fn,
                (long long)a->qkv_token_stride);
  if (a->q_token_stride < (int64_t)a->num_q_heads * a->head_dim)
    return fail(RA_ERR_INVALID_ARG, "%s: q_token_stride %lld smaller than num_q_heads * head_dim", fn,
                (long long)a->q_token_stride);
  if (a->num_tokens > (int64_t)(1 << 30) / (h3 * (a->head_dim / 16)))
    return fail(RA_ERR_INVALID_ARG, "%s: num_tokens * (Hq + 2 Hkv) * head_dim / 16 must not exceed 2^30; "
                "call in chunks", fn);
  if (a->num_tokens == 0) return RA_OK;
  if (!a->qkv || !a->positions || !a->rope_table || !a->q_out || !a->slot_mapping || !a->k_cache || !a->v_cache)
    return fail(RA_ERR_INVALID_ARG, "%s: qkv, positions, rope_table, q_out, slot_mapping, k_cache and v_cache "
                "must be non-NULL", fn);
  const bool tok = a->kv_dtype == RA_KV_INT8_TOKEN;
  if (tok && (!a->k_scales || !a->v_scales))
    return fail(RA_ERR_INVALID_ARG, "%s: per-token INT8 KV needs the k_scales and v_scales planes", fn);
  if (!aligned16(a->qkv) || !aligned16(a->q_out) || !aligned16(a->rope_table) || !aligned16(a->k_cache) ||
      !aligned16(a->v_cache) || (a->qkv_token_stride % 8) || (a->q_token_stride % 8) ||
      (tok && (!aligned16(a->k_scales) || !aligned16(a->v_scales))))
    return fail(RA_ERR_MISALIGNED, "%s: qkv, q_out, rope_table, the caches (and scale planes) must be 16-byte "
                "aligned and token strides multiples of 8", fn);
  const bool quant = per_layer_scales(a->kv_dtype);
  ra::RopeLaunch L{a->qkv, a->src_dtype == RA_BF16, a->qkv_token_stride, a->num_tokens, a->positions,
                   a->rope_table, a->max_position, a->rotary_dim, a->q_out, a->q_token_stride, a->slot_mapping,
                   a->k_cache, a->v_cache, kv_kind(a->kv_dtype), a->num_pages, a->num_q_heads, a->num_kv_heads,
                   a->head_dim, quant ? a->k_scale : 1.0f, quant ? a->v_scale : 1.0f, a->k_scales, a->v_scales};
  const hipError_t e = ra::launch_qkv_rope(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return RA_OK;
}

const char* ra_last_error(void) { return g_err.c_str(); }

int32_t ra_abi_version(void) { return RA_KV_ABI_VERSION * 1000 + RA_KV_LAYOUT_ID; }

}  // extern "C"
