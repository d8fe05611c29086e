/*
 * ra_kv.h -- paged, quantized-KV decode/verify attention for AMD MI355X (gfx950).
 *
 * C ABI of libra_kv.so.  Three operations make up one decode/verify step of a
 * serving engine's attention layer:
 *
 *   ra_kv_store     quantise this step's new K/V rows and scatter them into
 *                   16-token pages of the KV cache;
 *   ra_paged_attn   attention of each sequence's query block (1 + k verify
 *                   tokens, causal inside the block, grouped query heads) over
 *                   its paged, quantised context, optionally split into KV
 *                   partitions that emit partial (out, lse) pairs;
 *   ra_lse_merge    combine partial (out, lse) pairs by log-sum-exp;
 *   ra_qkv_rope_store  one pass over the new tokens' packed QKV rows: rotary
 *                   position embedding of Q and K (YaRN table), Q written
 *                   for attention, K/V quantised into the pages;
 *   ra_rope_table   (host) the RoPE / YaRN cos-sin table it reads.
 *
 * Sources of the operations (the ReVolta pages):
 *   - ReVolta README, intro list and "Weight and KV formats": the KV cache is
 *     stored as FP8 E4M3, FP16 or INT8 and converted to FP16 for the
 *     arithmetic; E4M3 uses calibrated per-layer K and V scales and strict mode
 *     refuses to run without them.
 *   - "ReVolta 0.1.3" release notes, "Known issues": 16-token kernel pages.
 *   - ReVolta README, intro list and "Quick start": MTP4 verifies 1 + 4 tokens
 *     per sequence per step; prefix caching shares pages between sequences;
 *     decode context parallelism (DCP2) splits one sequence's context and
 *     combines the parts' partial attention.
 *   - ReVolta README, "DFlash2 speculative decoding", and "ReVolta 0.1.3",
 *     "Behaviour changes": sliding-window and attention-sink layers.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer; the library never allocates or frees memory, never synchronises,
 *     and keeps no state other than a thread-local error message.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns at once.  Calls are safe from several host threads.
 *   - Every condition checkable on the host is checked BEFORE anything is
 *     enqueued.  On failure a non-zero ra_status is returned, ra_last_error()
 *     describes it, and no output byte is changed.
 *   - Conditions on device-resident data (block-table entries, context and
 *     query lengths, slots) cannot be checked on the host.  The kernels never
 *     read or write out of bounds because of them: an attention row whose
 *     sequence violates them is written as NaN (out and lse), and a store
 *     slot outside the cache is skipped.
 *   - Attention results are deterministic and, for each sequence, bitwise
 *     independent of the other sequences in the batch and of the batch size.
 *
 * Paged KV cache layout (identifier RA_KV_LAYOUT_ID)
 *   K and V are separate caches.  Each holds num_pages * Hkv blocks of
 *   16 * D * e bytes (e = 2 for FP16, 1 for E4M3 and INT8); block (page, head)
 *   starts at byte (page * Hkv + head) * 16 * D * e.  Within a block, element
 *   (t, d) -- token t of the page (0..15), dimension d -- is at byte
 *       offset = (b / 16) * 1024 + lane * 16 + (b % 16)
 *   with
 *       K:  lane = 16 * (d / (D/4)) + t,          b = (d % (D/4)) * e
 *       V:  lane = 16 * (t / 4) + d / (D/16),     b = ((d % (D/16)) * 4 + t % 4) * e
 *   Elements are little-endian FP16 bit patterns, E4M3 bytes or two's-complement
 *   int8.  A token's slot is page * 16 + t.  (Each 1 KiB of a block is one
 *   64-lane x 16-byte load of a wavefront and lands in registers already in
 *   the operand order of the gfx950 16x16x32 f16 matrix instruction.)
 *
 * Codes (the store's quantiser; bit-exact)
 *   y = fp32(x) / fp32(scale), IEEE correctly rounded (x is the fp16/bf16 input);
 *   E4M3 (OCP E4M3FN, bias 7, max 448): saturate to +-448 (+-inf -> +-448),
 *     round to nearest, ties to even code, sign of y kept (-0 -> 0x80),
 *     NaN -> 0x7F | sign;
 *   INT8: round half to even, clamp to [-127, 127], NaN -> 0;
 *   FP16 cache: IEEE round-to-nearest-even of fp32(x), no scale.
 *   Dequantised value = fp32(decode(code)) * fp32(scale).
 *
 * INT8 with runtime scales per token and head (RA_KV_INT8_TOKEN; ReVolta
 * README, "Weight and KV formats", INT8 KV): each (token, head) row of
 * head_dim values gets scale = fp32(max |x|) / fp32(127), correctly rounded,
 * and is quantised as INT8 above with that scale (a row of zeros: scale 0,
 * codes 0).  The codes use the INT8 layout; the scales live in two fp32
 * planes beside the caches, k_scales and v_scales [num_pages][num_kv_heads][16],
 * the scale of (slot, head) at float index (page * num_kv_heads + head) * 16
 * + slot % 16.
 */
#ifndef RA_KV_H_
#define RA_KV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_KV_ABI_VERSION 7
#define RA_KV_LAYOUT_ID 1
#define RA_KV_PAGE_SIZE 16
#define RA_KV_MAX_SPLITS 4096

/* Status codes (int32_t return value of every entry point). */
enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent argument  */
  RA_ERR_UNSUPPORTED = 2,   /* head_dim not 64/128, page size not 16, dtype   */
  RA_ERR_MISALIGNED = 3,    /* a pointer or stride breaks 16-byte alignment   */
  RA_ERR_WORKSPACE = 4,     /* partial buffers missing or too small           */
  RA_ERR_HIP = 5            /* the HIP runtime refused the launch             */
};

/* Activation dtypes (queries, new K/V, attention output). */
enum { RA_F16 = 1, RA_BF16 = 2, RA_F32 = 3 };

/* KV cache element formats. */
enum { RA_KV_F16 = 1, RA_KV_FP8_E4M3 = 2, RA_KV_INT8 = 3, RA_KV_INT8_TOKEN = 4 };

/*
 * ra_kv_store -- quantise new K/V rows and scatter them into the paged caches.
 *
 * k, v          [num_tokens][num_kv_heads][head_dim] of src_dtype (RA_F16 or
 *               RA_BF16); the token stride is k_token_stride / v_token_stride
 *               ELEMENTS (so K/V may be views into a fused QKV buffer), heads
 *               are head_dim apart, dims contiguous.  16-byte aligned, strides
 *               multiples of 8.
 * slot_mapping  int64 [num_tokens]; slot = page * 16 + token-in-page.  slot < 0
 *               skips the token (padding).  Slots >= num_pages * 16 are
 *               skipped.  Slots must be unique within one call.
 * k_cache, v_cache  caches in the layout above, kv_dtype elements, 16-byte
 *               aligned, num_pages * num_kv_heads * 16 * head_dim elements each.
 * k_scale, v_scale  (host) per-layer scales; required finite and > 0 for
 *               E4M3 / INT8 (there is no fallback to 1.0), ignored for FP16.
 * head_dim in {64, 128}; page_size must be 16.  One call stores at most
 * 2^30 / (num_kv_heads * head_dim / 8) tokens (RA_ERR_INVALID_ARG beyond:
 * store in chunks).
 * Bytes of tokens not stored are left unchanged.
 */
int32_t ra_kv_store(const void* k, const void* v, int32_t src_dtype,
                    int64_t k_token_stride, int64_t v_token_stride,
                    const int64_t* slot_mapping, int64_t num_tokens,
                    void* k_cache, void* v_cache, int32_t kv_dtype,
                    int64_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                    int32_t page_size, float k_scale, float v_scale, void* stream);

/*
 * ra_kv_store_int8_token -- ra_kv_store for RA_KV_INT8_TOKEN caches: quantise
 * new K/V rows with their own per-(token, head) scales (layout and rule above),
 * scatter the codes into k_cache / v_cache and the scales into k_scales /
 * v_scales.  Arguments as ra_kv_store, with the scale planes (fp32,
 * num_pages * num_kv_heads * 16 each, 16-byte aligned) in place of the
 * per-layer scales.  Non-finite inputs give unspecified codes.
 */
int32_t ra_kv_store_int8_token(const void* k, const void* v, int32_t src_dtype,
                               int64_t k_token_stride, int64_t v_token_stride,
                               const int64_t* slot_mapping, int64_t num_tokens,
                               void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                               int64_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, void* stream);

/*
 * ra_rope_table -- (host only; enqueues nothing) fill the HOST buffer
 * out [max_position][2][rotary_dim / 2] fp32 with cos(p * f_i) and
 * sin(p * f_i) times the attention temperature m, computed in double and
 * rounded once.  Plain RoPE (factor <= 1): f_i = base^(-2 i / rotary_dim),
 * m = 1.  YaRN (factor > 1; ReVolta README, "Quick start", step 2: factor 2
 * over original_max_position = 262,144 positions): with
 * d(beta) = rotary_dim * ln(original_max_position / (2 pi beta)) / (2 ln base),
 * lo = max(floor(d(beta_fast)), 0), hi = min(ceil(d(beta_slow)), rotary_dim - 1)
 * and ramp_i = clamp((i - lo) / (hi - lo), 0, 1):
 * f_i = base^(-2 i / rotary_dim) * (1 - ramp_i + ramp_i / factor) and
 * m = 0.1 ln(factor) + 1.  (beta_fast = 32, beta_slow = 1 are the usual
 * values.)  rotary_dim even and > 0; max_position >= 1; base > 1.  Copy the
 * table to device memory for ra_qkv_rope_store.
 */
int32_t ra_rope_table(float* out, int32_t max_position, int32_t rotary_dim, double base,
                      double factor, int32_t original_max_position, double beta_fast,
                      double beta_slow);

/*
 * Arguments of ra_qkv_rope_store.  Set struct_size = sizeof(ra_qkv_rope_args).
 *
 * qkv         [num_tokens] rows of (num_q_heads + 2 * num_kv_heads) * head_dim
 *             src_dtype elements (RA_F16 or RA_BF16): Q heads, then K heads,
 *             then V heads, as a fused QKV projection writes them; rows are
 *             qkv_token_stride ELEMENTS apart.
 * positions   int64 [num_tokens]: each token's position in its sequence.
 * rope_table  fp32 [max_position][2][rotary_dim / 2] (see ra_rope_table).
 *             rotary_dim is a multiple of 16 and <= head_dim; dim i < R/2
 *             pairs with dim i + R/2 (R = rotary_dim) and the pair turns as
 *             y_i = x_i cos - x_{i+R/2} sin, y_{i+R/2} = x_{i+R/2} cos + x_i sin,
 *             in fp32 without fused multiply-add; dims >= R pass through.
 * q_out       [num_tokens][num_q_heads][head_dim] src_dtype (rounded to
 *             nearest even), rows q_token_stride ELEMENTS apart: the rotated
 *             queries, ready for ra_paged_attn.
 * slot_mapping, k_cache, v_cache, kv_dtype, k_scale, v_scale, k_scales,
 *             v_scales, num_pages: as ra_kv_store (per-layer scales for E4M3 /
 *             INT8, scale planes for RA_KV_INT8_TOKEN, neither for FP16); the
 *             rotated K rows and the V rows are quantised and stored exactly
 *             as ra_kv_store stores fp32 values.
 * head_dim in {64, 128}; page_size 16.  qkv, q_out, rope_table, the caches
 * and the planes are 16-byte aligned; strides are multiples of 8.  A token
 * whose position is outside [0, max_position) gets a NaN Q row and stores
 * nothing; slot < 0 (or >= num_pages * 16) stores nothing, Q is still
 * written.  One call handles at most 2^30 / ((num_q_heads + 2 *
 * num_kv_heads) * head_dim / 16) tokens.
 * (ReVolta README, DFlash2 settings list: the verifier's Q/K/V rows packed
 * by one copy kernel; "Quick start", step 2: YaRN position scaling.)
 */
typedef struct ra_qkv_rope_args {
  uint32_t struct_size;
  const void* qkv;
  int32_t src_dtype;
  int64_t qkv_token_stride;
  int64_t num_tokens;
  const int64_t* positions;
  const float* rope_table;
  int32_t max_position;
  int32_t rotary_dim;
  void* q_out;
  int64_t q_token_stride;
  const int64_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  int32_t kv_dtype;
  float k_scale;
  float v_scale;
  float* k_scales;
  float* v_scales;
  int64_t num_pages;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
} ra_qkv_rope_args;

int32_t ra_qkv_rope_store(const ra_qkv_rope_args* args, void* stream);

/*
 * Arguments of ra_paged_attn.  Set struct_size = sizeof(ra_attn_args).
 *
 * For sequence b: q_len_b = query_start_loc[b+1] - query_start_loc[b] and
 * ctx_b = context_lens[b], which INCLUDES this step's q_len_b tokens (store
 * them first, or pass them for the fused store below).  Query i of the block sits at position pos = ctx_b - q_len_b + i;
 * query head h reads KV head h / (num_q_heads / num_kv_heads).  Key j is
 * visible iff j <= pos and (window_left < 0 or pos - j < window_left or
 * j < num_sinks).  out = softmax(softmax_scale * q . k) v over visible keys,
 * lse = natural log of the softmax denominator (max-shifted form); a row with
 * no visible key gets out = 0, lse = -inf.
 *
 * Context parallelism (ReVolta README, "Quick start", DCP2): a GPU may hold
 * only a range of each sequence's keys.  Then kv_pos0[b] gives the global
 * position of the cache's key 0 and q_pos0[b] the global position of the
 * block's first query (query i at q_pos0[b] + i); ctx_b counts the keys this
 * cache holds (q_len_b <= ctx_b is then not required, and a GPU holding
 * none of a sequence's keys passes ctx_b = 0).  Visibility, windows and sinks
 * use global positions.  Each GPU's (out, lse), with out = NULL its partials,
 * combine across GPUs with ra_lse_merge.  NULL arrays mean kv_pos0 = 0 and
 * q_pos0 = ctx_b - q_len_b.
 *
 * Splitting: the keys of sequence b are cut into partitions of P_b tokens;
 * num_splits = S > 0 gives P_b = 16 * ceil(ceil(ctx_b / S) / 16) (S slots per
 * sequence); num_splits = 0 lets the library choose P_b from the sequence's
 * own ctx_b and q_len_b and the head counts, never from the rest of the batch:
 *   rows_b = (Hq / Hkv) * q_len_b < 16 (decode): about 32 partitions of ctx_b,
 *     P_b clamped to [512, 2048] tokens;
 *   rows_b >= 16: P_b = max(2048, 16 * ceil(ceil(ctx_b / n_b) / 16)) with
 *     n_b = ceil(2048 / u_b) partitions wanted, u_b = Hkv * ceil(rows_b / 48)
 *     workgroups per partition (n_b = 1 once u_b >= 2048: a long prefill
 *     chunk is attended in one pass);
 *   with a window (window_left >= 0), whatever the rows: only the sinks and
 *     the window span hold visible keys, so the partitions cut that span
 *     instead of [0, ctx_b): with base = 16 * floor(max(0, pos_first -
 *     window_left + 1) / 16) (pos_first the block's first query), partition
 *     s covers [base + s * P, base + (s + 1) * P), partition 0 starting at 0
 *     so that it also holds the sinks, P = max(256, 16 * ceil(ceil(window_left
 *     / 32) / 16)).
 * The grid's slot count follows from max_context_len, max_q_len and
 * min_q_len; a sequence whose q_len_b is below min_q_len is written as NaN.
 *
 * Fused store: with new_k non-NULL the launch first does what ra_kv_store
 * would do with new_k / new_v / new_slots for the query tokens (row q of
 * new_k and new_v is the K and V of query token q, slot new_slots[q]; slot
 * < 0 or >= num_pages * 16 stores nothing), each token stored by the
 * workgroups of the partition holding its position, before they read it; the
 * separate ra_kv_store call and its launch go away.  The fused store WRITES
 * k_cache and v_cache (and, for RA_KV_INT8_TOKEN, k_scales and v_scales) at
 * the new tokens' slots; without new_k the launch only reads them.  A page
 * that receives a new token must be read by no other sequence of the same
 * launch (a partly filled page shared between sequences through prefix
 * caching must not take new tokens): the other sequence's workgroups could
 * read it before or after the store.  The slot of query i of
 * sequence b must be the block table's slot for its position p (local to this
 * cache): block_tables[b][p / 16] * 16 + p % 16.  Tokens whose position lies
 * outside [0, ctx_b) are not stored (they belong to another context-parallel
 * shard).  Supported for decode and verify blocks, (Hq / Hkv) * max_q_len <=
 * 48; longer blocks (prefill) return RA_ERR_UNSUPPORTED and are stored with
 * ra_kv_store first.  The store's format, scales and rounding are those of
 * ra_kv_store (per-token INT8 writes its scale planes too).
 *
 * RoPE on the fused path: with rope_table non-NULL (and new_k), query token
 * q's Q rows and its K rows are rotated by the table row positions[q] exactly
 * as ra_qkv_rope_store rotates them (same pairing, fp32 without fused
 * multiply-add, rotated Q rounded to q_dtype) before use: one launch then
 * does the whole of ra_qkv_rope_store + ra_paged_attn for a decode or verify
 * step.  q (q_token_stride elements between tokens) and new_k / new_v may
 * point into the packed QKV projection rows.  A position outside
 * [0, rope_max_position) gives NaN rows for that token and stores nothing.
 * With more than
 * one partition slot the kernel writes partial_out [slots][total_q][Hq][D] and
 * partial_lse [slots][total_q][Hq] (fp32; out already normalised; an empty
 * partition writes out = 0, lse = -inf) and, if `out` is non-NULL, merges them
 * into out / lse on the same stream.  With one slot and `out` non-NULL the
 * result is written directly.
 */
typedef struct ra_attn_args {
  uint32_t struct_size;
  int32_t q_dtype;                 /* RA_F16 or RA_BF16; also the dtype of out   */
  const void* q;                   /* [total_q][num_q_heads][head_dim]           */
  void* out;                       /* [total_q][num_q_heads][head_dim] or NULL   */
  float* lse;                      /* [total_q][num_q_heads] or NULL             */
  void* k_cache;                   /* paged layout above; read, and written by   */
  void* v_cache;                   /* the fused store (see above)                */
  int32_t kv_dtype;                /* RA_KV_*                                    */
  float k_scale;                   /* (host) > 0, finite for E4M3 / INT8         */
  float v_scale;
  const int32_t* block_tables;     /* [batch][block_table_stride] page ids       */
  int32_t block_table_stride;      /* entries >= ceil(ctx_b / 16) never read     */
  const int32_t* context_lens;     /* [batch]                                    */
  const int32_t* query_start_loc;  /* [batch + 1], non-decreasing, last = total_q*/
  int32_t batch;
  int32_t total_q;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;                /* 64 or 128                                  */
  int32_t page_size;               /* 16                                         */
  int64_t num_pages;               /* pages in each cache                        */
  int32_t max_q_len;               /* (host) >= every q_len_b                    */
  int32_t min_q_len;               /* (host) <= every q_len_b; 0 if unknown      */
  int32_t max_context_len;         /* (host) >= every ctx_b, <= stride * 16      */
  float softmax_scale;             /* > 0                                        */
  int32_t window_left;             /* < 0: no window                             */
  int32_t num_sinks;               /* >= 0; used only with a window              */
  int32_t num_splits;              /* 0 = auto, 1..RA_KV_MAX_SPLITS              */
  float* partial_out;              /* workspace, see above                       */
  float* partial_lse;
  int32_t partial_slots;           /* slots the partial buffers hold             */
  float* k_scales;                 /* RA_KV_INT8_TOKEN: scale planes (layout     */
  float* v_scales;                 /* above; written by the fused store too);    */
                                   /* ignored by the other formats               */
  const int32_t* kv_pos0;          /* [batch] or NULL: global position of key 0  */
  const int32_t* q_pos0;           /* [batch] or NULL: global position of query 0*/
  /* Fused store (decode and verify): the query tokens' own K/V rows, stored
     by the launch itself before it reads them; new_k = NULL stores nothing. */
  const void* new_k;               /* [total_q][num_kv_heads][head_dim] or NULL  */
  const void* new_v;
  int32_t new_dtype;               /* RA_F16 or RA_BF16                          */
  int64_t new_k_stride;            /* elements between tokens, multiple of 8     */
  int64_t new_v_stride;
  const int64_t* new_slots;        /* [total_q] cache slot of each query token   */
  int64_t q_token_stride;          /* elements between query tokens; 0: Hq * D   */
  /* RoPE on the fused path: q and new_k hold rows before the rotation; NULL
     rope_table rotates nothing.  Needs new_k (decode and verify blocks). */
  const float* rope_table;         /* [rope_max_position][2][rotary_dim / 2]     */
  int32_t rope_max_position;
  int32_t rotary_dim;              /* multiple of 16, <= head_dim                */
  const int64_t* positions;        /* [total_q] RoPE position of each query token*/
} ra_attn_args;

/*
 * ra_paged_attn -- decode/verify attention over the paged, quantised cache.
 * Argument meaning, layouts and the split rule are given with ra_attn_args.
 * Host checks: non-null pointers; 16-byte aligned q, out and caches;
 * Hq % Hkv == 0; head_dim in {64, 128}; page_size == 16; known dtypes; finite
 * positive scales for E4M3 / INT8; non-null, 16-byte aligned scale planes for
 * RA_KV_INT8_TOKEN (k_scale / v_scale are then ignored); 1 <= max_q_len;
 * max_context_len <=
 * block_table_stride * 16; num_splits in [0, RA_KV_MAX_SPLITS]; partial
 * buffers present and partial_slots >= the slots needed when more than one
 * slot is used.
 */
int32_t ra_paged_attn(const ra_attn_args* args, void* stream);

/*
 * ra_paged_attn_workspace -- (host only, enqueues nothing) number of partition
 * slots ra_paged_attn will use for these arguments, and the fp32 element counts
 * of partial_out and partial_lse it needs (0 when one slot and out != NULL).
 */
int32_t ra_paged_attn_workspace(const ra_attn_args* args, int32_t* slots,
                                int64_t* partial_out_floats,
                                int64_t* partial_lse_floats);

/*
 * ra_paged_attn_noalloc -- ra_paged_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same attention, kernels and results, but the
 * partials of a split call live in a scratch array of the library's own,
 * RA_KV_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the library's first
 * use on that GPU until the process ends; partial_out, partial_lse and
 * partial_slots are ignored.  out must be non-NULL (RA_ERR_INVALID_ARG).  A
 * call whose partials, slots * total_q * num_q_heads * (head_dim + 1) * 4
 * bytes, exceed the scratch returns RA_ERR_WORKSPACE before anything is
 * enqueued.  The call allocates and frees nothing.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race and must not be
 * issued; calls ordered on one stream are safe.  Uses the device that is
 * current on the calling thread (it must be the stream's device).
 */
#define RA_KV_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t ra_paged_attn_noalloc(const ra_attn_args* args, void* stream);

/*
 * ra_lse_merge -- merge partial attention results by log-sum-exp.
 *
 * partial_out [num_partitions][rows][head_dim] fp32, partial_lse
 * [num_partitions][rows] fp32 (natural log; -inf marks an empty partition,
 * whose out adds nothing whatever it holds, though the buffer is read).  For
 * each row: M = max_s lse_s; if M = -inf the
 * result is out = 0, lse = -inf; else a_s = exp(lse_s - M),
 * out = sum_s a_s out_s / sum_s a_s, lse = M + ln sum_s a_s, summed in the
 * order s = 0, 1, ...  out [rows][head_dim] of out_dtype (RA_F16, RA_BF16 or
 * RA_F32), lse_out [rows] fp32 or NULL.  head_dim in {64, 128};
 * num_partitions in [1, RA_KV_MAX_SPLITS]; rows in [0, 2^31 - 16];
 * 16-byte aligned buffers.
 * (ReVolta README, "Quick start" and "Hardware": decode context parallelism
 * combines the partial attention of context parts.)
 */
int32_t ra_lse_merge(const float* partial_out, const float* partial_lse,
                     int32_t num_partitions, int64_t rows, int32_t head_dim,
                     void* out, int32_t out_dtype, float* lse_out, void* stream);

/*
 * ra_kv_gather_dequant -- (test and debugging aid) read one sequence's K or V
 * back through its block-table row and dequantise it exactly.
 * which: 0 = K cache, 1 = V cache.  out [ctx][num_kv_heads][head_dim] fp32 =
 * fp32(decode(code)) * scale (FP16 caches: the fp16 value, scale ignored;
 * RA_KV_INT8_TOKEN: the (slot, head) scale from the plane `scales`, which is
 * ignored, and may be NULL, for the other formats).
 * Positions whose page id is outside [0, num_pages) are written as NaN.
 */
int32_t ra_kv_gather_dequant(const void* cache, int32_t which, int32_t kv_dtype,
                             float scale, const float* scales, const int32_t* block_table_row,
                             int32_t ctx, int64_t num_pages, int32_t num_kv_heads,
                             int32_t head_dim, float* out, void* stream);

/* Message describing the last non-OK status returned on this thread. */
const char* ra_last_error(void);

/* RA_KV_ABI_VERSION * 1000 + RA_KV_LAYOUT_ID. */
int32_t ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_KV_H_ */
