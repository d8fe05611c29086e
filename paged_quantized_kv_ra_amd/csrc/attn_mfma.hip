// attn_mfma.hip -- decode and verify attention on the gfx950 matrix cores.
//
// One (sequence, KV head) unit has g * q_len query rows: the pages' MTP4
// verify block of 1 + 4 tokens times the query heads of one KV head (ReVolta
// README, intro list and "Quick start"), or g rows for plain decode.  Rows are
// processed in 16-row tiles; a decode unit with fewer rows uses one padded
// tile (the path is bound by HBM, not by the matrix cores).  The KV cache is
// converted exactly to FP16 operands in registers (the pages' V100 converts
// stored KV to FP16 for the arithmetic: ReVolta README, "Weight and KV
// formats").
//
// Per wavefront and 16-token page, for each 16-row tile of query rows:
//   S^T[16 keys][16 rows] = K[16][D] . Q^T[D][16]      v_mfma_f32_16x16x32_f16 (D/32 steps)
//   P^T = exp2(c * S^T - c * m)                       online softmax, fp32, rescaled lazily
// and per pair of pages (32 keys; a lone last page uses the 16x16x16 form):
//   O^T[D][16 rows]      += V^T[D][32] . P^T[32][16]   v_mfma_f32_16x16x32_f16 (D/16 tiles)
// The cache layout puts every lane's 16-byte piece of a page directly in the
// operand order of both products: a K lane holds one token's contiguous D/4
// dims, a V lane holds four consecutive tokens of D/16 dims, and the S^T
// accumulator layout (lane = row + 16 * token-quad) is exactly the P^T operand
// layout, so no data moves between lanes in the hot loop.  Pages stream into a
// per-wave LDS ring by DMA (global_load_lds), NRING - 1 pages in flight per
// wave, and each lane reads back its own 16-byte pieces.
//
// A workgroup has 8 waves (two per SIMD) that take contiguous shares of the
// unit's pages; their partial (m, l, O) are combined through LDS in a fixed
// order at the end.
#include "attn_common.h"

#ifdef RA_TIMELINE
// Timing build (compiled only with -DRA_TIMELINE): every workgroup records,
// from lane 0 of the marking wave, the 100 MHz real-time counter at fixed
// points of its life into slots of ra_timeline[block][kTlSlots], for the
// per-phase breakdown bench.py --timeline prints.  The product build has none
// of it.
#ifndef RA_TIMELINE_BLOCKS
#define RA_TIMELINE_BLOCKS 8192
#endif
constexpr int kTlSlots = 40;
__device__ uint64_t ra_timeline[RA_TIMELINE_BLOCKS * kTlSlots];
enum TlSlot {
  TL_ENTRY = 0, TL_HWID = 1, TL_XCC = 2, TL_META = 3, TL_IDSQ = 4, TL_FIRST = 5, TL_PAGES = 6, TL_UNIT = 7,
  TL_LOOP = 8,     // + wave: the wave left its page loop
  TL_COMB = 16,    // every wave's (m, l) published (first combine barrier passed), wave 0
  TL_ML = 17,      // wave 0 has the common row maxima and sums
  TL_P0W = 18,     // + pass (0, 1): the pass's LDS writes and barrier done, wave 0
  TL_P0R = 20,     // + pass: wave 0's sums and stores of the pass issued
  TL_END = 24,     // + wave: the wave's last store issued
  TL_PLAN = 32,    // wave 0 has its partition and page ranges
  TL_IDISS = 33,   // wave 0 has requested its page ids and query loads
  TL_IDLAND = 34,  // wave 0's page ids have landed (early page request only)
  TL_PGISS = 35,   // wave 0 has requested its first ring pages (early page request only)
};
#define TL_MARK(slot)                                                                      \
  do {                                                                                     \
    if ((threadIdx.x & 63) == 0 && blockIdx.x < RA_TIMELINE_BLOCKS)                        \
      ra_timeline[blockIdx.x * kTlSlots + (slot)] = __builtin_amdgcn_s_memrealtime();      \
  } while (0)
#define TL_VALUE(slot, v)                                                                  \
  do {                                                                                     \
    if ((threadIdx.x & 63) == 0 && blockIdx.x < RA_TIMELINE_BLOCKS)                        \
      ra_timeline[blockIdx.x * kTlSlots + (slot)] = (uint64_t)(v);                         \
  } while (0)
#else
#define TL_MARK(slot) do {} while (0)
#define TL_VALUE(slot, v) do {} while (0)
#endif

namespace ra {
namespace {

#ifndef RA_MFMA_WAVES
#define RA_MFMA_WAVES 8
#endif
constexpr int kWaves = RA_MFMA_WAVES;   // waves per workgroup
static_assert(kWaves == 8 || kWaves == 4, "8 or 4 waves per workgroup");
constexpr int kSlab = 1024; // bytes of one wavefront-wide 16-byte load
typedef __attribute__((address_space(3))) uint8_t lds_u8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;   // log2 headroom before the running max is refreshed
constexpr int kCpolNt = 2;      // cache-policy operand of a load: nontemporal

#ifndef RA_MFMA_RING_KIB
#define RA_MFMA_RING_KIB 8
#endif

template <int KV, int D>
struct Geo {
  static constexpr int E = KV == KV_F16 ? 2 : 1;
  static constexpr int SLABS = D * E / 64;       // 16-byte loads per lane per page (K, and again V)
  static constexpr int KS = D / 32;              // k-steps of the QK product
  static constexpr int MT = D / 16;              // 16-dim tiles of the PV product
  static constexpr int BLK = kPage * D * E;      // bytes per (page, head) block
  static constexpr int NSL = 2 * SLABS;          // 1 KiB slabs per page (K, then V)
  // depth of the per-wave LDS page ring: RA_MFMA_RING_KIB of LDS per wave,
  // 2 .. 8 pages; NRING - 1 pages are in flight while one computes
  static constexpr int NRING_RAW = RA_MFMA_RING_KIB / NSL;
  static constexpr int NRING = NRING_RAW > 8 ? 8 : (NRING_RAW < 2 ? 2 : NRING_RAW);
  // vector-memory operations per page: the slabs, plus the loads of the
  // page's 16 K and 16 V scales for per-token INT8
  static constexpr int OPS = NSL + (KV == KV_I8T ? 2 : 0);
};

template <int KV, int D>
struct PageRegs {
  u32x4 k[Geo<KV, D>::SLABS];
  u32x4 v[Geo<KV, D>::SLABS];
  f32x4 ks, vs;   // per-token INT8: the K and V scales of the lane's 4 tokens
};

// Page ids of the pages one wave visits, staged 64 at a time in LDS by the
// same DMA path as the pages, so that the wave's vector-memory counter only
// tracks loads whose order the ring accounts for.  Lane j of chunk c holds the
// raw block-table entry of the wave's (64 c + j)-th page; chunk c + 1 is
// requested when chunk c is taken up.
struct IdRing {
  int32_t cur;     // per-lane ids of chunk `chunk`
  int32_t chunk;
};

// The unit's pages a wave visits: its k-th page (k < count) is the unit's
// logical page first + stride * k.
struct WaveSpan {
  int32_t first, stride, count;
  __device__ __forceinline__ int32_t page(int32_t k) const { return first + stride * k; }
};

// The lane's entry of an id chunk that LDS DMA wrote: read from assembly (and
// waited for in the same block), because for an ordinary LDS read the compiler
// would first wait for every outstanding DMA of the wave, page loads and
// query rows included; the caller's vmcnt wait retires the chunk's DMA.
__device__ __forceinline__ int32_t read_id(const int32_t* slot, int lane) {
  int32_t v;
  asm volatile(
      "ds_read_b32 %0, %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(v)
      : "v"((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int32_t*)(slot + lane))
      : "memory");
  return v;
}

// The KS query operands of one 16-row tile (1 KiB apart in LDS), read from
// assembly and waited for in the same block, for the reason given above.
template <int KS>
__device__ __forceinline__ void read_q_tile(const void* base, u32x4 (&w)[KS]) {
  const uint32_t adr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)base;
  if constexpr (KS == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
        : "v"(adr)
        : "memory");
  } else {
    static_assert(KS == 2, "two or four k-steps");
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1])
        : "v"(adr)
        : "memory");
  }
}

__device__ __forceinline__ void id_dma(int32_t* slot, const UnitPages& pg, const WaveSpan& ws, const int32_t* bt_row,
                                       int32_t chunk, int lane) {
  const int32_t k = chunk * 64 + lane;
  if (k < ws.count) __builtin_amdgcn_global_load_lds(bt_row + pg.page(ws.page(k)), (lds_u8*)slot, 4, 0, 0);
}

// Checked physical id of the wave's k-th page (k non-decreasing).  On entry to
// a new chunk its DMA must have retired: the caller waits for every load older
// than the last NRING - 1 pages, and a chunk is requested 64 pages before use.
// An id outside [0, num_pages) makes the unit bad and reads page 0 instead.
__device__ __forceinline__ int32_t ring_page_id(IdRing& r, int32_t (*sm_id)[64], const AttnLaunch& a,
                                                const UnitPages& pg, const WaveSpan& ws, const int32_t* bt_row,
                                                int32_t k, int lane, bool& bad) {
  const int32_t ch = k >> 6;
  if (ch != r.chunk) {       // wave-uniform, once per 64 pages
    r.chunk = ch;
    r.cur = read_id(sm_id[ch & 1], lane);
    id_dma(sm_id[(ch + 1) & 1], pg, ws, bt_row, ch + 1, lane);
  }
  int32_t id = __builtin_amdgcn_readlane(r.cur, k & 63);
  if (id < 0 || id >= a.num_pages) {
    bad = true;
    id = 0;
  }
  return id;
}

// Issue the loads of the wave's i-th page (i < the wave's page count)
// straight into the LDS ring slot `ring`: one global_load_lds_dwordx4 per 1 KiB
// slab, lane L writing bytes L*16 .. L*16+15 of the slab, the lane order the
// cache layout has in HBM.
// Per-token INT8 adds two 16-lane loads of the (page, head)'s 16 K scales and
// 16 V scales into the slot's 128-byte scale area `scl`.
// With NTP the page slabs are read with the nontemporal cache policy: a
// launch whose units each read a page once (one row group per sequence and
// KV head) streams its pages at about 6.8 TB/s this way against 6.1 TB/s with
// the default policy (random 2 KiB blocks), while units that re-read pages
// (several row groups of a long query block) need them kept in L2.
template <int KV, int D, bool NTP>
__device__ __forceinline__ void issue_page(uint8_t (*ring)[kSlab], float* scl, IdRing& ids, int32_t (*sm_id)[64],
                                           const AttnLaunch& a, const UnitPages& pg, const WaveSpan& ws,
                                           int32_t i, const int32_t* bt_row, int h, int lane, bool& bad) {
  using G = Geo<KV, D>;
  const int32_t pid = ring_page_id(ids, sm_id, a, pg, ws, bt_row, i, lane, bad);
  if constexpr (KV == KV_I8T) {
    if (lane < 16) {   // two 16-lane loads from uniform plane bases: K scales, then V scales
      const int64_t so = ((int64_t)pid * a.hkv + h) * kPage + lane;
      __builtin_amdgcn_global_load_lds(a.k_scales + so, (lds_u8*)scl, 4, 0, 0);
      __builtin_amdgcn_global_load_lds(a.v_scales + so, (lds_u8*)(scl + 16), 4, 0, 0);
    }
  }
  const int64_t blk = ((int64_t)pid * a.hkv + h) * G::BLK;
  const uint8_t* kp = a.k_cache + blk + (uint32_t)lane * 16u;
  const uint8_t* vp = a.v_cache + blk + (uint32_t)lane * 16u;
  constexpr int cpol = NTP ? kCpolNt : 0;
#pragma unroll
  for (int j = 0; j < G::SLABS; ++j) __builtin_amdgcn_global_load_lds(kp + j * kSlab, (lds_u8*)ring[j], 16, 0, cpol);
#pragma unroll
  for (int j = 0; j < G::SLABS; ++j)
    __builtin_amdgcn_global_load_lds(vp + j * kSlab, (lds_u8*)ring[G::SLABS + j], 16, 0, cpol);
}

// Wait until at most `n` of this wave's vector-memory operations are
// outstanding (the LDS ring's loads retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14;
  // expcnt (bits 6:4) and lgkmcnt (bits 11:8) left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt at their maxima
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// The lane's 16-byte pieces of one ring slot: the K slabs, then the V slabs.
// The reads are issued from inline assembly, each block waiting for its own
// LDS returns (lgkmcnt(0)) before it ends.  The slot was written by LDS DMA,
// which the compiler tracks only coarsely: for an ordinary LDS read of the
// ring it would wait for every outstanding DMA (vmcnt(0)), including the
// pages still in flight to the other slots, and the ring would stop
// overlapping loads with arithmetic.  The caller's explicit vmcnt wait is the
// one that retires this slot's loads.
template <int KV, int D>
__device__ __forceinline__ void read_page(PageRegs<KV, D>& r, const uint8_t (*ring)[kSlab], const float* scl,
                                          uint32_t lane_off, int kgrp) {
  using G = Geo<KV, D>;
  const uint32_t adr = lds_addr(ring[0]) + lane_off;
  if constexpr (G::SLABS == 1) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.k[0]), "=&v"(r.v[0])
        : "v"(adr)
        : "memory");
  } else if constexpr (G::SLABS == 2) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.k[0]), "=&v"(r.k[1]), "=&v"(r.v[0]), "=&v"(r.v[1])
        : "v"(adr)
        : "memory");
  } else {
    static_assert(G::SLABS == 4, "one, two or four 1 KiB slabs per page half");
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\t"
        "ds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.k[0]), "=&v"(r.k[1]), "=&v"(r.k[2]), "=&v"(r.k[3]), "=&v"(r.v[0]), "=&v"(r.v[1]),
          "=&v"(r.v[2]), "=&v"(r.v[3])
        : "v"(adr)
        : "memory");
  }
  if constexpr (KV == KV_I8T) {
    const uint32_t sadr = lds_addr(scl + 4 * kgrp);
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.ks), "=&v"(r.vs)
        : "v"(sadr)
        : "memory");
  }
}

// K operand of k-step ks: the lane's token, dims kgrp * D/4 + 8 ks .. + 8.
template <int KV, int D>
__device__ __forceinline__ f16x8 k_operand(const PageRegs<KV, D>& r, int ks) {
  if constexpr (KV == KV_F16) {
    return as<f16x8>(r.k[ks]);
  } else {
    const u32x4 w = r.k[ks >> 1];
    const uint32_t d0 = (ks & 1) ? w[2] : w[0];
    const uint32_t d1 = (ks & 1) ? w[3] : w[1];
    const f16x4 lo = codes4_to_f16x4<KV>(d0);
    const f16x4 hi = codes4_to_f16x4<KV>(d1);
    return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// V operand of dim tile mt: tokens 4 kgrp .. 4 kgrp + 3 of the lane's dim.
template <int KV, int D>
__device__ __forceinline__ f16x4 v_operand(const u32x4 (&v)[Geo<KV, D>::SLABS], int mt) {
  if constexpr (KV == KV_F16) {
    const u32x4 w = v[mt >> 1];
    const uint32_t a = (mt & 1) ? w[2] : w[0];
    const uint32_t b = (mt & 1) ? w[3] : w[1];
    const f16x2 lo = as<f16x2>(a);
    const f16x2 hi = as<f16x2>(b);
    return f16x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    const u32x4 w = v[mt >> 2];
    return codes4_to_f16x4<KV>(w[mt & 3]);
  }
}

// Row sums of P ride on the matrix cores as one more PV tile whose V operand
// is all ones (every lane of that tile then holds its row's whole sum), except
// for per-token INT8, whose P carries the V scales and is summed on the VALU.
template <int KV>
constexpr bool kOnesSum = KV != KV_I8T;

template <int KV, int D, int NT>
struct Acc {
  f32x4 o[Geo<KV, D>::MT][NT];
  f32x4 ls[NT];   // row sums by the ones tile
  float m[NT];
  float mc[NT];   // c * m, or 0 while m = -inf: the rows' exponent offset
  float l[NT];    // the lane's partial row sums (per-token INT8)
  // Per-token INT8: the V scales ride on P relative to a power-of-two
  // reference vref (wave-uniform), so that the fp16 operand p * vs / vref
  // stays in fp16's normal range whatever the magnitude of V: every V scale
  // seen is at most 2^7 vref, hence p * vs / vref <= 2^8 * 2^7, and O
  // holds sums in units of vref.  0 until the first non-zero scale.
  float vref, vinv;
};

// Per-token INT8: take up a page's V scales into the wave's power-of-two
// reference.  When a scale exceeds 2^7 vref the reference moves to 2^(e - 7)
// for the page's largest scale f * 2^e (f in [0.5, 1)).  Returns the factor,
// old reference over new (a power of two, 0 before the first scale, 1 when
// the reference stays), by which what was accumulated in units of the old
// reference (O, and the pending page's probabilities) must be rescaled; the
// softmax applies it together with its own max-refresh factor.
template <int KV, int D, int NT>
__device__ __forceinline__ float take_v_scales(Acc<KV, D, NT>& acc, const f32x4& vs) {
  float vm = fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3]));
  vm = fmaxf(vm, __shfl_xor(vm, 16));   // the lanes' token quads: kgrp = lane bits 4, 5
  vm = fmaxf(vm, __shfl_xor(vm, 32));
  vm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vm)));   // (the builtin takes an int)
  if (!(vm > acc.vref * 128.0f)) return 1.0f;
  int32_t e = (int32_t)((__float_as_uint(vm) >> 23) & 0xFFu) - 126;   // vm = f * 2^e, f in [0.5, 1)
  e = min(max(e, -119), 120);                                         // vref and 1 / vref stay normal
  const float ninv = __uint_as_float((uint32_t)(7 - e + 127) << 23);
  const float f = acc.vref * ninv;                                    // old / new: a power of two, or 0
  acc.vref = __uint_as_float((uint32_t)(e - 7 + 127) << 23);
  acc.vinv = ninv;
  return f;
}

// QK, masks and the online softmax of one page.  p receives the page's
// unnormalised probabilities (times the per-token V scales for per-token
// INT8); a refresh of the running max also rescales `pend`, the
// probabilities of an earlier page whose PV product is still to come.
template <int KV, int D, int NT>
__device__ __forceinline__ void scores_softmax(Acc<KV, D, NT>& acc, PageRegs<KV, D>& r,
                                               const f16x8 (&qf)[NT][Geo<KV, D>::KS],
                                               const AttnLaunch& a, const UnitPages& pg, int32_t n, int32_t ctx,
                                               const SeqFrame& fr, const int32_t (&pos)[NT], int kgrp, float c,
                                               float thr, float (&p)[NT][4], float (&pend)[NT][4]) {
  using G = Geo<KV, D>;
  // ---- scores S^T for the page's 16 keys
  f32x4 s[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) s[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const f16x8 kop = k_operand<KV, D>(r, ks);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qf[nt][ks], s[nt], 0, 0, 0);
  }
  if constexpr (KV == KV_I8T) {   // per-token K scales
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s[nt] *= r.ks;
  }
  // ---- masks (only on pages that can hold an invisible key).  Keys past ctx
  // (stale bytes of the last page) also get their V codes zeroed so that
  // 0 * garbage cannot produce NaN.
  // ---- online softmax with lazy max refresh (per-token INT8: and with a
  // move of the V-scale reference, fv != 1, which rescales O and the pending
  // probabilities but not the row sums)
  const auto softmax = [&](float fv) {
    float mx[NT];
    bool trig = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mx[nt] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[nt][0], s[nt][1]),
                                             __builtin_elementwise_maximum(s[nt][2], s[nt][3]));
      trig |= mx[nt] > acc.m[nt] + thr;
    }
    if (__any(trig) || (KV == KV_I8T && fv != 1.0f)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float rm = mx[nt];
        rm = __builtin_elementwise_maximum(rm, __shfl_xor(rm, 16));
        rm = __builtin_elementwise_maximum(rm, __shfl_xor(rm, 32));
        const bool upd = rm > acc.m[nt] + thr;
        const float alpha =
            upd ? (acc.m[nt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((acc.m[nt] - rm) * c)) : 1.0f;
        acc.m[nt] = upd ? rm : acc.m[nt];
        acc.mc[nt] = acc.m[nt] == -INFINITY ? 0.0f : acc.m[nt] * c;
        if constexpr (kOnesSum<KV>) acc.ls[nt] *= alpha;
        else acc.l[nt] *= alpha;
        const float ao = KV == KV_I8T ? alpha * fv : alpha;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) acc.o[mt][nt] *= ao;
#pragma unroll
        for (int i = 0; i < 4; ++i) pend[nt][i] *= ao;
      }
    }
    float vsn[4];   // per-token INT8: the V scales in units of the reference
#pragma unroll
    for (int i = 0; i < 4; ++i) vsn[i] = KV == KV_I8T ? r.vs[i] * acc.vinv : 1.0f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[nt][i], c, -acc.mc[nt]));
        if constexpr (!kOnesSum<KV>) ps += e;
        p[nt][i] = KV == KV_I8T ? e * vsn[i] : e;   // per-token V scales ride on P
      }
      if constexpr (!kOnesSum<KV>) acc.l[nt] += ps;
    }
  };
  const int32_t tok0 = pg.page(n) * kPage;
  const bool need_mask = (tok0 + kPage - 1 > fr.pmin) || (tok0 + kPage - 1 >= ctx) ||
                         (a.window >= 0 && tok0 <= fr.pmax - a.window);
  if (need_mask) {
    const int32_t tb = tok0 + 4 * kgrp;
    uint32_t keep8 = 0, keep_lo = 0, keep_hi = 0;   // byte / half masks of the lane's 4 tokens
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t j = tb + i;
      const bool data = j < ctx;   // keys past ctx are stale bytes, whatever the query positions
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[nt][i] = data && key_visible(a, fr, j, pos[nt]) ? s[nt][i] : -INFINITY;
      if constexpr (KV == KV_I8T) r.vs[i] = data ? r.vs[i] : 0.0f;   // the scale plane past ctx is not data
      keep8 |= data ? 0xFFu << (8 * i) : 0u;
      if (i < 2) keep_lo |= data ? 0xFFFFu << (16 * i) : 0u;
      else keep_hi |= data ? 0xFFFFu << (16 * (i - 2)) : 0u;
    }
#pragma unroll
    for (int sl = 0; sl < G::SLABS; ++sl)
#pragma unroll
      for (int w = 0; w < 4; ++w) r.v[sl][w] &= KV == KV_F16 ? ((w & 1) ? keep_hi : keep_lo) : keep8;
  }
  float fv = 1.0f;
  if constexpr (KV == KV_I8T) fv = take_v_scales<KV, D, NT>(acc, r.vs);
  softmax(fv);
}

// Fused store: quantise the unit's head's K and V rows of the query tokens
// whose (local) positions fall in the partition [lo, hi) and write them at
// their slots exactly as the KV store kernel does, before any page of the
// partition is read.  32 threads per token for D = 128 (16 for K, 16 for V,
// 8 dims each).  Returns whether anything was stored (workgroup-uniform).
template <int KV, int D>
__device__ __forceinline__ bool store_new_tokens(const AttnLaunch& a, int h, int32_t q0, int32_t q_len,
                                                 int32_t pmin, int32_t lo, int32_t hi) {
  constexpr int CH = D / 8;         // lanes per row
  constexpr int E = KV == KV_F16 ? 2 : 1;
  const int32_t i0 = max(0, lo - pmin), i1 = min(q_len, hi - pmin);
  if (i0 >= i1) return false;
  const int t = threadIdx.x;
  const int c = t % CH;
  const bool is_v = (t / CH) & 1;
  const int64_t limit = a.num_pages * kPage;
  for (int32_t base = i0; base < i1; base += kWaves * kWave / (2 * CH)) {
    const int32_t i = base + t / (2 * CH);
    if (i < i1) {   // whole rows of lanes are in or out
      const int64_t row = q0 + i;
      const uint16_t* src = reinterpret_cast<const uint16_t*>(is_v ? a.new_v : a.new_k) +
                            row * (is_v ? a.new_v_stride : a.new_k_stride) + (int64_t)h * D + 8 * c;
      const u32x4 raw = load16(src);
      const int64_t slot = a.new_slots[row];
      asm volatile("" ::"v"(raw), "v"(slot));   // both requests in flight before the first wait
      float x[8];
      src8_to_f32(raw, a.new_bf16, x);
      bool pos_ok = true;
      if (a.rope != nullptr) {   // RoPE on the fused path: rotate K (V passes through)
        const int64_t rp = a.positions[row];
        pos_ok = rp >= 0 && rp < a.rope_max_pos;
        const int d0 = 8 * c;
        if (!is_v && pos_ok && d0 < a.rot) {
          const int half = a.rot / 2;
          float partner[8];
          src8_to_f32(load16(src + (d0 < half ? half : -half)), a.new_bf16, partner);
          rope8(x, partner, a.rope + rp * a.rot, d0, a.rot);
        }
      }
      float sc = is_v ? a.v_scale : a.k_scale;
      if constexpr (KV == KV_I8T) sc = row_absmax(x, CH) / 127.0f;   // correctly rounded division
      if (pos_ok && slot >= 0 && slot < limit) {
        const int64_t page = slot >> 4;
        const int tp = (int)(slot & 15);
        if constexpr (KV == KV_I8T) {
          if (c == 0) (is_v ? a.v_scales : a.k_scales)[(page * a.hkv + h) * kPage + tp] = sc;
        }
        uint8_t* blk = (is_v ? a.v_cache : a.k_cache) + (page * a.hkv + h) * (int64_t)(kPage * D * E);
        store_row8<KV, D>(blk, tp, 8 * c, x, sc, is_v);
      }
    }
  }
  return true;
}

// O^T += V^T . P^T for one page (16 keys): D/16 x NT 16x16x16 products.
template <int KV, int D, int NT>
__device__ __forceinline__ void pv_single(Acc<KV, D, NT>& acc, const u32x4 (&v)[Geo<KV, D>::SLABS],
                                          const float (&p)[NT][4]) {
  using G = Geo<KV, D>;
  f16x4 pf[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[nt][i] = (f16)p[nt][i];
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt) {
    const f16x4 vop = v_operand<KV, D>(v, mt);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc.o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop, pf[nt], acc.o[mt][nt], 0, 0, 0);
  }
  if constexpr (kOnesSum<KV>) {
    const f16x4 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc.ls[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pf[nt], acc.ls[nt], 0, 0, 0);
  }
}

// O^T += V^T . P^T for two pages at once with the 16x16x32 product (twice the
// 16x16x16 rate): the contraction runs over 32 keys, the lane's k-slots 0-3
// holding its 4 keys of page A and slots 4-7 the same keys of page B, in the
// V operand and the P operand alike.
template <int KV, int D, int NT>
__device__ __forceinline__ void pv_pair(Acc<KV, D, NT>& acc, const u32x4 (&va)[Geo<KV, D>::SLABS],
                                        const float (&pa)[NT][4], const u32x4 (&vb)[Geo<KV, D>::SLABS],
                                        const float (&pb)[NT][4]) {
  using G = Geo<KV, D>;
  f16x8 pf[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[nt][i] = (f16)pa[nt][i];
      pf[nt][4 + i] = (f16)pb[nt][i];
    }
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt) {
    const f16x4 x = v_operand<KV, D>(va, mt);
    const f16x4 y = v_operand<KV, D>(vb, mt);
    const f16x8 vop = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc.o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pf[nt], acc.o[mt][nt], 0, 0, 0);
  }
  if constexpr (kOnesSum<KV>) {
    const f16x8 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc.ls[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[nt], acc.ls[nt], 0, 0, 0);
  }
}

// A decode tile (NT = 1) whose page ring takes at most 8 KiB per wave keeps
// to 128 VGPRs, so that two workgroups share a CU.
template <int KV, int D, int NT>
constexpr int kWavesPerSimd = (NT == 1 && Geo<KV, D>::NRING * Geo<KV, D>::NSL <= 8) ? 4 : 2;

// The cross-wave merge of O.  A wave's O is C = NT * MT chunks of one f32x4
// per lane (1 KiB per wave): chunk q = nt * MT + j, with i = j / (MT / 4) and
// k = j % (MT / 4), holds acc.o[4k .. 4k + 3][nt][i], the dims
// (4 kgrp + i) * MT + 4k .. + 4 of row nt * 16 + ncol: four consecutive dims,
// stored by the lane in one 16-byte write.  The chunks cross LDS
// unscaled in at most two passes, chunks [0, CA) and then [CA, C).  Within a
// pass a wave keeps its chunks in slabs of its own: the first R in its page
// ring, the next X in an area past all the rings.  So the first pass is stored
// as soon as the wave's own page loop ends, while other waves still stream.
// Chunk q of a pass is summed by wave q % kWaves (each SIMD then sums the
// same number of chunks when a pass holds a multiple of 4).
template <int N>
struct IntC {
  static constexpr int value = N;
};

template <int KV, int D, int NT>
struct MergePlan {
  using G = Geo<KV, D>;
  static constexpr int R = G::NRING * G::NSL;
  static constexpr int C = NT * G::MT;
  // LDS of one workgroup: the CU's 160 KiB over the workgroups it holds
  static constexpr int kWgPerCu = kWavesPerSimd<KV, D, NT> * 4 / kWaves;
  static constexpr int kLimit = 163840 / kWgPerCu;
  // the kernel's other LDS arrays, with slack for their alignment
  static constexpr int kOther = 2 * (2 * NT * 16 * kWaves * 4) + kWaves * 2 * 64 * 4 +
                                (KV == KV_I8T ? kWaves * G::NRING * 32 * 4 : 16) + 2 * kWaves * 4 +
                                NT * G::KS * kWave * 16 + 256;
  static constexpr int kMaxPerWave = (kLimit - kOther) / (kWaves * kSlab);
  static constexpr int kFit = (kMaxPerWave / 4) * 4;
  static constexpr int CA = C <= kMaxPerWave ? C : (kFit > R ? kFit : R);
  static constexpr int X = CA > R ? CA - R : 0;
  static constexpr int CB = C - CA;
  static constexpr int kSlabs = kWaves * (R + X);
  static_assert(CB <= CA, "two passes hold every chunk");
  static_assert(kSlabs * kSlab + kOther <= kLimit, "LDS budget");
  // first slab of wave w's chunk c (index within its pass)
  static __device__ __forceinline__ int slab(int w, int c) {
    return c < R ? w * R + c : kWaves * R + w * X + (c - R);
  }
};

template <int KV, int D, int NT, bool NTP>
__global__ void __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<KV, D, NT>)))
attn_mfma_kernel(AttnLaunch a, int32_t row_groups) {
  using G = Geo<KV, D>;
  using MP = MergePlan<KV, D, NT>;
  // LDS: the per-wave page rings, then the merge's extra slabs (see MergePlan)
  __shared__ __attribute__((aligned(16))) uint8_t sm_raw[MP::kSlabs][kSlab];
  __shared__ f32x4 sm_m[NT * 16][kWaves / 4];       // per row: the waves' running maxima
  __shared__ f32x4 sm_fs[2][NT * 16][kWaves / 4];   // per row: the waves' O weights f (x vref) and f * l
  __shared__ int32_t sm_ids[kWaves][2][64];
  // per-token INT8: each ring slot's 16 K and 16 V scales
  __shared__ __attribute__((aligned(16))) float sm_scl[KV == KV_I8T ? kWaves * G::NRING * 32 : 4];
  __shared__ __attribute__((aligned(16))) int32_t sm_bad[kWaves];
  // the workgroup's query fragments, [nt][ks][lane] in operand order
  __shared__ f16x8 sm_q[NT][G::KS][kWave];

  // one field of each 64-byte line of the launch arguments, so that the
  // scalar loads of all of them are in flight together before the first branch
  asm volatile("" ::"s"(a.q), "s"(a.batch), "s"(a.slots), "s"(a.kv_pos0), "s"(a.positions));
  if (threadIdx.x < 64) TL_MARK(TL_ENTRY);
  UnitId u;
  if (!decode_unit(a, row_groups, u)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = lane >> 4;
  const int ncol = lane & 15;

  // the sequence's metadata in one round of loads (all four addresses are
  // valid for any b < batch), before the first branch that depends on them
  const int32_t q0 = a.qsl[u.b], q1 = a.qsl[u.b + 1];
  const int32_t ctx = a.context_lens[u.b];
  const int32_t kv0 = a.kv_pos0 ? a.kv_pos0[u.b] : 0;
  const int32_t qp0 = a.q_pos0 ? a.q_pos0[u.b] : 0;
  asm volatile("" ::"v"(q0), "v"(q1), "v"(ctx), "v"(kv0), "v"(qp0));
  if (q0 < 0 || q1 < q0 || q1 > a.total_q) return;      // rows not addressable
#ifdef RA_TIMELINE
  if (threadIdx.x < 64) {
    TL_MARK(TL_META);
    TL_VALUE(TL_HWID, __builtin_amdgcn_s_getreg((31 << 11) | 4));    // HW_ID
    TL_VALUE(TL_XCC, __builtin_amdgcn_s_getreg((31 << 11) | 20));    // XCC_ID
    TL_VALUE(TL_UNIT, ((uint64_t)u.b << 32) | ((uint64_t)u.h << 24) | ((uint64_t)u.rg << 16) | (uint64_t)u.s);
  }
#endif
  const int32_t g = (int32_t)a.fd_g.d;
  const int32_t q_len = q1 - q0;
  const int32_t rows = g * q_len;
  if (rows == 0) return;
  const int32_t row0 = u.rg * kMfmaRowsPerBlock;
  if (row0 >= rows) return;
  if (prefill_sequence(a, rows, ctx, q_len)) return;   // the prefill kernel's sequence
  bool bad = !seq_ok(a, ctx, q0, q1, kv0, qp0);
  const SeqFrame fr = seq_frame(a, ctx, q_len, kv0, qp0);
  // the row group's own queries i = row0 / g .. (last row) / g bound the keys
  // it can see: a long block (chunked prefill) skips pages past its last query
  // and masks only pages past its first
  SeqFrame frg = fr;
  frg.pmin = fr.pmin + (int32_t)fdiv(a.fd_g, (uint32_t)row0);
  frg.pmax = fr.pmin + (int32_t)fdiv(a.fd_g, (uint32_t)(min(row0 + kMfmaRowsPerBlock, rows) - 1));

  // partition and visible pages
  int32_t lo = 0, hi = 0;
  UnitPages pg{0, 0, 0, 0};
  if (!bad) {
    if (a.num_splits == 0 && a.window >= 0) {
      // windowed block, automatic partitions: cut the window span from its
      // first page; partition 0 starts at key 0 so that it also holds the sinks
      const int32_t P = a.part_window;
      const int32_t base = (max(fr.pmin - a.window + 1, 0) / kPage) * kPage;
      lo = u.s == 0 ? 0 : base + u.s * P;
      hi = min(base + (u.s + 1) * P, ctx);
    } else {
      const int32_t P = partition_tokens(a, ctx, rows);
      lo = u.s * P;
      hi = min(lo + P, ctx);
    }
    pg = unit_pages(a, frg, lo, hi);
  }
  const int32_t npages = pg.count();
  const int32_t* bt_row = a.block_tables + (int64_t)u.b * a.bt_stride;
  if (wave == 0) TL_MARK(TL_PLAN);

  // first two chunks of the wave's page ids (DMA into LDS)
  int32_t (*sm_id)[64] = sm_ids[wave];
  // Each wave takes a contiguous share of the unit's pages.  On each SIMD the
  // older wave (0-3) wins issue arbitration over its partner (4-7) and runs
  // about a fifth faster, so it takes 9 of every 16 pages of the pair: both
  // then finish together.  The split depends only on the page count.
  // (With four waves, one per SIMD, the shares are equal.)
  constexpr int32_t kFast = kWaves == 8 ? 9 : 16, kSlow = kWaves == 8 ? 16 - kFast : 16;
  const int32_t cum0 = wave < 4 ? wave * kFast : 4 * kFast + (wave - 4) * kSlow;
  const int32_t cum1 = cum0 + (wave < 4 ? kFast : kSlow);
  const int32_t p0 = (int32_t)(((int64_t)npages * cum0) >> 6), p1 = (int32_t)(((int64_t)npages * cum1) >> 6);
  const WaveSpan ws{p0, 1, p1 - p0};
  id_dma(sm_id[0], pg, ws, bt_row, 0, lane);
  id_dma(sm_id[1], pg, ws, bt_row, 1, lane);
  const uint32_t lane_off = (uint32_t)lane * 16u;

  // query fragments: lane (kgrp, ncol) holds row ncol of each 16-row tile,
  // dims kgrp * D/4 + 8 * ks .. + 8.  The workgroup loads the tile once, by
  // LDS DMA straight into operand order (one instruction per (tile, k-step)
  // fills a 1 KiB slab, lane L's 16 bytes at L * 16), in flight together with
  // the id DMA; the instructions are spread over the waves, each wave issuing
  // the same number kQOps of them (some issued twice, writing the same bytes)
  // so that its wait counts are exact.  (RoPE on the fused path rotates the
  // tile into the same slabs instead.)
  constexpr int kQInst = NT * G::KS;
  constexpr int kQOps = (kQInst + kWaves - 1) / kWaves;
  int32_t pos[NT];
  bool qlive[NT];
  const uint16_t* qp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int32_t r = row0 + nt * 16 + ncol;
    qlive[nt] = r < rows && !bad;
    const int32_t ri = (int32_t)fdiv(a.fd_g, (uint32_t)r), rj = r - ri * g;   // query token, head in group
    pos[nt] = fr.pmin + (qlive[nt] ? ri : 0);
    const int64_t qtok = qlive[nt] ? q0 + ri : 0, qhead = qlive[nt] ? u.h * g + rj : 0;
    qp[nt] = reinterpret_cast<const uint16_t*>(a.q) + qtok * a.q_stride + qhead * D + kgrp * (D / 4);
  }
  if (a.rope == nullptr) {
#pragma unroll
    for (int j = 0; j < kQOps; ++j) {
      const int i = (wave + j * kWaves) % kQInst;   // uniform
      const int qt = i / G::KS, ks = i % G::KS;
      const uint16_t* src = qp[0];
#pragma unroll
      for (int t = 1; t < NT; ++t)
        if (qt == t) src = qp[t];
      __builtin_amdgcn_global_load_lds(src + 8 * ks, (lds_u8*)&sm_q[qt][ks][0], 16, 0, 0);
    }
  }
  if (wave == 0) TL_MARK(TL_IDISS);
  // the fused store of the query tokens' own K/V (decode and verify blocks)
  bool stored = false;
  if (a.new_k != nullptr && !bad) stored = store_new_tokens<KV, D>(a, u.h, q0, q_len, fr.pmin, lo, hi);
  const int32_t my_pages = ws.count;
  constexpr int NR = G::NRING;
  uint8_t (*ring)[kSlab] = &sm_raw[wave * NR * G::NSL];
  float* scl = &sm_scl[KV == KV_I8T ? wave * NR * 32 : 0];
  // Without a store or RoPE here, the first ring pages are requested as soon
  // as the page ids have landed, and the query rows (requested after the
  // ids, so that waiting for the ids leaves them in flight) arrive meanwhile.
  const bool early = !stored && a.rope == nullptr;
  IdRing ids{0, 0};
  if (early) {
    wait_vmcnt<kQOps>();   // the id chunks, older than this wave's kQOps query loads, have landed
    if (wave == 0) TL_MARK(TL_IDLAND);
    ids.cur = read_id(sm_id[0], lane);
#pragma unroll
    for (int j = 0; j < NR; ++j)
      if (j < my_pages)
        issue_page<KV, D, NTP>(ring + j * G::NSL, scl + j * 32, ids, sm_id, a, pg, ws, j, bt_row, u.h, lane, bad);
    if (wave == 0) TL_MARK(TL_PGISS);
    // this wave's query loads, older than the pages just requested; then
    // every wave's (a plain barrier: the pages stay in flight)
    if (my_pages >= NR)
      wait_vmcnt<NR * G::OPS>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  } else {
    // the first id chunks and the query rows have landed and the stores have
    // completed, in every wave: no page load can read a stored token before
    wait_vmcnt<0>();
    __syncthreads();
  }
  if (wave == 0) {
    TL_MARK(TL_IDSQ);
    TL_VALUE(TL_PAGES, npages);
  }
  f16x8 qf[NT][G::KS];
  if (a.rope == nullptr) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      u32x4 qraw[G::KS];
      read_q_tile<G::KS>(&sm_q[nt][0][lane], qraw);
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        const u32x4 w = qlive[nt] ? qraw[ks] : u32x4{0, 0, 0, 0};
        if (a.q_bf16) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t word = w[i >> 1];
            qf[nt][ks][i] = (f16)bf16_to_f32((uint16_t)(word >> (16 * (i & 1))));
          }
        } else {
          qf[nt][ks] = as<f16x8>(w);
        }
      }
    }
  } else {
    // RoPE on the fused path: the workgroup rotates its query tile once,
    // (row, 8-dim chunk) per task, as the fused QKV kernel does (fp32, no
    // fused multiply-add, rounded to the query dtype), into LDS
    constexpr int kTasks = NT * 16 * (D / 8);
    for (int task = threadIdx.x; task < kTasks; task += kWaves * kWave) {
      const int rr = task / (D / 8), ch = task % (D / 8);
      const int32_t r = row0 + rr;
      const int d0 = 8 * ch;
      f16x8 outv = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < rows && !bad) {
        const int32_t ri = (int32_t)fdiv(a.fd_g, (uint32_t)r);
        const int64_t tok = q0 + ri;
        const uint16_t* rowp =
            reinterpret_cast<const uint16_t*>(a.q) + tok * a.q_stride + (int64_t)(u.h * g + r - ri * g) * D;
        float x[8];
        src8_to_f32(load16(rowp + d0), a.q_bf16, x);
        const int64_t rp = a.positions[tok];
        if (rp >= 0 && rp < a.rope_max_pos) {
          if (d0 < a.rot) {
            const int half = a.rot / 2;
            float partner[8];
            src8_to_f32(load16(rowp + d0 + (d0 < half ? half : -half)), a.q_bf16, partner);
            rope8(x, partner, a.rope + rp * a.rot, d0, a.rot);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = __builtin_nanf("");
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) outv[i] = a.q_bf16 ? (f16)bf16_to_f32(f32_to_bf16(x[i])) : (f16)x[i];
      }
      // operand slot: tile rr / 16, k-step ch % (D / 32), lane (ch / (D / 32)) * 16 + rr % 16
      sm_q[rr / 16][ch % (D / 32)][(ch / (D / 32)) * 16 + rr % 16] = outv;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qf[nt][ks] = sm_q[nt][ks][lane];
  }

  Acc<KV, D, NT> acc;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    acc.m[nt] = -INFINITY;
    acc.mc[nt] = 0.0f;
    acc.l[nt] = 0.0f;
    acc.ls[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) acc.o[mt][nt] = f32x4{0, 0, 0, 0};
  }
  acc.vref = acc.vinv = 0.0f;
  const float c = a.softmax_scale * a.k_scale * kLog2e;
  const float thr = kLazy / c;

  // ---- main loop over the wave's pages through the LDS
  // ring: page k computes from slot k % NRING while pages k + 1 .. k + NRING - 1
  // are in flight; once its slab reads have retired, page k + NRING is issued
  // into the slot it freed.
  if (!early) {
    ids.cur = read_id(sm_id[0], lane);
#pragma unroll
    for (int j = 0; j < NR; ++j)
      if (j < my_pages)
        issue_page<KV, D, NTP>(ring + j * G::NSL, scl + j * 32, ids, sm_id, a, pg, ws, j, bt_row, u.h, lane, bad);
  }
  if (my_pages > 0) {
    // pages are taken in pairs for the PV product: the even page of a pair
    // waits (its masked V codes and probabilities in registers) for the odd
    // one; an odd count leaves the last page to a single-page product
    static_assert(NR % 2 == 0, "page pairs must not straddle ring rounds");
    u32x4 pend_v[G::SLABS];
    float pend_p[NT][4];
#pragma unroll
    for (int sl = 0; sl < G::SLABS; ++sl) pend_v[sl] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pend_p[nt][i] = 0.0f;
    for (int32_t i = 0; i < my_pages; i += NR) {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int32_t k = i + j;
        if (k < my_pages) {
          // page k's loads retire before the (NR - 1) * OPS loads issued after
          // them, unless the tail issued fewer
          if (k + NR - 1 < my_pages)
            wait_vmcnt<(NR - 1) * G::OPS>();
          else
            wait_vmcnt<0>();
#ifdef RA_TIMELINE
          if (k == 0 && wave == 0) TL_MARK(TL_FIRST);
#endif
          PageRegs<KV, D> r;
          read_page<KV, D>(r, ring + j * G::NSL, scl + j * 32, lane_off, kgrp);
          float p[NT][4];
          scores_softmax<KV, D, NT>(acc, r, qf, a, pg, ws.page(k), ctx, frg, pos, kgrp, c, thr, p, pend_p);
          if (j & 1) {   // k odd (the ring depth is even): the pair is complete
            pv_pair<KV, D, NT>(acc, pend_v, pend_p, r.v, p);
          } else {
#pragma unroll
            for (int sl = 0; sl < G::SLABS; ++sl) pend_v[sl] = r.v[sl];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i) pend_p[nt][i] = p[nt][i];
          }
          // the slot's reads have returned (their values were consumed) before
          // the next load may overwrite it
          wait_lgkmcnt0();
          if (k + NR < my_pages)
            issue_page<KV, D, NTP>(ring + j * G::NSL, scl + j * 32, ids, sm_id, a, pg, ws, k + NR, bt_row, u.h, lane,
                              bad);
        }
      }
    }
    if (my_pages & 1) pv_single<KV, D, NT>(acc, pend_v, pend_p);
  }
  wait_vmcnt<0>();   // no ring load may land after the ring becomes the merge buffer
  TL_MARK(TL_LOOP + wave);

  // The lane's row and dim group, recomputed here (mbcnt) rather than kept
  // live in registers across the page loop.
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int kgrp_e = lane_e >> 4;
  const int ncol_e = lane_e & 15;
  // ---- combine the waves (MergePlan).  (1) Every wave publishes its rows'
  // running maxima and its bad flag, and stores the first pass's chunks of its
  // O, unscaled, into its own slabs: its ring reads have all returned.
  f32x4* slabs = reinterpret_cast<f32x4*>(&sm_raw[0][0]);   // [slab][lane]
  float lrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l;
    if constexpr (kOnesSum<KV>) {
      l = acc.ls[nt][0];   // the whole row's sum in every lane_e of the row
    } else {
      l = acc.l[nt];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
    }
    lrow[nt] = l;
    if (kgrp_e == 0) reinterpret_cast<float*>(&sm_m[nt * 16 + ncol_e][0])[wave] = acc.m[nt];
  }
  if (lane_e == 0) sm_bad[wave] = bad ? 1 : 0;
  wait_lgkmcnt0();
#pragma unroll
  for (int q = 0; q < MP::CA; ++q) {
    const int nt = q / G::MT, j = q % G::MT, i = j / (G::MT / 4), k = j % (G::MT / 4);
    slabs[MP::slab(wave, q) * kWave + lane_e] =
        f32x4{acc.o[4 * k][nt][i], acc.o[4 * k + 1][nt][i], acc.o[4 * k + 2][nt][i], acc.o[4 * k + 3][nt][i]};
  }
  __syncthreads();
  if (wave == 0) TL_MARK(TL_COMB);
  // (2) Every wave takes the rows' common maxima M and publishes its own
  // weights: f = 2^((m - M) c) for its O (times its V reference for
  // per-token INT8, whose O is in units of it) and f * l for the row sums.
  {
    const int4 b4a = *reinterpret_cast<const int4*>(&sm_bad[0]);
    bad = bad || (b4a.x | b4a.y | b4a.z | b4a.w) != 0;
    if constexpr (kWaves == 8) {
      const int4 b4b = *reinterpret_cast<const int4*>(&sm_bad[4]);
      bad = bad || (b4b.x | b4b.y | b4b.z | b4b.w) != 0;
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rr = nt * 16 + ncol_e;
    float M = -INFINITY;
#pragma unroll
    for (int qd = 0; qd < kWaves / 4; ++qd) {
      const f32x4 m4 = sm_m[rr][qd];
      M = fmaxf(M, fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    }
    float f = acc.m[nt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((acc.m[nt] - M) * c);
    const float fl = f * lrow[nt];
    if constexpr (KV == KV_I8T) f *= acc.vref;
    if (kgrp_e == 0) {
      reinterpret_cast<float*>(&sm_fs[0][rr][0])[wave] = f;
      reinterpret_cast<float*>(&sm_fs[1][rr][0])[wave] = fl;
    }
  }
  __syncthreads();
  if (wave == 0) {
    TL_MARK(TL_ML);
    TL_MARK(TL_P0W);
  }
  // (3) Sum chunk q over the waves in wave order, weighted, and write that
  // slice of the output (out and lse, or the partition's partials).  A wave's
  // chunks of a pass are summed together (their LDS reads in flight at once),
  // then written.
  const float vs = a.v_scale;
  const auto sum_chunk = [&](int q, int cpass, float (&v)[4], float& L) {
    const int rr = (q / G::MT) * 16 + ncol_e;
    float fw[kWaves];
    L = 0.0f;
#pragma unroll
    for (int qd = 0; qd < kWaves / 4; ++qd) {
      const f32x4 f4 = sm_fs[0][rr][qd], l4 = sm_fs[1][rr][qd];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fw[4 * qd + t] = f4[t];
        L += l4[t];
      }
    }
    f32x4 x[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x[w] = slabs[MP::slab(w, cpass) * kWave + lane_e];
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = fmaf(x[w][t], fw[w], v[t]);
  };
  const auto emit_chunk = [&](int q, float (&v)[4], float L) {
    const int nt = q / G::MT, j = q % G::MT, i = j / (G::MT / 4), k = j % (G::MT / 4);
    const int rr = nt * 16 + ncol_e;
    const int32_t r = row0 + rr;
    if (r < rows) {
      const int32_t qi = (int32_t)fdiv(a.fd_g, (uint32_t)r), hj = r - qi * g;
      const int64_t orow = (int64_t)(q0 + qi) * a.hq + u.h * g + hj;
      // a row with no visible key has L = 0 (out 0, lse -inf); NaN scores
      // leave L = NaN, and the row stays NaN in out and lse
      const float inv = L > 0.0f ? vs / L : (L == L ? 0.0f : __builtin_nanf(""));
      const int d0 = (4 * kgrp_e + i) * G::MT + 4 * k;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = bad ? __builtin_nanf("") : v[t] * inv;
      if (a.direct) {
        uint16_t hv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) hv[t] = a.q_bf16 ? f32_to_bf16(v[t]) : as<uint16_t>((f16)v[t]);
        u32x2 w2;
        w2[0] = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
        w2[1] = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + orow * D + d0) = w2;
      } else {
        float* op = a.part_out + ((int64_t)u.s * a.total_q * a.hq + orow) * D + d0;
        *reinterpret_cast<f32x4*>(op) = f32x4{v[0], v[1], v[2], v[3]};
      }
      if (kgrp_e == 0 && j == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int qd = 0; qd < kWaves / 4; ++qd) {
          const f32x4 m4 = sm_m[rr][qd];
          M = fmaxf(M, fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
        }
        float lse = L > 0.0f ? (M * c + log2f(L)) * kLn2 : (L == L ? -INFINITY : __builtin_nanf(""));
        if (bad) lse = __builtin_nanf("");
        if (a.direct) {
          if (a.lse) a.lse[orow] = lse;
        } else {
          a.part_lse[(int64_t)u.s * a.total_q * a.hq + orow] = lse;
        }
      }
    }
  };
  // chunks [QA, QB) of a pass: this wave's are QA + wave + t * kWaves
  const auto reduce_pass = [&](auto qa, auto qb) {
    constexpr int QA = decltype(qa)::value, QB = decltype(qb)::value;
    constexpr int kPer = (QB - QA + kWaves - 1) / kWaves;
    constexpr bool kFull = (QB - QA) % kWaves == 0;
    float v[kPer][4], L[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int q = QA + wave + t * kWaves;
      if (kFull || q < QB) sum_chunk(q, q - QA, v[t], L[t]);
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int q = QA + wave + t * kWaves;
      if (kFull || q < QB) emit_chunk(q, v[t], L[t]);
    }
  };
  reduce_pass(IntC<0>{}, IntC<MP::CA>{});
  if (wave == 0) TL_MARK(TL_P0R);
  if constexpr (MP::CB > 0) {
    // (4) the second pass, through the same slabs once every wave has read
    // the first
    __syncthreads();
#pragma unroll
    for (int q = MP::CA; q < MP::C; ++q) {
      const int nt = q / G::MT, j = q % G::MT, i = j / (G::MT / 4), k = j % (G::MT / 4);
      slabs[MP::slab(wave, q - MP::CA) * kWave + lane_e] =
          f32x4{acc.o[4 * k][nt][i], acc.o[4 * k + 1][nt][i], acc.o[4 * k + 2][nt][i], acc.o[4 * k + 3][nt][i]};
    }
    __syncthreads();
    if (wave == 0) TL_MARK(TL_P0W + 1);
    reduce_pass(IntC<MP::CA>{}, IntC<MP::C>{});
    if (wave == 0) TL_MARK(TL_P0R + 1);
  }
  TL_MARK(TL_END + wave);
}

template <int KV, int D, int NT>
hipError_t launch_t(const AttnLaunch& a, int32_t row_groups, hipStream_t s) {
  const int64_t units = (int64_t)a.slots * a.hkv * row_groups * a.batch;
  // one row group: every page is read by one workgroup, once (nontemporal)
  if (row_groups == 1)
    hipLaunchKernelGGL((attn_mfma_kernel<KV, D, NT, true>), dim3(padded_grid(units)), dim3(kWaves * kWave), 0, s,
                       a, row_groups);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<KV, D, NT, false>), dim3(padded_grid(units)), dim3(kWaves * kWave), 0, s,
                       a, row_groups);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_nt(const AttnLaunch& a, int nt, int32_t row_groups, hipStream_t s) {
  switch (nt) {
    case 1: return launch_t<KV, D, 1>(a, row_groups, s);
    case 2: return launch_t<KV, D, 2>(a, row_groups, s);
    default: return launch_t<KV, D, 3>(a, row_groups, s);
  }
}

template <int KV>
hipError_t launch_d(const AttnLaunch& a, int nt, int32_t row_groups, hipStream_t s) {
  return a.head_dim == 64 ? launch_nt<KV, 64>(a, nt, row_groups, s) : launch_nt<KV, 128>(a, nt, row_groups, s);
}

}  // namespace

hipError_t launch_attn_mfma(const AttnLaunch& a0, hipStream_t s) {
  const int32_t g = a0.hq / a0.hkv;
  const int32_t rows_max = g * a0.max_q_len;
  const int32_t rows_blk = rows_max < kMfmaRowsPerBlock ? rows_max : kMfmaRowsPerBlock;
  const int nt = (rows_blk + 15) / 16;
  const int32_t row_groups = (rows_max + kMfmaRowsPerBlock - 1) / kMfmaRowsPerBlock;
  AttnLaunch a = a0;
  a.fd_g = make_fastdiv((uint32_t)g);
  a.fd_batch = make_fastdiv((uint32_t)a.batch);
  a.fd_hkv = make_fastdiv((uint32_t)a.hkv);
  a.fd_rg = make_fastdiv((uint32_t)row_groups);
  switch (a.kv) {
    case KV_F16: return launch_d<KV_F16>(a, nt, row_groups, s);
    case KV_E4M3: return launch_d<KV_E4M3>(a, nt, row_groups, s);
    case KV_I8T: return launch_d<KV_I8T>(a, nt, row_groups, s);
    default: return launch_d<KV_I8>(a, nt, row_groups, s);
  }
}

}  // namespace ra

#ifdef RA_TIMELINE
// Timing build only: copy the timeline to host memory, or clear it.
extern "C" int32_t ra_timeline_read(void* host, size_t bytes) {
  if (bytes > sizeof(ra_timeline)) bytes = sizeof(ra_timeline);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(ra_timeline), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0 : 5;
}
extern "C" int32_t ra_timeline_clear(void) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(ra_timeline)) != hipSuccess) return 5;
  if (hipMemset(p, 0, sizeof(ra_timeline)) != hipSuccess) return 5;
  return hipDeviceSynchronize() == hipSuccess ? 0 : 5;
}
extern "C" int32_t ra_timeline_layout(int32_t* blocks, int32_t* slots) {
  *blocks = RA_TIMELINE_BLOCKS;
  *slots = kTlSlots;
  return 0;
}
#endif
