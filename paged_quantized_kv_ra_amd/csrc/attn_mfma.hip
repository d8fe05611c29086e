// attn_mfma.hip -- grouped verify attention on the gfx950 matrix cores.
//
// Used when a (sequence, KV head) unit has g * q_len >= 16 query rows (the
// pages' MTP4 verify block of 1 + 4 tokens times the query heads of one KV
// head: ReVolta README, intro list and "Quick start").  The KV cache is read
// once, straight into registers, and converted exactly to FP16 operands (the
// pages' V100 converts stored KV to FP16 for the arithmetic: ReVolta README,
// "Weight and KV formats").
//
// Per wavefront and 16-token page, for each 16-row tile of query rows:
//   S^T[16 keys][16 rows] = K[16][D] . Q^T[D][16]      v_mfma_f32_16x16x32_f16 (D/32 steps)
//   P^T = exp2(c * S^T - c * m)                       online softmax, fp32, rescaled lazily
//   O^T[D][16 rows]      += V^T[D][16] . P^T[16][16]   v_mfma_f32_16x16x16_f16 (D/16 tiles)
// The cache layout puts every lane's 16-byte loads directly in the operand
// order of both products: a K lane holds one token's contiguous D/4 dims, a V
// lane holds four consecutive tokens of D/16 dims, and the S^T accumulator
// layout (lane = row + 16 * token-quad) is exactly the P^T operand layout, so
// no data moves between lanes or through LDS in the hot loop.  Pages stream
// through a ring of NBUF register buffers, NBUF - 1 pages in flight per wave.
//
// A workgroup has 8 waves (two per SIMD) that take pages round-robin; their partial
// (m, l, O) are combined through LDS in a fixed order at the end.
#include "attn_common.h"

namespace ra {
namespace {

constexpr int kWaves = 8;   // waves per workgroup (two per SIMD)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;   // log2 headroom before the running max is refreshed

// depth of the per-wave page ring (tuning constants)
#ifndef RA_MFMA_RING_8BIT
#define RA_MFMA_RING_8BIT 2
#endif
#ifndef RA_MFMA_RING_16BIT
#define RA_MFMA_RING_16BIT 2
#endif

template <int KV, int D>
struct Geo {
  static constexpr int E = KV == KV_F16 ? 2 : 1;
  static constexpr int SLABS = D * E / 64;       // 16-byte loads per lane per page (K, and again V)
  static constexpr int KS = D / 32;              // k-steps of the QK product
  static constexpr int MT = D / 16;              // 16-dim tiles of the PV product
  static constexpr int BLK = kPage * D * E;      // bytes per (page, head) block
  // register buffers of the page ring: one page (K and V) is 8 * SLABS VGPRs
  static constexpr int NBUF = E == 1 ? RA_MFMA_RING_8BIT : RA_MFMA_RING_16BIT;
};

template <int KV, int D>
struct PageRegs {
  u32x4 k[Geo<KV, D>::SLABS];
  u32x4 v[Geo<KV, D>::SLABS];
};

// Issue the loads of the wave's i-th page (logical page wave + 4 i of the
// unit).  Branch-free: a page past the unit's end loads page 0 and is never
// computed, so the compiler can keep the next pages' loads in flight.
template <int KV, int D>
__device__ __forceinline__ void load_page(PageRegs<KV, D>& r, PageIdChunks& ids, const AttnLaunch& a,
                                          const UnitPages& pg, int32_t npages, int32_t wave, int32_t i,
                                          const int32_t* bt_row, int h, uint32_t lane_off, int lane, bool& bad) {
  using G = Geo<KV, D>;
  const bool live = wave_page<1, kWaves>(wave, i) < npages;
  const int32_t pid = page_id<1, kWaves>(ids, a, pg, npages, bt_row, wave, i, lane, live, bad);
  const int64_t blk = ((int64_t)pid * a.hkv + h) * G::BLK;
  const uint8_t* kp = a.k_cache + blk + lane_off;
  const uint8_t* vp = a.v_cache + blk + lane_off;
#pragma unroll
  for (int j = 0; j < G::SLABS; ++j) r.k[j] = load16(kp + j * 1024);
#pragma unroll
  for (int j = 0; j < G::SLABS; ++j) r.v[j] = load16(vp + j * 1024);
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
__device__ __forceinline__ f16x4 v_operand(const PageRegs<KV, D>& r, int mt) {
  if constexpr (KV == KV_F16) {
    const u32x4 w = r.v[mt >> 1];
    const uint32_t a = (mt & 1) ? w[2] : w[0];
    const uint32_t b = (mt & 1) ? w[3] : w[1];
    const f16x2 lo = as<f16x2>(a);
    const f16x2 hi = as<f16x2>(b);
    return f16x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    const u32x4 w = r.v[mt >> 2];
    return codes4_to_f16x4<KV>(w[mt & 3]);
  }
}

template <int KV, int D, int NT>
struct Acc {
  f32x4 o[Geo<KV, D>::MT][NT];
  float m[NT];
  float l[NT];
};

template <int KV, int D, int NT>
__device__ __forceinline__ void compute_page(Acc<KV, D, NT>& acc, PageRegs<KV, D>& r,
                                             const f16x8 (*sm_q)[Geo<KV, D>::KS][kWave], int lane,
                                             const AttnLaunch& a, const UnitPages& pg, int32_t n, int32_t ctx,
                                             int32_t q_len, const int32_t (&pos)[NT], int kgrp, float c,
                                             float thr) {
  using G = Geo<KV, D>;
  // ---- scores S^T for the page's 16 keys
  f32x4 s[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) s[nt] = f32x4{0, 0, 0, 0};
  // the query fragments are re-read from LDS for every page (an opaque index
  // keeps the compiler from hoisting them into registers for the whole loop)
  int li = lane;
  asm volatile("" : "+v"(li));
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const f16x8 kop = k_operand<KV, D>(r, ks);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, sm_q[nt][ks][li], s[nt], 0, 0, 0);
  }
  // ---- masks (only on pages that can hold an invisible key).  Keys past ctx
  // (stale bytes of the last page) also get their V codes zeroed so that
  // 0 * garbage cannot produce NaN.
  const int32_t tok0 = pg.page(n) * kPage;
  const bool need_mask = (tok0 + kPage - 1 > ctx - q_len) || (a.window >= 0 && tok0 <= ctx - 1 - a.window);
  if (need_mask) {
    const int32_t tb = tok0 + 4 * kgrp;
    uint32_t keep8 = 0, keep_lo = 0, keep_hi = 0;   // byte / half masks of the lane's 4 tokens
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t j = tb + i;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[nt][i] = key_visible(a, j, pos[nt]) ? s[nt][i] : -INFINITY;
      const bool data = j < ctx;
      keep8 |= data ? 0xFFu << (8 * i) : 0u;
      if (i < 2) keep_lo |= data ? 0xFFFFu << (16 * i) : 0u;
      else keep_hi |= data ? 0xFFFFu << (16 * (i - 2)) : 0u;
    }
#pragma unroll
    for (int sl = 0; sl < G::SLABS; ++sl)
#pragma unroll
      for (int w = 0; w < 4; ++w) r.v[sl][w] &= KV == KV_F16 ? ((w & 1) ? keep_hi : keep_lo) : keep8;
  }
  // ---- online softmax with lazy max refresh
  float mx[NT];
  bool trig = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    mx[nt] = fmaxf(fmaxf(s[nt][0], s[nt][1]), fmaxf(s[nt][2], s[nt][3]));
    trig |= mx[nt] > acc.m[nt] + thr;
  }
  if (__any(trig)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float rm = mx[nt];
      rm = fmaxf(rm, __shfl_xor(rm, 16));
      rm = fmaxf(rm, __shfl_xor(rm, 32));
      const bool upd = rm > acc.m[nt] + thr;
      const float alpha = upd ? (acc.m[nt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((acc.m[nt] - rm) * c))
                              : 1.0f;
      acc.m[nt] = upd ? rm : acc.m[nt];
      acc.l[nt] *= alpha;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) acc.o[mt][nt] *= alpha;
    }
  }
  f16x4 pf[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float mc = acc.m[nt] == -INFINITY ? 0.0f : acc.m[nt] * c;
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(s[nt][i], c, -mc));
      ps += e;
      pf[nt][i] = (f16)e;
    }
    acc.l[nt] += ps;
  }
  // ---- O^T += V^T . P^T
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt) {
    const f16x4 vop = v_operand<KV, D>(r, mt);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc.o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop, pf[nt], acc.o[mt][nt], 0, 0, 0);
  }
}

template <int KV, int D, int NT>
__global__ void __launch_bounds__(kWaves * kWave) attn_mfma_kernel(AttnLaunch a, int32_t row_groups) {
  using G = Geo<KV, D>;
  __shared__ float sm_ml[2][kWaves][NT * 16];
  __shared__ f32x4 sm_o[kWaves / 2][G::MT * NT][kWave];
  __shared__ f16x8 sm_q[NT][G::KS][kWave];

  UnitId u;
  if (!decode_unit(a, row_groups, u)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = lane >> 4;
  const int ncol = lane & 15;

  const int32_t q0 = a.qsl[u.b], q1 = a.qsl[u.b + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.total_q) return;      // rows not addressable
  const int32_t g = a.hq / a.hkv;
  const int32_t q_len = q1 - q0;
  const int32_t rows = g * q_len;
  if (rows < kMfmaMinRows) return;                      // the vector kernel's unit
  const int32_t row0 = u.rg * kMfmaRowsPerBlock;
  if (row0 >= rows) return;
  const int32_t ctx = a.context_lens[u.b];
  bool bad = !seq_ok(a, ctx, q0, q1);

  // partition and visible pages
  int32_t lo = 0, hi = 0;
  UnitPages pg{0, 0, 0, 0};
  if (!bad) {
    const int32_t P = partition_tokens(a, ctx);
    lo = u.s * P;
    hi = min(lo + P, ctx);
    pg = unit_pages(a, ctx, q_len, lo, hi);
  }
  const int32_t npages = pg.count();
  const int32_t* bt_row = a.block_tables + (int64_t)u.b * a.bt_stride;

  // query fragments: lane (kgrp, ncol) holds row ncol of each 16-row tile,
  // dims kgrp * D/4 + 8 * ks .. + 8.  They are the same for the 4 waves, so
  // wave 0 converts them once into LDS and every wave reads them per pair
  // (keeping registers for the load pipeline).
  int32_t pos[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int32_t r = row0 + nt * 16 + ncol;
    pos[nt] = (r < rows && !bad) ? ctx - q_len + r / g : ctx - 1;
  }
  if (wave == 0) {
    u32x4 qraw[NT][G::KS];
    bool qlive[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int32_t r = row0 + nt * 16 + ncol;
      qlive[nt] = r < rows && !bad;
      const int64_t qrow = qlive[nt] ? ((int64_t)(q0 + r / g) * a.hq + u.h * g + r % g) : 0;
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qrow * D + kgrp * (D / 4);
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qraw[nt][ks] = load16(qp + 8 * ks);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        const u32x4 w = qlive[nt] ? qraw[nt][ks] : u32x4{0, 0, 0, 0};
        f16x8 h;
        if (a.q_bf16) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t word = w[i >> 1];
            h[i] = (f16)bf16_to_f32((uint16_t)(word >> (16 * (i & 1))));
          }
        } else {
          h = as<f16x8>(w);
        }
        sm_q[nt][ks][lane] = h;
      }
    }
  }
  __syncthreads();

  Acc<KV, D, NT> acc;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    acc.m[nt] = -INFINITY;
    acc.l[nt] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) acc.o[mt][nt] = f32x4{0, 0, 0, 0};
  }
  const float c = a.softmax_scale * a.k_scale * kLog2e;
  const float thr = kLazy / c;
  const uint32_t lane_off = (uint32_t)lane * 16u;

  // ---- main loop over the wave's pages (page wave + 4 i) through a ring of
  // NBUF register buffers: the loads of pages i + 1 .. i + NBUF - 1 are in
  // flight while page i computes.
  PageIdChunks ids;
  init_ids<1, kWaves>(ids, pg, npages, bt_row, wave, lane);
  const int32_t my_pages = npages > wave ? (npages - wave + kWaves - 1) / kWaves : 0;
  if (my_pages > 0) {
    constexpr int NB = G::NBUF;
    PageRegs<KV, D> buf[NB];
#pragma unroll
    for (int j = 0; j < NB - 1; ++j)
      load_page<KV, D>(buf[j], ids, a, pg, npages, wave, j, bt_row, u.h, lane_off, lane, bad);
    for (int32_t i = 0;; i += NB) {
      bool done = false;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (!done) {
          load_page<KV, D>(buf[(j + NB - 1) % NB], ids, a, pg, npages, wave, i + j + NB - 1, bt_row, u.h,
                           lane_off, lane, bad);
          compute_page<KV, D, NT>(acc, buf[j], sm_q, lane, a, pg, wave + kWaves * (i + j), ctx, q_len, pos,
                                  kgrp, c, thr);
          done = i + j + 1 >= my_pages;
        }
      }
      if (done) break;
    }
  }

  // ---- combine the waves: rows' (m, l), then O in a fixed tree order
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = acc.l[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    acc.l[nt] = l;
    if (kgrp == 0) {
      sm_ml[0][wave][nt * 16 + ncol] = acc.m[nt];
      sm_ml[1][wave][nt * 16 + ncol] = l;
    }
  }
  bad = __syncthreads_or(bad ? 1 : 0) != 0;
  float Mrow[NT], Lrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rr = nt * 16 + ncol;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[0][w][rr]);
    float L = 0.0f, fself = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_ml[0][w][rr];
      const float f = (mw == -INFINITY) ? 0.0f : exp2f((mw - M) * c);
      L += f * sm_ml[1][w][rr];
      if (w == wave) fself = f;
    }
    Mrow[nt] = M;
    Lrow[nt] = L;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) acc.o[mt][nt] *= fself;
  }
  // fixed-order tree: in each round the upper half of the live waves hands its
  // O to the lower half through LDS ((O0 + O4) + (O2 + O6)) + ((O1 + O5) + (O3 + O7))
#pragma unroll
  for (int half = kWaves / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sm_o[wave - half][mt * NT + nt][lane] = acc.o[mt][nt];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc.o[mt][nt] += sm_o[wave][mt * NT + nt][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // ---- epilogue: lane writes row (nt, ncol), dims (4*kgrp+i)*MT .. +MT
  const float vs = a.v_scale;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int32_t r = row0 + nt * 16 + ncol;
    if (r >= rows) continue;
    const int32_t qi = r / g, hj = r % g;
    const int64_t orow = (int64_t)(q0 + qi) * a.hq + u.h * g + hj;
    const float L = Lrow[nt];
    const float inv = L > 0.0f ? vs / L : 0.0f;
    float lse = L > 0.0f ? (Mrow[nt] * c + log2f(L)) * kLn2 : -INFINITY;
    if (bad) lse = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = (4 * kgrp + i) * G::MT;
      float v[G::MT];
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) v[mt] = bad ? __builtin_nanf("") : acc.o[mt][nt][i] * inv;
      if (a.direct) {
        uint16_t hv[G::MT];
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
          hv[mt] = a.q_bf16 ? f32_to_bf16(v[mt]) : as<uint16_t>((f16)v[mt]);
        uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + orow * D + d0;
#pragma unroll
        for (int k = 0; k < G::MT / 8; ++k) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = (uint32_t)hv[8 * k + 2 * j] | ((uint32_t)hv[8 * k + 2 * j + 1] << 16);
          *reinterpret_cast<u32x4*>(op + 8 * k) = w;
        }
        if constexpr (G::MT % 8 != 0) {
          u32x2 w;
          w[0] = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
          w[1] = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
          *reinterpret_cast<u32x2*>(op) = w;
        }
      } else {
        float* op = a.part_out + ((int64_t)u.s * a.total_q * a.hq + orow) * D + d0;
#pragma unroll
        for (int k = 0; k < G::MT / 4; ++k)
          *reinterpret_cast<f32x4*>(op + 4 * k) = f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
      }
    }
    if (kgrp == 0) {
      if (a.direct) {
        if (a.lse) a.lse[orow] = lse;
      } else {
        a.part_lse[(int64_t)u.s * a.total_q * a.hq + orow] = lse;
      }
    }
  }
}

template <int KV, int D, int NT>
hipError_t launch_t(const AttnLaunch& a, int32_t row_groups, hipStream_t s) {
  const int64_t units = (int64_t)a.slots * a.hkv * row_groups * a.batch;
  hipLaunchKernelGGL((attn_mfma_kernel<KV, D, NT>), dim3(padded_grid(units)), dim3(kWaves * kWave), 0, s,
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

hipError_t launch_attn_mfma(const AttnLaunch& a, hipStream_t s) {
  const int32_t g = a.hq / a.hkv;
  const int32_t rows_max = g * a.max_q_len;
  const int32_t rows_blk = rows_max < kMfmaRowsPerBlock ? rows_max : kMfmaRowsPerBlock;
  const int nt = (rows_blk + 15) / 16;
  const int32_t row_groups = (rows_max + kMfmaRowsPerBlock - 1) / kMfmaRowsPerBlock;
  switch (a.kv) {
    case KV_F16: return launch_d<KV_F16>(a, nt, row_groups, s);
    case KV_E4M3: return launch_d<KV_E4M3>(a, nt, row_groups, s);
    default: return launch_d<KV_I8>(a, nt, row_groups, s);
  }
}

}  // namespace ra
