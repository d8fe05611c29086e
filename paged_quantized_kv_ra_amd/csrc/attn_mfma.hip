// attn_mfma.hip -- grouped verify attention on the gfx950 matrix cores.
//
// Used when a (sequence, KV head) unit has g * q_len >= 16 query rows (the
// pages' MTP4 verify block of 1 + 4 tokens times the query heads of one KV
// head: ReVolta README, intro list and "Quick start").  The KV cache is read
// once, straight into registers, and converted exactly to FP16 operands (the
// pages' V100 converts stored KV to FP16 for the arithmetic: ReVolta README,
// "Weight and KV formats").
//
// Per wavefront and pair of 16-token pages:
//   S^T[32 keys][16 rows]  = K[32][D] . Q^T[D][16]     v_mfma_f32_16x16x32_f16, per 16-row tile
//   P^T = exp2(c * S^T - c * m)   (online softmax, fp32, rescaled lazily)
//   O^T[D][16 rows]       += V^T[D][32] . P^T[32][16]
// The cache layout puts every lane's 16-byte loads directly in the operand
// order of both products: a K lane holds one token's contiguous D/4 dims, a V
// lane holds four consecutive tokens of D/16 dims, and the S^T accumulator
// layout (lane = row + 16 * token-quad) is exactly the P^T operand layout, so
// no data moves between lanes or through LDS in the hot loop.
//
// A workgroup has 4 waves that take page pairs round-robin; their partial
// (m, l, O) are combined through LDS in a fixed order at the end.
#include "attn_common.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;   // log2 headroom before the running max is refreshed

template <int KV, int D>
struct Geo {
  static constexpr int E = KV == KV_F16 ? 2 : 1;
  static constexpr int SLABS = D * E / 64;       // 16-byte loads per lane per page
  static constexpr int KS = D / 32;              // k-steps of the QK product
  static constexpr int MT = D / 16;              // 16-dim tiles of the PV product
  static constexpr int BLK = kPage * D * E;      // bytes per (page, head) block
};

template <int KV, int D>
struct PairRegs {
  u32x4 k[2][Geo<KV, D>::SLABS];
  u32x4 v[2][Geo<KV, D>::SLABS];
};

// Issue the loads of page pair `p` (logical pages 2p, 2p+1 of the unit).
template <int KV, int D>
__device__ __forceinline__ void load_pair(PairRegs<KV, D>& r, const AttnLaunch& a, const UnitPages& pg,
                                          int32_t npages, int32_t p, const int32_t* bt_row, int h,
                                          uint32_t lane_off, bool& bad) {
  using G = Geo<KV, D>;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int32_t n = 2 * p + x;
    int32_t pid = -1;
    if (n < npages) {
      pid = bt_row[pg.page(n)];
      if (pid < 0 || pid >= a.num_pages) { bad = true; pid = -1; }
    }
    if (pid >= 0) {
      const int64_t blk = ((int64_t)pid * a.hkv + h) * G::BLK;
      const uint8_t* kp = a.k_cache + blk + lane_off;
      const uint8_t* vp = a.v_cache + blk + lane_off;
#pragma unroll
      for (int j = 0; j < G::SLABS; ++j) r.k[x][j] = load16(kp + j * 1024);
#pragma unroll
      for (int j = 0; j < G::SLABS; ++j) r.v[x][j] = load16(vp + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < G::SLABS; ++j) { r.k[x][j] = u32x4{0, 0, 0, 0}; r.v[x][j] = u32x4{0, 0, 0, 0}; }
    }
  }
}

template <int KV, int D>
__device__ __forceinline__ f16x8 k_operand(const PairRegs<KV, D>& r, int x, int ks) {
  if constexpr (KV == KV_F16) {
    return as<f16x8>(r.k[x][ks]);
  } else {
    const u32x4 w = r.k[x][ks >> 1];
    const uint32_t d0 = (ks & 1) ? w[2] : w[0];
    const uint32_t d1 = (ks & 1) ? w[3] : w[1];
    const f16x4 lo = codes4_to_f16x4<KV>(d0);
    const f16x4 hi = codes4_to_f16x4<KV>(d1);
    return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Four consecutive tokens (of page x) of dim tile mt, as fp16.
template <int KV, int D>
__device__ __forceinline__ f16x4 v_quad(const PairRegs<KV, D>& r, int x, int mt) {
  if constexpr (KV == KV_F16) {
    const u32x4 w = r.v[x][mt >> 1];
    const uint32_t a = (mt & 1) ? w[2] : w[0];
    const uint32_t b = (mt & 1) ? w[3] : w[1];
    const f16x2 lo = as<f16x2>(a);
    const f16x2 hi = as<f16x2>(b);
    return f16x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    const u32x4 w = r.v[x][mt >> 2];
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
__device__ __forceinline__ void compute_pair(Acc<KV, D, NT>& acc, const PairRegs<KV, D>& r,
                                             const f16x8 (&qf)[NT][Geo<KV, D>::KS],
                                             const AttnLaunch& a, const UnitPages& pg, int32_t npages,
                                             int32_t p, int32_t ctx, int32_t q_len,
                                             const int32_t (&pos)[NT], int kgrp, float c, float thr) {
  using G = Geo<KV, D>;
  // ---- scores: S^T tiles for both pages
  f32x4 s[2][NT];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s[x][nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      const f16x8 kop = k_operand<KV, D>(r, x, ks);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        s[x][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qf[nt][ks], s[x][nt], 0, 0, 0);
    }
  }
  // ---- masks (only for pairs that can hold an invisible key)
  const int32_t n0 = 2 * p;
  const bool has_b = n0 + 1 < npages;
  const int32_t tok0 = pg.page(n0) * kPage;
  const int32_t tok1 = has_b ? pg.page(n0 + 1) * kPage : tok0;
  const bool need_mask = !has_b || (tok1 + kPage - 1 > ctx - q_len) ||
                         (a.window >= 0 && tok0 <= ctx - q_len - a.window);
  uint32_t vlive[2] = {0xFu, 0xFu};   // per page: bit i set where token 4*kgrp+i holds data
  bool sanitize = false;
  if (need_mask) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int32_t tb = (x == 0 ? tok0 : tok1) + 4 * kgrp;
      const bool live = x == 0 || has_b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t j = tb + i;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bool vis = live && key_visible(a, j, pos[nt]);
          s[x][nt][i] = vis ? s[x][nt][i] : -INFINITY;
        }
        if (!(live && j < ctx)) vlive[x] &= ~(1u << i);
      }
    }
    sanitize = true;
  }
  // ---- online softmax with lazy max refresh
  float mx[NT];
  bool trig = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float v = fmaxf(fmaxf(s[0][nt][0], s[0][nt][1]), fmaxf(s[0][nt][2], s[0][nt][3]));
    v = fmaxf(v, fmaxf(fmaxf(s[1][nt][0], s[1][nt][1]), fmaxf(s[1][nt][2], s[1][nt][3])));
    mx[nt] = v;
    trig |= v > acc.m[nt] + thr;
  }
  if (__any(trig)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float rm = mx[nt];
      rm = fmaxf(rm, __shfl_xor(rm, 16));
      rm = fmaxf(rm, __shfl_xor(rm, 32));
      const bool upd = rm > acc.m[nt] + thr;
      const float alpha = upd ? (acc.m[nt] == -INFINITY ? 0.0f : exp2f((acc.m[nt] - rm) * c)) : 1.0f;
      acc.m[nt] = upd ? rm : acc.m[nt];
      acc.l[nt] *= alpha;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) acc.o[mt][nt] *= alpha;
    }
  }
  f16x8 pf[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float mc = acc.m[nt] == -INFINITY ? 0.0f : acc.m[nt] * c;
    float ps = 0.0f;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2f(fmaf(s[x][nt][i], c, -mc));
        ps += e;
        pf[nt][4 * x + i] = (f16)e;
      }
    }
    acc.l[nt] += ps;
  }
  // ---- O^T += V^T . P^T
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt) {
    f16x4 v0 = v_quad<KV, D>(r, 0, mt);
    f16x4 v1 = v_quad<KV, D>(r, 1, mt);
    if (sanitize) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v0[i] = (vlive[0] >> i) & 1u ? v0[i] : (f16)0.0f;
        v1[i] = (vlive[1] >> i) & 1u ? v1[i] : (f16)0.0f;
      }
    }
    const f16x8 vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc.o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pf[nt], acc.o[mt][nt], 0, 0, 0);
  }
}

template <int KV, int D, int NT>
__global__ void __launch_bounds__(kWaves * kWave) attn_mfma_kernel(AttnLaunch a, int32_t row_groups) {
  using G = Geo<KV, D>;
  __shared__ float sm_ml[2][kWaves][NT * 16];
  __shared__ f32x4 sm_o[2][G::MT * NT][kWave];

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
  const int32_t npairs = (npages + 1) / 2;
  const int32_t* bt_row = a.block_tables + (int64_t)u.b * a.bt_stride;

  // query fragments: lane (kgrp, ncol) holds row ncol of each 16-row tile,
  // dims kgrp * D/4 + 8 * ks .. + 8
  f16x8 qf[NT][G::KS];
  int32_t pos[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int32_t r = row0 + nt * 16 + ncol;
    const bool live = r < rows && !bad;
    const int32_t qi = live ? r / g : 0;
    const int32_t hj = live ? r % g : 0;
    pos[nt] = live ? ctx - q_len + qi : ctx - 1;
    const int64_t qbase = (((int64_t)(q0 + qi) * a.hq + u.h * g + hj) * D) + kgrp * (D / 4);
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      if (!live) { qf[nt][ks] = f16x8{0, 0, 0, 0, 0, 0, 0, 0}; continue; }
      const u32x4 w = load16(reinterpret_cast<const uint16_t*>(a.q) + qbase + 8 * ks);
      if (a.q_bf16) {
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (f16)bf16_to_f32((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
        qf[nt][ks] = h;
      } else {
        qf[nt][ks] = as<f16x8>(w);
      }
    }
  }

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

  // ---- main loop: two register buffers, the next pair loads while one computes
  PairRegs<KV, D> ra{}, rb{};   // zeroed: no path carries undefined registers into the loop
  int32_t p = wave;
  if (p < npairs) load_pair<KV, D>(ra, a, pg, npages, p, bt_row, u.h, lane_off, bad);
  for (; p < npairs; p += 2 * kWaves) {
    if (p + kWaves < npairs) load_pair<KV, D>(rb, a, pg, npages, p + kWaves, bt_row, u.h, lane_off, bad);
    compute_pair<KV, D, NT>(acc, ra, qf, a, pg, npages, p, ctx, q_len, pos, kgrp, c, thr);
    if (p + kWaves >= npairs) break;
    if (p + 2 * kWaves < npairs) load_pair<KV, D>(ra, a, pg, npages, p + 2 * kWaves, bt_row, u.h, lane_off, bad);
    compute_pair<KV, D, NT>(acc, rb, qf, a, pg, npages, p + kWaves, ctx, q_len, pos, kgrp, c, thr);
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
  // round 1: waves 2, 3 -> waves 0, 1
  if (wave >= 2) {
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sm_o[wave - 2][mt * NT + nt][lane] = acc.o[mt][nt];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc.o[mt][nt] += sm_o[wave][mt * NT + nt][lane];
  }
  __syncthreads();
  // round 2: wave 1 -> wave 0
  if (wave == 1) {
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sm_o[0][mt * NT + nt][lane] = acc.o[mt][nt];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc.o[mt][nt] += sm_o[0][mt * NT + nt][lane];

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
