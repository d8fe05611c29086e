// attn_vec.hip -- decode attention for units with fewer than 16 query rows.
//
// A (sequence, KV head) unit with g * q_len < 16 rows (plain decode, q_len 1,
// of the pages' serving loop: ReVolta README, intro list) is too thin for a
// 16-row matrix tile, so this kernel computes it on the vector ALUs.  It reads
// the same paged layout as the matrix-core kernel with the same 16-byte
// loads: lane (kgrp, t) holds token t's dims [kgrp * D/4, +D/4) of K, and lane
// (kq, m) holds tokens 4*kq .. 4*kq+3 of dims [m * D/16, +D/16) of V.
//
// Per wavefront and 16-token page:
//   partial q.k over the lane's D/4 dims (fp16 x fp16 -> fp32 fused products),
//   summed over the 4 lane groups with cross-lane shuffles;
//   online softmax (fp32, lazy max refresh) per (row, token);
//   probabilities exchanged through a per-wave LDS row, then
//   acc[row][dim] += p * v over the lane's 4 tokens.
// Up to 8 rows per workgroup; wider units use more row groups.
#include "attn_common.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;

template <int KV, int D>
struct VGeo {
  static constexpr int E = KV == KV_F16 ? 2 : 1;
  static constexpr int SLABS = D * E / 64;
  static constexpr int QD = D / 4;      // K dims per lane
  static constexpr int MT = D / 16;     // V dims per lane
  static constexpr int BLK = kPage * D * E;
};

template <int KV, int D>
struct PageRegs {
  u32x4 k[VGeo<KV, D>::SLABS];
  u32x4 v[VGeo<KV, D>::SLABS];
};

// Issue the loads of the wave's i-th page (page wave + 4 i of the unit).
// Branch-free: a page past the unit's end loads page 0 and is masked later.
template <int KV, int D>
__device__ __forceinline__ void load_page(PageRegs<KV, D>& r, PageIdChunks& ids, const AttnLaunch& a,
                                          const UnitPages& pg, int32_t npages, int32_t wave, int32_t i,
                                          const int32_t* bt_row, int h, uint32_t lane_off, int lane, bool& bad) {
  using G = VGeo<KV, D>;
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

// The lane's K dims as fp16 pairs (QD / 2 words).
template <int KV, int D>
__device__ __forceinline__ void k_halves(const PageRegs<KV, D>& r, f16x2 (&kh)[VGeo<KV, D>::QD / 2]) {
  using G = VGeo<KV, D>;
  if constexpr (KV == KV_F16) {
#pragma unroll
    for (int i = 0; i < G::QD / 2; ++i) kh[i] = as<f16x2>(r.k[i / 4][i % 4]);
  } else {
#pragma unroll
    for (int w = 0; w < G::QD / 4; ++w) {
      const f16x4 h = codes4_to_f16x4<KV>(r.k[w / 4][w % 4]);
      kh[2 * w] = f16x2{h[0], h[1]};
      kh[2 * w + 1] = f16x2{h[2], h[3]};
    }
  }
}

// V tokens 4kq..4kq+3 of the lane's dim mt.
template <int KV, int D>
__device__ __forceinline__ f16x4 v_quad_vec(const PageRegs<KV, D>& r, int mt) {
  if constexpr (KV == KV_F16) {
    const u32x4 w = r.v[mt >> 1];
    const f16x2 lo = as<f16x2>((mt & 1) ? w[2] : w[0]);
    const f16x2 hi = as<f16x2>((mt & 1) ? w[3] : w[1]);
    return f16x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    return codes4_to_f16x4<KV>(r.v[mt >> 2][mt & 3]);
  }
}

template <int D, int RP>
struct VAcc {
  float o[RP][D / 16];
  float m[RP];
  float l[RP];
};

template <int KV, int D, int RP>
__device__ __forceinline__ void compute_page(VAcc<D, RP>& acc, PageRegs<KV, D>& r,
                                             const f16x2 (&qh)[RP][VGeo<KV, D>::QD / 2],
                                             const AttnLaunch& a, const UnitPages& pg, int32_t npages,
                                             int32_t n, int32_t ctx, int32_t q_len, const int32_t (&pos)[RP],
                                             int lane, float c, float thr, float* sm_p) {
  using G = VGeo<KV, D>;
  const int t = lane & 15;
  const int kq = lane >> 4;
  // ---- scores: s[r] for (row r, token t)
  f16x2 kh[G::QD / 2];
  k_halves<KV, D>(r, kh);
  float s[RP];
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
    float x = 0.0f;
#pragma unroll
    for (int i = 0; i < G::QD / 2; ++i) {
      x = fmaf((float)qh[rr][i][0], (float)kh[i][0], x);
      x = fmaf((float)qh[rr][i][1], (float)kh[i][1], x);
    }
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    s[rr] = x;
  }
  const int32_t tok0 = pg.page(n) * kPage;
  const bool need_mask = (tok0 + kPage - 1 > ctx - q_len) ||
                         (a.window >= 0 && tok0 <= ctx - 1 - a.window);
  if (need_mask) {
    const int32_t j = tok0 + t;
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) s[rr] = key_visible(a, j, pos[rr]) ? s[rr] : -INFINITY;
  }
  // ---- lazy online softmax
  bool trig = false;
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) trig |= s[rr] > acc.m[rr] + thr;
  if (__any(trig)) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      float rm = s[rr];
      rm = fmaxf(rm, __shfl_xor(rm, 1));
      rm = fmaxf(rm, __shfl_xor(rm, 2));
      rm = fmaxf(rm, __shfl_xor(rm, 4));
      rm = fmaxf(rm, __shfl_xor(rm, 8));
      const bool upd = rm > acc.m[rr] + thr;
      const float alpha = upd ? (acc.m[rr] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((acc.m[rr] - rm) * c)) : 1.0f;
      acc.m[rr] = upd ? rm : acc.m[rr];
      acc.l[rr] *= alpha;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) acc.o[rr][mt] *= alpha;
    }
  }
  float p[RP];
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
    const float mc = acc.m[rr] == -INFINITY ? 0.0f : acc.m[rr] * c;
    p[rr] = __builtin_amdgcn_exp2f(fmaf(s[rr], c, -mc));
    acc.l[rr] += p[rr];       // every lane group holds the same p; group 0's sum is used
  }
  // ---- exchange p through LDS: sm_p[row][token]
  if (kq == 0) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) sm_p[rr * 16 + t] = p[rr];
  }
  __builtin_amdgcn_wave_barrier();      // LDS requests of one wave complete in order
  // tokens 4kq .. 4kq+3 beyond ctx carry stale data: zero their V codes
  const int32_t jq = tok0 + 4 * kq;
  if (jq + 3 >= ctx) {
    uint32_t keep8 = 0, keep_lo = 0, keep_hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool data = jq + i < ctx;
      keep8 |= data ? 0xFFu << (8 * i) : 0u;
      if (i < 2) keep_lo |= data ? 0xFFFFu << (16 * i) : 0u;
      else keep_hi |= data ? 0xFFFFu << (16 * (i - 2)) : 0u;
    }
#pragma unroll
    for (int sl = 0; sl < G::SLABS; ++sl)
#pragma unroll
      for (int w = 0; w < 4; ++w) r.v[sl][w] &= KV == KV_F16 ? ((w & 1) ? keep_hi : keep_lo) : keep8;
  }
  f32x4 pr[RP];
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) pr[rr] = *reinterpret_cast<const f32x4*>(sm_p + rr * 16 + 4 * kq);
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt) {
    const f16x4 v = v_quad_vec<KV, D>(r, mt);
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      float x = acc.o[rr][mt];
      x = fmaf(pr[rr][0], (float)v[0], x);
      x = fmaf(pr[rr][1], (float)v[1], x);
      x = fmaf(pr[rr][2], (float)v[2], x);
      x = fmaf(pr[rr][3], (float)v[3], x);
      acc.o[rr][mt] = x;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

template <int KV, int D, int RP>
__global__ void __launch_bounds__(kWaves * kWave) attn_vec_kernel(AttnLaunch a, int32_t row_groups) {
  using G = VGeo<KV, D>;
  __shared__ __attribute__((aligned(16))) float sm_p[kWaves][RP * 16];
  __shared__ float sm_ml[2][kWaves][RP];
  __shared__ float sm_o[2][RP * G::MT][kWave];

  UnitId u;
  if (!decode_unit(a, row_groups, u)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = lane >> 4;

  const int32_t q0 = a.qsl[u.b], q1 = a.qsl[u.b + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.total_q) return;
  const int32_t g = a.hq / a.hkv;
  const int32_t q_len = q1 - q0;
  const int32_t rows = g * q_len;
  if (rows == 0 || rows >= kMfmaMinRows) return;       // nothing, or the matrix-core kernel's unit
  const int32_t row0 = u.rg * RP;
  if (row0 >= rows) return;
  const int32_t ctx = a.context_lens[u.b];
  bool bad = !seq_ok(a, ctx, q0, q1);

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

  // queries: row rr, the lane's K dims kgrp * D/4 .. + D/4, as fp16 pairs.
  // All loads are issued before any is used.
  f16x2 qh[RP][G::QD / 2];
  u32x4 qraw[RP][G::QD / 8];
  bool qlive[RP];
  int32_t pos[RP];
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
    const int32_t r = row0 + rr;
    qlive[rr] = r < rows && !bad;
    pos[rr] = qlive[rr] ? ctx - q_len + r / g : ctx - 1;
    const int64_t qrow = qlive[rr] ? ((int64_t)(q0 + r / g) * a.hq + u.h * g + r % g) : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qrow * D + kgrp * G::QD;
#pragma unroll
    for (int w = 0; w < G::QD / 8; ++w) qraw[rr][w] = load16(qp + 8 * w);
  }
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
#pragma unroll
    for (int w = 0; w < G::QD / 8; ++w) {
      const u32x4 x = qlive[rr] ? qraw[rr][w] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = x[i];
        if (a.q_bf16) {
          qh[rr][4 * w + i] = f16x2{(f16)bf16_to_f32((uint16_t)(word & 0xFFFFu)),
                                    (f16)bf16_to_f32((uint16_t)(word >> 16))};
        } else {
          qh[rr][4 * w + i] = as<f16x2>(word);
        }
      }
    }
  }

  VAcc<D, RP> acc;
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
    acc.m[rr] = -INFINITY;
    acc.l[rr] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) acc.o[rr][mt] = 0.0f;
  }
  const float c = a.softmax_scale * a.k_scale * kLog2e;
  const float thr = kLazy / c;
  const uint32_t lane_off = (uint32_t)lane * 16u;
  float* smp = sm_p[wave];

  // main loop over the wave's pages (page wave + 4 i): two register buffers,
  // the next page's loads are in flight while one page computes
  PageIdChunks ids;
  init_ids<1, kWaves>(ids, pg, npages, bt_row, wave, lane);
  const int32_t my_pages = npages > wave ? (npages - wave + kWaves - 1) / kWaves : 0;
  if (my_pages > 0) {
    PageRegs<KV, D> ra, rb;
    load_page<KV, D>(ra, ids, a, pg, npages, wave, 0, bt_row, u.h, lane_off, lane, bad);
    for (int32_t i = 0;; i += 2) {
      load_page<KV, D>(rb, ids, a, pg, npages, wave, i + 1, bt_row, u.h, lane_off, lane, bad);
      compute_page<KV, D, RP>(acc, ra, qh, a, pg, npages, wave + kWaves * i, ctx, q_len, pos, lane, c, thr, smp);
      if (i + 1 >= my_pages) break;
      load_page<KV, D>(ra, ids, a, pg, npages, wave, i + 2, bt_row, u.h, lane_off, lane, bad);
      compute_page<KV, D, RP>(acc, rb, qh, a, pg, npages, wave + kWaves * (i + 1), ctx, q_len, pos, lane, c, thr,
                              smp);
      if (i + 2 >= my_pages) break;
    }
  }

  // ---- per wave: sum o over the 4 token quads, l over the 16 tokens
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      float x = acc.o[rr][mt];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc.o[rr][mt] = x;
    }
    float l = acc.l[rr];
    l += __shfl_xor(l, 1);
    l += __shfl_xor(l, 2);
    l += __shfl_xor(l, 4);
    l += __shfl_xor(l, 8);
    acc.l[rr] = l;
    if (lane == 0) {
      sm_ml[0][wave][rr] = acc.m[rr];
      sm_ml[1][wave][rr] = l;
    }
  }
  bad = __syncthreads_or(bad ? 1 : 0) != 0;
  float Mrow[RP], Lrow[RP];
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
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
    Mrow[rr] = M;
    Lrow[rr] = L;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) acc.o[rr][mt] *= fself;
  }
  if (wave >= 2) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr)
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) sm_o[wave - 2][rr * G::MT + mt][lane] = acc.o[rr][mt];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr)
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) acc.o[rr][mt] += sm_o[wave][rr * G::MT + mt][lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int rr = 0; rr < RP; ++rr)
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) sm_o[0][rr * G::MT + mt][lane] = acc.o[rr][mt];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int rr = 0; rr < RP; ++rr)
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) acc.o[rr][mt] += sm_o[0][rr * G::MT + mt][lane];

  // ---- epilogue: lanes 0..15 (m) write dims m * MT .. + MT of every row
  if (lane >= 16) return;
  const int mcol = lane;
  const float vs = a.v_scale;
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
    const int32_t r = row0 + rr;
    if (r >= rows) continue;
    const int32_t qi = r / g, hj = r % g;
    const int64_t orow = (int64_t)(q0 + qi) * a.hq + u.h * g + hj;
    const float L = Lrow[rr];
    const float inv = L > 0.0f ? vs / L : 0.0f;
    float lse = L > 0.0f ? (Mrow[rr] * c + log2f(L)) * kLn2 : -INFINITY;
    if (bad) lse = __builtin_nanf("");
    const int d0 = mcol * G::MT;
    float v[G::MT];
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) v[mt] = bad ? __builtin_nanf("") : acc.o[rr][mt] * inv;
    if (a.direct) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + orow * D + d0;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
        op[mt] = a.q_bf16 ? f32_to_bf16(v[mt]) : as<uint16_t>((f16)v[mt]);
      if (mcol == 0 && a.lse) a.lse[orow] = lse;
    } else {
      float* op = a.part_out + ((int64_t)u.s * a.total_q * a.hq + orow) * D + d0;
#pragma unroll
      for (int k = 0; k < G::MT / 4; ++k)
        *reinterpret_cast<f32x4*>(op + 4 * k) = f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
      if (mcol == 0) a.part_lse[(int64_t)u.s * a.total_q * a.hq + orow] = lse;
    }
  }
}

template <int KV, int D, int RP>
hipError_t launch_t(const AttnLaunch& a, int32_t row_groups, hipStream_t s) {
  const int64_t units = (int64_t)a.slots * a.hkv * row_groups * a.batch;
  hipLaunchKernelGGL((attn_vec_kernel<KV, D, RP>), dim3(padded_grid(units)), dim3(kWaves * kWave), 0, s,
                     a, row_groups);
  return hipGetLastError();
}

template <int KV>
hipError_t launch_d(const AttnLaunch& a, int rp, int32_t row_groups, hipStream_t s) {
  if (a.head_dim == 64)
    return rp == 4 ? launch_t<KV, 64, 4>(a, row_groups, s) : launch_t<KV, 64, 8>(a, row_groups, s);
  return rp == 4 ? launch_t<KV, 128, 4>(a, row_groups, s) : launch_t<KV, 128, 8>(a, row_groups, s);
}

}  // namespace

hipError_t launch_attn_vec(const AttnLaunch& a, hipStream_t s) {
  const int32_t g = a.hq / a.hkv;
  int32_t rows_max = g * a.max_q_len;
  if (rows_max >= kMfmaMinRows) rows_max = kMfmaMinRows - 1;   // larger units are not ours
  const int rp = rows_max <= 4 ? 4 : kVecRowsPerBlock;
  const int32_t row_groups = (rows_max + rp - 1) / rp;
  switch (a.kv) {
    case KV_F16: return launch_d<KV_F16>(a, rp, row_groups, s);
    case KV_E4M3: return launch_d<KV_E4M3>(a, rp, row_groups, s);
    default: return launch_d<KV_I8>(a, rp, row_groups, s);
  }
}

}  // namespace ra
