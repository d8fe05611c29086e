// attn_prefill.hip -- long query blocks (prefill and chunked prefill) over the
// paged FP8 E4M3 / INT8 cache, on the gfx950 matrix cores.
//
// A prompt, or a chunk of one, attends causally to the cached context and to
// itself (ReVolta README, intro table: cold 8K and 131K prompt prefill;
// "Quick start": chunked long prefills).  Such a block has g * q_len rows per
// KV head, far more than one workgroup's tiles, so the work is cut by rows:
// a workgroup of 4 waves owns 128 rows (each wave 32 rows, two 16-row tiles)
// of one (sequence, KV head, partition) and walks the partition's keys 64 at
// a time (4 pages).  Per 64-key tile:
//   - each wave requests one page of the next tile into the other LDS stage
//     by DMA (global_load_lds), so loads run one tile ahead;
//   - the 256 threads convert the tile's codes once, exactly, to fp16 MFMA
//     operands in LDS (a K operand per (page, k-step, lane), a V operand per
//     (page pair, dim tile, lane) with the two pages' four keys side by side);
//   - every wave then computes its rows against the shared tile:
//     S^T = K . Q^T (v_mfma_f32_16x16x32_f16, 4 key tiles x 2 row tiles x 4
//     k-steps), masks on the diagonal and past the context, the online
//     softmax with lazy max refresh, and O^T += V^T . P^T over 32-key pairs
//     (v_mfma_f32_16x16x32_f16, with one more tile of ones for the row sums).
// A wave owns its rows outright, so there is no cross-wave combine: each wave
// writes its rows (out and lse, or one partition's partials) at the end.
// Decoding the tile once per workgroup rather than once per wave (as the
// decode kernel does, whose waves split the keys) takes the fp8 conversions,
// which bound that kernel on long blocks, off the critical path.
#include "attn_common.h"

namespace ra {
namespace {

constexpr int kPW = 4;                  // waves per workgroup
constexpr int kPThreads = kPW * kWave;
constexpr int kPNT = 2;                 // 16-row tiles per wave
constexpr int kPTileKeys = 64;          // keys per iteration
constexpr int kPTilePages = kPTileKeys / kPage;
constexpr int kPD = 128;                // head_dim of this kernel
constexpr int kPKS = kPD / 32;          // k-steps of QK
constexpr int kPMT = kPD / 16;          // dim tiles of PV
constexpr int kPSlab = 1024;
constexpr int kPSlabs = kPD / 64;       // 1 KiB slabs per K (or V) page of 1-byte codes
constexpr float kPLog2e = 1.4426950408889634f;
constexpr float kPLn2 = 0.6931471805599453f;
constexpr float kPLazy = 8.0f;
typedef __attribute__((address_space(3))) uint8_t lds8;

static_assert(kPTilePages == kPW, "each wave loads one page of the tile");

template <int KV>
__device__ __forceinline__ f16x4 dec4(uint32_t x) {
  return codes4_to_f16x4<KV>(x);
}

template <int KV>
__global__ void __launch_bounds__(kPThreads) attn_prefill_kernel(AttnLaunch a, int32_t row_groups) {
  // raw pages by DMA: [stage][page][K, V][slab][1 KiB]
  __shared__ __attribute__((aligned(16))) uint8_t raw[2][kPTilePages][2][kPSlabs][kPSlab];
  // fp16 operands: K [page][k-step][lane], V [page pair][dim tile][lane]
  __shared__ f16x8 kop_s[kPTilePages][kPKS][kWave];
  __shared__ f16x8 vop_s[kPTilePages / 2][kPMT][kWave];
  __shared__ int32_t sm_bad_page;   // a block-table entry outside [0, num_pages) was met

  // unit: logical id ((s * row_groups + (row_groups - 1 - rg)) * Hkv + h) * batch + b,
  // the latest (heaviest) row groups first, in dispatch order
  const int64_t total = (int64_t)a.slots * a.hkv * row_groups * a.batch;
  const int64_t id0 = blockIdx.x;
  if (id0 >= total) return;
  int64_t id = id0;
  const int32_t b = (int32_t)(id % a.batch); id /= a.batch;
  const int32_t h = (int32_t)(id % a.hkv); id /= a.hkv;
  const int32_t rg = row_groups - 1 - (int32_t)(id % row_groups); id /= row_groups;
  const int32_t s = (int32_t)id;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = lane >> 4;
  const int ncol = lane & 15;

  const int32_t q0 = a.qsl[b], q1 = a.qsl[b + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.total_q) return;      // rows not addressable
  const int32_t g = a.hq / a.hkv;
  const int32_t q_len = q1 - q0;
  const int32_t rows = g * q_len;
  const int32_t row0 = rg * (kPW * kPNT * 16);
  if (row0 >= rows) return;
  const int32_t ctx = a.context_lens[b];
  if (!prefill_sequence(a, rows, ctx, q_len)) return;   // the decode kernel's sequence
  const int32_t kv0 = a.kv_pos0 ? a.kv_pos0[b] : 0;
  const int32_t qp0 = a.q_pos0 ? a.q_pos0[b] : 0;
  bool bad = !seq_ok(a, ctx, q0, q1, kv0, qp0);
  const SeqFrame fr = seq_frame(a, ctx, q_len, kv0, qp0);
  const int32_t last_row = min(row0 + kPW * kPNT * 16, rows) - 1;
  const int32_t pmax_wg = fr.pmin + last_row / g;       // the workgroup's last query

  // the partition's keys the workgroup's queries can see: [lo, hi)
  int32_t lo = 0, hi = 0;
  if (!bad) {
    const int32_t P = partition_tokens(a, ctx, rows);
    lo = s * P;
    hi = min(min(lo + P, ctx), pmax_wg + 1);
  }
  const int32_t ntiles = hi > lo ? (hi - lo + kPTileKeys - 1) / kPTileKeys : 0;
  const int32_t* bt_row = a.block_tables + (int64_t)b * a.bt_stride;
  const int32_t page_end = (hi + kPage - 1) / kPage;    // pages past it are never loaded

  // the wave's rows and their query fragments (as in the decode kernel)
  int32_t pos[kPNT];
  bool qlive[kPNT];
  f16x8 qf[kPNT][kPKS];
#pragma unroll
  for (int nt = 0; nt < kPNT; ++nt) {
    const int32_t r = row0 + wave * (kPNT * 16) + nt * 16 + ncol;
    qlive[nt] = r < rows && !bad;
    pos[nt] = fr.pmin + (qlive[nt] ? r / g : 0);
    const int64_t qtok = qlive[nt] ? q0 + r / g : 0, qhead = qlive[nt] ? h * g + r % g : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qtok * a.q_stride + qhead * kPD + kgrp * (kPD / 4);
#pragma unroll
    for (int ks = 0; ks < kPKS; ++ks) {
      const u32x4 w = qlive[nt] ? load16(qp + 8 * ks) : u32x4{0, 0, 0, 0};
      if (a.q_bf16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[nt][ks][i] = (f16)bf16_to_f32((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
      } else {
        qf[nt][ks] = as<f16x8>(w);
      }
    }
  }
  const int32_t w_row_last = min(row0 + wave * (kPNT * 16) + kPNT * 16, rows) - 1;
  const int32_t wpmin = fr.pmin + min(row0 + wave * (kPNT * 16), rows - 1) / g;   // the wave's first query
  const int32_t wpmax = fr.pmin + max(w_row_last, 0) / g;                          // and its last

  f32x4 o[kPMT][kPNT], ls[kPNT];
  float m[kPNT], mc[kPNT];
#pragma unroll
  for (int nt = 0; nt < kPNT; ++nt) {
    m[nt] = -INFINITY;
    mc[nt] = 0.0f;
    ls[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int mt = 0; mt < kPMT; ++mt) o[mt][nt] = f32x4{0, 0, 0, 0};
  }
  const float c = a.softmax_scale * a.k_scale * kPLog2e;
  const float thr = kPLazy / c;
  const uint32_t lane_off = (uint32_t)lane * 16u;

  // wave w requests page w of tile t into stage st (pages past the keys are skipped)
  auto issue = [&](int32_t t, int st) {
    const int32_t pg = lo / kPage + t * kPTilePages + wave;
    if (pg < page_end) {
      int32_t pid = bt_row[pg];
      if (pid < 0 || pid >= a.num_pages) {   // a violated precondition: read page 0, write NaN rows
        pid = 0;
        sm_bad_page = 1;
      }
      const int64_t blk = ((int64_t)pid * a.hkv + h) * (kPage * kPD);
      const uint8_t* kp = a.k_cache + blk + lane_off;
      const uint8_t* vp = a.v_cache + blk + lane_off;
#pragma unroll
      for (int j = 0; j < kPSlabs; ++j)
        __builtin_amdgcn_global_load_lds(kp + j * kPSlab, (lds8*)raw[st][wave][0][j], 16, 0, 0);
#pragma unroll
      for (int j = 0; j < kPSlabs; ++j)
        __builtin_amdgcn_global_load_lds(vp + j * kPSlab, (lds8*)raw[st][wave][1][j], 16, 0, 0);
    }
  };
  if (threadIdx.x == 0) sm_bad_page = 0;
  __syncthreads();
  if (ntiles > 0) issue(0, 0);

  for (int32_t t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    const int32_t base = lo + t * kPTileKeys;   // key of the tile's first slot
    __builtin_amdgcn_s_waitcnt((0 & 15) | 0x70 | 0xF00);   // vmcnt(0): this wave's page of tile t has landed
    __syncthreads();   // every page of tile t has landed; every wave is done with tile t - 1's operands
    if (t + 1 < ntiles) issue(t + 1, st ^ 1);

    // ---- decode tile t once: 256 threads, 2 K items and 2 V items each
    const int32_t valid_end = min(hi, ctx);   // keys at or past it hold no data of this partition
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int x = threadIdx.x + it * kPThreads;   // (page, slab, lane)
      const int p = x / (kPSlabs * kWave), j = (x / kWave) % kPSlabs, L = x % kWave;
      // K: 16 codes = dims (L / 16) * 32 + 16 j .. + 16 of key L % 16
      const u32x4 kw = *reinterpret_cast<const u32x4*>(&raw[st][p][0][j][L * 16]);
      const f16x4 k0 = dec4<KV>(kw[0]), k1 = dec4<KV>(kw[1]), k2 = dec4<KV>(kw[2]), k3 = dec4<KV>(kw[3]);
      kop_s[p][2 * j][L] = f16x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      kop_s[p][2 * j + 1][L] = f16x8{k2[0], k2[1], k2[2], k2[3], k3[0], k3[1], k3[2], k3[3]};
      // V: 16 codes = dims (L % 16) * 8 + 4 j + q (q = 0..3), each for keys
      // 4 (L / 16) .. + 3; keys past the data are zeroed (their scores are
      // masked, and 0 * garbage must not make NaN)
      const int32_t key0 = base + p * kPage + 4 * (L >> 4);
      const bool loaded = lo / kPage + t * kPTilePages + p < page_end;
      uint32_t keep = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) keep |= (loaded && key0 + i < valid_end) ? 0xFFu << (8 * i) : 0u;
      const u32x4 vw = *reinterpret_cast<const u32x4*>(&raw[st][p][1][j][L * 16]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x4 v4 = dec4<KV>(vw[q] & keep);
        f16* dst = reinterpret_cast<f16*>(&vop_s[p >> 1][4 * j + q][L]) + 4 * (p & 1);
        *reinterpret_cast<f16x4*>(dst) = v4;
      }
    }
    __syncthreads();   // the tile's operands are in LDS

    // ---- the wave's rows against tile t
    if (base > wpmax) continue;   // none of the wave's queries sees these keys (uniform per wave)
    f32x4 sc[kPTilePages][kPNT];
#pragma unroll
    for (int p = 0; p < kPTilePages; ++p)
#pragma unroll
      for (int nt = 0; nt < kPNT; ++nt) sc[p][nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < kPTilePages; ++p)
#pragma unroll
      for (int ks = 0; ks < kPKS; ++ks) {
        const f16x8 kop = kop_s[p][ks][lane];
#pragma unroll
        for (int nt = 0; nt < kPNT; ++nt) sc[p][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qf[nt][ks], sc[p][nt], 0, 0, 0);
      }
    // masks: only tiles that reach the wave's first query or the data's end
    if (base + kPTileKeys - 1 > wpmin || base + kPTileKeys > valid_end) {
#pragma unroll
      for (int p = 0; p < kPTilePages; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t j = base + p * kPage + 4 * kgrp + i;
#pragma unroll
          for (int nt = 0; nt < kPNT; ++nt) sc[p][nt][i] = (j < valid_end && j <= pos[nt]) ? sc[p][nt][i] : -INFINITY;
        }
    }
    // online softmax with lazy max refresh
    float mx[kPNT];
    bool trig = false;
#pragma unroll
    for (int nt = 0; nt < kPNT; ++nt) {
      float v = -INFINITY;
#pragma unroll
      for (int p = 0; p < kPTilePages; ++p)
        v = __builtin_elementwise_maximum(v, __builtin_elementwise_maximum(
                                                 __builtin_elementwise_maximum(sc[p][nt][0], sc[p][nt][1]),
                                                 __builtin_elementwise_maximum(sc[p][nt][2], sc[p][nt][3])));
      mx[nt] = v;
      trig |= v > m[nt] + thr;
    }
    if (__any(trig)) {
#pragma unroll
      for (int nt = 0; nt < kPNT; ++nt) {
        float rm = mx[nt];
        rm = __builtin_elementwise_maximum(rm, __shfl_xor(rm, 16));
        rm = __builtin_elementwise_maximum(rm, __shfl_xor(rm, 32));
        const bool upd = rm > m[nt] + thr;
        const float alpha = upd ? (m[nt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m[nt] - rm) * c)) : 1.0f;
        m[nt] = upd ? rm : m[nt];
        mc[nt] = m[nt] == -INFINITY ? 0.0f : m[nt] * c;
        ls[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < kPMT; ++mt) o[mt][nt] *= alpha;
      }
    }
    f16x8 pf[kPTilePages / 2][kPNT];
#pragma unroll
    for (int p = 0; p < kPTilePages; ++p)
#pragma unroll
      for (int nt = 0; nt < kPNT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pf[p >> 1][nt][4 * (p & 1) + i] = (f16)__builtin_amdgcn_exp2f(fmaf(sc[p][nt][i], c, -mc[nt]));
    // O^T += V^T . P^T over the two 32-key pairs, and the row sums
    const f16x8 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int pr = 0; pr < kPTilePages / 2; ++pr) {
#pragma unroll
      for (int mt = 0; mt < kPMT; ++mt) {
        const f16x8 vop = vop_s[pr][mt][lane];
#pragma unroll
        for (int nt = 0; nt < kPNT; ++nt)
          o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pf[pr][nt], o[mt][nt], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < kPNT; ++nt) ls[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[pr][nt], ls[nt], 0, 0, 0);
    }
  }
  __syncthreads();
  bad = bad || sm_bad_page != 0;

  // ---- the wave's rows: out and lse (one partition slot) or this partition's partials
  const float vs = a.v_scale;
#pragma unroll
  for (int nt = 0; nt < kPNT; ++nt) {
    const int32_t r = row0 + wave * (kPNT * 16) + nt * 16 + ncol;
    if (r >= rows) continue;
    const int32_t qi = r / g, hj = r % g;
    const int64_t orow = (int64_t)(q0 + qi) * a.hq + h * g + hj;
    const float L = ls[nt][0];
    const float inv = L > 0.0f ? vs / L : (L == L ? 0.0f : __builtin_nanf(""));   // NaN scores: NaN row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[kPMT];
#pragma unroll
      for (int mt = 0; mt < kPMT; ++mt) v[mt] = bad ? __builtin_nanf("") : o[mt][nt][i] * inv;
      const int d0 = (4 * kgrp + i) * kPMT;
      if (a.direct) {
        u32x4 w;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t lo16 = a.q_bf16 ? f32_to_bf16(v[2 * jj]) : as<uint16_t>((f16)v[2 * jj]);
          const uint32_t hi16 = a.q_bf16 ? f32_to_bf16(v[2 * jj + 1]) : as<uint16_t>((f16)v[2 * jj + 1]);
          w[jj] = lo16 | (hi16 << 16);
        }
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + orow * kPD + d0) = w;
      } else {
        float* op = a.part_out + ((int64_t)s * a.total_q * a.hq + orow) * kPD + d0;
        *reinterpret_cast<f32x4*>(op) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(op + 4) = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
    if (kgrp == 0) {
      float lse = L > 0.0f ? (m[nt] * c + log2f(L)) * kPLn2 : (L == L ? -INFINITY : __builtin_nanf(""));
      if (bad) lse = __builtin_nanf("");
      if (a.direct) {
        if (a.lse) a.lse[orow] = lse;
      } else {
        a.part_lse[(int64_t)s * a.total_q * a.hq + orow] = lse;
      }
    }
  }
}

}  // namespace

bool prefill_kernel_serves(const AttnLaunch& a) {
  return (a.kv == KV_E4M3 || a.kv == KV_I8) && a.head_dim == kPD && a.window < 0;
}

hipError_t launch_attn_prefill(const AttnLaunch& a, hipStream_t s) {
  const int64_t rows_max = (int64_t)(a.hq / a.hkv) * a.max_q_len;
  const int32_t row_groups = (int32_t)((rows_max + kPW * kPNT * 16 - 1) / (kPW * kPNT * 16));
  const int64_t units = (int64_t)a.slots * a.hkv * row_groups * a.batch;
  if (units == 0) return hipSuccess;
  if (a.kv == KV_E4M3)
    hipLaunchKernelGGL((attn_prefill_kernel<KV_E4M3>), dim3((unsigned)units), dim3(kPThreads), 0, s, a, row_groups);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<KV_I8>), dim3((unsigned)units), dim3(kPThreads), 0, s, a, row_groups);
  return hipGetLastError();
}

}  // namespace ra
