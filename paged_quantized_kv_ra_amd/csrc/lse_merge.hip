// lse_merge.hip -- combine split-KV partial attention by log-sum-exp.
//
// The pages run decode context parallelism (DCP2): one sequence's context is
// split and the parts' partial attention is combined (ReVolta README, "Quick
// start" and "Hardware").  Each partial is (out_s, lse_s) with out_s already
// normalised; the combination is
//   M = max_s lse_s,  a_s = exp(lse_s - M),
//   out = sum_s a_s out_s / sum_s a_s,  lse = M + ln sum_s a_s,
// summed in the fixed order s = 0, 1, ...  Partitions with lse = -inf add
// nothing, whatever their out holds.  A NaN lse (a partial whose sequence
// broke a precondition) makes the row NaN.
//
// One single-wave workgroup per row (rather than several rows per workgroup,
// so that the launch spreads over every CU; about 1 us less per step on the
// split workloads): lane s holds lse_s for a chunk of 64 partitions, the
// weights are broadcast with a lane shuffle, each lane accumulates D/64 dims;
// sixteen partial rows are in flight at a time.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

template <int D, int OUT>
__global__ void __launch_bounds__(64) lse_merge_kernel(MergeLaunch a) {
  constexpr int PER = D / 64;
  constexpr int BATCH = 16;                    // partial rows in flight per lane
  // every launch argument in one round of scalar loads, ahead of the first branch
  asm volatile("" ::"s"(a.part_out), "s"(a.part_lse), "s"(a.parts), "s"(a.rows), "s"(a.out), "s"(a.lse));
  const int64_t row = blockIdx.x;
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const float* base_o = a.part_out + row * D + lane * PER;
  const int64_t pstride = a.rows * D;

  // BATCH partial rows are loaded together (a partition of weight 0, with no
  // visible key, is loaded but adds nothing, whatever its out holds); the
  // first batch is requested together with the lse values
  auto load_batch = [&](float (&v)[BATCH][PER], int first, int n) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const float* o = base_o + (int64_t)(first + min(j, n - 1)) * pstride;
      if constexpr (PER == 2) {
        const float2 x = *reinterpret_cast<const float2*>(o);
        v[j][0] = x.x;
        v[j][1] = x.y;
      } else {
        v[j][0] = o[0];
      }
    }
  };
  float v[BATCH][PER];
  load_batch(v, 0, min(a.parts, 64));

  // lane s holds lse_s of the first 64 partitions (the common case keeps
  // them for the weights); later chunks are re-read
  const float ls0 = lane < a.parts ? a.part_lse[(int64_t)lane * a.rows + row] : -INFINITY;
  float M = ls0;
  bool nan = !(ls0 == ls0);
  for (int s = lane + 64; s < a.parts; s += 64) {
    const float x = a.part_lse[(int64_t)s * a.rows + row];
    nan |= !(x == x);
    M = fmaxf(M, x);
  }
  M = wave_max(M);
  nan = __any(nan);

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float den = 0.0f;
  if (!nan && M != -INFINITY) {
    for (int base = 0; base < a.parts; base += 64) {
      const float ls = base == 0 ? ls0
                                 : (base + lane < a.parts ? a.part_lse[(int64_t)(base + lane) * a.rows + row]
                                                          : -INFINITY);
      const float w_l = ls == -INFINITY ? 0.0f : expf(ls - M);
      const int n = min(64, a.parts - base);
      for (int k0 = 0; k0 < n; k0 += BATCH) {
        if (base != 0 || k0 != 0) load_batch(v, base + k0, n - k0);
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const float w = k0 + j < n ? __shfl(w_l, k0 + j) : 0.0f;
          if (w != 0.0f) {
            den += w;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, v[j][i], acc[i]);
          }
        }
      }
    }
  }
  float lse;
  float res[PER];
  if (nan) {
    lse = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < PER; ++i) res[i] = __builtin_nanf("");
  } else if (den > 0.0f) {
    lse = M + logf(den);
#pragma unroll
    for (int i = 0; i < PER; ++i) res[i] = acc[i] / den;
  } else {
    lse = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) res[i] = 0.0f;
  }
  if (OUT == 3) {
    float* o = reinterpret_cast<float*>(a.out) + row * D + lane * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = res[i];
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + row * D + lane * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      o[i] = OUT == 2 ? f32_to_bf16(res[i]) : as<uint16_t>((f16)res[i]);
  }
  if (lane == 0 && a.lse) a.lse[row] = lse;
}

template <int D>
hipError_t launch_out(const MergeLaunch& a, hipStream_t s) {
  const dim3 g((unsigned)a.rows), b(64);
  switch (a.out_dtype) {
    case 1: hipLaunchKernelGGL((lse_merge_kernel<D, 1>), g, b, 0, s, a); break;
    case 2: hipLaunchKernelGGL((lse_merge_kernel<D, 2>), g, b, 0, s, a); break;
    default: hipLaunchKernelGGL((lse_merge_kernel<D, 3>), g, b, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeLaunch& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  return a.head_dim == 64 ? launch_out<64>(a, s) : launch_out<128>(a, s);
}

}  // namespace ra
