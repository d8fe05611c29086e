// lse_merge.hip -- combine split-KV partial attention by log-sum-exp.
//
// The pages run decode context parallelism (DCP2): one sequence's context is
// split and the parts' partial attention is combined (ReVolta README, "Quick
// start" and "Hardware").  Each partial is (out_s, lse_s) with out_s already
// normalised; the combination is
//   M = max_s lse_s,  a_s = exp(lse_s - M),
//   out = sum_s a_s out_s / sum_s a_s,  lse = M + ln sum_s a_s,
// summed in the fixed order s = 0, 1, ...  Partitions with lse = -inf are
// skipped without reading their out.  A NaN lse (a partial whose sequence
// broke a precondition) makes the row NaN.
//
// One wavefront per row: lane s holds lse_s for a chunk of 64 partitions, the
// weights are broadcast with readlane, each lane accumulates D/64 dims.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

template <int D, int OUT>
__global__ void __launch_bounds__(256) lse_merge_kernel(MergeLaunch a) {
  constexpr int PER = D / 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;

  float M = -INFINITY;
  bool nan = false;
  for (int s = lane; s < a.parts; s += 64) {
    const float v = a.part_lse[(int64_t)s * a.rows + row];
    nan |= !(v == v);
    M = fmaxf(M, v);
  }
  M = wave_max(M);
  nan = __any(nan);

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float den = 0.0f;
  if (!nan && M != -INFINITY) {
    for (int base = 0; base < a.parts; base += 64) {
      const int s_l = base + lane;
      const float ls = s_l < a.parts ? a.part_lse[(int64_t)s_l * a.rows + row] : -INFINITY;
      const float w_l = ls == -INFINITY ? 0.0f : expf(ls - M);
      const int n = min(64, a.parts - base);
      for (int k = 0; k < n; ++k) {
        const float w = __shfl(w_l, k);
        if (w == 0.0f) continue;             // empty partition: its out is not read
        den += w;
        const float* o = a.part_out + ((int64_t)(base + k) * a.rows + row) * D + lane * PER;
        if constexpr (PER == 2) {
          const float2 v = *reinterpret_cast<const float2*>(o);
          acc[0] = fmaf(w, v.x, acc[0]);
          acc[1] = fmaf(w, v.y, acc[1]);
        } else {
          acc[0] = fmaf(w, o[0], acc[0]);
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
  const dim3 g((unsigned)((a.rows + 3) / 4)), b(256);
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
