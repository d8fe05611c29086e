// kv_store.hip -- quantise new K/V rows and scatter them into 16-token pages,
// and the exact gather-dequantise read-back used to check the cache.
//
// The KV cache is written as FP16, FP8 E4M3 or INT8 with per-layer K and V
// scales (ReVolta README, intro list and "Weight and KV formats"; "Running
// FP4-Local on 4 x V100 32 GB (Volta) with ReVolta", "What it takes", for the
// per-layer target K/V scale pack), or as INT8 with a scale per token and head
// computed here at store time (ReVolta README, "Weight and KV formats", INT8
// KV), into 16-token pages ("ReVolta 0.1.3", "Known issues").
//
// One thread handles 8 consecutive dimensions of one head for TPT consecutive
// source tokens: it reads 16 bytes of K and 16 of V per token, quantises with
// a correctly rounded fp32 divide, and writes each token's K codes as one 8-
// or 16-byte store (a K row slice is contiguous in the layout).  V interleaves
// four tokens per dimension.  Large stores (bulk fills) take TPT = 4 tokens
// per thread: when those four slots are one 4-token group of a page (tokens
// written in order), their V codes go out as whole 16-byte pieces
// (store_v_quad).  Any other group, and smaller stores, whose launches need
// every thread they can get in flight (a prompt's store is latency-bound),
// store V element by element.  The bytes written are the same either way.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

template <int KV, int D, bool BF16, int TPT>
__global__ void __launch_bounds__(256) kv_store_kernel(StoreLaunch a) {
  constexpr int E = KV == KV_F16 ? 2 : 1;
  constexpr int CH = D / 8;                       // 8-dim chunks per head
  // every launch argument in one round of scalar loads, ahead of the first branch
  asm volatile("" ::"s"(a.k), "s"(a.v), "s"(a.k_stride), "s"(a.v_stride), "s"(a.slots), "s"(a.num_tokens),
               "s"(a.k_cache), "s"(a.v_cache), "s"(a.num_pages), "s"(a.hkv), "s"(a.k_scale), "s"(a.v_scale),
               "s"(gridDim.x), "s"(blockDim.x), "s"(a.k_scales), "s"(a.v_scales));
  // the host guarantees num_tokens * hkv * CH < 2^31
  static_assert(TPT == 1 || TPT == 4, "tokens per thread");
  const int64_t T = a.num_tokens;
  const int32_t units = (int32_t)((T + TPT - 1) / TPT * a.hkv * CH);
  const int64_t limit = a.num_pages * kPage;
  for (int32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += gridDim.x * blockDim.x) {
    const int c = u % CH;
    const int32_t th = u / CH;
    const int h = th % a.hkv;
    const int64_t t0 = TPT * (int64_t)(th / a.hkv);   // the group's first source token
    const int nt = (int)min((int64_t)TPT, T - t0);
    const int d0 = c * 8;
    // the group's source rows and slots are requested together (a short last
    // group repeats its last token; only tokens j < nt are stored)
    u32x4 kr[TPT], vr[TPT];
    int64_t slot[TPT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int64_t t = t0 + min(j, nt - 1);
      kr[j] = load16(reinterpret_cast<const uint16_t*>(a.k) + t * a.k_stride + (int64_t)h * D + d0);
      vr[j] = load16(reinterpret_cast<const uint16_t*>(a.v) + t * a.v_stride + (int64_t)h * D + d0);
      slot[j] = a.slots[t];
    }
#pragma unroll
    for (int j = 0; j < TPT; ++j) asm volatile("" ::"v"(kr[j]), "v"(vr[j]), "v"(slot[j]));   // all in flight
    float kf[TPT][8], vf[TPT][8];
#pragma unroll
    for (int j = 0; j < TPT; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t kb = (uint16_t)(kr[j][i >> 1] >> (16 * (i & 1)));
        const uint16_t vb = (uint16_t)(vr[j][i >> 1] >> (16 * (i & 1)));
        if constexpr (BF16) {
          kf[j][i] = bf16_to_f32(kb);
          vf[j][i] = bf16_to_f32(vb);
        } else {
          kf[j][i] = (float)as<f16>(kb);
          vf[j][i] = (float)as<f16>(vb);
        }
      }
    // per-token INT8: each (token, head) row's scale is max |x| / 127 over its
    // CH threads (consecutive lanes of one wave, all active or all skipped)
    float ks[TPT], vs[TPT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      ks[j] = a.k_scale;
      vs[j] = a.v_scale;
      if constexpr (KV == KV_I8T) {
        ks[j] = row_absmax(kf[j], CH) / 127.0f;   // correctly rounded (built with -fhip-fp32-correctly-rounded-divide-sqrt)
        vs[j] = row_absmax(vf[j], CH) / 127.0f;
      }
    }
    uint8_t* const k0 = reinterpret_cast<uint8_t*>(a.k_cache);
    uint8_t* const v0 = reinterpret_cast<uint8_t*>(a.v_cache);
    bool whole = false;
    if constexpr (TPT == 4)
      whole = nt == 4 && slot[0] >= 0 && slot[0] + 3 < limit && (slot[0] & 3) == 0 && slot[1] == slot[0] + 1 &&
              slot[2] == slot[0] + 2 && slot[3] == slot[0] + 3;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      if (j >= nt || slot[j] < 0 || slot[j] >= limit) continue;
      const int64_t page = slot[j] >> 4;
      const int tp = (int)(slot[j] & 15);
      const int64_t blk = (page * a.hkv + h) * (int64_t)(kPage * D * E);
      if constexpr (KV == KV_I8T) {
        if (c == 0) {
          const int64_t si = (page * a.hkv + h) * kPage + tp;
          a.k_scales[si] = ks[j];
          a.v_scales[si] = vs[j];
        }
      }
      store_row8<KV, D>(k0 + blk, tp, d0, kf[j], ks[j], false);
      if (!whole) store_row8<KV, D>(v0 + blk, tp, d0, vf[j], vs[j], true);
    }
    if constexpr (TPT == 4) {
      if (whole) {
        const int64_t page = slot[0] >> 4;
        store_v_quad<KV, D>(v0 + (page * a.hkv + h) * (int64_t)(kPage * D * E), (int)(slot[0] & 15) >> 2, d0, vf,
                            vs);
      }
    }
  }
}

// out[j][h][d] = fp32(decode(code)) * scale, through the block-table row.
template <int KV, int D, bool IS_V>
__global__ void __launch_bounds__(256) kv_gather_kernel(GatherLaunch a) {
  constexpr int E = KV == KV_F16 ? 2 : 1;
  const int64_t n = (int64_t)a.ctx * a.hkv * (D / 4);   // 4 dims per thread
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int d0 = (int)(u % (D / 4)) * 4;
    const int64_t jh = u / (D / 4);
    const int h = (int)(jh % a.hkv);
    const int j = (int)(jh / a.hkv);
    float* o = a.out + ((int64_t)j * a.hkv + h) * D + d0;
    const int32_t page = a.bt_row[j >> 4];
    if (page < 0 || page >= a.num_pages) {
      for (int i = 0; i < 4; ++i) o[i] = __builtin_nanf("");
      continue;
    }
    const int t = j & 15;
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.cache) +
                         ((int64_t)page * a.hkv + h) * (int64_t)(kPage * D * E);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = IS_V ? v_elem_offset<D, E>(t, d0 + i) : k_elem_offset<D, E>(t, d0 + i);
      float val;
      if constexpr (KV == KV_F16) {
        val = (float)as<f16>(*reinterpret_cast<const uint16_t*>(blk + off));
      } else {
        // decode through the same fp16 converters the attention kernels use
        const f16x4 h4 = codes4_to_f16x4<KV>((uint32_t)blk[off]);
        const float sc = KV == KV_I8T ? a.scales[((int64_t)page * a.hkv + h) * kPage + t] : a.scale;
        val = __fmul_rn((float)h4[0], sc);
      }
      o[i] = val;
    }
  }
}

// Stores of at least this many (token, head) rows take four tokens per
// thread: that still puts 32 waves of 64 threads on each of the 256 CUs (at
// D = 128, 16 threads per row and token).
constexpr int64_t kQuadRows = 256 * 32 * 64 * 4 / 16;

dim3 grid_for(int64_t units) {
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;   // grid-stride beyond this
  if (blocks < 1) blocks = 1;
  return dim3((unsigned)blocks);
}

template <int KV, int D, int TPT>
hipError_t store_dispatch_src(const StoreLaunch& a, hipStream_t s, dim3 b) {
  const dim3 g = grid_for((a.num_tokens + TPT - 1) / TPT * a.hkv * (D / 8));
  if (a.src_bf16) hipLaunchKernelGGL((kv_store_kernel<KV, D, true, TPT>), g, b, 0, s, a);
  else hipLaunchKernelGGL((kv_store_kernel<KV, D, false, TPT>), g, b, 0, s, a);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t store_dispatch_tpt(const StoreLaunch& a, hipStream_t s, dim3 b) {
  return a.num_tokens * a.hkv >= kQuadRows ? store_dispatch_src<KV, D, 4>(a, s, b)
                                           : store_dispatch_src<KV, D, 1>(a, s, b);
}

template <int KV>
hipError_t store_dispatch_d(const StoreLaunch& a, hipStream_t s, dim3 b) {
  return a.head_dim == 64 ? store_dispatch_tpt<KV, 64>(a, s, b) : store_dispatch_tpt<KV, 128>(a, s, b);
}

template <int KV, int D>
hipError_t gather_dispatch_which(const GatherLaunch& a, hipStream_t s, dim3 g, dim3 b) {
  if (a.which) hipLaunchKernelGGL((kv_gather_kernel<KV, D, true>), g, b, 0, s, a);
  else hipLaunchKernelGGL((kv_gather_kernel<KV, D, false>), g, b, 0, s, a);
  return hipGetLastError();
}

template <int KV>
hipError_t gather_dispatch_d(const GatherLaunch& a, hipStream_t s, dim3 g, dim3 b) {
  return a.head_dim == 64 ? gather_dispatch_which<KV, 64>(a, s, g, b)
                          : gather_dispatch_which<KV, 128>(a, s, g, b);
}

}  // namespace

hipError_t launch_kv_store(const StoreLaunch& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const dim3 b(256);
  switch (a.kv) {
    case KV_F16: return store_dispatch_d<KV_F16>(a, s, b);
    case KV_E4M3: return store_dispatch_d<KV_E4M3>(a, s, b);
    case KV_I8T: return store_dispatch_d<KV_I8T>(a, s, b);
    default: return store_dispatch_d<KV_I8>(a, s, b);
  }
}

hipError_t launch_kv_gather(const GatherLaunch& a, hipStream_t s) {
  if (a.ctx == 0) return hipSuccess;
  const dim3 g = grid_for((int64_t)a.ctx * a.hkv * (a.head_dim / 4)), b(256);
  switch (a.kv) {
    case KV_F16: return gather_dispatch_d<KV_F16>(a, s, g, b);
    case KV_E4M3: return gather_dispatch_d<KV_E4M3>(a, s, g, b);
    case KV_I8T: return gather_dispatch_d<KV_I8T>(a, s, g, b);
    default: return gather_dispatch_d<KV_I8>(a, s, g, b);
  }
}

}  // namespace ra
