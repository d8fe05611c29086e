// qkv_rope.hip -- one pass over a step's new tokens: split the packed QKV
// projection rows, apply rotary position embedding (RoPE, with YaRN scaling
// baked into the table) to Q and K, write Q contiguously for the attention
// kernel, and quantise + scatter K and V into the paged caches.
//
// Sources: ReVolta README, DFlash2 settings list (the verifier's Q/K/V rows
// packed by one copy kernel); "Quick start", step 2 (YaRN, factor 2 over a
// 262,144-token native context).  The rotation pairs dim i with dim
// i + R/2 over the first R = rotary_dim dims (the half-split form of the
// Qwen family); the table is fp32 [max_position][2][R/2] (cos, then sin, the
// YaRN temperature already folded in).
//
// One thread owns 16 dims of one (token, head): for i0 = 8c < R/2 the pairs
// [i0, i0 + 8) and [R/2 + i0, R/2 + i0 + 8); past the rotary part, 16
// consecutive dims.  It reads them as two 16-byte loads, rotates in fp32
// with no fused multiply-add (y1 = x1 c - x2 s, y2 = x2 c + x1 s), and then
// either writes Q (two 16-byte stores) or quantises K/V exactly as the KV
// store does (correctly rounded fp32 division by the scale).  Rows of a
// head take D / 16 consecutive lanes, so the per-token INT8 row maximum is a
// shuffle reduction inside that lane group.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {
namespace {

template <bool BF16>
__device__ __forceinline__ void unpack8(const u32x4& r, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t b = (uint16_t)(r[i >> 1] >> (16 * (i & 1)));
    x[i] = BF16 ? bf16_to_f32(b) : (float)as<f16>(b);
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack8(const float (&y)[8]) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = BF16 ? f32_to_bf16(y[2 * j]) : as<uint16_t>((f16)y[2 * j]);
    const uint32_t hi = BF16 ? f32_to_bf16(y[2 * j + 1]) : as<uint16_t>((f16)y[2 * j + 1]);
    w[j] = lo | (hi << 16);
  }
  return w;
}

template <int KV, int D, bool BF16>
__global__ void __launch_bounds__(256) qkv_rope_kernel(RopeLaunch a) {
  constexpr int E = KV == KV_F16 ? 2 : 1;
  constexpr int CP = D / 16;                     // lanes per head
  const int32_t H3 = a.hq + 2 * a.hkv;
  // the host guarantees num_tokens * H3 * CP < 2^31
  const int32_t units = (int32_t)(a.num_tokens * H3 * CP);
  const int64_t limit = a.num_pages * kPage;
  const int half = a.rot / 2;
  for (int32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += gridDim.x * blockDim.x) {
    const int c = u % CP;
    const int32_t th = u / CP;
    const int hh = th % H3;
    const int32_t t = th / H3;
    const bool rotary = 16 * c < a.rot;
    const int da = rotary ? 8 * c : a.rot + 16 * (c - a.rot / 16);
    const int db = rotary ? half + 8 * c : da + 8;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(a.qkv) + t * a.qkv_stride + (int64_t)hh * D;
    const u32x4 ra = load16(src + da);
    const u32x4 rb = load16(src + db);
    const int64_t pos = a.positions[t];
    const bool pos_ok = pos >= 0 && pos < a.max_pos;
    float xa[8], xb[8];
    unpack8<BF16>(ra, xa);
    unpack8<BF16>(rb, xb);
    const bool is_v = hh >= a.hq + a.hkv;
    if (rotary && !is_v && pos_ok) {
      const float* cs = a.table + pos * a.rot + 8 * c;
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + half);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + half + 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float co = i < 4 ? c0[i & 3] : c1[i & 3];
        const float si = i < 4 ? s0[i & 3] : s1[i & 3];
        const float y1 = rope_first(xa[i], xb[i], co, si);
        const float y2 = rope_second(xa[i], xb[i], co, si);
        xa[i] = y1;
        xb[i] = y2;
      }
    }
    if (hh < a.hq) {                              // Q: contiguous [T][Hq][D] rows
      if (!pos_ok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) xa[i] = xb[i] = __builtin_nanf("");
      }
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.q_out) + t * a.q_stride + (int64_t)hh * D;
      *reinterpret_cast<u32x4*>(dst + da) = pack8<BF16>(xa);
      *reinterpret_cast<u32x4*>(dst + db) = pack8<BF16>(xb);
      continue;
    }
    // K or V of KV head h: the whole lane group of the (token, head) takes
    // this branch together (same token), so the shuffles below see it whole
    const int h = is_v ? hh - a.hq - a.hkv : hh - a.hq;
    const int64_t slot = a.slots[t];
    if (!pos_ok || slot < 0 || slot >= limit) continue;
    const int64_t page = slot >> 4;
    const int tp = (int)(slot & 15);
    float sc = is_v ? a.v_scale : a.k_scale;
    if constexpr (KV == KV_I8T) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fmaxf(fabsf(xa[i]), fabsf(xb[i])));
#pragma unroll
      for (int o = 1; o < CP; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      sc = m / 127.0f;   // correctly rounded (built with -fhip-fp32-correctly-rounded-divide-sqrt)
      if (c == 0) (is_v ? a.v_scales : a.k_scales)[(page * a.hkv + h) * kPage + tp] = sc;
    }
    uint8_t* blk = reinterpret_cast<uint8_t*>(is_v ? a.v_cache : a.k_cache) +
                   (page * a.hkv + h) * (int64_t)(kPage * D * E);
    store_row8<KV, D>(blk, tp, da, xa, sc, is_v);
    store_row8<KV, D>(blk, tp, db, xb, sc, is_v);
  }
}

template <int KV, int D>
hipError_t dispatch_src(const RopeLaunch& a, hipStream_t s, dim3 g, dim3 b) {
  if (a.src_bf16) hipLaunchKernelGGL((qkv_rope_kernel<KV, D, true>), g, b, 0, s, a);
  else hipLaunchKernelGGL((qkv_rope_kernel<KV, D, false>), g, b, 0, s, a);
  return hipGetLastError();
}

template <int KV>
hipError_t dispatch_d(const RopeLaunch& a, hipStream_t s, dim3 g, dim3 b) {
  return a.head_dim == 64 ? dispatch_src<KV, 64>(a, s, g, b) : dispatch_src<KV, 128>(a, s, g, b);
}

}  // namespace

hipError_t launch_qkv_rope(const RopeLaunch& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const int64_t units = a.num_tokens * (a.hq + 2 * a.hkv) * (a.head_dim / 16);
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;   // grid-stride beyond this
  const dim3 g((unsigned)blocks), b(256);
  switch (a.kv) {
    case KV_F16: return dispatch_d<KV_F16>(a, s, g, b);
    case KV_E4M3: return dispatch_d<KV_E4M3>(a, s, g, b);
    case KV_I8T: return dispatch_d<KV_I8T>(a, s, g, b);
    default: return dispatch_d<KV_I8>(a, s, g, b);
  }
}

}  // namespace ra
