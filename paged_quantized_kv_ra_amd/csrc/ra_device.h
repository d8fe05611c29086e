// ra_device.h -- device-side types and helpers shared by the gfx950 kernels.
//
// KV element formats (ReVolta README, intro list and "Weight and KV formats"):
// FP16, FP8 E4M3 (OCP E4M3FN) and INT8, with per-layer scalar scales; the
// arithmetic runs on FP16 operands converted exactly from the stored codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPage = 16;
constexpr int kWave = 64;

// Bit reinterpretation through a by-value copy.  (hipcc's __builtin_bit_cast
// applied directly to a vector-element subscript such as v[i] reads element 0;
// passing the value through a parameter sidesteps that.)
template <class To, class From>
__device__ __forceinline__ To as(From x) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, x);
}

// ---------------------------------------------------------------------------
// Encoders (the store's quantiser).  Bit-level, independent of any table.

// fp32 -> OCP E4M3 byte: saturate to +-448, round to nearest even, keep the
// sign, NaN -> 0x7F | sign.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu | sign;            // NaN
  const float af = __uint_as_float(a);
  uint32_t mag;
  if (af >= 448.0f) {
    mag = 0x7Eu;                                       // saturate (inf too)
  } else if (af < 0.015625f) {                         // below 2^-6: steps of 2^-9
    mag = (uint32_t)__builtin_rintf(af * 512.0f);      // exact scaling, RNE; 8 = 2^-6
  } else {
    // keep 3 mantissa bits: round the low 20 bits to nearest even
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    mag = (r >> 20) - (120u << 3);                     // rebias exponent 127 -> 7
  }
  return mag | sign;
}

// fp32 -> int8 code: round half to even, clamp to [-127, 127], NaN -> 0.
__device__ __forceinline__ int32_t i8_encode(float y) {
  if (!(y == y)) return 0;
  float r = __builtin_rintf(y);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int32_t)r;
}

// ---------------------------------------------------------------------------
// Exact decoders to FP16 operands.

// Four E4M3 bytes (little-endian in x) -> four fp16 values, exactly (every
// E4M3 value, subnormals included, is an fp16 value).  The gfx950 scaled
// conversion with scale 1.0 is exact.
__device__ __forceinline__ f16x4 e4m3x4_to_f16x4(uint32_t x) {
  const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
  const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true);
  return f16x4{lo[0], lo[1], hi[0], hi[1]};
}

// Four int8 bytes -> four fp16 values, exactly: 0x6400 | (b ^ 0x80) is the
// fp16 number 1024 + (b + 128); subtracting 1152 leaves b.
__device__ __forceinline__ f16x4 i8x4_to_f16x4(uint32_t x) {
  const uint32_t ux = x ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, ux, 0x04010400u);  // [b1' 64 b0' 64]
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, ux, 0x04030402u);  // [b3' 64 b2' 64]
  f16x2 l = as<f16x2>(lo);
  f16x2 h = as<f16x2>(hi);
  const f16x2 off = {(f16)1152.0f, (f16)1152.0f};
  l = l - off;
  h = h - off;
  return f16x4{l[0], l[1], h[0], h[1]};
}

template <int KV>
__device__ __forceinline__ f16x4 codes4_to_f16x4(uint32_t x) {
  if constexpr (KV == KV_E4M3) return e4m3x4_to_f16x4(x);
  else return i8x4_to_f16x4(x);
}

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// Paged layout: byte offsets of an element inside its (page, head) block.

template <int D, int E>
__device__ __forceinline__ uint32_t k_elem_offset(int t, int d) {
  constexpr int Q = D / 4;
  const int lane = 16 * (d / Q) + t;
  const int b = (d % Q) * E;
  return (uint32_t)((b >> 4) * 1024 + lane * 16 + (b & 15));
}

template <int D, int E>
__device__ __forceinline__ uint32_t v_elem_offset(int t, int d) {
  constexpr int W = D / 16;
  const int lane = 16 * (t / 4) + d / W;
  const int b = ((d % W) * 4 + (t % 4)) * E;
  return (uint32_t)((b >> 4) * 1024 + lane * 16 + (b & 15));
}

// ---------------------------------------------------------------------------
// The store's quantiser for one cache element: FP16 cache: RNE cast; E4M3 /
// INT8: correctly rounded fp32 division by the scale, then the encoder (a
// per-token INT8 row of scale 0, all zeros, codes to 0).
template <int KV>
__device__ __forceinline__ uint32_t encode_code(float x, float scale) {
  if constexpr (KV == KV_F16) return as<uint16_t>((f16)x);
  else if constexpr (KV == KV_E4M3) return e4m3_encode(x / scale);
  else if constexpr (KV == KV_I8) return (uint32_t)i8_encode(x / scale) & 0xFFu;
  else return scale > 0.0f ? (uint32_t)i8_encode(x / scale) & 0xFFu : 0u;
}

// Quantise dims d0 .. d0 + 7 of one token's row and write them into the
// (page, head) block `blk` at token-in-page tp.  K: the 8 dims are contiguous
// inside one 16-byte piece of the layout (one 8- or 16-byte store).  V:
// four tokens interleave per dim, so one store per element.
template <int KV, int D>
__device__ __forceinline__ void store_row8(uint8_t* blk, int tp, int d0, const float (&x)[8], float scale,
                                           bool is_v) {
  constexpr int E = KV == KV_F16 ? 2 : 1;
  uint32_t code[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) code[i] = encode_code<KV>(x[i], scale);
  if (!is_v) {
    uint8_t* p = blk + k_elem_offset<D, E>(tp, d0);
    if constexpr (E == 2) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = code[2 * j] | (code[2 * j + 1] << 16);
      *reinterpret_cast<u32x4*>(p) = w;
    } else {
      u32x2 w;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        w[j] = code[4 * j] | (code[4 * j + 1] << 8) | (code[4 * j + 2] << 16) | (code[4 * j + 3] << 24);
      *reinterpret_cast<u32x2*>(p) = w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = v_elem_offset<D, E>(tp, d0 + i);
      if constexpr (E == 2) *reinterpret_cast<uint16_t*>(blk + off) = (uint16_t)code[i];
      else blk[off] = (uint8_t)code[i];
    }
  }
}


// Quantise dims d0 .. d0 + 7 (d0 a multiple of 8) of the four tokens of token
// quad gq of one page (tokens 4 gq .. 4 gq + 3, x[j] the row of token
// 4 gq + j, scale[j] its scale) and write their V codes.  The four tokens
// interleave per dim in the layout, so together they fill whole 16-byte
// pieces: 2 E of them in one lane's row at D = 128, E in each of two lanes
// at D = 64, each written with one store.
template <int KV, int D>
__device__ __forceinline__ void store_v_quad(uint8_t* blk, int gq, int d0, const float (&x)[4][8],
                                             const float (&scale)[4]) {
  constexpr int E = KV == KV_F16 ? 2 : 1;
  constexpr int W = D / 16;                     // dims per lane row
  constexpr int NL = W >= 8 ? 1 : 8 / W;        // lane rows the 8 dims span
  constexpr int NP = 2 * E / NL;                // 16-byte pieces per lane row
  static_assert(W == 8 || W == 4, "head_dim 128 or 64");
  u32x4 piece[NL][NP];
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int p = 0; p < NP; ++p) piece[l][p] = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // v_elem_offset(4 gq + j, d0 + i): lane row 16 gq + (d0 + i) / W, byte b
      const int l = W >= 8 ? 0 : i / W;
      const int b = ((i % W) * 4 + j) * E;
      piece[l][b >> 4][(b & 15) >> 2] |= encode_code<KV>(x[j][i], scale[j]) << (8 * (b & 3));
    }
  const int lane0 = 16 * gq + d0 / W;
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int p = 0; p < NP; ++p) *reinterpret_cast<u32x4*>(blk + p * 1024 + (lane0 + l) * 16) = piece[l][p];
}

// ---------------------------------------------------------------------------
// Rotary position embedding (half-split pairing, dim i with i + R/2): the
// pair turns as y1 = x1 c - x2 s, y2 = x2 c + x1 s, evaluated as written in
// fp32 (two roundings per product, one per sum: no fused multiply-add).
__device__ __forceinline__ float rope_first(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
  return x1 * c - x2 * s;
}
__device__ __forceinline__ float rope_second(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
  return x2 * c + x1 * s;
}

// Rotate the 8 dims d0 .. d0 + 7 (d0 a multiple of 8) of one row in place,
// given the row's 8 partner dims (d0 + R/2, or d0 - R/2 in the second half)
// and the row's table entry `cs` ([2][R/2] fp32: cos, then sin).  Dims past R
// pass through.
__device__ __forceinline__ void rope8(float (&x)[8], const float (&partner)[8], const float* cs, int d0, int rot) {
  if (d0 >= rot) return;
  const int half = rot / 2;
  const bool first = d0 < half;
  const int i0 = first ? d0 : d0 - half;
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + i0);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + i0 + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + half + i0);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + half + i0 + 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float co = i < 4 ? c0[i & 3] : c1[i & 3];
    const float si = i < 4 ? s0[i & 3] : s1[i & 3];
    x[i] = first ? rope_first(x[i], partner[i], co, si) : rope_second(partner[i], x[i], co, si);
  }
}

// 8 source elements (fp16, or bf16 bit patterns) -> fp32, exactly
__device__ __forceinline__ void src8_to_f32(const u32x4& r, bool bf, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t b = (uint16_t)(r[i >> 1] >> (16 * (i & 1)));
    const float hv = (float)as<f16>(b), bv = bf16_to_f32(b);
    x[i] = bf ? bv : hv;
  }
}

// fp32 max |x| of a per-token INT8 row spread over `lanes` consecutive lanes
// (a power of two; all of them active) holding 8 values each.
__device__ __forceinline__ float row_absmax(const float (&x)[8], int lanes) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  for (int o = 1; o < lanes; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// ---------------------------------------------------------------------------
// 16-byte global load (one lane's piece of a 1 KiB wavefront slab).

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace ra
