// read_ceiling.hip -- HBM read-rate probe for the attention's page stream
// (libra_probe.so; a measurement aid, not part of the library's ABI).
//
// Reads whole blocks of `block_bytes` (2, 4 or 8 KiB) at the positions of a
// permutation of the blocks of a buffer, the way the attention kernel reads
// (page, head) blocks through a block table, and reports nothing but an XOR of
// what it read.  Workgroups have 8 waves (512 threads); every wave takes
// blocks wave_id, wave_id + waves, ... of the permutation and keeps two of
// them in flight:
//   mode 0: LDS DMA (global_load_lds_dwordx4) into a per-wave ring, default
//           cache policy;
//   mode 1: the same with the nontemporal policy;
//   mode 2: plain 16-byte loads into registers, default policy;
//   mode 3: plain loads, nontemporal;
//   mode 4: plain loads, nontemporal, blocks in buffer order (a streaming read).
// A lane reads bytes 16 L .. 16 L + 15 of every 1 KiB of a block (one
// wavefront-wide load per KiB, as the cache layout is read).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// LDS DMA ring: two blocks of SL KiB per wave
template <int SL, int CPOL>
__global__ void __launch_bounds__(512) lds_ring(const uint8_t* buf, const int32_t* ids, int32_t nblk, uint32_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[8][2][SL * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * 8 + wave;
  const int64_t nw = (int64_t)gridDim.x * 8;
  uint32_t acc = 0;
  int32_t idv = 0, chunk = -1;
  auto issue = [&](int64_t k) {
    if (gw + k * nw >= nblk) return;
    if ((int32_t)(k >> 6) != chunk) {   // ids of the wave's next 64 blocks, one per lane
      chunk = (int32_t)(k >> 6);
      const int64_t bl = gw + (64 * (int64_t)chunk + lane) * nw;
      idv = bl < nblk ? ids[bl] : 0;
      wait_vmcnt<0>();
    }
    const int32_t id = __builtin_amdgcn_readlane(idv, (int)(k & 63));
    const uint8_t* p = buf + (int64_t)id * (SL * 1024) + lane * 16;
#pragma unroll
    for (int s = 0; s < SL; ++s)
      __builtin_amdgcn_global_load_lds(p + s * 1024, (lds_u8*)(ring[wave][k & 1] + s * 1024), 16, 0, CPOL);
  };
  issue(0);
  issue(1);
  for (int64_t k = 0; gw + k * nw < nblk; ++k) {
    wait_vmcnt<SL>();   // block k landed; block k + 1 may be in flight
    if (gw + (k + 1) * nw >= nblk) wait_vmcnt<0>();
    const uint32_t adr = (uint32_t)(uintptr_t)(const lds_u8*)&ring[wave][k & 1][lane * 16];
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(adr) : "memory");
    acc ^= x[0] ^ x[3];
    issue(k + 2);
  }
  wait_vmcnt<0>();
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = acc;
}

// plain loads: two blocks of SL KiB per wave in registers
template <int SL, bool NT, bool SEQ>
__global__ void __launch_bounds__(512) plain(const uint8_t* buf, const int32_t* ids, int32_t nblk, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * 8;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t i = gw; i < nblk; i += 2 * nw) {
    const int64_t i2 = i + nw < nblk ? i + nw : i;
    const int64_t b0 = SEQ ? i : ids[i], b1 = SEQ ? i2 : ids[i2];
    const uint8_t* p = buf + b0 * (SL * 1024) + lane * 16;
    const uint8_t* q = buf + b1 * (SL * 1024) + lane * 16;
    u32x4 a[SL], b[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      a[s] = NT ? __builtin_nontemporal_load((const u32x4*)(p + s * 1024)) : *(const u32x4*)(p + s * 1024);
      b[s] = NT ? __builtin_nontemporal_load((const u32x4*)(q + s * 1024)) : *(const u32x4*)(q + s * 1024);
    }
#pragma unroll
    for (int s = 0; s < SL; ++s) acc ^= a[s] ^ b[s];
  }
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <int SL>
hipError_t launch(int mode, const uint8_t* buf, const int32_t* ids, int32_t nblk, int32_t grid, uint32_t dyn,
                  uint32_t* out, hipStream_t s) {
  switch (mode) {
    case 0: hipLaunchKernelGGL((lds_ring<SL, 0>), dim3(grid), dim3(512), dyn, s, buf, ids, nblk, out); break;
    case 1: hipLaunchKernelGGL((lds_ring<SL, 2>), dim3(grid), dim3(512), dyn, s, buf, ids, nblk, out); break;
    case 2: hipLaunchKernelGGL((plain<SL, false, false>), dim3(grid), dim3(512), dyn, s, buf, ids, nblk, out); break;
    case 3: hipLaunchKernelGGL((plain<SL, true, false>), dim3(grid), dim3(512), dyn, s, buf, ids, nblk, out); break;
    default: hipLaunchKernelGGL((plain<SL, true, true>), dim3(grid), dim3(512), dyn, s, buf, ids, nblk, out); break;
  }
  return hipGetLastError();
}

}  // namespace

// buf: nblk * block_bytes device bytes; ids: a permutation of [0, nblk) in
// device memory (unused in mode 4); out: grid * 512 uint32 of device memory;
// dyn_lds: extra LDS bytes per workgroup (unused by the kernel), which bounds
// how many workgroups share a CU.  Returns 0, 1 for a bad argument, 5 for a
// refused launch.
extern "C" int32_t ra_probe_read_blocks(const void* buf, const int32_t* ids, int32_t nblk, int32_t block_bytes,
                                        int32_t mode, int32_t grid, int32_t dyn_lds, uint32_t* out, void* stream) {
  if (!buf || !out || (!ids && mode != 4) || nblk < 1 || grid < 1 || grid > 65536 || mode < 0 || mode > 4 ||
      dyn_lds < 0 || dyn_lds > 96 * 1024)
    return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  hipError_t e;
  switch (block_bytes) {
    case 2048: e = launch<2>(mode, b, ids, nblk, grid, (uint32_t)dyn_lds, out, s); break;
    case 4096: e = launch<4>(mode, b, ids, nblk, grid, (uint32_t)dyn_lds, out, s); break;
    case 8192: e = launch<8>(mode, b, ids, nblk, grid, (uint32_t)dyn_lds, out, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 5;
}
