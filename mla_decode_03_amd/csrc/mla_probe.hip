// HBM streaming-read probe: the read bandwidth this device delivers to a plain stream,
// reported beside the decode's as the ceiling it is measured against.  Not part of the
// decode path.
//
// Each workgroup (256 threads) reads its own contiguous chunk of the source once, in one
// of two ways:
//   mode 0  16-byte vector loads into registers, four in flight per thread;
//   mode 1  the decode's copy instruction: wave-wide global->LDS copies of 1 KB (64 lanes
//           x 16 B) into a 128 KB LDS ring, up to 32 copies in flight per wave, which is
//           what the decode's page stream is built from.
// The loaded values feed a condition that is practically never true, so no load can be
// removed; `sink` is written only then.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_args.h"
#include "mla_device.h"

namespace mla {

constexpr int kProbeRingBytes = 131072;   // mode 1: LDS ring, 128 slots of 1 KB
constexpr int kProbeDepth = 32;           // mode 1: copies in flight per wave
constexpr uint32_t kProbeMagic = 0x9e3779b9u;

__global__ __launch_bounds__(256) void mla_probe_loads_kernel(const uint8_t* __restrict__ src,
                                                              size_t chunk, uint32_t* sink) {
  const u32x4* p = (const u32x4*)(src + (size_t)blockIdx.x * chunk);
  const size_t n = chunk / 16;   // 16-byte elements, a multiple of 4 x 256
  uint32_t acc = 0;
  for (size_t i = threadIdx.x; i < n; i += 4 * 256) {
    const u32x4 a = p[i], b = p[i + 256], c = p[i + 512], d = p[i + 768];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^
           d[2] ^ d[3];
  }
  if (acc == kProbeMagic) sink[blockIdx.x] = acc;
}

// The decode's copy form: lane i's 16 bytes at base + voff land at LDS lds + 16 i.
__device__ __forceinline__ void probe_copy(const uint8_t* base, uint32_t voff, MLA_LDS uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

__global__ __launch_bounds__(256, 1) void mla_probe_lds_kernel(const uint8_t* __restrict__ src, size_t chunk,
                                                               uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kProbeRingBytes];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)ring;
  const int w = wave_id(), l = threadIdx.x & 63;
  const uint8_t* base = src + (size_t)blockIdx.x * chunk;
  // wave w copies KB k = 4j + w of the chunk into ring slot (4j + w) mod 128, so slot s is
  // rewritten kProbeDepth copies later by the same wave, after its earlier copy landed
  const int per_wave = (int)(chunk / 4096);
  for (int j = 0; j < per_wave; ++j) {
    if (j >= kProbeDepth) asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kProbeDepth - 1) : "memory");
    const uint32_t kb = 4u * (uint32_t)j + (uint32_t)w;
    probe_copy(base, kb * 1024u + 16u * (uint32_t)l, lds + (kb % 128u) * 1024u);
  }
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  __syncthreads();
  const uint32_t v = ((const MLA_LDS uint32_t*)lds)[threadIdx.x];
  if (v == kProbeMagic) sink[blockIdx.x] = v;
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_probe(const void* src, size_t bytes, int mode, int num_wg,
                                                    uint32_t* sink, hipStream_t stream) {
  const size_t chunk = bytes / (size_t)num_wg;
  const uint8_t* s = static_cast<const uint8_t*>(src);
  if (mode == 0)
    hipLaunchKernelGGL(mla::mla_probe_loads_kernel, dim3(num_wg), dim3(256), 0, stream, s, chunk, sink);
  else
    hipLaunchKernelGGL(mla::mla_probe_lds_kernel, dim3(num_wg), dim3(256), 0, stream, s, chunk, sink);
  return hipGetLastError();
}
