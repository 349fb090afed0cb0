// mla_read_probe.hip -- measurement helper, built as its own library (libmla_read_probe.so)
// next to the attention library: the plain-read probe behind mla_hbm_read_probe, i.e. the
// rate at which the device delivers a given number of bytes to a kernel that only reads
// them.  Not part of the attention boundary.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_read_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Work-group g reads words [g * per_wg, min((g + 1) * per_wg, n16)); eight 16-byte
// loads per thread are in flight per iteration, each wave-wide load a contiguous 1 KB,
// with the nontemporal hint (the fastest plain read measured on this chip: about
// 6.6 TB/s at 512 work-groups against 5.6 - 5.8 TB/s without the hint).  The xor keeps
// the loads alive.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* __restrict__ src,
                                                         size_t n16, size_t per_wg,
                                                         uint32_t* __restrict__ sink) {
  constexpr int kUnroll = 8;
  const size_t beg = (size_t)blockIdx.x * per_wg;
  const size_t end = beg + per_wg < n16 ? beg + per_wg : n16;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (size_t i = beg + threadIdx.x; i < end; i += 256 * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + 256 * (size_t)u;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : (u32x4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" int mla_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid,
                                  void* stream) {
  if (!src || !sink || grid < 1 || grid > 65536) return -1;
  if (bytes % 16 != 0 || ((uintptr_t)src & 15) != 0) return -1;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  const size_t per = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4_t*)src, n16, per, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
