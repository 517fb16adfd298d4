// Measurement helper: the streaming-read rate this chip sustains for the decode
// kernel's access pattern (wave64, 16-byte non-temporal loads, 1 KB contiguous
// per load instruction, about four workgroups per CU). It is the achievable
// denominator next to the 8 TB/s HBM3E figure; nothing on the attention path
// calls it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rswa_internal.h"

namespace rswa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4_t *buf, int64_t nvec, float *sink) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 * 8 + threadIdx.x; base < nvec; base += stride) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < nvec ? __builtin_nontemporal_load(buf + i) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one value per workgroup keeps the loads alive
  acc ^= __shfl_xor(acc, 1, 64) ^ __shfl_xor(acc, 2, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(acc & 0xffff);
}

}  // namespace

hipError_t launch_probe_read(const void *buf, size_t bytes, float *sink, int32_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(workgroups), dim3(256), 0, s, static_cast<const u32x4_t *>(buf),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace rswa
