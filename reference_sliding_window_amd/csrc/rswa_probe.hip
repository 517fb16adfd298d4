// Measurement helpers (nothing on the attention path calls them):
//  * the streaming-read rate this chip sustains for the decode kernel's access
//    pattern (wave64, 16-byte non-temporal loads, 1 KB contiguous per load
//    instruction, about four workgroups per CU): the achievable denominator next
//    to the 8 TB/s HBM3E figure;
//  * the bf16 matrix-core rate the chip sustains at the clock it holds under
//    matrix load: the packed kernels' own instruction, v_mfma_f32_32x32x16_bf16,
//    issued back to back from two waves per SIMD with nothing else in the loop.
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Each wave runs `iters` rounds of 4 independent 32x32x16 bf16 products (four
// accumulators, so each product's result is next needed 4 products later) on
// operands that depend on its lane, and folds the accumulators into one value
// per workgroup so the products are not optimised away.
__global__ __launch_bounds__(256) void probe_mfma_kernel(float *sink, int32_t iters) {
  const float x = (float)(threadIdx.x & 63) * 0.001f;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(x + 0.01f * i);
    b[i] = (__bf16)(0.5f - x);
  }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += acc[j][e];
  r += __shfl_xor(r, 1, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = r;
}

}  // namespace

hipError_t launch_probe_mfma(float *sink, int32_t workgroups, int32_t iters, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(256), 0, s, sink, iters);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void *buf, size_t bytes, float *sink, int32_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(workgroups), dim3(256), 0, s, static_cast<const u32x4_t *>(buf),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace rswa
