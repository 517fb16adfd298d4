// Measurement helpers (nothing on the attention path calls them):
//  * the streaming-read rate this chip sustains for the decode kernel's access
//    pattern (wave64, 16-byte non-temporal loads, 1 KB contiguous per load
//    instruction, about four workgroups per CU): the achievable denominator next
//    to the 8 TB/s HBM3E figure;
//  * the bf16 matrix-core rate the chip sustains at the clock it holds under
//    matrix load: the packed kernels' own instruction, v_mfma_f32_32x32x16_bf16,
//    issued back to back from two waves per SIMD with nothing else in the loop;
//  * per-CU rates, in shader-clock cycles, of the other units the packed kernels
//    lean on: LDS reads with their two access patterns (16-byte row fragments and
//    transposing reads, on the same swizzled 256-byte-row tiles), v_exp_f32 and
//    v_fma_f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rswa_internal.h"
#include "rswa_tile.h"

namespace rswa {
namespace {

using namespace tile;

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

// All 16 values handed to one empty asm statement: the reads are issued back to
// back and waited for once, and nothing is computed from them.
__device__ __forceinline__ void keep16(const u32x4_t (&v)[16]) {
  asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
               "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
}

// One workgroup of 8 waves per CU (two per SIMD, the packed forward's wave
// count; 96 KB of LDS keeps a second workgroup off the CU, so one workgroup's
// cycles are the CU's). After a barrier every wave runs `iters` rounds of one
// kind of instruction and the workgroup records the shader-clock cycles the
// rounds took (s_memtime, wave 0)
// next to a fold of the arithmetic results; each LDS read result is handed to
// an empty asm statement, which keeps the read without any arithmetic on it:
//   kind 0: 16 ds_read_b128 row-fragment reads per round (16 KB per wave, the
//           forward's K-fragment pattern over two 64-row tiles);
//   kind 1: 32 ds_read_b64_tr_b16 transposing reads per round (16 KB per wave,
//           the forward's V^T pattern);
//   kind 2: 8 independent v_exp_f32 per round; kind 3: 8 independent v_fma_f32.
// out[2 g] = cycles of workgroup g, out[2 g + 1] = its fold.
__global__ __launch_bounds__(512, 1) void probe_cu_kernel(uint32_t *out, int32_t iters, int32_t kind) {
  __shared__ uint16_t sm[6 * 64 * kD];  // 96 KB; the reads use the first 32 KB
  for (int i = threadIdx.x; i < 2 * 64 * kD / 8; i += 512)
    reinterpret_cast<u32x4_t *>(sm)[i] = u32x4_t{(uint32_t)i, (uint32_t)i * 3u, (uint32_t)i ^ 0x55u, 7u};
  __syncthreads();
  const int lane = threadIdx.x & 63, hi = lane >> 5, l32 = lane & 31;
  uint32_t koff[kD / 16], toff[kD / 32][2];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) koff[ks] = row_frag_off(l32, hi, ks);
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
    toff[db][0] = tr_off(lane, db, 0);
    toff[db][1] = tr_off(lane, db, 1);
  }
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = (float)(lane + k) * (1.f / 128.f);
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (kind == 0) {
    uint32_t base = 0;
    for (int it = 0; it < iters; ++it) {
      asm volatile("" : "+v"(base));  // the compiler may not hoist the reads out of the loop
      const char *tb = reinterpret_cast<const char *>(sm) + base;
      u32x4_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = *reinterpret_cast<const u32x4_t *>(tb + koff[i % 8] + (i / 8) * 32 * kRowBytes);
      keep16(v);
    }
  } else if (kind == 1) {
    uint32_t base = 0;
    for (int it = 0; it < iters; ++it) {
      asm volatile("" : "+v"(base));
      const char *tb = reinterpret_cast<const char *>(sm) + base;
      u32x4_t v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[j] = __builtin_bit_cast(u32x4_t, tr_operand(tb, toff[j & 3][0], toff[j & 3][1], j >> 2));
      keep16(v);
    }
  } else if (kind == 2) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);  // stays in (0.5, 1]
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = fmaf(x[k], 0.999f, 0.001f);
    }
  }
  float fsum = 0.f;  // positive for every kind that computes (x stays in (0.5, 1] or tends to 1)
#pragma unroll
  for (int k = 0; k < 8; ++k) fsum += x[k];
  fsum += __shfl_xor(fsum, 1, 64);
  const uint32_t fold = __float_as_uint(fsum);
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = (uint32_t)(t1 - t0);
    out[2 * blockIdx.x + 1] = fold;
  }
}

}  // namespace

hipError_t launch_probe_cu(uint32_t *out, int32_t workgroups, int32_t iters, int32_t kind, hipStream_t s) {
  hipLaunchKernelGGL(probe_cu_kernel, dim3(workgroups), dim3(512), 0, s, out, iters, kind);
  return hipGetLastError();
}

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
