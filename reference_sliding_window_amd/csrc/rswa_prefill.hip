// Prefill -> decode hand-off: after the packed forward of a pack whose sample b
// is cache sequence b's reference segment followed by its first T0 outputs,
// write the cache state T0 decode steps would have left (yhxrc and 夜雨聆风
// pages: the reference is written once; the window keeps the latest n outputs,
// the oldest evicted first; WeThinkIn "Unlimited OCR Works：一篇读懂 R-SWA…",
// section 方法展开.4, Eq. (6): L_m + min(n, T0) occupied slots):
//   reference row r (0 <= r < L_m)            -> slot r
//   output t (T0 - min(n, T0) < t <= T0)      -> slot L_m + ((t - 1) mod n)
// and step[b] = T0. Output t is row L_m + t - 1 of the sample (the token whose
// query is q_t). Bit-exact copies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rswa_internal.h"

namespace rswa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Grid (row blocks of 32, H, B); 256 threads copy 16-byte vectors.
template <int kElemBytes, int D>
__global__ __launch_bounds__(256) void prefill_handoff_kernel(HandoffParams p) {
  constexpr int kRows = 32;
  constexpr int kVecPerRow = D * kElemBytes / 16;
  constexpr int kEpv = 16 / kElemBytes;  // elements per 16-byte vector
  const int b = blockIdx.z, h = blockIdx.y;
  const int32_t L = p.ref_len[b];
  const int64_t base = p.seq_base[b];
  const int32_t row0 = p.cu_seqlens[b], row1 = p.cu_seqlens[b + 1];
  const int32_t rows = row1 - row0;
  int err = 0;
  if (L < 0 || L > p.max_ref_len) err |= RSWA_DEVERR_REF_LEN;
  if (base < 0 || (base % kEpv) != 0) err |= RSWA_DEVERR_ALIGN;
  if (row0 < 0 || row1 < row0 || row1 > p.total_tokens || rows > p.max_seq_len || L > rows)
    err |= RSWA_DEVERR_PACK;
  if (err) {
    if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0) atomicOr(p.error, err);
    return;
  }
  const int32_t T0 = rows - L;
  if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0) p.step[b] = T0;
  // Rows of the sample that land in the cache: the reference, then the last
  // min(n, T0) outputs.
  const int32_t keep_from = L + (T0 > p.window ? T0 - p.window : 0);
  const int r0 = blockIdx.x * kRows;
  const int r1 = min(rows, r0 + kRows);
  const int64_t src_stride = (int64_t)p.heads * D * kElemBytes;  // bytes per packed row
  const char *ks = static_cast<const char *>(p.k_src) + (int64_t)row0 * src_stride + (int64_t)h * D * kElemBytes;
  const char *vs = static_cast<const char *>(p.v_src) + (int64_t)row0 * src_stride + (int64_t)h * D * kElemBytes;
  char *kd = static_cast<char *>(p.k) + (base + (int64_t)h * (L + p.window) * D) * kElemBytes;
  char *vd = static_cast<char *>(p.v) + (base + (int64_t)h * (L + p.window) * D) * kElemBytes;
  for (int i = threadIdx.x; i < kRows * kVecPerRow; i += 256) {
    const int r = r0 + i / kVecPerRow, c = i % kVecPerRow;
    if (r >= r1) break;
    if (r >= L && r < keep_from) continue;  // outputs already evicted after T0 steps
    const int slot = r < L ? r : L + (r - L) % p.window;  // output t = r - L + 1
    const int64_t src = (int64_t)r * src_stride + 16 * c;
    const int64_t dst = (int64_t)slot * D * kElemBytes + 16 * c;
    *reinterpret_cast<u32x4_t *>(kd + dst) = *reinterpret_cast<const u32x4_t *>(ks + src);
    *reinterpret_cast<u32x4_t *>(vd + dst) = *reinterpret_cast<const u32x4_t *>(vs + src);
  }
}

template <int kElemBytes, int D>
hipError_t launch_handoff_t(const HandoffParams &p, hipStream_t s) {
  const int row_blocks = p.max_seq_len > 0 ? (p.max_seq_len + 31) / 32 : 1;
  hipLaunchKernelGGL((prefill_handoff_kernel<kElemBytes, D>), dim3(row_blocks, p.heads, p.batch),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_handoff(const HandoffParams &p, int32_t dtype, int32_t head_dim, hipStream_t s) {
  if (dtype == RSWA_BF16) return head_dim == 128 ? launch_handoff_t<2, 128>(p, s) : launch_handoff_t<2, 64>(p, s);
  return head_dim == 128 ? launch_handoff_t<4, 128>(p, s) : launch_handoff_t<4, 64>(p, s);
}

}  // namespace rswa
