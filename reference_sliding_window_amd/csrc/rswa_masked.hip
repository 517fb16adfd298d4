// Packed (teacher-forced) R-SWA forward on gfx950 matrix cores.
//
// Row i of a packed sequence attends to key j iff j <= i and (j < L_m or
// i - j < n): for an output row this is N(t) = P ∪ D_n(t) of WeThinkIn
// "Unlimited OCR Works：一篇读懂 R-SWA…", section 方法展开.3, Eqs. (1)-(2), for
// the query formed at position i; prefix rows (not covered by Eq. (1)) are
// causal, or see the whole prefix in RSWA_PREFIX_FULL mode. Softmax and the
// weighted sum follow Eqs. (3)-(4).
//
// Design (one workgroup = 128 query rows of one head, 4 waves x 32 rows):
//  * Only key blocks that intersect the two-segment mask are visited: the
//    prefix range [0, min(L_m, q_end)) and the window range
//    [max(L_m, first_output_row - n + 1), q_end). Everything else is skipped.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as the A operand, the wave's Q rows resident in VGPRs as the B operand),
//    so lane l owns query l % 32: the softmax row max and sum are in-register
//    plus one exchange with lane l ^ 32.
//  * O^T += V^T P^T reuses the S^T accumulators as the B operand after the
//    exp2 and the bf16 conversion; the key order inside each 16-key MFMA step
//    is permuted to match the accumulator layout, and V is stored transposed
//    in LDS so that the A operand is two 8-byte LDS reads.
//  * Global loads of the next key block are issued before the MFMAs of the
//    current one (register double buffering).
//  * Workgroups are ordered so that all query blocks of a head run on the same
//    XCD (hardware places workgroup i on XCD i mod 8), keeping that head's
//    prefix K/V resident in the XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rswa_internal.h"

namespace rswa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;          // head dim
constexpr int kBM = 128;         // query rows per workgroup
constexpr int kBN = 64;          // keys per block
constexpr int kKPitch = kD + 8;  // LDS row pitch of K (elements): conflict-free b128 reads
constexpr int kVPitch = kBN + 4; // LDS row pitch of V^T (elements)
constexpr float kNegInf = -__builtin_huge_valf();

struct Smem {
  uint16_t k[kBN * kKPitch];   // K block, row-major [key][d]
  uint16_t vt[kD * kVPitch];   // V block transposed [d][key]
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

struct Range {
  int lo, hi;
};

__global__ __launch_bounds__(256) void masked_attn_kernel(MaskedParams p) {
  __shared__ Smem sm;
  const int N = p.seq_len, H = p.heads, Lm = p.ref_len, n = p.window;
  const int nqb = (N + kBM - 1) / kBM;
  const int G = nqb * H;
  // XCD-aware order: logical work item w -> (head, query block)
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int h = w / nqb;
  const int qb = w % nqb;
  const int q0 = qb * kBM;
  const int q_end = min(N, q0 + kBM);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5;   // lane half
  const int l32 = lane & 31;
  const int64_t row_stride = (int64_t)H * kD;
  const uint16_t *Qg = static_cast<const uint16_t *>(p.q) + (int64_t)h * kD;
  const uint16_t *Kg = static_cast<const uint16_t *>(p.k) + (int64_t)h * kD;
  const uint16_t *Vg = static_cast<const uint16_t *>(p.v) + (int64_t)h * kD;
  uint16_t *Og = static_cast<uint16_t *>(p.out) + (int64_t)h * kD;

  // Key ranges that intersect the mask for this query block.
  Range ranges[2];
  int nr = 0;
  {
    const int pre_hi = (p.prefix_mode == RSWA_PREFIX_FULL && q0 < Lm) ? Lm : min(Lm, q_end);
    if (pre_hi > 0) ranges[nr++] = {0, pre_hi};
    if (q_end > Lm) {
      const int first_out = max(q0, Lm);
      ranges[nr++] = {max(Lm, first_out - n + 1), q_end};
    }
  }

  // This wave's 32 queries; lane l owns query qi.
  const int qi = q0 + wave * 32 + l32;
  const bool q_ok = qi < N;
  bf16x8_t qf[kD / 16];
  {
    const uint16_t *qrow = Qg + (int64_t)(q_ok ? qi : 0) * row_stride;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      uint4 u = q_ok ? *reinterpret_cast<const uint4 *>(qrow + ks * 16 + hi * 8)
                     : make_uint4(0, 0, 0, 0);
      qf[ks] = as_bf16x8(u);
    }
  }

  f32x16_t o[kD / 32];
#pragma unroll
  for (int j = 0; j < kD / 32; ++j) o[j] = f32x16_t{};
  float m = kNegInf, l = 0.f;

  // Global->register staging of one key block: thread t loads rows
  // (t >> 4) + 16 * i (i = 0..3), 16-byte column chunk t & 15, of K and V.
  const int ld_row = tid >> 4, ld_col = (tid & 15) * 8;
  uint4 kst[4], vst[4];
  auto load_block = [&](int kb0, int kend) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = kb0 + ld_row + 16 * i;
      r = r < kend ? r : kend - 1;
      kst[i] = *reinterpret_cast<const uint4 *>(Kg + (int64_t)r * row_stride + ld_col);
      vst[i] = *reinterpret_cast<const uint4 *>(Vg + (int64_t)r * row_stride + ld_col);
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_row + 16 * i;
      *reinterpret_cast<uint4 *>(&sm.k[r * kKPitch + ld_col]) = kst[i];
      const uint32_t w4[4] = {vst[i].x, vst[i].y, vst[i].z, vst[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.vt[(ld_col + 2 * e) * kVPitch + r] = static_cast<uint16_t>(w4[e] & 0xffffu);
        sm.vt[(ld_col + 2 * e + 1) * kVPitch + r] = static_cast<uint16_t>(w4[e] >> 16);
      }
    }
  };

  // Flattened list of key blocks over the (at most two) ranges.
  int nb0 = nr > 0 ? (ranges[0].hi - ranges[0].lo + kBN - 1) / kBN : 0;
  int nb1 = nr > 1 ? (ranges[1].hi - ranges[1].lo + kBN - 1) / kBN : 0;
  const int nblocks = nb0 + nb1;
  auto block_of = [&](int bi, int &kb0, int &kend) {
    if (bi < nb0) {
      kb0 = ranges[0].lo + bi * kBN;
      kend = ranges[0].hi;
    } else {
      kb0 = ranges[1].lo + (bi - nb0) * kBN;
      kend = ranges[1].hi;
    }
  };

  const bool full_prefix = p.prefix_mode == RSWA_PREFIX_FULL;
  if (nblocks > 0) {
    int kb0, kend;
    block_of(0, kb0, kend);
    load_block(kb0, kend);
  }
  for (int bi = 0; bi < nblocks; ++bi) {
    int kb0, kend;
    block_of(bi, kb0, kend);
    __syncthreads();  // previous block's LDS reads are done
    store_block();
    __syncthreads();
    if (bi + 1 < nblocks) {
      int nb, ne;
      block_of(bi + 1, nb, ne);
      load_block(nb, ne);
    }

    // S^T tiles: 2 x (32 keys x 32 queries)
    f32x16_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16_t{};
      const uint16_t *krow = &sm.k[(kt * 32 + l32) * kKPitch + hi * 8];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4 *>(krow + ks * 16));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kt], 0, 0, 0);
      }
    }

    // Mask, scale, block max. Accumulator element r of tile kt holds
    // key kb0 + 32 kt + 8 (r / 4) + 4 hi + (r % 4) for query qi.
    float bmax = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kb0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        bool vis = (j < kend) && (j <= qi);
        if (qi >= Lm) {
          vis = vis && (j < Lm || qi - j < n);
        } else if (full_prefix) {
          vis = (j < kend) && (j < Lm);
        }
        const float x = vis ? s[kt][r] * p.scale_log2 : kNegInf;
        s[kt][r] = x;
        bmax = fmaxf(bmax, x);
      }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(m, bmax);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - mu);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int j = 0; j < kD / 32; ++j) o[j] *= alpha;

    // P^T as bf16 B operands: step (kt, half) uses accumulator elements
    // 8*half .. 8*half+7, i.e. keys 32kt + 16half + {4hi..4hi+3, 8+4hi..8+4hi+3}.
    bf16x8_t pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(s[kt][8 * half + 2 * e] - mu);
          const float p1 = __builtin_amdgcn_exp2f(s[kt][8 * half + 2 * e + 1] - mu);
          l += p0 + p1;
          w4[e] = pack_bf16(p0, p1);
        }
        pb[2 * kt + half] = as_bf16x8(make_uint4(w4[0], w4[1], w4[2], w4[3]));
      }
    }

    // O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
      const uint16_t *vrow = &sm.vt[(db * 32 + l32) * kVPitch + 4 * hi];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int key0 = 16 * st;  // st = 2 kt + half
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + key0);
        const uint2 hi8 = *reinterpret_cast<const uint2 *>(vrow + key0 + 8);
        const bf16x8_t a = as_bf16x8(make_uint4(lo.x, lo.y, hi8.x, hi8.y));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[db], 0, 0, 0);
      }
    }
  }

  // Normalise and store: accumulator element r of o[db] is d = 32 db + 8 (r/4) + 4 hi + r%4.
  l += __shfl_xor(l, 32, 64);
  if (!q_ok) return;
  const float inv = 1.f / l;
  uint16_t *orow = Og + (int64_t)qi * row_stride;
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * hi;
      uint2 w2;
      w2.x = pack_bf16(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv);
      w2.y = pack_bf16(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
      *reinterpret_cast<uint2 *>(orow + d0) = w2;
    }
  }
}

}  // namespace

hipError_t launch_masked(const MaskedParams &p, int32_t head_dim, hipStream_t s) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int nqb = (p.seq_len + kBM - 1) / kBM;
  const int64_t G = (int64_t)nqb * p.heads;
  hipLaunchKernelGGL(masked_attn_kernel, dim3((unsigned)G), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace rswa
