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
//    [max(L_m, first_output_row - n + 1), q_end). Only blocks that cut the
//    mask (partial blocks, the causal diagonal of prefix rows, the window)
//    evaluate the mask; all other blocks run unmasked.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as the A operand, the wave's Q rows resident in VGPRs as the B operand),
//    so lane l owns query l % 32: the softmax row max and sum are in-register
//    plus one exchange with lane l ^ 32.
//  * O^T += V^T P^T reuses the S^T accumulators as the B operand after the
//    exp2 and the packed bf16 convert; V is stored transposed in LDS.
//  * Keys sit in LDS in a permuted order: with R = block / 16 rows staged per
//    thread, LDS row rho holds key rho / R + 16 (rho mod R). A thread that
//    loads keys u, u+16, ... (coalesced rows) then writes them as one packed
//    word of V^T per d (8 bytes for 64-key blocks, 4 for 32-key blocks).
//    The contraction over keys does not depend on their order; the mask uses
//    the true key index.
//  * Softmax in base 2 with the scale folded into one FMA before exp2. The
//    running max used for exponentiation is only raised (and O, l rescaled)
//    when a block's max exceeds it by more than 8 (a factor 2^8), which keeps
//    every probability below 2^8 and skips most rescales.
//  * LDS is double buffered: the next block's global loads are issued before
//    the current block's MFMAs and written to the other buffer after them;
//    one barrier per block.
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
// Native vectors for 16- and 8-byte moves (HIP's uint4 is a struct whose copies
// go through private memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#ifndef RSWA_MASKED_BN
#define RSWA_MASKED_BN 64  // keys per block: 32 or 64
#endif
#ifndef RSWA_MASKED_OCC
#define RSWA_MASKED_OCC 2  // workgroups per CU the register budget is sized for
#endif

constexpr int kD = 128;           // head dim
constexpr int kBM = 128;          // query rows per workgroup
constexpr int kBN = RSWA_MASKED_BN;
constexpr int kRpt = kBN / 16;    // key rows staged per thread
constexpr int kKPitch = kD + 8;   // LDS row pitch of K (elements)
constexpr int kVPitch = kBN + 4;  // LDS row pitch of V^T (elements)
static_assert(kBN == 32 || kBN == 64, "key block of 32 or 64");
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleThreshold = 8.f;  // log2 units

struct Buf {
  uint16_t k[kBN * kKPitch];   // K block, [rho][d]
  uint16_t vt[kD * kVPitch];   // V block transposed, [d][rho]
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// true key offset (within the block) of LDS row rho
__device__ __forceinline__ int key_of_row(int rho) { return rho / kRpt + 16 * (rho % kRpt); }

struct Block {
  int kb0;      // first key of the block
  int kend;     // end of the key range the block belongs to
  bool window;  // block of the window range (keys >= L_m)
};

__global__ __launch_bounds__(256, RSWA_MASKED_OCC) void masked_attn_kernel(MaskedParams p) {
  __shared__ Buf sm[2];
  const int N = p.seq_len, H = p.heads, Lm = p.ref_len, n = p.window;
  const bool full_prefix = p.prefix_mode == RSWA_PREFIX_FULL;
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
  const int hi = lane >> 5;  // lane half
  const int l32 = lane & 31;
  const int64_t row_stride = (int64_t)H * kD;
  const uint16_t *Qg = static_cast<const uint16_t *>(p.q) + (int64_t)h * kD;
  const uint16_t *Kg = static_cast<const uint16_t *>(p.k) + (int64_t)h * kD;
  const uint16_t *Vg = static_cast<const uint16_t *>(p.v) + (int64_t)h * kD;
  uint16_t *Og = static_cast<uint16_t *>(p.out) + (int64_t)h * kD;

  // Key ranges that intersect the mask for this query block.
  const int pre_hi = (full_prefix && q0 < Lm) ? Lm : min(Lm, q_end);
  const int win_lo = max(Lm, max(q0, Lm) - n + 1);
  const int win_hi = q_end > Lm ? q_end : win_lo;
  const int nb_pre = (pre_hi + kBN - 1) / kBN;
  const int nb_win = (win_hi - win_lo + kBN - 1) / kBN;
  const int nblocks = nb_pre + nb_win;
  auto block_of = [&](int bi) -> Block {
    if (bi < nb_pre) return {bi * kBN, pre_hi, false};
    return {win_lo + (bi - nb_pre) * kBN, win_hi, true};
  };

  // This wave's 32 queries; lane l owns query qi.
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const bool q_ok = qi < N;
  bf16x8_t qf[kD / 16];
  {
    const uint16_t *qrow = Qg + (int64_t)(q_ok ? qi : 0) * row_stride;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const u32x4_t u = q_ok ? *reinterpret_cast<const u32x4_t *>(qrow + ks * 16 + hi * 8)
                             : u32x4_t{0, 0, 0, 0};
      qf[ks] = as_bf16x8(u);
    }
  }

  f32x16_t o[kD / 32];
#pragma unroll
  for (int j = 0; j < kD / 32; ++j) o[j] = f32x16_t{};
  float m = kNegInf;  // running max (raw scores) used for exponentiation
  float l = 0.f;      // this lane's part of the row sum

  // Staging: thread t loads keys u + 16 i (i < kRpt), u = t >> 4, 16-byte
  // column chunk c = t & 15, of K and V.
  const int su = tid >> 4, sc = tid & 15;
  u32x4_t kst[kRpt], vst[kRpt];
  auto load_block = [&](const Block &bk) {
#pragma unroll
    for (int i = 0; i < kRpt; ++i) {
      int r = bk.kb0 + su + 16 * i;
      r = r < bk.kend ? r : bk.kend - 1;
      kst[i] = *reinterpret_cast<const u32x4_t *>(Kg + (int64_t)r * row_stride + sc * 8);
      vst[i] = *reinterpret_cast<const u32x4_t *>(Vg + (int64_t)r * row_stride + sc * 8);
    }
  };
  auto store_block = [&](Buf &b) {
#pragma unroll
    for (int i = 0; i < kRpt; ++i)
      *reinterpret_cast<u32x4_t *>(&b.k[(kRpt * su + i) * kKPitch + sc * 8]) = kst[i];
    const u32x4_t *v = vst;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      // d = 8 sc + 2 k2 (low halves) and d + 1 (high halves) of keys u + 16 i
      const int d = sc * 8 + 2 * k2;
      if constexpr (kRpt == 4) {
        const u32x2_t even = {__builtin_amdgcn_perm(v[1][k2], v[0][k2], 0x05040100u),
                              __builtin_amdgcn_perm(v[3][k2], v[2][k2], 0x05040100u)};
        const u32x2_t odd = {__builtin_amdgcn_perm(v[1][k2], v[0][k2], 0x07060302u),
                             __builtin_amdgcn_perm(v[3][k2], v[2][k2], 0x07060302u)};
        *reinterpret_cast<u32x2_t *>(&b.vt[d * kVPitch + kRpt * su]) = even;
        *reinterpret_cast<u32x2_t *>(&b.vt[(d + 1) * kVPitch + kRpt * su]) = odd;
      } else {
        *reinterpret_cast<uint32_t *>(&b.vt[d * kVPitch + kRpt * su]) =
            __builtin_amdgcn_perm(v[1][k2], v[0][k2], 0x05040100u);
        *reinterpret_cast<uint32_t *>(&b.vt[(d + 1) * kVPitch + kRpt * su]) =
            __builtin_amdgcn_perm(v[1][k2], v[0][k2], 0x07060302u);
      }
    }
  };

  const float c = p.scale_log2;
  if (nblocks > 0) {
    load_block(block_of(0));
    store_block(sm[0]);
  }
  for (int bi = 0; bi < nblocks; ++bi) {
    const Block bk = block_of(bi);
    __syncthreads();  // sm[bi & 1] is complete; sm[(bi + 1) & 1] is no longer read
    const bool has_next = bi + 1 < nblocks;
    if (has_next) load_block(block_of(bi + 1));
    const Buf &b = sm[bi & 1];

    // S^T tiles: kBN / 32 x (32 keys x 32 queries)
    constexpr int kTiles = kBN / 32;
    f32x16_t s[kTiles];
#pragma unroll
    for (int kt = 0; kt < kTiles; ++kt) {
      s[kt] = f32x16_t{};
      const uint16_t *krow = &b.k[(kt * 32 + l32) * kKPitch + hi * 8];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t *>(krow + ks * 16));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kt], 0, 0, 0);
      }
    }

    // Does this block cut the mask for any query of the wave? (wave-uniform)
    const bool partial = bk.kb0 + kBN > bk.kend;
    const bool diag = !full_prefix && qw0 < Lm && qw0 < bk.kb0 + kBN - 1;
    if (bk.window || partial || diag) {
      // Accumulator element r of tile kt is LDS row rho = 32 kt + 8 (r/4) + 4 hi + r%4.
#pragma unroll
      for (int kt = 0; kt < kTiles; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rho = kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const int j = bk.kb0 + key_of_row(rho);
          bool vis = j < bk.kend;
          if (bk.window) {
            vis = vis && j <= qi && qi - j < n;
          } else {
            vis = vis && (qi >= Lm || full_prefix || j <= qi);
          }
          s[kt][r] = vis ? s[kt][r] : kNegInf;
        }
      }
    }

    float bmax = kNegInf;
#pragma unroll
    for (int kt = 0; kt < kTiles; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[kt][r]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    // Raise the exponentiation max only when a score exceeds it by > 2^8.
    const bool raise = bmax != kNegInf && (m == kNegInf || (bmax - m) * c > kRescaleThreshold);
    if (__ballot(raise) != 0) {
      const float m_new = fmaxf(m, bmax);
      const float alpha = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < kD / 32; ++j) o[j] *= alpha;
      m = m_new;
    }
    const float mc = (m == kNegInf) ? 0.f : m * c;

    // P^T as bf16 B operands: step (kt, half) uses accumulator elements
    // 8 half .. 8 half + 7 (LDS rows 32 kt + 16 half + {4 hi.., 8 + 4 hi..}).
    bf16x8_t pb[2 * kTiles];
#pragma unroll
    for (int kt = 0; kt < kTiles; ++kt) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * half + 2 * e], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * half + 2 * e + 1], c, -mc));
          l += p0 + p1;
          w4[e] = pack_bf16(p0, p1);
        }
        pb[2 * kt + half] = as_bf16x8(u32x4_t{w4[0], w4[1], w4[2], w4[3]});
      }
    }

    // O^T[d][q] += V^T[d][rho] P^T[rho][q]
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
      const uint16_t *vrow = &b.vt[(db * 32 + l32) * kVPitch + 4 * hi];
#pragma unroll
      for (int st = 0; st < 2 * kTiles; ++st) {
        const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow + 16 * st);
        const u32x2_t hi8 = *reinterpret_cast<const u32x2_t *>(vrow + 16 * st + 8);
        const bf16x8_t a = as_bf16x8(u32x4_t{lo.x, lo.y, hi8.x, hi8.y});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[db], 0, 0, 0);
      }
    }

    if (has_next) store_block(sm[(bi + 1) & 1]);
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
      const u32x2_t w2 = {pack_bf16(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv),
                          pack_bf16(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
      *reinterpret_cast<u32x2_t *>(orow + d0) = w2;
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
