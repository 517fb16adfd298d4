// Packed (teacher-forced) R-SWA forward on gfx950 matrix cores.
//
// Row i of a packed sequence attends to key j iff j <= i and (j < L_m or
// i - j < n): for an output row this is N(t) = P ∪ D_n(t) of WeThinkIn
// "Unlimited OCR Works：一篇读懂 R-SWA…", section 方法展开.3, Eqs. (1)-(2), for
// the query formed at position i; prefix rows (not covered by Eq. (1)) are
// causal, or see the whole prefix in RSWA_PREFIX_FULL mode. Softmax and the
// weighted sum follow Eqs. (3)-(4).
//
// Design (one workgroup = 128 query rows of one head, 4 waves x 32 rows,
// two workgroups per CU):
//  * Only the 64-key blocks that intersect the two-segment mask are visited:
//    the prefix range [0, min(L_m, q_end)) and the window range
//    [max(L_m, first_output_row - n + 1), q_end). Each wave runs three loops:
//    prefix blocks that hide no key from any of its queries (no mask code at
//    all), prefix blocks that cut the mask (partial block, causal diagonal of
//    prefix rows), and window blocks.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as the A operand, the wave's Q rows resident in VGPRs as the B operand),
//    so lane l owns query l % 32: the softmax row max and sum are in-register
//    plus one exchange with lane l ^ 32.
//  * O^T += V^T P^T reuses the S^T accumulators as the B operand after the
//    exp2 and the packed bf16 convert, one 16-key step at a time, so that the
//    MFMAs of one step overlap the exponentials of the next.
//  * Keys sit in LDS in a permuted order: LDS row rho of a block holds key
//    rho / 4 + 16 (rho mod 4), so a thread that loads the coalesced rows
//    u, u+16, u+32, u+48 writes them as one 8-byte word of V^T per d. Inside
//    a V^T row, bits 2 and 3 of rho are swapped (the 8 keys an MFMA lane
//    needs per step become 16 contiguous bytes) and bits 4-5 are XOR-ed with
//    (d >> 5) to spread the transposing stores over the LDS banks. The
//    contraction over keys does not depend on their order; the mask uses the
//    true key index.
//  * Softmax in base 2 with the scale folded into one FMA before exp2. The
//    running max used for exponentiation is only raised (and O, l rescaled)
//    when a block's max exceeds it by more than 8 (a factor 2^8), which keeps
//    every probability below 2^8 and skips most rescales. The row sum is
//    taken with v_dot2 over the same bf16 probabilities that enter PV.
//  * LDS is double buffered: the next block's global loads are issued before
//    the current block's MFMAs and written to the other buffer after them;
//    one barrier per block.
//  * Workgroups are ordered so that all query blocks of a head run on the same
//    XCD (hardware places workgroup i on XCD i mod 8), keeping that head's
//    prefix K/V resident in the XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

constexpr int kD = 128;           // head dim
constexpr int kBM = 128;          // query rows per workgroup
constexpr int kBN = 64;           // keys per block
constexpr int kTiles = kBN / 32;  // 32-key S^T tiles per block
constexpr int kKPitch = kD + 8;   // LDS row pitch of K (elements)
constexpr int kVPitch = kBN + 8;  // LDS row pitch of V^T (elements; rows stay 16-byte aligned)
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleThreshold = 8.f;  // log2 units

struct Buf {
  uint16_t k[kBN * kKPitch];   // K block, [rho][d]
  uint16_t vt[kD * kVPitch];   // V block transposed, [d][vt_col]
};

__device__ constexpr bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// true key offset (within the block) of LDS row rho
__device__ __forceinline__ int key_of_row(int rho) { return (rho >> 2) + 16 * (rho & 3); }

// Physical V^T column of LDS key row rho in row d (see the header comment).
__device__ __forceinline__ int vt_col(int d, int rho) {
  const int swapped = (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
  return swapped ^ (16 * ((d >> 5) & 3));
}

// Sets to -inf the scores of keys the two-segment mask hides from query qi.
// Accumulator element r of tile kt is LDS row rho = 32 kt + 8 (r/4) + 4 hi + r%4.
template <bool kWindow>
__device__ __forceinline__ void apply_mask(f32x16_t (&s)[kTiles], int kb0, int kend, int qi, int n,
                                           bool sees_prefix, int hi) {
#pragma unroll
  for (int kt = 0; kt < kTiles; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rho = kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const int j = kb0 + key_of_row(rho);
      const bool vis = kWindow ? (j < kend && j <= qi && qi - j < n)
                               : (j < kend && (sees_prefix || j <= qi));
      s[kt][r] = vis ? s[kt][r] : kNegInf;
    }
  }
}

struct Block {
  int kb0;   // first key of the block
  int kend;  // end of the key range the block belongs to
};

__global__ __launch_bounds__(256, 2) void masked_attn_kernel(MaskedParams p) {
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
    if (bi < nb_pre) return {bi * kBN, pre_hi};
    return {win_lo + (bi - nb_pre) * kBN, win_hi};
  };

  // This wave's 32 queries; lane l owns query qi.
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const bool q_ok = qi < N;
  const bool sees_prefix = qi >= Lm || full_prefix;  // every prefix key is visible
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

  // Staging: thread t loads keys u + 16 i (i = 0..3), u = t >> 4, 16-byte
  // column chunk c = t & 15, of K and V. Element offsets fit in 32 bits (the
  // host rejects tensors of 2^31 elements or more).
  const int su = tid >> 4, sc = tid & 15;
  const uint32_t stride32 = (uint32_t)row_stride;
  u32x4_t kst[4], vst[4];
  auto load_block = [&](const Block &bk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = min(bk.kb0 + su + 16 * i, bk.kend - 1);
      const uint32_t off = __umul24((uint32_t)r, stride32) + sc * 8;
      kst[i] = *reinterpret_cast<const u32x4_t *>(Kg + off);
      vst[i] = *reinterpret_cast<const u32x4_t *>(Vg + off);
    }
  };
  const int vcol = vt_col(sc * 8, 4 * su);  // same for all 8 d of the thread's chunk
  auto store_block = [&](Buf &b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t *>(&b.k[(4 * su + i) * kKPitch + sc * 8]) = kst[i];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      // d = 8 sc + 2 k2 (low halves) and d + 1 (high halves) of keys u + 16 i
      const int d = sc * 8 + 2 * k2;
      const u32x2_t even = {__builtin_amdgcn_perm(vst[1][k2], vst[0][k2], 0x05040100u),
                            __builtin_amdgcn_perm(vst[3][k2], vst[2][k2], 0x05040100u)};
      const u32x2_t odd = {__builtin_amdgcn_perm(vst[1][k2], vst[0][k2], 0x07060302u),
                           __builtin_amdgcn_perm(vst[3][k2], vst[2][k2], 0x07060302u)};
      *reinterpret_cast<u32x2_t *>(&b.vt[d * kVPitch + vcol]) = even;
      *reinterpret_cast<u32x2_t *>(&b.vt[(d + 1) * kVPitch + vcol]) = odd;
    }
  };

  const float c = p.scale_log2;
  if (nblocks > 0) {
    load_block(block_of(0));
    store_block(sm[0]);
  }

  // One key block. kMode 0: no key of the block is hidden from any query of
  // the wave; 1: prefix block that cuts the mask (partial block, or the causal
  // diagonal of prefix rows); 2: window block.
  auto body = [&](int bi, auto mode) {
    constexpr int kMode = decltype(mode)::value;
    const Block bk = block_of(bi);
    __syncthreads();  // sm[bi & 1] is complete; sm[(bi + 1) & 1] is no longer read
    const bool has_next = bi + 1 < nblocks;
    if (has_next) load_block(block_of(bi + 1));
    const Buf &b = sm[bi & 1];

    // S^T tiles: kTiles x (32 keys x 32 queries)
    f32x16_t s[kTiles];
#pragma unroll
    for (int kt = 0; kt < kTiles; ++kt) {
      const uint16_t *krow = &b.k[(kt * 32 + l32) * kKPitch + hi * 8];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t *>(krow + ks * 16));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? f32x16_t{} : s[kt],
                                                        0, 0, 0);
      }
    }
    if constexpr (kMode == 1) apply_mask<false>(s, bk.kb0, bk.kend, qi, n, sees_prefix, hi);
    if constexpr (kMode == 2) apply_mask<true>(s, bk.kb0, bk.kend, qi, n, sees_prefix, hi);

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

    // Per 16-key step st = 2 kt + half: P^T as a bf16 B operand from accumulator
    // elements 8 half .. 8 half + 7 of tile kt (LDS rows 32 kt + 16 half +
    // {4 hi.., 8 + 4 hi..}), then O^T[d][q] += V^T[d][rho] P^T[rho][q] for the
    // four 32-row d blocks.
#pragma unroll
    for (int st = 0; st < 2 * kTiles; ++st) {
      const int kt = st >> 1, half = st & 1;
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * half + 2 * e], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * half + 2 * e + 1], c, -mc));
        w4[e] = pack_bf16(p0, p1);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4[e]), kOnes, l, false);
      }
      const bf16x8_t pb = as_bf16x8(u32x4_t{w4[0], w4[1], w4[2], w4[3]});
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) {
        // vt_col(d, 16 st + 4 hi) = (16 st ^ 16 db) + 8 hi for every d of this
        // d block: one 16-byte read at a compile-time offset from a lane base
        const uint16_t *vrow = &b.vt[(db * 32 + l32) * kVPitch + 8 * hi];
        const bf16x8_t a =
            as_bf16x8(*reinterpret_cast<const u32x4_t *>(vrow + ((16 * st) ^ (16 * db))));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
      }
    }

    if (has_next) store_block(sm[(bi + 1) & 1]);
  };

  // Prefix blocks [0, nb_clear) hide no key from any query of this wave: they
  // are whole and, for causal prefix rows, lie left of the wave's diagonal.
  // Different waves may split differently; every wave still runs nblocks
  // iterations, hence the same barriers.
  int nb_clear = pre_hi / kBN;
  if (!full_prefix && qw0 < Lm) nb_clear = min(nb_clear, (qw0 + 1) / kBN);
  // Drain every outstanding load (the Q fragments among them) before the loop,
  // so that the loop's waits only cover the block prefetch.
  __builtin_amdgcn_s_waitcnt(0);
  int bi = 0;
  for (; bi < nb_clear; ++bi) body(bi, std::integral_constant<int, 0>{});
  for (; bi < nb_pre; ++bi) body(bi, std::integral_constant<int, 1>{});
  for (; bi < nblocks; ++bi) body(bi, std::integral_constant<int, 2>{});

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
