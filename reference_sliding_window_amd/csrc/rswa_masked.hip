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
//  * K and V blocks go from global memory straight into LDS by DMA
//    (global_load_lds_dwordx4), double buffered: the next block is in flight
//    while the current one is multiplied; one barrier per block. Tiles are
//    row-major with 256-byte rows and XOR-swizzled 16-byte chunks, so the
//    fragment reads below are free of bank conflicts.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K fragments
//    from LDS as the A operand, the wave's Q rows resident in VGPRs as the B
//    operand), so lane l owns query l % 32: the softmax row max and sum are
//    in-register plus one exchange with lane l ^ 32.
//  * O^T += V^T P^T reuses the S^T accumulators as the B operand after the
//    exp2 and the packed bf16 convert, one 16-key step at a time; the V^T A
//    operand comes from the row-major V tile through transposing LDS reads
//    (ds_read_b64_tr_b16, two per operand).
//  * Softmax in base 2 with the scale folded into one FMA before exp2. The
//    running max used for exponentiation is only raised (and O, l rescaled)
//    when a block's max exceeds it by more than 8 (a factor 2^8), which keeps
//    every probability below 2^8 and skips most rescales. The row sum is
//    taken with v_dot2 over the same bf16 probabilities that enter PV.
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
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleThreshold = 8.f;  // log2 units
constexpr int kRowBytes = kD * 2;         // 256-byte K and V rows in LDS, no padding

// K and V blocks, row-major, rows = LDS key rows; 16-byte chunks swizzled (see chunk_swz).
struct Buf {
  uint16_t k[kBN * kD];
  uint16_t v[kBN * kD];
};

// Physical 16-byte chunk of logical chunk c in row r: c ^ (4 (r mod 4) + (r / 4) mod 4).
// Eight consecutive rows read at one chunk (K fragments) and four consecutive rows
// read at four neighbouring chunks (transposing V reads) then hit distinct banks.
__device__ __forceinline__ int chunk_swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ constexpr bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
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
      const int j = kb0 + rho;
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

  // Global -> LDS by DMA (global_load_lds_dwordx4: lane L's 16 bytes land at the
  // wave-uniform LDS base + 16 L). Wave w fills rows 16 w .. 16 w + 15 of the K and
  // V tiles with 4 instructions each; instruction j covers rows 16 w + 4 j + L / 16,
  // physical chunk L % 16, i.e. logical chunk (L % 16) ^ chunk_swz(row).
  // Element offsets fit in 32 bits (the host rejects tensors of 2^31 elements or more).
  const uint32_t stride32 = (uint32_t)row_stride;
  int dma_row[4];
  uint32_t dma_col[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    dma_row[j] = 16 * wave + 4 * j + (lane >> 4);
    dma_col[j] = 8u * (uint32_t)((lane & 15) ^ chunk_swz(dma_row[j]));
  }
  auto dma_block = [&](const Block &bk, Buf &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = min(bk.kb0 + dma_row[j], bk.kend - 1);
      const uint32_t off = __umul24((uint32_t)r, stride32) + dma_col[j];
      char *kdst = reinterpret_cast<char *>(b.k) + (16 * wave + 4 * j) * kRowBytes;
      char *vdst = reinterpret_cast<char *>(b.v) + (16 * wave + 4 * j) * kRowBytes;
      __builtin_amdgcn_global_load_lds(Kg + off, (lds_void_t *)kdst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Vg + off, (lds_void_t *)vdst, 16, 0, 0);
    }
  };
  // K fragment of step ks for S^T tile 0: row l32, logical chunk 2 ks + hi.
  uint32_t koff[kD / 16];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks)
    koff[ks] = l32 * kRowBytes + 16 * ((2 * ks + hi) ^ chunk_swz(l32));
  // Transposing V reads: the A operand of 16-key step st and d block db is two
  // ds_read_b64_tr_b16. In each, lane s addresses row 16 st + 8 h2 + 4 (G / 2) + e,
  // d = 32 db + 16 (G % 2) + 4 q (G = s / 16, e = s / 4 mod 4, q = s mod 4) and
  // lane i of each 16-lane group receives d = 32 db + l % 32 of the four rows
  // base + e; the row-dependent part of the swizzle does not depend on st.
  uint32_t voff[kD / 32][2];
  {
    const int G = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int row = 8 * h2 + 4 * (G >> 1) + e;
        const int chunk = (4 * db + 2 * (G & 1) + (q >> 1)) ^ chunk_swz(row);
        voff[db][h2] = row * kRowBytes + 16 * chunk + 8 * (q & 1);
      }
  }

  const float c = p.scale_log2;
  if (nblocks > 0) dma_block(block_of(0), sm[0]);

  // One key block. kMode 0: no key of the block is hidden from any query of
  // the wave; 1: prefix block that cuts the mask (partial block, or the causal
  // diagonal of prefix rows); 2: window block.
  auto body = [&](int bi, auto mode) {
    constexpr int kMode = decltype(mode)::value;
    const Block bk = block_of(bi);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's DMA into sm[bi & 1] landed
    __syncthreads();  // sm[bi & 1] is complete; sm[(bi + 1) & 1] is no longer read
    const bool has_next = bi + 1 < nblocks;
    if (has_next) dma_block(block_of(bi + 1), sm[(bi + 1) & 1]);
    const Buf &b = sm[bi & 1];
    // let the scheduler interleave the LDS fragment reads with the MFMAs
    __builtin_amdgcn_iglp_opt(0);
    const char *kb = reinterpret_cast<const char *>(b.k);
    const char *vb = reinterpret_cast<const char *>(b.v);

    // S^T tiles: kTiles x (32 keys x 32 queries)
    f32x16_t s[kTiles];
#pragma unroll
    for (int kt = 0; kt < kTiles; ++kt) {
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8_t a = as_bf16x8(
            *reinterpret_cast<const u32x4_t *>(kb + koff[ks] + kt * 32 * kRowBytes));
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
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t *)(vb + voff[db][0] + 16 * st * kRowBytes));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t *)(vb + voff[db][1] + 16 * st * kRowBytes));
        const u32x2_t a0 = __builtin_bit_cast(u32x2_t, v0), a1 = __builtin_bit_cast(u32x2_t, v1);
        const bf16x8_t a = as_bf16x8(u32x4_t{a0.x, a0.y, a1.x, a1.y});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
      }
    }

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
  if (p.lse != nullptr && hi == 0)  // natural log of sum_j 2^(c s_j) = (c m + log2 l) ln 2
    p.lse[(int64_t)h * N + qi] = (m * c + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
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
