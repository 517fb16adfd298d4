// Packed (teacher-forced) R-SWA forward on gfx950 matrix cores.
//
// Row i of a packed sequence attends to key j iff j <= i and (j < L_m or
// i - j < n): for an output row this is N(t) = P ∪ D_n(t) of WeThinkIn
// "Unlimited OCR Works：一篇读懂 R-SWA…", section 方法展开.3, Eqs. (1)-(2), for
// the query formed at position i; prefix rows (not covered by Eq. (1)) are
// causal, or see the whole prefix in RSWA_PREFIX_FULL mode. Softmax and the
// weighted sum follow Eqs. (3)-(4).
//
// Design (one workgroup = 128 query rows of one head, 4 waves x 32 rows, two
// independent workgroups per CU, so that one's VALU work overlaps the other's
// matrix products):
//  * Only the 64-key blocks that intersect the two-segment mask are visited:
//    the prefix range [0, min(L_m, q_end)) and the window range
//    [max(L_m, first_output_row - n + 1), q_end). Inside a block the keys a
//    row sees form one interval, so masking is one unsigned compare per score,
//    and only in blocks that cut some row's interval.
//  * K and V blocks go from global memory straight into LDS by DMA
//    (global_load_lds_dwordx4) through two-stage rings, one for K and one for
//    V: while block bi's V is multiplied, block bi + 1's K is multiplied, and
//    K of block bi + 2 and V of block bi + 1 are in flight (a full block of
//    lead); one barrier per block. Tiles are row-major with 256-byte rows and
//    XOR-swizzled 16-byte chunks, so the fragment reads are free of bank
//    conflicts.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K fragments
//    from LDS as the A operand, the wave's Q rows resident in VGPRs as the B
//    operand), so lane l owns query l % 32: the softmax row max and sum are
//    in-register plus one exchange with lane l ^ 32 (v_permlane32_swap).
//  * Software pipeline: the S^T products of block bi + 1 are issued next to the
//    exp2 / convert / row-sum work of block bi, then O^T += V^T P^T for block
//    bi takes the packed bf16 probabilities as the B operand and V^T from
//    transposing LDS reads (ds_read_b64_tr_b16, two per operand). The
//    compiler's schedule is kept: with two workgroups per CU it measured a
//    little faster than a hand-fixed order.
//  * Softmax in base 2 with the scale folded into one FMA before exp2. A
//    block's probabilities are formed against the running max as it stands,
//    with no max taken first: only when some lane's share of the block's
//    probabilities sums above 2^15 or is not finite (always the case while a
//    row has no max yet) does the block take the row max, raise the running
//    max, rescale O and l, and form its probabilities again. Every probability
//    that enters PV is thus at most 2^15. The row sum is taken with v_dot2 over
//    the same bf16 probabilities that enter PV.
//  * Workgroups are ordered so that all query blocks of a head run on the same
//    XCD (hardware places workgroup i on XCD i mod 8), keeping that head's
//    prefix K/V resident in the XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rswa_internal.h"
#include "rswa_tile.h"

namespace rswa {
namespace {

using namespace tile;

constexpr int kWaves = 4;                 // waves per workgroup, 32 query rows each
constexpr int kBM = 32 * kWaves;          // query rows per workgroup
constexpr int kBN = 64;                   // keys per block
constexpr int kTiles = kBN / 32;          // 32-key S^T tiles per block
constexpr float kSumHi = 32768.f;  // a lane's block sum above this raises the running max

typedef uint16_t Tile[kBN * kD];  // one 64-row K or V block

__global__ __launch_bounds__(64 * kWaves, 2) void masked_attn_kernel(MaskedParams p) {
  __shared__ Tile k_sm[2], v_sm[2];
  const int H = p.heads, n = p.window;
  const bool full_prefix = p.prefix_mode == RSWA_PREFIX_FULL;
  const int nqb = max(1, (p.max_seq_len + kBM - 1) / kBM);
  const int G = p.num_seqs * H * nqb;
  // XCD-aware order: logical work item w -> (head, sample, query block). An XCD
  // takes a contiguous range of w: the query blocks of one (sample, head) share
  // its L2, and with heads outermost every XCD gets the same heads of every
  // sample, so samples of different sizes do not unbalance the XCDs. Within a
  // (sample, head) the last query block comes first: with a causal prefix the
  // later blocks see the most keys, and the cheap prefix blocks then fill the
  // tail of the launch.
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int h = w / (p.num_seqs * nqb);
  const int sample = (w / nqb) % p.num_seqs;
  const int q0 = (nqb - 1 - w % nqb) * kBM;
  // One sample of the pack: rows [row0, row0 + N) with its own reference
  // length; no row sees another sample's keys.
  int row0 = 0, N = p.seq_len, Lm = p.ref_len;
  bool handoff = false;
  if (p.cu_seqlens != nullptr) {
    row0 = p.cu_seqlens[sample];
    const int row1 = p.cu_seqlens[sample + 1];
    Lm = p.ref_lens[sample];
    N = row1 - row0;
    const bool pack_bad = row0 < 0 || row1 < row0 || row1 > p.seq_len || N > p.max_seq_len || Lm > N;
    if (p.cache_k != nullptr) {
      // Prefill hand-off: the per-sequence checks of the cache calls; one
      // workgroup of the sequence (head 0, work item 0 of its query blocks)
      // publishes step[b] = T0 or the error.
      int err = pack_bad ? RSWA_DEVERR_PACK : 0;
      if (Lm < 0 || Lm > p.max_ref_len) err |= RSWA_DEVERR_REF_LEN;
      const int64_t cb = p.seq_base[sample];
      if (cb < 0 || (cb & 7) != 0) err |= RSWA_DEVERR_ALIGN;
      if (w % nqb == 0 && h == 0 && threadIdx.x == 0) {
        if (err != 0) {
          atomicOr(p.error, err);
        } else {
          p.step[sample] = N - Lm;
          if (p.arrive != nullptr) p.arrive[sample] = 0;
        }
      }
      handoff = err == 0;
    }
    // device-side metadata: a malformed sample is skipped
    if (pack_bad || Lm < 0) return;
  }
  if (q0 >= N) return;
  const int q_end = min(N, q0 + kBM);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const uint32_t stride = (uint32_t)H * kD;
  const int64_t base = (int64_t)row0 * stride + (int64_t)h * kD;
  const uint16_t *Qg = static_cast<const uint16_t *>(p.q) + base;
  const uint16_t *Kg = static_cast<const uint16_t *>(p.k) + base;
  const uint16_t *Vg = static_cast<const uint16_t *>(p.v) + base;
  uint16_t *Og = static_cast<uint16_t *>(p.out) + base;

  // Key blocks: the reference segment [0, pre_hi), then the output keys
  // [win_lo, win_hi) some row of this workgroup sees.
  const int pre_hi = (full_prefix && q0 < Lm) ? Lm : min(Lm, q_end);
  const int win_lo = max(Lm, max(q0, Lm) - n + 1);
  const int win_hi = q_end > Lm ? q_end : win_lo;
  const int nb_pre = (pre_hi + kBN - 1) / kBN;
  const int nblocks = nb_pre + (win_hi - win_lo + kBN - 1) / kBN;
  auto kb0_of = [&](int bi) __attribute__((always_inline)) {
    return bi < nb_pre ? bi * kBN : win_lo + (bi - nb_pre) * kBN;
  };
  auto kend_of = [&](int bi) __attribute__((always_inline)) { return bi < nb_pre ? pre_hi : win_hi; };

  // This wave's 32 queries; lane l owns query qi.
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const bool q_ok = qi < N;
  bf16x8_t qf[kD / 16];
  {
    const int64_t r = (int64_t)(q_ok ? qi : 0) * stride;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const u32x4_t zero = {0, 0, 0, 0};
      qf[ks] = as_bf16x8(q_ok ? *reinterpret_cast<const u32x4_t *>(Qg + r + ks * 16 + hi * 8) : zero);
    }
  }

  // The keys row qi sees inside each segment form one interval [lo, lo + span):
  // the reference segment up to L_m (or up to the row itself for a causal row
  // below L_m), and the n output keys ending at the row.
  const uint32_t span_p = (uint32_t)((full_prefix || qi >= Lm) ? Lm : qi + 1);
  const int lo_w = max(Lm, qi - n + 1);
  const uint32_t span_w = (uint32_t)max(0, qi + 1 - lo_w);
  // Reference-segment blocks no row of this wave masks. Waves may differ; each
  // still runs every block, hence the same barriers.
  const int nb_clear = min((!full_prefix && qw0 < Lm) ? qw0 + 1 : Lm, pre_hi) / kBN;

  f32x16_t o[kD / 32];
#pragma unroll
  for (int j = 0; j < kD / 32; ++j) o[j] = f32x16_t{};
  float m = kNegInf;  // running max (raw scores) used for exponentiation
  float l = 0.f;      // this lane's part of the row sum
  const float c = p.scale_log2;

  uint32_t koff[kD / 16], toff[kD / 32][2];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) koff[ks] = row_frag_off(l32, hi, ks);
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
    toff[db][0] = tr_off(lane, db, 0);
    toff[db][1] = tr_off(lane, db, 1);
  }

  // DMA of one 64-row K or V block: wave w fills rows 16 w .. 16 w + 15, 4
  // instructions per wave. The tensor's base stays in scalar registers; each
  // lane adds the byte offset of its row (clamped to the segment's last row)
  // and of its swizzled 16-byte chunk, which is fixed for the kernel. Byte
  // offsets fit in 32 bits and the row product in the 24-bit multiplier (the
  // host rejects tensors of 2^31 elements or more and 2^16 heads or more).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t c16[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c16[j] = 16u * (uint32_t)((lane & 15) ^ chunk_swz(16 * wave + 4 * j + (lane >> 4)));
  const uint32_t stride2 = 2u * stride;
  const uint32_t k_lds[2] = {lds_addr(&k_sm[0][0]), lds_addr(&k_sm[1][0])};
  const uint32_t v_lds[2] = {lds_addr(&v_sm[0][0]), lds_addr(&v_sm[1][0])};
  uint32_t c16r[4];  // instruction j: its chunk offset plus its 4 j rows
#pragma unroll
  for (int j = 0; j < 4; ++j) c16r[j] = c16[j] + 4u * (uint32_t)j * stride2;
  auto dma_tile = [&](const uint16_t *src, int bi, uint32_t t_lds) __attribute__((always_inline)) {
    const int kb0 = kb0_of(bi), kend = kend_of(bi);
    if (kb0 + kBN <= kend) {  // a whole block: one row product per lane
      const uint32_t rb = __umul24((uint32_t)(kb0 + 16 * wv + (lane >> 4)), stride2);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16(src, rb + c16r[j], t_lds + (uint32_t)((16 * wv + 4 * j) * kRowBytes));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row0 = 16 * wv + 4 * j;
        const uint32_t r = (uint32_t)min(kb0 + row0 + (lane >> 4), kend - 1);
        dma16(src, __umul24(r, stride2) + c16[j], t_lds + (uint32_t)(row0 * kRowBytes));
      }
    }
  };

  // S^T = K Q^T of the block in K stage ks_stage, two 32-key tiles: element r of
  // tile kt is key kb0 + 32 kt + 8 (r/4) + 4 hi + r%4 of that block, query qi.
  auto qk = [&](const Tile &kt_sm, f32x16_t (&s)[kTiles]) __attribute__((always_inline)) {
    const char *kb = reinterpret_cast<const char *>(kt_sm);
#pragma unroll
    for (int kt = 0; kt < kTiles; ++kt)
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8_t ka = as_bf16x8(*reinterpret_cast<const u32x4_t *>(kb + koff[ks] + kt * 32 * kRowBytes));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16_t{} : s[kt], 0, 0, 0);
      }
  };

  // One pipeline step for block bi (P = bi & 1), its S^T computed the step
  // before: wait for K of block bi + 1 and V of block bi, start the DMA of K of
  // block bi + 2 and V of block bi + 1, mask, then the S^T products of block
  // bi + 1 next to this block's exp2 / convert / row sum, then O^T += V^T P^T.
  auto step = [&](int bi, auto parity, f32x16_t (&s_cur)[kTiles], f32x16_t (&s_nxt)[kTiles])
      __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    wait_vmcnt<0>();  // everything issued one step ago landed
    block_barrier();  // for every wave; K stage P and V stage 1 - P are free
    if (bi + 2 < nblocks) dma_tile(Kg, bi + 2, k_lds[P]);
    if (bi + 1 < nblocks) dma_tile(Vg, bi + 1, v_lds[1 - P]);
    float xs[kTiles * 16];
#pragma unroll
    for (int kt = 0; kt < kTiles; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[16 * kt + r] = s_cur[kt][r];
    if (bi >= nb_clear) {
      const bool win = bi >= nb_pre;
      const uint32_t t = (uint32_t)(kb0_of(bi) + 4 * hi - (win ? lo_w : 0));
      const uint32_t span = win ? span_w : span_p;
#pragma unroll
      for (int e = 0; e < kTiles * 16; ++e) {
        const int kt = e >> 4, r = e & 15;
        xs[e] = t + (uint32_t)(32 * kt + 8 * (r >> 2) + (r & 3)) < span ? xs[e] : kNegInf;
      }
    }
    // Probabilities against the running max as it stands (m = -inf, before the
    // row has a max, gives non-finite ones and so the rare path below).
    const float mc = m * c;
    // S^T of block bi + 1 (a stale stage after the last block; result unused),
    // K fragments two products ahead; two probabilities per product.
    const char *kn = reinterpret_cast<const char *>(k_sm[1 - P]);
    constexpr int kSteps = kTiles * (kD / 16);
    bf16x8_t ka[kSteps];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ka[i] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(kn + koff[i % 8] + (i / 8) * 32 * kRowBytes));
    uint32_t pw[kTiles * 8];
    float lb = 0.f;  // this lane's share of the block's probabilities
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int kt = i / 8, ks = i % 8;
      if (i + 2 < kSteps)
        ka[i + 2] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(kn + koff[(i + 2) % 8] + ((i + 2) / 8) * 32 * kRowBytes));
      s_nxt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qf[ks], ks == 0 ? f32x16_t{} : s_nxt[kt], 0, 0, 0);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(xs[2 * i], c, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(xs[2 * i + 1], c, -mc));
      pw[i] = pack_bf16(p0, p1);
      lb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]), kOnes, lb, false);
    }
    if (__ballot(!(lb <= kSumHi)) != 0) {
      // Rare: raise the running max to the block's row max, rescale O and l,
      // and form the block's probabilities again.
      float bmax = xs[0];
#pragma unroll
      for (int e = 1; e < kTiles * 16; ++e) bmax = fmaxf(bmax, xs[e]);
      bmax = swap_halves_max(bmax);
      const float m_new = fmaxf(m, bmax);
      const float alpha = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < kD / 32; ++j) o[j] *= alpha;
      m = m_new;
      const float mc2 = (m == kNegInf) ? 0.f : m * c;
      lb = 0.f;
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(xs[2 * i], c, -mc2));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(xs[2 * i + 1], c, -mc2));
        pw[i] = pack_bf16(p0, p1);
        lb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]), kOnes, lb, false);
      }
    }
    l += lb;
    // O^T[d][q] += V^T[d][key] P^T[key][q] over 16-key steps stp (elements
    // 8 (stp%2) .. + 7 of tile stp/2 = pw[4 stp .. 4 stp + 3]); transposing V
    // reads one product ahead.
    const char *vb = reinterpret_cast<const char *>(v_sm[P]);
    constexpr int kPv = 2 * kTiles * (kD / 32);
    bf16x8_t tv[2];
    tv[0] = tr_operand(vb, toff[0][0], toff[0][1], 0);
#pragma unroll
    for (int j = 0; j < kPv; ++j) {
      const int stp = j >> 2, db = j & 3;
      if (j + 1 < kPv) tv[(j + 1) & 1] = tr_operand(vb, toff[(j + 1) & 3][0], toff[(j + 1) & 3][1], (j + 1) >> 2);
      const bf16x8_t pb = as_bf16x8(u32x4_t{pw[4 * stp], pw[4 * stp + 1], pw[4 * stp + 2], pw[4 * stp + 3]});
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tv[j & 1], pb, o[db], 0, 0, 0);
    }
  };

  wait_vmcnt<0>();  // resident Q rows landed (the compiler does not count the DMA)
  f32x16_t sa[kTiles] = {}, sb[kTiles] = {};
  if (nblocks > 0) {
    dma_tile(Kg, 0, k_lds[0]);
    dma_tile(Vg, 0, v_lds[0]);
    if (nblocks > 1) dma_tile(Kg, 1, k_lds[1]);
    wait_vmcnt<0>();
    block_barrier();
    qk(k_sm[0], sa);
  }
  int bi = 0;
  for (; bi + 1 < nblocks; bi += 2) {
    step(bi, std::integral_constant<int, 0>{}, sa, sb);
    step(bi + 1, std::integral_constant<int, 1>{}, sb, sa);
  }
  if (bi < nblocks) step(bi, std::integral_constant<int, 0>{}, sa, sb);

  // Prefill hand-off: this workgroup's own rows [q0, q_end) of head h that the
  // cache keeps -- reference row r -> slot r, output t = r - L_m + 1 among the
  // last min(n, T0) -> slot L_m + ((t - 1) mod n) -- copied bit for bit. The
  // workgroup has just streamed these rows, so they come from its XCD's L2.
  if (handoff) {
    const int keep_from = Lm + max(0, N - Lm - n);
    const int64_t cb = p.seq_base[sample] + (int64_t)h * (Lm + n) * kD;
    uint16_t *ck = static_cast<uint16_t *>(p.cache_k) + cb;
    uint16_t *cv = static_cast<uint16_t *>(p.cache_v) + cb;
    constexpr int kPer = kBM * (kD / 8) / (64 * kWaves);  // 16-byte chunks per thread and tensor
    u32x4_t kx[kPer], vx[kPer];
    int64_t dst[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * 64 * kWaves;
      const int r = q0 + i / (kD / 8), c = i % (kD / 8);
      const bool keep = r < q_end && (r < Lm || r >= keep_from);
      dst[j] = keep ? (int64_t)(r < Lm ? r : Lm + (r - Lm) % n) * kD + 8 * c : -1;
      if (keep) {
        const int64_t src = (int64_t)r * stride + 8 * c;
        kx[j] = *reinterpret_cast<const u32x4_t *>(Kg + src);
        vx[j] = *reinterpret_cast<const u32x4_t *>(Vg + src);
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (dst[j] >= 0) {
        *reinterpret_cast<u32x4_t *>(ck + dst[j]) = kx[j];
        *reinterpret_cast<u32x4_t *>(cv + dst[j]) = vx[j];
      }
    }
  }

  // Normalise and store: accumulator element r of o[db] is d = 32 db + 8 (r/4) + 4 hi + r%4.
  l = swap_halves_sum(l);
  if (!q_ok) return;
  const float inv = 1.f / l;
  if (p.lse != nullptr && hi == 0)  // natural log of sum_j 2^(c s_j) = (c m + log2 l) ln 2
    p.lse[(int64_t)h * p.seq_len + row0 + qi] = (m * c + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
  uint16_t *orow = Og + (int64_t)qi * stride;
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
  const int nqb = p.max_seq_len > 0 ? (p.max_seq_len + kBM - 1) / kBM : 1;
  const int64_t G = (int64_t)nqb * p.heads * p.num_seqs;
  if (G == 0) return hipSuccess;
  hipLaunchKernelGGL(masked_attn_kernel, dim3((unsigned)G), dim3(64 * kWaves), 0, s, p);
  return hipGetLastError();
}

}  // namespace rswa
