// Backward of the packed (teacher-forced) R-SWA forward on gfx950 matrix cores.
//
// For the loss sum(dO * O) of the forward O_i = softmax(scale K_J q_i) V_J over
// the two-segment visible set J(i) (WeThinkIn "Unlimited OCR Works：一篇读懂
// R-SWA…", section 方法展开.3, Eqs. (1)-(4)), with P_ij the softmax weights:
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   D_i = dO_i . O_i,
//   dS_ij = P_ij (dP_ij - D_i),   dQ_i = scale sum_j dS_ij k_j,
//   dK_j = scale sum_i dS_ij q_i.
// P is recomputed from the forward's per-row log-sum-exp. Two kernels (and a
// reduction when the long walks are split):
//  * bwd_dq_kernel: one workgroup per 128 query rows x head, the forward's
//    block walk; it first forms D_i and -lse_i / scale of its rows (stored for
//    the next kernel), then per 32-key tile S^T = K Q^T and dP^T = V dO^T on
//    matrix cores (K and V row fragments from LDS, Q and dO rows resident),
//    dS^T in registers, dQ^T += K^T dS^T with K^T from transposing LDS reads;
//  * bwd_dkdv_kernel: one workgroup per 128 keys x head walking the 32-row
//    query blocks that see any of its keys; producer waves (K and V rows of 32
//    keys resident) form S = Q K^T and dP = dO V^T (Q, dO row fragments from
//    LDS) and P, dS; consumer waves (dK, dV of the same keys resident) take P
//    and dS through LDS and run dV += P^T dO and dK += dS^T Q with dO and Q
//    from transposing LDS reads.
// Q/dO and K/V tiles reach LDS by DMA (global_load_lds_dwordx4) through rings
// of four (dQ) and five (dK/dV) stages, into 256-byte rows with swizzled
// 16-byte chunks (rswa_tile.h). The same kernels serve one sequence or a pack
// of independent samples (device row offsets and reference lengths per
// sample; a row never sees another sample's keys).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rswa_internal.h"
#include "rswa_tile.h"

namespace rswa {
namespace {

using namespace tile;

// --------------------------------------------------------------- dQ kernel
constexpr int kBMq = 128;    // query rows per workgroup (4 waves x 32)
constexpr int kBNq = 32;     // keys per block
constexpr int kStagesQ = 4;  // LDS ring of key blocks: one in use, one computed ahead, two in flight

struct DqStage {
  uint16_t k[kBNq * kD];
  uint16_t v[kBNq * kD];
};

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(MaskedBwdParams p) {
  __shared__ DqStage sm[kStagesQ];
  const int H = p.heads, n = p.window;
  const bool full_prefix = p.prefix_mode == RSWA_PREFIX_FULL;
  const int samples = p.cu_seqlens != nullptr ? p.num_seqs : 1;
  const int nqb = ((p.cu_seqlens != nullptr ? p.max_seq_len : p.seq_len) + kBMq - 1) / kBMq;
  const int G = samples * H * nqb;
  // Work item w -> (head, sample, query block); an XCD takes a contiguous range of
  // w, and within a (sample, head) the last query block (the most keys) comes first.
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int h = w / (samples * nqb);
  const int sample = (w / nqb) % samples;
  const int q0 = (nqb - 1 - w % nqb) * kBMq;
  // One sample of a pack: rows [row0, row0 + N) with its own reference length.
  int row0 = 0, N = p.seq_len, Lm = p.ref_len;
  if (p.cu_seqlens != nullptr) {
    row0 = p.cu_seqlens[sample];
    const int row1 = p.cu_seqlens[sample + 1];
    Lm = p.ref_lens[sample];
    N = row1 - row0;
    // device-side metadata: a malformed sample is skipped
    if (row0 < 0 || row1 < row0 || row1 > p.seq_len || N > p.max_seq_len || Lm < 0 || Lm > N) return;
  }
  if (q0 >= N) return;
  const int q_end = min(N, q0 + kBMq);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const uint32_t stride = (uint32_t)H * kD;
  const int64_t base = (int64_t)row0 * stride + (int64_t)h * kD;
  const uint16_t *Qg = static_cast<const uint16_t *>(p.q) + base;
  const uint16_t *Kg = static_cast<const uint16_t *>(p.k) + base;
  const uint16_t *Vg = static_cast<const uint16_t *>(p.v) + base;
  const uint16_t *Gg = static_cast<const uint16_t *>(p.dout) + base;

  // Key blocks: the reference segment [0, pre_hi), then the output keys
  // [win_lo, win_hi) some row of this workgroup sees.
  const int pre_hi = (full_prefix && q0 < Lm) ? Lm : min(Lm, q_end);
  const int win_lo = max(Lm, max(q0, Lm) - n + 1);
  const int win_hi = q_end > Lm ? q_end : win_lo;
  const int nb_pre = (pre_hi + kBNq - 1) / kBNq;
  const int nblocks = nb_pre + (win_hi - win_lo + kBNq - 1) / kBNq;
  auto kb0_of = [&](int bi) __attribute__((always_inline)) {
    return bi < nb_pre ? bi * kBNq : win_lo + (bi - nb_pre) * kBNq;
  };
  auto kend_of = [&](int bi) __attribute__((always_inline)) { return bi < nb_pre ? pre_hi : win_hi; };

  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const bool q_ok = qi < N;
  bf16x8_t qf[kD / 16], gf[kD / 16];
  {
    const int64_t r = (int64_t)(q_ok ? qi : 0) * stride;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const u32x4_t zero = {0, 0, 0, 0};
      qf[ks] = as_bf16x8(q_ok ? *reinterpret_cast<const u32x4_t *>(Qg + r + ks * 16 + hi * 8) : zero);
      gf[ks] = as_bf16x8(q_ok ? *reinterpret_cast<const u32x4_t *>(Gg + r + ks * 16 + hi * 8) : zero);
    }
  }
  // D_i = dO_i . O_i of this lane's row (the lane holds half of the row's dO,
  // at the same places as its O loaded here; lane l ^ 32 the other half) and
  // -lse_i / scale, computed here and stored for the dK/dV pass, whose
  // products start from them.
  float dpart = 0.f;
  if (q_ok) {
    const uint16_t *Orow = static_cast<const uint16_t *>(p.out) + base + (int64_t)qi * stride;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const u32x4_t o = *reinterpret_cast<const u32x4_t *>(Orow + ks * 16 + hi * 8);
      const u32x4_t g = __builtin_bit_cast(u32x4_t, gf[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dpart = fmaf(__uint_as_float(g[e] << 16), __uint_as_float(o[e] << 16), dpart);
        dpart = fmaf(__uint_as_float(g[e] & 0xffff0000u), __uint_as_float(o[e] & 0xffff0000u), dpart);
      }
    }
  }
  const float Dq = swap_halves_sum(dpart);
  const float nls_q = q_ok ? -p.lse[(int64_t)h * p.seq_len + row0 + qi] / p.scale : 0.f;
  if (q_ok && hi == 0) {
    const int64_t rq = (int64_t)h * p.n_pad + row0 + qi;
    p.nd_row[rq] = -Dq;
    p.nls[rq] = nls_q;
  }
  const float c = p.scale_log2;
  const float nlc = nls_q * c;  // -lse in base 2

  // The keys row qi sees inside each segment form one interval [lo, lo + span):
  // the reference segment up to L_m (or up to the row itself for a causal row
  // below L_m), and the n output keys ending at the row.
  const int pv = (full_prefix || qi >= Lm) ? Lm : qi + 1;
  const uint32_t span_p = (uint32_t)pv;
  const int lo_w = max(Lm, qi - n + 1);
  const uint32_t span_w = (uint32_t)max(0, qi + 1 - lo_w);
  // Reference-segment blocks no row of this wave masks.
  const int nb_clear = min((!full_prefix && qw0 < Lm) ? qw0 + 1 : Lm, pre_hi) / kBNq;

  f32x16_t dq[kD / 32];
#pragma unroll
  for (int j = 0; j < kD / 32; ++j) dq[j] = f32x16_t{};

  uint32_t koff[kD / 16], toff[kD / 32][2];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) koff[ks] = row_frag_off(l32, hi, ks);
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
    toff[db][0] = tr_off(lane, db, 0);
    toff[db][1] = tr_off(lane, db, 1);
  }

  // DMA of one 32-key block: wave w fills rows 8 w .. 8 w + 7 of the K and V
  // tiles, 4 instructions per wave and block. Tensor bases stay scalar; a lane
  // adds the byte offset of its row (clamped to the segment's last row) and of
  // its swizzled 16-byte chunk (fixed for the kernel). Byte offsets fit in 32
  // bits and the row product in the 24-bit multiplier (the host rejects tensors
  // of 2^31 elements or more and 2^16 heads or more).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t stride2 = 2u * stride;
  uint32_t c16[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) c16[j] = 16u * (uint32_t)((lane & 15) ^ chunk_swz(8 * wave + 4 * j + (lane >> 4)));
  const uint32_t sm_lds = lds_addr(&sm[0]);
  const uint32_t c16r1 = c16[1] + 4u * stride2;  // instruction 1: four rows further
  auto dma_block = [&](int bi, int stg) __attribute__((always_inline)) {
    const int kb0 = kb0_of(bi), kend = kend_of(bi);
    const uint32_t k_lds = sm_lds + (uint32_t)(stg * sizeof(DqStage) + offsetof(DqStage, k));
    const uint32_t v_lds = sm_lds + (uint32_t)(stg * sizeof(DqStage) + offsetof(DqStage, v));
    uint32_t off[2];
    if (kb0 + kBNq <= kend) {  // a whole block: one row product per lane
      const uint32_t rb = __umul24((uint32_t)(kb0 + 8 * wv + (lane >> 4)), stride2);
      off[0] = rb + c16[0];
      off[1] = rb + c16r1;
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t r = (uint32_t)min(kb0 + 8 * wv + 4 * j + (lane >> 4), kend - 1);
        off[j] = __umul24(r, stride2) + c16[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t row_lds = (uint32_t)((8 * wv + 4 * j) * kRowBytes);
      dma16(Kg, off[j], k_lds + row_lds);
      dma16(Vg, off[j], v_lds + row_lds);
    }
  };

  // S^T = K Q^T and dP^T = V dO^T of the block in stage stg: element r is key
  // kb0 + 8 (r/4) + 4 hi + r%4 of that block, query qi.
  auto sdp = [&](int stg, f32x16_t &s, f32x16_t &dp) __attribute__((always_inline)) {
    const char *kb = reinterpret_cast<const char *>(sm[stg].k);
    const char *vb = reinterpret_cast<const char *>(sm[stg].v);
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const bf16x8_t ka = as_bf16x8(*reinterpret_cast<const u32x4_t *>(kb + koff[ks]));
      const bf16x8_t va = as_bf16x8(*reinterpret_cast<const u32x4_t *>(vb + koff[ks]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16_t{} : s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], ks == 0 ? f32x16_t{} : dp, 0, 0, 0);
    }
  };

  // One pipeline step for block bi (stage bi & 3), its S^T and dP^T computed the
  // step before: wait for block bi + 1, start the DMA of block bi + 3, then
  // S^T/dP^T of block bi + 1 interleaved (hand-ordered) with this block's dS,
  // then dQ^T += K^T dS^T.
  auto step = [&](int bi, f32x16_t &s_cur, f32x16_t &dp_cur, f32x16_t &s_nxt, f32x16_t &dp_nxt)
      __attribute__((always_inline)) {
    const DqStage &st = sm[bi & 3];
    if (bi + 2 < nblocks)
      wait_vmcnt<4>();  // only block bi + 2's four may be outstanding
    else
      wait_vmcnt<0>();
    block_barrier();  // every wave's part of block bi + 1 landed; stage (bi + 3) & 3 is free
    if (bi + 3 < nblocks) dma_block(bi + 3, (bi + 3) & 3);
    float xs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) xs[r] = s_cur[r];
    if (bi >= nb_clear) {
      const bool win = bi >= nb_pre;
      const uint32_t t = (uint32_t)(kb0_of(bi) + 4 * hi - (win ? lo_w : 0));
      const uint32_t span = win ? span_w : span_p;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xs[r] = t + (uint32_t)(8 * (r >> 2) + (r & 3)) < span ? xs[r] : kNegInf;
    }
    __builtin_amdgcn_sched_barrier(0);
    const char *kn = reinterpret_cast<const char *>(sm[(bi + 1) & 3].k);
    const char *vn = reinterpret_cast<const char *>(sm[(bi + 1) & 3].v);
    bf16x8_t ka[kD / 16], va[kD / 16];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      ka[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(kn + koff[ks]));
      va[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(vn + koff[ks]));
    }
    uint32_t dw[8];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      if (ks + 2 < kD / 16) {
        ka[ks + 2] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(kn + koff[ks + 2]));
        va[ks + 2] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(vn + koff[ks + 2]));
      }
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], ks == 0 ? f32x16_t{} : s_nxt, 0, 0, 0);
      dp_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks], gf[ks], ks == 0 ? f32x16_t{} : dp_nxt, 0, 0, 0);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(xs[2 * ks], c, nlc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(xs[2 * ks + 1], c, nlc));
      dw[ks] = pack_bf16(p0 * (dp_cur[2 * ks] - Dq), p1 * (dp_cur[2 * ks + 1] - Dq));
      __builtin_amdgcn_sched_barrier(0);
    }
    // dQ^T += K^T dS^T over two 16-key halves (elements 8 half .. 8 half + 7);
    // transposing reads of K one product ahead.
    const char *kb = reinterpret_cast<const char *>(st.k);
    bf16x8_t tk[2];
    tk[0] = tr_operand(kb, toff[0][0], toff[0][1], 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int half = j >> 2, db = j & 3;
      if (j + 1 < 8) tk[(j + 1) & 1] = tr_operand(kb, toff[(j + 1) & 3][0], toff[(j + 1) & 3][1], (j + 1) >> 2);
      const bf16x8_t dsb = as_bf16x8(u32x4_t{dw[4 * half], dw[4 * half + 1], dw[4 * half + 2], dw[4 * half + 3]});
      dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tk[j & 1], dsb, dq[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  wait_vmcnt<0>();  // resident Q/dO rows landed (the compiler does not count the DMA)
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < nblocks) dma_block(j, j);
  f32x16_t sa = {}, dpa = {}, sb = {}, dpb = {};
  if (nblocks > 0) {
    // block 0 landed: blocks 1 and 2 (four instructions each) may be outstanding
    if (nblocks > 2)
      wait_vmcnt<8>();
    else if (nblocks > 1)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    block_barrier();
    sdp(0, sa, dpa);
  }
  int bi = 0;
  for (; bi + 1 < nblocks; bi += 2) {
    step(bi, sa, dpa, sb, dpb);
    step(bi + 1, sb, dpb, sa, dpa);
  }
  if (bi < nblocks) step(bi, sa, dpa, sb, dpb);

  if (!q_ok) return;
  // dQ^T accumulator element r of dq[db] is d = 32 db + 8 (r/4) + 4 hi + r%4.
  uint16_t *orow = static_cast<uint16_t *>(p.dq) + base + (int64_t)qi * stride;
  const float sc = p.scale;
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * hi;
      const u32x2_t w2 = {pack_bf16(dq[db][4 * g4 + 0] * sc, dq[db][4 * g4 + 1] * sc),
                          pack_bf16(dq[db][4 * g4 + 2] * sc, dq[db][4 * g4 + 3] * sc)};
      *reinterpret_cast<u32x2_t *>(orow + d0) = w2;
    }
  }
}

// ------------------------------------------------------------- dK/dV kernel
constexpr int kBK = 128;    // keys per workgroup (4 key groups x 32)
constexpr int kBQ = 32;     // query rows per block
constexpr int kStages = 5;  // LDS ring of query blocks (see the step comment below)

struct DkdvStage {
  uint16_t q[kBQ * kD];
  uint16_t g[kBQ * kD];
  float ld[2 * kBQ];  // the block's rows: lse in base 2, then D
};

// P and dS of one query block, already in the layout of the dV/dK products'
// A operand: per key group, 16-row step and lane, 8 bf16 values (the lane's
// key against 8 rows of the step).
struct DkdvXchg {
  u32x4_t pd[4][2][2][64];  // [key group][16-row step][P, dS][lane]
};

// s_waitcnt with only lgkmcnt = 0 (this wave's LDS accesses performed).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Work of one workgroup: 128 keys of one head and a run of query blocks.
// Key blocks that hold reference-segment keys are seen by every later row; their
// walk is cut into `parts` runs of equal length whose fp32 partial sums a
// reduction adds up (parts > 1). Tasks are dealt to the 8 XCDs (block index mod
// 8) so that each (head, part) lands whole on one XCD, its key blocks walking the
// same Q/dO rows through one L2; the short output-segment tasks follow.
//
// Eight waves in two roles, one of each per SIMD: producer wave g (0..3) keeps
// the K and V rows of key group g resident, forms S and dP of a query block on
// the matrix cores and turns them into P and dS; consumer wave 4 + g keeps the
// dK and dV accumulators of the same 32 keys and runs the dV += P^T dO and
// dK += dS^T Q products of the block before, its A operands passed through LDS
// lane for lane. Each role fits in half the register file, so the SIMD overlaps
// one wave's exponentials and LDS reads with the other's products.
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(MaskedBwdParams p) {
  __shared__ DkdvStage sm[kStages];
  __shared__ DkdvXchg xc[2];
  const int H = p.heads, n = p.window;
  const bool full_prefix = p.prefix_mode == RSWA_PREFIX_FULL;
  const int S = p.parts;
  int N = p.seq_len, Lm = p.ref_len, row0 = 0;
  int h, kb, part;
  if (p.cu_seqlens != nullptr) {
    // Pack of samples: work item w -> (head, sample, 128-key block), an XCD
    // taking a contiguous range of w; walks are short, so never split.
    const int nkb = (p.max_seq_len + kBK - 1) / kBK;
    const int G = p.num_seqs * H * nkb;
    int w = blockIdx.x;
    if ((G & 7) == 0) w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    h = w / (p.num_seqs * nkb);
    const int sample = (w / nkb) % p.num_seqs;
    kb = w % nkb;
    part = -1;
    row0 = p.cu_seqlens[sample];
    const int row1 = p.cu_seqlens[sample + 1];
    Lm = p.ref_lens[sample];
    N = row1 - row0;
    // device-side metadata: a malformed sample is skipped
    if (row0 < 0 || row1 < row0 || row1 > p.seq_len || N > p.max_seq_len || Lm < 0 || Lm > N) return;
    if (kb * kBK >= N) return;
  } else {
    const int nkb_pre = p.nkb_pre, nkb_win = p.nkb_win;
    const int x = blockIdx.x & 7, kx = blockIdx.x >> 3;
    const int pairs = H * S;
    const int pre_x = (pairs > x ? (pairs - 1 - x) / 8 + 1 : 0) * nkb_pre;
    const int U = H * nkb_win;
    const int win_x = U > x ? (U - 1 - x) / 8 + 1 : 0;
    if (kx < pre_x) {
      const int pr = x + 8 * (kx / nkb_pre);
      kb = kx % nkb_pre;
      h = pr / S;
      part = pr % S;
    } else {
      const int k2 = kx - pre_x;
      if (k2 >= win_x) return;  // padding of this XCD's task list
      const int u = x + 8 * k2;
      h = u / nkb_win;
      kb = nkb_pre + u % nkb_win;
      part = -1;
    }
  }
  const int kw0 = kb * kBK;
  const int kmax = min(N, kw0 + kBK) - 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave & 3;
  const int hi = lane >> 5, l32 = lane & 31;
  const uint32_t stride = (uint32_t)H * kD;
  const int64_t base = (int64_t)row0 * stride + (int64_t)h * kD;
  const uint16_t *Qg = static_cast<const uint16_t *>(p.q) + base;
  const uint16_t *Gg = static_cast<const uint16_t *>(p.dout) + base;

  // Query blocks whose rows see some key of this workgroup, then this part of them.
  int b_lo, b_hi;
  if (kw0 < Lm) {
    b_lo = (full_prefix ? 0 : kw0) / kBQ;
    b_hi = (N + kBQ - 1) / kBQ;
  } else {
    b_lo = kw0 / kBQ;
    b_hi = (min(N, kmax + n) + kBQ - 1) / kBQ;
  }
  if (part >= 0 && S > 1) {
    const int len = b_hi - b_lo;
    const int s0 = b_lo + (int)((int64_t)len * part / S);
    b_hi = b_lo + (int)((int64_t)len * (part + 1) / S);
    b_lo = s0;
  }
  const int nblocks = max(0, b_hi - b_lo);
  const float *nls_h = p.nls + (int64_t)h * p.n_pad + row0;
  const float *d_h = p.nd_row + (int64_t)h * p.n_pad + row0;

  // DMA of one 32-row query block: wave w fills rows 4 w .. 4 w + 3 of the Q and
  // dO tiles (2 instructions) and, with its lanes 8 w .. 8 w + 7, an eighth of
  // the lse/D strip (1 instruction): 3 per wave and block. Row offsets as in
  // the dQ kernel's DMA (32-bit, from a 24-bit product).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t stride2 = 2u * stride;
  const uint32_t c16 = 16u * (uint32_t)((lane & 15) ^ chunk_swz(4 * wave + (lane >> 4)));
  const uint32_t sm_lds = lds_addr(&sm[0]);
  auto dma_block = [&](int bi, int stg) __attribute__((always_inline)) {
    const int qb0 = (b_lo + bi) * kBQ;
    const uint32_t st_lds = sm_lds + (uint32_t)(stg * sizeof(DkdvStage));
    const int row0 = 4 * wv;
    const uint32_t r = (uint32_t)min(qb0 + row0 + (lane >> 4), N - 1);
    const uint32_t off = __umul24(r, stride2) + c16;
    dma16(Qg, off, st_lds + (uint32_t)(offsetof(DkdvStage, q) + row0 * kRowBytes));
    dma16(Gg, off, st_lds + (uint32_t)(offsetof(DkdvStage, g) + row0 * kRowBytes));
    if ((lane >> 3) == wave) {
      // rows past the sequence's end repeat its last row, as the tile rows do
      // (their scores are masked, so P = dS = 0 whatever finite values sit here)
      const int rr = min(qb0 + (lane & 31), N - 1);
      const float *src = lane < 32 ? nls_h + rr : d_h + rr;
      dma4(src, st_lds + (uint32_t)offsetof(DkdvStage, ld));  // lane L's dword lands at ld[L]
    }
  };
  auto ring = [](int s, int k) __attribute__((always_inline)) { return s + k < kStages ? s + k : s + k - kStages; };

  // Step t (t = 0 .. nblocks, both roles, one barrier each): the producers form
  // P/dS of block t (its S/dP computed in step t - 1) next to S/dP of block
  // t + 1; the consumers run the products of block t - 1. Live stages: t - 1
  // (consumers) and t + 1 (Q, dO and the lse/D strip of the producers' next
  // S/dP); stage t is not read in step t; the other kStages - 3 hold blocks in flight
  // (DMA of block t + kStages - 2 issued in step t into the stage block t - 2
  // held, whose last reader finished in step t - 1). Step t's wait: this wave's
  // part of block t + 1 landed (loads return in order: the three instructions
  // of each later block may be outstanding); the barrier then makes every
  // wave's part visible, and P/dS of block t - 1 (written in step t - 1).
  constexpr int kAhead = kStages - 2;
  // Waits until at most nb blocks (three instructions each) of this wave's DMA
  // are outstanding.
  auto wait_blocks = [](int nb) __attribute__((always_inline)) {
    static_assert(kAhead <= 5, "vmcnt immediates below");
    if (nb <= 0)
      wait_vmcnt<0>();
    else if (nb == 1)
      wait_vmcnt<3>();
    else if (nb == 2)
      wait_vmcnt<6>();
    else if (nb == 3)
      wait_vmcnt<9>();
    else if (nb == 4)
      wait_vmcnt<12>();
    else
      wait_vmcnt<15>();
  };
  auto step_sync = [&](int t, int stg) __attribute__((always_inline)) {
    wait_blocks(min(kAhead - 2, nblocks - t - 2));
    wait_lgkmcnt0();
    block_barrier();
    if (t + kAhead < nblocks) dma_block(t + kAhead, ring(stg, kAhead));
  };
  // Step -1: blocks 0 .. kAhead - 1 requested, wait for block 0.
  auto first_sync = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (j < nblocks) dma_block(j, j);
    wait_blocks(min(kAhead - 1, nblocks - 1));
    block_barrier();
  };

  if (wave < 4) {
    // ------------------------------------------------------------ producer
    const uint16_t *Kg = static_cast<const uint16_t *>(p.k) + base;
    const uint16_t *Vg = static_cast<const uint16_t *>(p.v) + base;
    // This lane's key (B operand column / accumulator column of S and dP).
    const int kj = kw0 + 32 * grp + l32;
    const bool k_ok = kj < N;
    bf16x8_t kf[kD / 16], vf[kD / 16];
    {
      const int64_t r = (int64_t)(k_ok ? kj : 0) * stride;
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const u32x4_t zero = {0, 0, 0, 0};
        kf[ks] = as_bf16x8(k_ok ? *reinterpret_cast<const u32x4_t *>(Kg + r + ks * 16 + hi * 8) : zero);
        vf[ks] = as_bf16x8(k_ok ? *reinterpret_cast<const u32x4_t *>(Vg + r + ks * 16 + hi * 8) : zero);
      }
    }
    // Blocks that hide no (query, key) pair: all keys in the reference segment,
    // all rows output rows, block whole.
    int clear_lo = nblocks, clear_hi = nblocks;
    if (kmax < Lm) {
      clear_lo = min(nblocks, max(0, (Lm + kBQ - 1) / kBQ - b_lo));
      clear_hi = min(nblocks, max(clear_lo, N / kBQ - b_lo));
    }
    // Rows the lane's key is visible to form one interval [v_lo, v_hi): the whole
    // sequence tail from the key (reference-segment key), plus every row below
    // L_m with the full-prefix mode, or the n rows from the key (output key).
    const bool key_is_prefix = kj < Lm;
    int v_lo = kj, v_hi = key_is_prefix ? N : min(N, kj + n);
    if (key_is_prefix && full_prefix) v_lo = 0;
    if (!k_ok) v_hi = v_lo;
    const uint32_t v_span = (uint32_t)(v_hi - v_lo);
    uint32_t roff[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) roff[ks] = row_frag_off(l32, hi, ks);
    const float c = p.scale_log2;

    // S = Q K^T and dP = dO V^T of the block in stage stg: element r is query
    // qb0 + 8 (r/4) + 4 hi + r%4 of that block, key kj.
    // The products start from -lse/scale and -D of the element's row (the
    // block's strip holds them so), so S comes out as s - lse/scale and dP as
    // dP - D: P = exp2(c S) and dS = P dP need no subtraction per element.
    auto strip = [&](int stg, f32x16_t &nl, f32x16_t &nd) __attribute__((always_inline)) {
      const DkdvStage &st = sm[stg];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t *>(&st.ld[8 * g + 4 * hi]);
        const f32x4_t b = *reinterpret_cast<const f32x4_t *>(&st.ld[kBQ + 8 * g + 4 * hi]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nl[4 * g + e] = a[e];
          nd[4 * g + e] = b[e];
        }
      }
    };
    auto sdp = [&](int stg, f32x16_t &s, f32x16_t &dp) __attribute__((always_inline)) {
      const char *qb = reinterpret_cast<const char *>(sm[stg].q);
      const char *gb = reinterpret_cast<const char *>(sm[stg].g);
      f32x16_t nl, nd;
      strip(stg, nl, nd);
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8_t qa = as_bf16x8(*reinterpret_cast<const u32x4_t *>(qb + roff[ks]));
        const bf16x8_t ga = as_bf16x8(*reinterpret_cast<const u32x4_t *>(gb + roff[ks]));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], ks == 0 ? nl : s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], ks == 0 ? nd : dp, 0, 0, 0);
      }
    };

    // Producer step t: P and dS of block t (stage stg) from S/dP computed the
    // step before, two elements per k-step of block t + 1's S/dP products (about
    // the two products' time), order fixed by hand (sched_barrier).
    auto produce = [&](int t, int stg, f32x16_t &s_cur, f32x16_t &dp_cur, f32x16_t &s_nxt, f32x16_t &dp_nxt)
        __attribute__((always_inline)) {
      step_sync(t, stg);
      const int qb0 = (b_lo + t) * kBQ;
      float xs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[r] = s_cur[r];
      if (t < clear_lo || t >= clear_hi) {
        const uint32_t tt = (uint32_t)(qb0 + 4 * hi - v_lo);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          xs[r] = tt + (uint32_t)(8 * (r >> 2) + (r & 3)) < v_span ? xs[r] : kNegInf;
      }
      __builtin_amdgcn_sched_barrier(0);
      // S/dP of block t + 1 (a stale stage after the last block; result unused).
      const int nstg = ring(stg, 1);
      f32x16_t nl, nd;
      strip(nstg, nl, nd);
      const char *qn = reinterpret_cast<const char *>(sm[nstg].q);
      const char *gn = reinterpret_cast<const char *>(sm[nstg].g);
      bf16x8_t qa[kD / 16], ga[kD / 16];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qa[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(qn + roff[ks]));
        ga[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(gn + roff[ks]));
      }
      uint32_t pw[8], dw[8];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        if (ks + 2 < kD / 16) {
          qa[ks + 2] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(qn + roff[ks + 2]));
          ga[ks + 2] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(gn + roff[ks + 2]));
        }
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kf[ks], ks == 0 ? nl : s_nxt, 0, 0, 0);
        dp_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[ks], vf[ks], ks == 0 ? nd : dp_nxt, 0, 0, 0);
        // elements 2 ks, 2 ks + 1: rows 8 (ks/2) + 4 hi + 2 (ks%2) + {0, 1}
        const float p0 = __builtin_amdgcn_exp2f(xs[2 * ks] * c);
        const float p1 = __builtin_amdgcn_exp2f(xs[2 * ks + 1] * c);
        pw[ks] = pack_bf16(p0, p1);
        dw[ks] = pack_bf16(p0 * dp_cur[2 * ks], p1 * dp_cur[2 * ks + 1]);
        // Step st2 of the consumer's products uses elements 8 st2 .. 8 st2 + 7;
        // storing each half as soon as it exists keeps the arithmetic between
        // the products.
        if ((ks & 3) == 3) {
          const int st2 = ks >> 2;
          DkdvXchg &xo = xc[t & 1];
          xo.pd[grp][st2][0][lane] = u32x4_t{pw[4 * st2], pw[4 * st2 + 1], pw[4 * st2 + 2], pw[4 * st2 + 3]};
          xo.pd[grp][st2][1][lane] = u32x4_t{dw[4 * st2], dw[4 * st2 + 1], dw[4 * st2 + 2], dw[4 * st2 + 3]};
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (nblocks == 0) return;
    f32x16_t sa = {}, dpa = {}, sb = {}, dpb = {};
    first_sync();
    sdp(0, sa, dpa);
    int t = 0, stg = 0;
    for (; t + 1 < nblocks; t += 2) {
      produce(t, stg, sa, dpa, sb, dpb);
      stg = ring(stg, 1);
      produce(t + 1, stg, sb, dpb, sa, dpa);
      stg = ring(stg, 1);
    }
    if (t < nblocks) {
      produce(t, stg, sa, dpa, sb, dpb);
      stg = ring(stg, 1);
    }
    step_sync(nblocks, stg);  // hands P/dS of the last block to the consumers
    return;
  }

  // -------------------------------------------------------------- consumer
  f32x16_t dk[kD / 32], dv[kD / 32];
#pragma unroll
  for (int j = 0; j < kD / 32; ++j) {
    dk[j] = f32x16_t{};
    dv[j] = f32x16_t{};
  }
  uint32_t toff[kD / 32][2];
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
    toff[db][0] = tr_off(lane, db, 0);
    toff[db][1] = tr_off(lane, db, 1);
  }
  // dV += P^T dO and dK += dS^T Q of the block in stage stg over two 16-row
  // steps (st2 = j / 4, d block db = j % 4); the transposing reads run two
  // products ahead (order fixed by hand with sched_barrier).
  auto consume = [&](int stg, const DkdvXchg &xi) __attribute__((always_inline)) {
    const char *qb = reinterpret_cast<const char *>(sm[stg].q);
    const char *gb = reinterpret_cast<const char *>(sm[stg].g);
    bf16x8_t pa[2], da[2], tg[8], tq[8];
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2) {
      pa[st2] = as_bf16x8(xi.pd[grp][st2][0][lane]);
      da[st2] = as_bf16x8(xi.pd[grp][st2][1][lane]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      tg[j] = tr_operand(gb, toff[j][0], toff[j][1], 0);
      tq[j] = tr_operand(qb, toff[j][0], toff[j][1], 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int st2 = j >> 2, db = j & 3;
      if (j + 2 < 8) {
        const int jn = j + 2;
        tg[jn] = tr_operand(gb, toff[jn & 3][0], toff[jn & 3][1], jn >> 2);
        tq[jn] = tr_operand(qb, toff[jn & 3][0], toff[jn & 3][1], jn >> 2);
      }
      dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[st2], tg[j], dv[db], 0, 0, 0);
      dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[st2], tq[j], dk[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (nblocks > 0) {
    first_sync();
    int stg = 0;
    step_sync(0, stg);
    for (int t = 1; t <= nblocks; ++t) {
      const int prev = stg;
      stg = ring(stg, 1);
      step_sync(t, stg);
      consume(prev, xc[(t - 1) & 1]);
    }
  }

  // Accumulator element r of dk[db] is key kw0 + 32 grp + 8 (r/4) + 4 hi + r%4
  // and d = 32 db + l32: every lane stores, whatever its own score column.
  if (part >= 0 && S > 1) {
    const int64_t pbase = (((int64_t)part * H + h) * p.kpre + kw0 + 32 * grp) * kD;
    float *pk = p.part_dk + pbase;
    float *pv = p.part_dv + pbase;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) {
        pk[kl * kD + 32 * db + l32] = dk[db][r];
        pv[kl * kD + 32 * db + l32] = dv[db][r];
      }
    }
    return;
  }
  const float sc = p.scale;
  uint16_t *dkg = static_cast<uint16_t *>(p.dk) + base;
  uint16_t *dvg = static_cast<uint16_t *>(p.dv) + base;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kw0 + 32 * grp + 8 * (r >> 2) + 4 * hi + (r & 3);
    if (key >= N) continue;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
      const uint32_t kp = pack_bf16(dk[db][r] * sc, dv[db][r]);
      dkg[(int64_t)key * stride + 32 * db + l32] = static_cast<uint16_t>(kp & 0xffffu);
      dvg[(int64_t)key * stride + 32 * db + l32] = static_cast<uint16_t>(kp >> 16);
    }
  }
}

// Sums the parts' fp32 partials of the reference-segment key blocks and stores
// dK (times the scale) and dV in bf16. One thread per (key, head, 8 dims).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(MaskedBwdParams p) {
  const int H = p.heads;
  const int kval = min(p.seq_len, p.kpre);
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)kval * H * 16) return;
  const int c = (int)(t & 15);
  const int64_t kh = t >> 4;
  const int h = (int)(kh % H), key = (int)(kh / H);
  f32x4_t a0 = {}, a1 = {}, b0 = {}, b1 = {};
  for (int s = 0; s < p.parts; ++s) {
    const int64_t off = (((int64_t)s * H + h) * p.kpre + key) * kD + 8 * c;
    a0 += *reinterpret_cast<const f32x4_t *>(p.part_dk + off);
    a1 += *reinterpret_cast<const f32x4_t *>(p.part_dk + off + 4);
    b0 += *reinterpret_cast<const f32x4_t *>(p.part_dv + off);
    b1 += *reinterpret_cast<const f32x4_t *>(p.part_dv + off + 4);
  }
  const float sc = p.scale;
  const int64_t o = ((int64_t)key * H + h) * kD + 8 * c;
  *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(p.dk) + o) =
      u32x4_t{pack_bf16(a0[0] * sc, a0[1] * sc), pack_bf16(a0[2] * sc, a0[3] * sc),
              pack_bf16(a1[0] * sc, a1[1] * sc), pack_bf16(a1[2] * sc, a1[3] * sc)};
  *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(p.dv) + o) =
      u32x4_t{pack_bf16(b0[0], b0[1]), pack_bf16(b0[2], b0[3]), pack_bf16(b1[0], b1[1]),
              pack_bf16(b1[2], b1[3])};
}

}  // namespace

int64_t masked_bwd_dkdv_grid(int32_t heads, int32_t parts, int32_t nkb_pre, int32_t nkb_win) {
  const int64_t pairs = (int64_t)heads * parts, u = (int64_t)heads * nkb_win;
  return 8 * (((pairs + 7) / 8) * nkb_pre + (u + 7) / 8);
}

hipError_t launch_masked_bwd(const MaskedBwdParams &p, hipStream_t s) {
  const bool pack = p.cu_seqlens != nullptr;
  const int64_t rows_max = pack ? p.max_seq_len : p.seq_len;
  const int64_t samples = pack ? p.num_seqs : 1;
  const int64_t gq = samples * ((rows_max + kBMq - 1) / kBMq) * p.heads;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)gq), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t gk = pack ? samples * p.heads * ((rows_max + kBK - 1) / kBK)
                          : masked_bwd_dkdv_grid(p.heads, p.parts, p.nkb_pre, p.nkb_win);
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)gk), dim3(512), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.parts == 1 || p.nkb_pre == 0) return e;
  const int64_t kval = p.seq_len < p.kpre ? p.seq_len : p.kpre;
  const int64_t threads = kval * p.heads * 16;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace rswa
