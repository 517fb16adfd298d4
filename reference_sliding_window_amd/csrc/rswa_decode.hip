// Decode-side kernels of librswa for gfx950 (CDNA4, wave64):
//   * reference write   -- the reference segment is written once and never
//     updated (夜雨聆风 "多模态文档解析开源新进展:Unlimited OCR技术方案", section
//     "为什么它能”无限”读下去？关键在 KV cache 恒定");
//   * append / evict    -- the output window is a ring of n slots after the
//     reference, so the queue of capacity m+n that evicts position m+1 (same
//     section) is realised without moving entries;
//   * split-K decode    -- softmax attention of one query per (sequence, head)
//     over N(t) = P ∪ D_n(t) (WeThinkIn "Unlimited OCR Works：一篇读懂 R-SWA…",
//     section 方法展开.3, Eqs. (1)-(4)); with the ring layout N(t) is the
//     contiguous slot range [0, L_m + min(n, T)) (Eq. (6));
//   * split merge       -- combines the per-chunk softmax states; with a
//     single chunk per (sequence, head) the split kernel writes the output
//     itself and the last of a sequence's workgroups publishes its step
//     through the cache's arrival counter (one launch per step).
//
// Memory-bound design: each K/V row of d bf16 values (256 B at d = 128) is
// read by 16 lanes with one 16-byte load each, so a wave64 load instruction
// covers 4 consecutive rows = 1 KB contiguous. Every loaded element is used
// exactly once by the lane that loaded it, so K/V go straight to VGPRs with
// non-temporal loads (on MI355X they stream about 12 % faster than ordinary
// loads: nothing here is re-read); the 16-lane dot-product reduction uses DPP
// row operations (no LDS traffic).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rswa_internal.h"

namespace rswa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// Native 16-byte vector (HIP's uint4 is a struct whose copies can go through
// private memory, and the non-temporal builtin does not take it).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#ifndef RSWA_DECODE_U
#define RSWA_DECODE_U 8  // 16-byte K and V loads in flight per lane per tile
#endif
#ifndef RSWA_DECODE_NT
#define RSWA_DECODE_NT 1  // stream K/V with non-temporal loads (0: ordinary loads)
#endif

__device__ __forceinline__ u32x4_t stream_load(const u32x4_t *p) {
#if RSWA_DECODE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// ------------------------------------------------------------ element types
struct Bf16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;  // elements per 16-byte vector
  __device__ static inline void unpack(const u32x4_t &w, float *f) {
    const uint32_t x[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(x[i] << 16);
      f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
  }
  // float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
  __device__ static inline uint16_t round(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
};

struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  __device__ static inline void unpack(const u32x4_t &w, float *f) {
    f[0] = __uint_as_float(w[0]);
    f[1] = __uint_as_float(w[1]);
    f[2] = __uint_as_float(w[2]);
    f[3] = __uint_as_float(w[3]);
  }
};

// Stores one fp32 result into an output of the cache dtype (bf16: round to
// nearest even).
template <class E>
__device__ inline void store_out(void *out, int64_t i, float o) {
  if constexpr (E::kBytes == 2) {
    static_cast<uint16_t *>(out)[i] = Bf16::round(o);
  } else {
    static_cast<float *>(out)[i] = o;
  }
}

// ------------------------------------------------------------ lane reductions
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}

// Sum over groups of kLanes consecutive lanes (kLanes in {8, 16, 32}); every
// lane of a group receives the group's sum. Within a 16-lane DPP row:
// quad_perm [1,0,3,2] and [2,3,0,1] sum quads, row_half_mirror pairs the two
// quads of each 8-lane half, row_mirror pairs the two halves.
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (kLanes >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (kLanes >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// Merge of two base-2 online-softmax states (m = running max of the scaled
// scores, l = sum of 2^(s - m), acc = sum of 2^(s - m) v).
struct Rescale {
  float a, b;  // weights of the first and second state
};
__device__ __forceinline__ Rescale merge_weights(float m1, float m2, float &m_out) {
  const float m = fmaxf(m1, m2);
  const float mu = (m == kNegInf) ? 0.f : m;
  m_out = m;
  return {__builtin_amdgcn_exp2f(m1 - mu), __builtin_amdgcn_exp2f(m2 - mu)};
}

// ------------------------------------------------------------------ kernels
template <class E, int D>
struct Geometry {
  static constexpr int kEpl = E::kPerVec;   // elements per lane-load
  static constexpr int kLpr = D / kEpl;     // lanes per key row
  static constexpr int kRpl = 64 / kLpr;    // rows per wave-load
  static_assert(kLpr == 8 || kLpr == 16 || kLpr == 32, "unsupported row geometry");
};

__device__ __forceinline__ int seq_errors(int32_t L, int32_t max_ref_len, int64_t base,
                                          int align_elems) {
  int err = 0;
  if (L < 0 || L > max_ref_len) err |= RSWA_DEVERR_REF_LEN;
  if (base < 0 || (base % align_elems) != 0) err |= RSWA_DEVERR_ALIGN;
  return err;
}

// Reference write: grid (row blocks, H, B); 256 threads copy 16-byte vectors.
template <class E, int D>
__global__ __launch_bounds__(256) void cache_init_kernel(InitParams p) {
  using G = Geometry<E, D>;
  constexpr int kRows = 32;
  const int b = blockIdx.z, h = blockIdx.y;
  const int32_t L = p.ref_len[b];
  const int64_t base = p.seq_base[b];
  const int64_t rbase = p.max_ref_len > 0 ? p.ref_base[b] : 0;
  int err = seq_errors(L, p.max_ref_len, base, G::kEpl);
  if (rbase < 0 || (rbase % G::kEpl) != 0) err |= RSWA_DEVERR_ALIGN;
  if (err) {
    if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0) atomicOr(p.error, err);
    return;
  }
  if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0) {
    p.step[b] = 0;
    if (p.arrive != nullptr) p.arrive[b] = 0;
  }
  const int r0 = blockIdx.x * kRows;
  const int r1 = min(L, r0 + kRows);
  if (r0 >= r1) return;
  using S = typename E::storage;
  const S *ks = static_cast<const S *>(p.k_ref) + rbase + (int64_t)h * L * D;
  const S *vs = static_cast<const S *>(p.v_ref) + rbase + (int64_t)h * L * D;
  S *kd = static_cast<S *>(p.k) + base + (int64_t)h * (L + p.window) * D;
  S *vd = static_cast<S *>(p.v) + base + (int64_t)h * (L + p.window) * D;
  const int nvec = (r1 - r0) * G::kLpr;
  for (int i = threadIdx.x; i < nvec; i += 256) {
    const int64_t off = (int64_t)r0 * D + (int64_t)i * G::kEpl;
    *reinterpret_cast<u32x4_t *>(kd + off) = *reinterpret_cast<const u32x4_t *>(ks + off);
    *reinterpret_cast<u32x4_t *>(vd + off) = *reinterpret_cast<const u32x4_t *>(vs + off);
  }
}

// Append / evict: one block per sequence; bit-exact copy into slot
// L_m + (T mod n), then T += 1 (after every thread has read T).
template <class E, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  using G = Geometry<E, D>;
  const int b = blockIdx.x;
  if (p.active != nullptr && p.active[b] == 0) return;
  const int32_t L = p.ref_len[b];
  const int32_t T0 = p.step[b];
  const int64_t base = p.seq_base[b];
  int err = seq_errors(L, p.max_ref_len, base, G::kEpl);
  if (T0 < 0 || T0 == INT32_MAX) err |= RSWA_DEVERR_STEP;
  if (err) {
    if (threadIdx.x == 0) atomicOr(p.error, err);
    return;
  }
  const int slot = L + T0 % p.window;
  using S = typename E::storage;
  const S *kn = static_cast<const S *>(p.k_new) + (int64_t)b * p.heads * D;
  const S *vn = static_cast<const S *>(p.v_new) + (int64_t)b * p.heads * D;
  S *kd = static_cast<S *>(p.k) + base;
  S *vd = static_cast<S *>(p.v) + base;
  const int nvec = p.heads * G::kLpr;
  for (int i = threadIdx.x; i < nvec; i += 256) {
    const int h = i / G::kLpr, c = i % G::kLpr;
    const int64_t dst = ((int64_t)h * (L + p.window) + slot) * D + c * G::kEpl;
    const int64_t src = (int64_t)h * D + c * G::kEpl;
    *reinterpret_cast<u32x4_t *>(kd + dst) = *reinterpret_cast<const u32x4_t *>(kn + src);
    *reinterpret_cast<u32x4_t *>(vd + dst) = *reinterpret_cast<const u32x4_t *>(vn + src);
  }
  __syncthreads();
  if (threadIdx.x == 0) p.step[b] = T0 + 1;
}

// Per-sequence facts every decode kernel derives the same way: the error bits
// of sequence b and its visible slot count vis = L_m + min(n, T) (0 when flagged).
struct SeqFacts {
  int32_t L, T0, vis;
  int64_t base;
  int err;
};

template <int kEpl>
__device__ __forceinline__ SeqFacts seq_facts(const DecodeParams &p, int b) {
  SeqFacts f;
  f.L = p.ref_len[b];
  f.T0 = p.step[b];
  f.base = p.seq_base[b];
  const bool fused = p.k_new != nullptr;
  f.err = seq_errors(f.L, p.max_ref_len, f.base, kEpl);
  if (f.T0 < 0 || (fused && f.T0 == INT32_MAX)) f.err |= RSWA_DEVERR_STEP;
  const int32_t T = fused ? f.T0 + 1 : f.T0;
  f.vis = f.err ? 0 : f.L + min(p.window, T);
  if (!f.err && f.vis == 0) f.err |= RSWA_DEVERR_EMPTY;
  return f;
}

// Attention of one query (sequence b, head h) over the visible slots
// [start, end) (start < end), by one workgroup of 4 waves: its waves take tiles
// of kRpl*U rows round-robin; lane group g (kLpr lanes) of a wave follows rows
// g, g + kRpl, ... of each tile with its own online softmax state, so the loop
// needs no cross-row communication. The result is the chunk's partial state
// (po[d], pml = {max, sum}) or, with write_out, the normalised output row.
//
// Fused append: the slot receiving the new token, star = L_m + (T0 mod n),
// lies in exactly one chunk. That workgroup reads the new K/V from k_new/v_new
// instead of the slot and also writes them into the slot; no other workgroup
// reads the slot, so the evicted entry is never visible and there is no race.
template <class E, int D, int U>
__device__ __forceinline__ void attend_range(const DecodeParams &p, int b, int h, const SeqFacts &f,
                                             int start, int end, float *po, float *pml,
                                             bool write_out) {
  using G = Geometry<E, D>;
  using S = typename E::storage;
  constexpr int kEpl = G::kEpl, kLpr = G::kLpr, kRpl = G::kRpl;
  constexpr int kTile = kRpl * U;
  constexpr int kWaves = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / kLpr, c = lane % kLpr;
  const int64_t bh = (int64_t)b * p.heads + h;
  const bool fused = p.k_new != nullptr;
  const int32_t L = f.L;

  const int64_t head_off = f.base + (int64_t)h * (L + p.window) * D;
  const S *kb = static_cast<const S *>(p.k) + head_off;
  const S *vb = static_cast<const S *>(p.v) + head_off;
  const int star = fused ? L + f.T0 % p.window : -1;
  const S *kn = fused ? static_cast<const S *>(p.k_new) + bh * D : nullptr;
  const S *vn = fused ? static_cast<const S *>(p.v_new) + bh * D : nullptr;

  if (fused && star >= start && star < end && wave == 0 && lane < kLpr) {
    S *kd = static_cast<S *>(p.k) + head_off + (int64_t)star * D;
    S *vd = static_cast<S *>(p.v) + head_off + (int64_t)star * D;
    reinterpret_cast<u32x4_t *>(kd)[lane] = reinterpret_cast<const u32x4_t *>(kn)[lane];
    reinterpret_cast<u32x4_t *>(vd)[lane] = reinterpret_cast<const u32x4_t *>(vn)[lane];
  }

  float qf[kEpl];
  {
    const u32x4_t qv = reinterpret_cast<const u32x4_t *>(static_cast<const S *>(p.q) + bh * D)[c];
    E::unpack(qv, qf);
#pragma unroll
    for (int e = 0; e < kEpl; ++e) qf[e] *= p.scale_log2;
  }

  float m = kNegInf, l = 0.f;
  float acc[kEpl];
#pragma unroll
  for (int e = 0; e < kEpl; ++e) acc[e] = 0.f;

  for (int t0 = start + wave * kTile; t0 < end; t0 += kWaves * kTile) {
    u32x4_t kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = t0 + u * kRpl + g;
      valid[u] = row < end;
      const int rr = valid[u] ? row : end - 1;
      const bool is_new = (rr == star);
      const u32x4_t *kp = is_new ? reinterpret_cast<const u32x4_t *>(kn)
                               : reinterpret_cast<const u32x4_t *>(kb + (int64_t)rr * D);
      const u32x4_t *vp = is_new ? reinterpret_cast<const u32x4_t *>(vn)
                               : reinterpret_cast<const u32x4_t *>(vb + (int64_t)rr * D);
      kr[u] = stream_load(kp + c);
      vr[u] = stream_load(vp + c);
    }
    float s[U];
    float tmax = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[kEpl];
      E::unpack(kr[u], kf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < kEpl; ++e) dot = fmaf(qf[e], kf[e], dot);
      dot = group_sum<kLpr>(dot);
      s[u] = valid[u] ? dot : kNegInf;
      tmax = fmaxf(tmax, s[u]);
    }
    float m_new;
    const Rescale w = merge_weights(m, tmax, m_new);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = w.a;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = __builtin_amdgcn_exp2f(s[u] - mu);
      l += pu;
      float vf[kEpl];
      E::unpack(vr[u], vf);
#pragma unroll
      for (int e = 0; e < kEpl; ++e) acc[e] = fmaf(pu, vf[e], acc[e]);
    }
    m = m_new;
  }

  // Merge the kRpl row groups of the wave (lanes with equal column index c).
#pragma unroll
  for (int off = kLpr; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float l2 = __shfl_xor(l, off, 64);
    float mm;
    const Rescale w = merge_weights(m, m2, mm);
    l = l * w.a + l2 * w.b;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) {
      const float a2 = __shfl_xor(acc[e], off, 64);
      acc[e] = acc[e] * w.a + a2 * w.b;
    }
    m = mm;
  }

  // Merge the waves through LDS and write this chunk's partial state.
  __shared__ float sm_acc[kWaves][D];
  __shared__ float sm_m[kWaves], sm_l[kWaves];
  if (lane < kLpr) {
#pragma unroll
    for (int e = 0; e < kEpl; ++e) sm_acc[wave][c * kEpl + e] = acc[e];
    if (lane == 0) {
      sm_m[wave] = m;
      sm_l[wave] = l;
    }
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float M = kNegInf;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, sm_m[w2]);
    const float mu = (M == kNegInf) ? 0.f : M;
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const float a = __builtin_amdgcn_exp2f(sm_m[w2] - mu);
      o = fmaf(a, sm_acc[w2][threadIdx.x], o);
      lsum = fmaf(a, sm_l[w2], lsum);
    }
    if (write_out) {
      store_out<E>(p.out, bh * D + threadIdx.x, o / lsum);  // what the merge of one split computes
    } else {
      po[threadIdx.x] = o;
      if (threadIdx.x == 0) {
        pml[0] = M;
        pml[1] = lsum;
      }
    }
  }
  __syncthreads();  // the LDS above may be reused by the caller's next range
}

// Split-K decode. Grid (H, B, splits), 4 waves. Workgroup (b, h, sp) owns the
// key slots [sp*chunk, min(vis, (sp+1)*chunk)) of (b, h), vis = L_m + min(n, T).
template <class E, int D, int U>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  const int b = blockIdx.y, h = blockIdx.x, sp = blockIdx.z;
  const int64_t bh = (int64_t)b * p.heads + h;
  float *po = p.part_o + (bh * p.splits + sp) * D;
  float *pml = p.part_ml + (bh * p.splits + sp) * 2;
  const bool fused = p.k_new != nullptr;
  const SeqFacts f = seq_facts<Geometry<E, D>::kEpl>(p, b);
  if (sp == 0 && h == 0 && threadIdx.x == 0) {
    p.seq_state[b] = (f.err || !fused) ? -1 : f.T0 + 1;
    if (f.err) atomicOr(p.error, f.err);
  }

  const int start = sp * p.chunk;
  const int end = min(f.vis, start + p.chunk);
  if (f.err || start >= end) {  // empty partial state (one launch: a zero output)
    if (p.one_launch) {
      for (int i = threadIdx.x; i < D; i += 256) store_out<E>(p.out, bh * D + i, 0.f);
      return;
    }
    for (int i = threadIdx.x; i < D; i += 256) po[i] = 0.f;
    if (threadIdx.x == 0) {
      pml[0] = kNegInf;
      pml[1] = 0.f;
    }
    return;
  }
  attend_range<E, D, U>(p, b, h, f, start, end, po, pml, p.one_launch != 0);
  // One fused launch: every workgroup of sequence b read step[b] before it
  // counts itself here, so the last of the H may publish the new step.
  if (p.one_launch && fused && threadIdx.x == 0) {
    if (atomicAdd(&p.arrive[b], 1) == p.heads - 1) {
      atomicExch(&p.arrive[b], 0);
      p.step[b] = f.T0 + 1;
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int64_t wave_inclusive_sum(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Flat work list (a ragged batch). The visible slots of every (sequence, head),
// in order (b, h), form one list of T_all = H * sum_b vis_b slots; workgroup g
// of the G in the grid attends over slots [T_all g / G, T_all (g + 1) / G), so
// every workgroup streams the same number of bytes whatever the lengths. A
// workgroup may cover the end of one (sequence, head) and the start of the next:
// it writes one partial state per (sequence, head) it touches, at index g + s
// (s = b H + h), unique because a later workgroup never touches an earlier
// (sequence, head). Workgroup 0 also publishes the per-sequence prefix sums
// (seq_pre[b] = sum of vis over sequences before b, seq_pre[B] = the total), the
// new step counts for the merge, and the error bits.
template <class E, int D, int U>
__global__ __launch_bounds__(256) void decode_flat_kernel(DecodeParams p) {
  constexpr int kEpl = Geometry<E, D>::kEpl;
  const int lane = threadIdx.x & 63;
  const int gi = blockIdx.x, G = gridDim.x;
  const int B = p.batch, H = p.heads;
  const bool fused = p.k_new != nullptr;

  int64_t total = 0;  // sum of vis over the batch (every wave computes it)
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int64_t vis = 0;
    if (b < B) {
      const SeqFacts f = seq_facts<kEpl>(p, b);
      vis = f.vis;
      if (gi == 0 && threadIdx.x < 64) {
        p.seq_state[b] = (f.err || !fused) ? -1 : f.T0 + 1;
        if (f.err) atomicOr(p.error, f.err);
      }
    }
    const int64_t incl = wave_inclusive_sum(vis);
    if (gi == 0 && threadIdx.x < 64 && b < B) p.seq_pre[b] = total + incl - vis;
    total += __shfl(incl, 63, 64);
  }
  if (gi == 0 && threadIdx.x == 0) p.seq_pre[B] = total;

  const int64_t t_all = total * H;
  const int64_t lo = t_all * gi / G, hi = t_all * (gi + 1) / G;
  if (lo >= hi) return;  // an empty piece (the whole workgroup)

  // The sequence holding slot lo of the list: the first b whose prefix end
  // H * (pre_b + vis_b) exceeds lo.
  int b = 0;
  int64_t pre = 0;  // sum of vis before sequence b
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const int64_t vis = bb < B ? (int64_t)seq_facts<kEpl>(p, bb).vis : 0;
    const int64_t incl = wave_inclusive_sum(vis);
    const uint64_t past = __ballot((pre + incl) * H > lo && bb < B);
    if (past != 0) {
      const int first = __ffsll((unsigned long long)past) - 1;
      b = b0 + first;
      pre += __shfl(incl - vis, first, 64);
      break;
    }
    pre += __shfl(incl, 63, 64);
  }

  // Walk the (sequence, head) ranges of [lo, hi).
  int64_t pos = lo;
  while (pos < hi && b < B) {
    const SeqFacts f = seq_facts<kEpl>(p, b);
    const int64_t seq0 = pre * H;  // first list slot of sequence b
    if (f.vis > 0 && pos < seq0 + (int64_t)f.vis * H) {
      const int h = (int)((pos - seq0) / f.vis);
      const int start = (int)((pos - seq0) - (int64_t)h * f.vis);
      const int end = (int)min((int64_t)f.vis, start + (hi - pos));
      const int64_t idx = gi + (int64_t)b * H + h;
      attend_range<E, D, U>(p, b, h, f, start, end, p.part_o + idx * D, p.part_ml + idx * 2, false);
      pos += end - start;
    } else {
      pre += f.vis;
      ++b;
    }
  }
}

// Merge of the flat work list: grid (H, B), D threads. The list slots of
// (sequence b, head h) are [S, S + vis) with S = H pre_b + h vis; the workgroups
// that covered them are g0 .. g1 (those whose piece [T_all g / G, T_all (g+1) / G)
// is not empty), their partial states at g + b H + h.
template <class E, int D>
__global__ __launch_bounds__(128) void decode_merge_flat_kernel(DecodeParams p) {
  const int b = blockIdx.y, h = blockIdx.x, col = threadIdx.x;
  const int H = p.heads;
  const int64_t G = p.flat_wgs;
  const int64_t bh = (int64_t)b * H + h;
  const int64_t pre = p.seq_pre[b], vis = p.seq_pre[b + 1] - pre;
  const int64_t t_all = p.seq_pre[p.batch] * H;
  float o = 0.f;
  if (vis > 0) {
    const int64_t S = pre * H + (int64_t)h * vis;
    const int64_t g0 = ((S + 1) * G - 1) / t_all, g1 = ((S + vis) * G - 1) / t_all;
    float M = kNegInf;
    for (int64_t g = g0; g <= g1; ++g)
      if (t_all * g / G < t_all * (g + 1) / G) M = fmaxf(M, p.part_ml[(g + bh) * 2]);
    float num = 0.f, den = 0.f;
    for (int64_t g = g0; g <= g1; ++g) {
      if (t_all * g / G == t_all * (g + 1) / G) continue;  // empty piece: wrote nothing
      const float w = __builtin_amdgcn_exp2f(p.part_ml[(g + bh) * 2] - M);
      num = fmaf(w, p.part_o[(g + bh) * D + col], num);
      den = fmaf(w, p.part_ml[(g + bh) * 2 + 1], den);
    }
    o = num / den;
  }
  store_out<E>(p.out, bh * D + col, o);
  if (h == 0 && col == 0 && p.k_new != nullptr) {
    const int32_t next = p.seq_state[b];
    if (next >= 0) p.step[b] = next;
  }
}

// Split merge: grid (H, B), D threads. o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Block (b, 0) publishes the new step count of a fused append.
template <class E, int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
  const int b = blockIdx.y, h = blockIdx.x, col = threadIdx.x;
  const int64_t bh = (int64_t)b * p.heads + h;
  const float *pml = p.part_ml + bh * p.splits * 2;
  const float *po = p.part_o + bh * p.splits * D;
  float M = kNegInf;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, pml[2 * s]);
  float o = 0.f;
  if (M != kNegInf) {
    float num = 0.f, den = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      const float w = __builtin_amdgcn_exp2f(pml[2 * s] - M);
      num = fmaf(w, po[(int64_t)s * D + col], num);
      den = fmaf(w, pml[2 * s + 1], den);
    }
    o = num / den;
  }
  store_out<E>(p.out, bh * D + col, o);
  if (h == 0 && col == 0 && p.k_new != nullptr) {
    const int32_t next = p.seq_state[b];
    if (next >= 0) p.step[b] = next;
  }
}

__global__ void clear_word_kernel(int32_t *w) { *w = 0; }

template <class E, int D>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t s) {
  constexpr int kU = RSWA_DECODE_U;
  // Heads fastest: workgroup i lands on XCD i mod 8, so every sequence's chunks
  // spread over all XCDs whatever the split count (in a ragged batch the later
  // chunks are often empty; with splits fastest they would pile onto a few XCDs).
  if (p.flat_wgs > 0) {
    hipLaunchKernelGGL((decode_flat_kernel<E, D, kU>), dim3(p.flat_wgs), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_flat_kernel<E, D>), dim3(p.heads, p.batch), dim3(D), 0, s, p);
    return hipGetLastError();
  }
  dim3 grid(p.heads, p.batch, p.splits);
  hipLaunchKernelGGL((decode_split_kernel<E, D, kU>), grid, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.one_launch) return e;
  hipLaunchKernelGGL((decode_merge_kernel<E, D>), dim3(p.heads, p.batch), dim3(D), 0, s, p);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_init_t(const InitParams &p, hipStream_t s) {
  const int rows_blocks = p.max_ref_len > 0 ? (p.max_ref_len + 31) / 32 : 1;
  hipLaunchKernelGGL((cache_init_kernel<E, D>), dim3(rows_blocks, p.heads, p.batch), dim3(256), 0,
                     s, p);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_append_t(const AppendParams &p, hipStream_t s) {
  hipLaunchKernelGGL((append_kernel<E, D>), dim3(p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int32_t dtype, int32_t head_dim, hipStream_t s) {
  if (dtype == RSWA_BF16) {
    return head_dim == 128 ? launch_decode_t<Bf16, 128>(p, s) : launch_decode_t<Bf16, 64>(p, s);
  }
  return head_dim == 128 ? launch_decode_t<F32, 128>(p, s) : launch_decode_t<F32, 64>(p, s);
}

hipError_t launch_cache_init(const InitParams &p, int32_t dtype, int32_t head_dim, hipStream_t s) {
  if (dtype == RSWA_BF16) {
    return head_dim == 128 ? launch_init_t<Bf16, 128>(p, s) : launch_init_t<Bf16, 64>(p, s);
  }
  return head_dim == 128 ? launch_init_t<F32, 128>(p, s) : launch_init_t<F32, 64>(p, s);
}

hipError_t launch_append(const AppendParams &p, int32_t dtype, int32_t head_dim, hipStream_t s) {
  if (dtype == RSWA_BF16) {
    return head_dim == 128 ? launch_append_t<Bf16, 128>(p, s) : launch_append_t<Bf16, 64>(p, s);
  }
  return head_dim == 128 ? launch_append_t<F32, 128>(p, s) : launch_append_t<F32, 64>(p, s);
}

hipError_t launch_clear_word(int32_t *word, hipStream_t s) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, s, word);
  return hipGetLastError();
}

}  // namespace rswa
