// Host side of librswa: argument validation (before anything is enqueued),
// the decode split plan and workspace layout, and the extern "C" entry points
// declared in include/rswa.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "rswa_internal.h"

namespace rswa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

#ifndef RSWA_FLAT_WORKGROUPS
#define RSWA_FLAT_WORKGROUPS 512  // workgroups of a flat decode work list (2 per CU)
#endif
constexpr int32_t kMaxBwdParts = 64;

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The packed kernels (head_dim 128) form element offsets in 32 bits and each DMA
// row offset as a 24-bit product (row number times the row pitch of 256 H
// bytes): the tokens x heads x 128 elements stay below 2^31 and the heads below
// 2^16, which also keeps every row number below 2^24.
bool packed_sizes_fit(int64_t tokens, int64_t heads) {
  return tokens * heads * 128 < ((int64_t)1 << 31) && heads < ((int64_t)1 << 16);
}

// Host-visible checks of a cache descriptor (device arrays are checked by the kernels).
rswa_status_t check_cache(const rswa_cache_t *c) {
  if (c == nullptr) return RSWA_ERR_NULL;
  if (c->k == nullptr || c->v == nullptr || c->seq_base == nullptr || c->ref_len == nullptr ||
      c->step == nullptr || c->error == nullptr)
    return RSWA_ERR_NULL;
  if (c->dtype != RSWA_BF16 && c->dtype != RSWA_FP32) return RSWA_ERR_UNSUPPORTED;
  if (c->batch < 1 || c->num_heads < 1 || c->window < 1 || c->max_ref_len < 0)
    return RSWA_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return RSWA_ERR_UNSUPPORTED;
  // slot indices are int32; one sequence block must be addressable in int64
  const int64_t max_len = (int64_t)c->max_ref_len + c->window;
  if (max_len > INT32_MAX) return RSWA_ERR_CAPACITY;
  if ((int64_t)c->batch * c->num_heads > INT32_MAX / 2) return RSWA_ERR_CAPACITY;
  if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->error)) return RSWA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(c->arrive) & 3u) != 0) return RSWA_ERR_ALIGN;
  return RSWA_OK;
}

bool verbose() {
  const char *e = getenv("RSWA_LOG");
  return e != nullptr && e[0] == '1';
}

}  // namespace

SplitPlan plan_decode_splits(int32_t batch, int32_t heads, int32_t max_len, int32_t requested) {
  // Default: about 4 workgroups per CU (1024 over the 256 CUs) -- where a plain
  // non-temporal read stream peaks on MI355X -- but never chunks below 64 slots,
  // and never above 2048: per-sequence lengths live on the device, and in a
  // ragged batch a cap on the chunk keeps one long sequence from becoming one
  // long workgroup (measured: 64 sequences of 289..12960 slots, 0.58 ms with no
  // cap, 0.51 ms with 4096, 0.50 ms with 2048; a batch of 32 sequences of 16416
  // slots 624 -> 627 us with 2048; 4 sequences of 10400 slots unchanged).
  constexpr int64_t kTargetWorkgroups = 1024;
  constexpr int32_t kMinChunk = 64;
  constexpr int32_t kMaxChunk = 2048;
  const int64_t bh = (int64_t)batch * heads;
  const int32_t len = max_len > 0 ? max_len : 1;
  // One workgroup per (sequence, head), written out without a merge launch,
  // when the batch alone gives every CU two workgroups and every sequence fits
  // a chunk of 12288 slots (measured: 40-page batch 394 vs 399 us a step; a
  // ragged batch of up to 12960 slots keeps the split chunks, 526 vs 590 us).
  // Small steps keep many short chunks: there the kernel's own latency, not
  // the merge launch, sets the GPU time (one page, 12 layers in one graph:
  // 86 us with split chunks, 115 us with one chunk per head).
  constexpr int64_t kOneChunkMin = 512;
  constexpr int32_t kOneChunkMaxLen = 12288;
  if (requested <= 0 && bh >= kOneChunkMin && len <= kOneChunkMaxLen) return SplitPlan{1, len, 0};
  // Otherwise, for a large step (at least 4M slots of capacity), the flat work
  // list: every workgroup streams the same number of visible slots whatever the
  // per-sequence lengths (a ragged batch), with no empty workgroup and no long
  // tail (measured: the 64-sequence ragged batch 501 -> 491 us, 32 sequences of
  // 16416 slots 628 -> 623 us; smaller steps, e.g. 8 or 2 sequences of 10400
  // slots, keep the per-(sequence, head) chunks: 105 vs 116 us, 33 vs 41 us).
  constexpr int64_t kFlatWorkgroups = RSWA_FLAT_WORKGROUPS;
  constexpr int64_t kFlatMinSlots = (int64_t)1 << 22;
  if (requested <= 0 && bh * len >= kFlatMinSlots && bh * len < ((int64_t)1 << 50))
    return SplitPlan{0, 0, (int32_t)kFlatWorkgroups};
  int64_t s = requested > 0 ? requested : (kTargetWorkgroups + bh - 1) / bh;
  if (requested <= 0) {
    s = std::max<int64_t>(s, (len + kMaxChunk - 1) / kMaxChunk);
    s = std::min<int64_t>(s, (len + kMinChunk - 1) / kMinChunk);
  }
  s = std::max<int64_t>(1, std::min<int64_t>(s, len));
  int64_t chunk = (len + s - 1) / s;
  if (requested <= 0) chunk = round_up((size_t)chunk, kMinChunk);
  const int64_t splits = (len + chunk - 1) / chunk;
  return SplitPlan{(int32_t)splits, (int32_t)chunk, 0};
}

WorkspaceLayout decode_workspace_layout(int32_t batch, int32_t heads, int32_t head_dim,
                                        const SplitPlan &plan) {
  WorkspaceLayout w{};
  const size_t bh = (size_t)batch * heads;
  const size_t units = plan.flat_wgs > 0 ? plan.flat_wgs + bh : bh * plan.splits;
  w.part_o = 0;
  w.part_ml = round_up(units * head_dim * sizeof(float), 256);
  w.seq_state = w.part_ml + round_up(units * 2 * sizeof(float), 256);
  w.seq_pre = w.seq_state + round_up((size_t)batch * sizeof(int32_t), 256);
  w.total = w.seq_pre + (plan.flat_wgs > 0 ? round_up(((size_t)batch + 1) * sizeof(int64_t), 256) : 0);
  return w;
}

BwdPlan plan_masked_bwd(int32_t seq_len, int32_t ref_len, int32_t heads, int32_t requested_parts) {
  BwdPlan b{};
  b.n_pad = (seq_len + 31) / 32 * 32;
  b.nkb_pre = (ref_len + 127) / 128;
  b.nkb_win = (seq_len + 127) / 128 - b.nkb_pre;
  b.kpre = 128 * b.nkb_pre;
  // A reference-segment key block walks up to ceil(seq_len / 32) query blocks;
  // runs of about 256 blocks keep those walks from setting the kernel's length.
  int32_t parts = requested_parts;
  if (parts == 0) parts = ((seq_len + 31) / 32 + 255) / 256;
  if (parts < 1) parts = 1;
  if (b.nkb_pre == 0) parts = 1;
  b.parts = parts;
  b.bytes_rows = 2 * (size_t)heads * b.n_pad * sizeof(float);
  b.bytes_parts = parts > 1 ? 2 * (size_t)parts * heads * b.kpre * 128 * sizeof(float) : 0;
  return b;
}

}  // namespace rswa

using namespace rswa;

extern "C" {

int32_t rswa_abi_version(void) { return RSWA_ABI_VERSION; }

const char *rswa_status_str(int32_t status) {
  switch (status) {
    case RSWA_OK: return "ok";
    case RSWA_ERR_NULL: return "required pointer is NULL";
    case RSWA_ERR_SHAPE: return "size or shape argument out of range";
    case RSWA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim or mode";
    case RSWA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case RSWA_ERR_CAPACITY: return "sizes overflow the index range";
    case RSWA_ERR_WORKSPACE: return "workspace missing or too small";
    case RSWA_ERR_STATE: return "device-side state invalid";
    case RSWA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

rswa_status_t rswa_cache_init(const rswa_cache_t *cache, const void *k_ref, const void *v_ref,
                              const int64_t *ref_base, void *stream) {
  rswa_status_t st = check_cache(cache);
  if (st != RSWA_OK) return st;
  // An empty reference (max_ref_len == 0) needs no source buffers.
  if (cache->max_ref_len > 0 && (k_ref == nullptr || v_ref == nullptr || ref_base == nullptr))
    return RSWA_ERR_NULL;
  if (!aligned16(k_ref) || !aligned16(v_ref)) return RSWA_ERR_ALIGN;
  InitParams p{};
  p.k_ref = k_ref;
  p.v_ref = v_ref;
  p.ref_base = ref_base;
  p.k = cache->k;
  p.v = cache->v;
  p.seq_base = cache->seq_base;
  p.ref_len = cache->ref_len;
  p.step = cache->step;
  p.error = cache->error;
  p.arrive = cache->arrive;
  p.batch = cache->batch;
  p.heads = cache->num_heads;
  p.window = cache->window;
  p.max_ref_len = cache->max_ref_len;
  const hipError_t e = launch_cache_init(p, cache->dtype, cache->head_dim,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_append_kv(const rswa_cache_t *cache, const void *k_new, const void *v_new,
                             const uint8_t *active, void *stream) {
  rswa_status_t st = check_cache(cache);
  if (st != RSWA_OK) return st;
  if (k_new == nullptr || v_new == nullptr) return RSWA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return RSWA_ERR_ALIGN;
  AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.active = active;
  p.k = cache->k;
  p.v = cache->v;
  p.seq_base = cache->seq_base;
  p.ref_len = cache->ref_len;
  p.step = cache->step;
  p.error = cache->error;
  p.batch = cache->batch;
  p.heads = cache->num_heads;
  p.window = cache->window;
  p.max_ref_len = cache->max_ref_len;
  const hipError_t e = launch_append(p, cache->dtype, cache->head_dim,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

size_t rswa_workspace_size(int32_t batch, int32_t num_heads, int32_t head_dim, int32_t max_len) {
  if (batch < 1 || num_heads < 1 || (head_dim != 64 && head_dim != 128) || max_len < 1) return 0;
  if ((int64_t)batch * num_heads > INT32_MAX / 2) return 0;
  const SplitPlan plan = plan_decode_splits(batch, num_heads, max_len, 0);
  return decode_workspace_layout(batch, num_heads, head_dim, plan).total;
}

size_t rswa_decode_workspace_size(const rswa_cache_t *cache, int32_t num_splits) {
  if (check_cache(cache) != RSWA_OK || num_splits < 0) return 0;
  const SplitPlan plan = plan_decode_splits(cache->batch, cache->num_heads,
                                            cache->max_ref_len + cache->window, num_splits);
  return decode_workspace_layout(cache->batch, cache->num_heads, cache->head_dim, plan).total;
}

}  // extern "C"

namespace rswa {
namespace {

// Checks of a decode call that do not involve its workspace.
rswa_status_t check_decode_args(const rswa_cache_t *cache, const void *q, const void *out,
                                const void *k_new, const void *v_new, float scale,
                                int32_t num_splits) {
  rswa_status_t st = check_cache(cache);
  if (st != RSWA_OK) return st;
  if (q == nullptr || out == nullptr) return RSWA_ERR_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return RSWA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out)) return RSWA_ERR_ALIGN;
  if (k_new != nullptr && (!aligned16(k_new) || !aligned16(v_new))) return RSWA_ERR_ALIGN;
  if (!isfinite(scale)) return RSWA_ERR_SHAPE;
  if (num_splits < 0) return RSWA_ERR_SHAPE;
  return RSWA_OK;
}

// ---------------------------------------------------------------------------
// Library-owned decode workspace for callers that cannot allocate device
// memory (rswa_decode_attn_noalloc). Each GPU holds its own copy of `scratch`
// until the process ends; host code uses only the device address looked up
// per device, never the array's name (a host-side stand-in).
constexpr size_t kScratchBytes = (size_t)RSWA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up once per device, under a lock).
rswa_status_t scratch_for_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return RSWA_ERR_HIP;
  if (dev >= kMaxDevices) return RSWA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return RSWA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RSWA_OK;
}

}  // namespace
}  // namespace rswa

extern "C" {

rswa_status_t rswa_decode_attn(const rswa_cache_t *cache, const void *q, void *out,
                               const void *k_new, const void *v_new, float scale,
                               int32_t num_splits, void *workspace, size_t workspace_bytes,
                               void *stream) {
  const rswa_status_t st = check_decode_args(cache, q, out, k_new, v_new, scale, num_splits);
  if (st != RSWA_OK) return st;
  const SplitPlan plan = plan_decode_splits(cache->batch, cache->num_heads,
                                            cache->max_ref_len + cache->window, num_splits);
  const WorkspaceLayout ws = decode_workspace_layout(cache->batch, cache->num_heads,
                                                     cache->head_dim, plan);
  if (workspace == nullptr) return RSWA_ERR_WORKSPACE;
  if (workspace_bytes < ws.total) return RSWA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RSWA_ERR_ALIGN;
  char *wsb = static_cast<char *>(workspace);
  DecodeParams p{};
  p.q = q;
  p.out = out;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k = cache->k;
  p.v = cache->v;
  p.seq_base = cache->seq_base;
  p.ref_len = cache->ref_len;
  p.step = cache->step;
  p.error = cache->error;
  p.part_o = reinterpret_cast<float *>(wsb + ws.part_o);
  p.part_ml = reinterpret_cast<float *>(wsb + ws.part_ml);
  p.seq_state = reinterpret_cast<int32_t *>(wsb + ws.seq_state);
  p.seq_pre = reinterpret_cast<int64_t *>(wsb + ws.seq_pre);
  p.flat_wgs = plan.flat_wgs;
  p.arrive = cache->arrive;
  p.one_launch = plan.flat_wgs == 0 && plan.splits == 1 && (k_new == nullptr || cache->arrive != nullptr);
  p.batch = cache->batch;
  p.heads = cache->num_heads;
  p.window = cache->window;
  p.max_ref_len = cache->max_ref_len;
  p.splits = plan.splits;
  p.chunk = plan.chunk;
  const float sc = scale == 0.f ? 1.f / sqrtf((float)cache->head_dim) : scale;
  p.scale_log2 = sc * kLog2e;
  if (verbose()) {
    fprintf(stderr, "[rswa] decode B=%d H=%d d=%d n=%d maxL=%d splits=%d chunk=%d flat_wgs=%d fused=%d one_launch=%d\n",
            p.batch, p.heads, cache->head_dim, p.window, p.max_ref_len, p.splits, p.chunk,
            p.flat_wgs, k_new != nullptr, p.one_launch);
  }
  const hipError_t e = launch_decode(p, cache->dtype, cache->head_dim,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_decode_attn_noalloc(const rswa_cache_t *cache, const void *q, void *out,
                                       const void *k_new, const void *v_new, float scale,
                                       int32_t num_splits, void *stream) {
  const rswa_status_t st = check_decode_args(cache, q, out, k_new, v_new, scale, num_splits);
  if (st != RSWA_OK) return st;
  if (rswa_decode_workspace_size(cache, num_splits) > kScratchBytes) return RSWA_ERR_WORKSPACE;
  void *ws = nullptr;
  const rswa_status_t sst = scratch_for_current_device(&ws);
  if (sst != RSWA_OK) return sst;
  return rswa_decode_attn(cache, q, out, k_new, v_new, scale, num_splits, ws, kScratchBytes, stream);
}

rswa_status_t rswa_masked_attn(const void *q, const void *k, const void *v, void *out,
                               float *lse, int32_t seq_len, int32_t ref_len, int32_t window,
                               int32_t num_heads, int32_t head_dim, int32_t dtype,
                               int32_t prefix_mode, float scale, void *stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return RSWA_ERR_NULL;
  if (seq_len < 0 || ref_len < 0 || ref_len > seq_len || window < 1 || num_heads < 1)
    return RSWA_ERR_SHAPE;
  if (dtype != RSWA_BF16 || head_dim != 128) return RSWA_ERR_UNSUPPORTED;
  if (prefix_mode != RSWA_PREFIX_CAUSAL && prefix_mode != RSWA_PREFIX_FULL)
    return RSWA_ERR_UNSUPPORTED;
  if (!packed_sizes_fit(seq_len, num_heads)) return RSWA_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RSWA_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return RSWA_ERR_ALIGN;
  if (!isfinite(scale) || scale < 0.f) return RSWA_ERR_SHAPE;  // see rswa_masked_attn
  if (seq_len == 0) return RSWA_OK;
  MaskedParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.num_seqs = 1;
  p.max_seq_len = seq_len;
  p.seq_len = seq_len;
  p.ref_len = ref_len;
  p.window = window;
  p.heads = num_heads;
  p.prefix_mode = prefix_mode;
  const float sc = scale == 0.f ? 1.f / sqrtf((float)head_dim) : scale;
  p.scale_log2 = sc * kLog2e;
  const hipError_t e = launch_masked(p, head_dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_masked_attn_varlen(const void *q, const void *k, const void *v, void *out,
                                      float *lse, const int32_t *cu_seqlens,
                                      const int32_t *ref_lens, int32_t num_seqs,
                                      int32_t total_tokens, int32_t max_seq_len, int32_t window,
                                      int32_t num_heads, int32_t head_dim, int32_t dtype,
                                      int32_t prefix_mode, float scale, void *stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || cu_seqlens == nullptr ||
      ref_lens == nullptr)
    return RSWA_ERR_NULL;
  if (num_seqs < 0 || total_tokens < 0 || max_seq_len < 0 || window < 1 || num_heads < 1)
    return RSWA_ERR_SHAPE;
  if (dtype != RSWA_BF16 || head_dim != 128) return RSWA_ERR_UNSUPPORTED;
  if (prefix_mode != RSWA_PREFIX_CAUSAL && prefix_mode != RSWA_PREFIX_FULL)
    return RSWA_ERR_UNSUPPORTED;
  if (!packed_sizes_fit(total_tokens, num_heads)) return RSWA_ERR_CAPACITY;
  if ((int64_t)num_seqs * num_heads * ((max_seq_len + 127) / 128) >= ((int64_t)1 << 31))
    return RSWA_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RSWA_ERR_ALIGN;
  if (((reinterpret_cast<uintptr_t>(cu_seqlens) | reinterpret_cast<uintptr_t>(ref_lens)) & 3u) != 0)
    return RSWA_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return RSWA_ERR_ALIGN;
  if (!isfinite(scale) || scale < 0.f) return RSWA_ERR_SHAPE;  // see rswa_masked_attn
  if (num_seqs == 0 || total_tokens == 0 || max_seq_len == 0) return RSWA_OK;
  MaskedParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.ref_lens = ref_lens;
  p.num_seqs = num_seqs;
  p.max_seq_len = max_seq_len;
  p.seq_len = total_tokens;
  p.window = window;
  p.heads = num_heads;
  p.prefix_mode = prefix_mode;
  const float sc = scale == 0.f ? 1.f / sqrtf((float)head_dim) : scale;
  p.scale_log2 = sc * kLog2e;
  const hipError_t e = launch_masked(p, head_dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_prefill(const rswa_cache_t *cache, const void *q, const void *k, const void *v,
                           void *out, float *lse, const int32_t *cu_seqlens, int32_t total_tokens,
                           int32_t max_seq_len, int32_t prefix_mode, float scale, void *stream) {
  const rswa_status_t st = check_cache(cache);
  if (st != RSWA_OK) return st;
  if (cache->dtype != RSWA_BF16 || cache->head_dim != 128) return RSWA_ERR_UNSUPPORTED;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || cu_seqlens == nullptr)
    return RSWA_ERR_NULL;
  if (total_tokens < 0 || max_seq_len < 0) return RSWA_ERR_SHAPE;
  if (prefix_mode != RSWA_PREFIX_CAUSAL && prefix_mode != RSWA_PREFIX_FULL)
    return RSWA_ERR_UNSUPPORTED;
  if (!packed_sizes_fit(total_tokens, cache->num_heads)) return RSWA_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RSWA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return RSWA_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return RSWA_ERR_ALIGN;
  if (!isfinite(scale) || scale < 0.f) return RSWA_ERR_SHAPE;  // see rswa_masked_attn
  const int64_t qblocks = max_seq_len > 0 ? (max_seq_len + 127) / 128 : 1;
  if ((int64_t)cache->batch * cache->num_heads * qblocks >= ((int64_t)1 << 31)) return RSWA_ERR_CAPACITY;
  // One launch: the packed forward with the hand-off fused in (every sequence
  // gets at least one workgroup per head, so empty samples still publish step[b]).
  MaskedParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.ref_lens = cache->ref_len;
  p.num_seqs = cache->batch;
  p.max_seq_len = max_seq_len;
  p.seq_len = total_tokens;
  p.window = cache->window;
  p.heads = cache->num_heads;
  p.prefix_mode = prefix_mode;
  const float sc = scale == 0.f ? 1.f / sqrtf((float)cache->head_dim) : scale;
  p.scale_log2 = sc * kLog2e;
  p.cache_k = cache->k;
  p.cache_v = cache->v;
  p.seq_base = cache->seq_base;
  p.step = cache->step;
  p.error = cache->error;
  p.arrive = cache->arrive;
  p.max_ref_len = cache->max_ref_len;
  const hipError_t e = launch_masked(p, cache->head_dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

size_t rswa_masked_bwd_workspace_size(int32_t seq_len, int32_t ref_len, int32_t num_heads,
                                      int32_t num_parts) {
  if (seq_len < 0 || ref_len < 0 || ref_len > seq_len || num_heads < 1 || num_parts < 0 ||
      num_parts > kMaxBwdParts || !packed_sizes_fit(seq_len, num_heads))
    return 0;
  const BwdPlan b = plan_masked_bwd(seq_len, ref_len, num_heads, num_parts);
  return b.bytes_rows + b.bytes_parts;
}

rswa_status_t rswa_masked_attn_bwd(const void *q, const void *k, const void *v, const void *out,
                                   const void *dout, const float *lse, void *dq, void *dk,
                                   void *dv, int32_t seq_len, int32_t ref_len, int32_t window,
                                   int32_t num_heads, int32_t head_dim, int32_t dtype,
                                   int32_t prefix_mode, float scale, int32_t num_parts,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr ||
      lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return RSWA_ERR_NULL;
  if (seq_len < 0 || ref_len < 0 || ref_len > seq_len || window < 1 || num_heads < 1)
    return RSWA_ERR_SHAPE;
  if (dtype != RSWA_BF16 || head_dim != 128) return RSWA_ERR_UNSUPPORTED;
  if (prefix_mode != RSWA_PREFIX_CAUSAL && prefix_mode != RSWA_PREFIX_FULL)
    return RSWA_ERR_UNSUPPORTED;
  if (!packed_sizes_fit(seq_len, num_heads)) return RSWA_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return RSWA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return RSWA_ERR_ALIGN;
  if (!isfinite(scale) || scale < 0.f) return RSWA_ERR_SHAPE;  // see rswa_masked_attn
  if (num_parts < 0 || num_parts > kMaxBwdParts) return RSWA_ERR_SHAPE;
  if (seq_len == 0) return RSWA_OK;
  const BwdPlan plan = plan_masked_bwd(seq_len, ref_len, num_heads, num_parts);
  const size_t need = plan.bytes_rows + plan.bytes_parts;
  if (workspace == nullptr) return RSWA_ERR_NULL;
  if (!aligned16(workspace)) return RSWA_ERR_ALIGN;
  if (workspace_bytes < need) return RSWA_ERR_WORKSPACE;
  MaskedBwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.seq_len = seq_len;
  p.n_pad = plan.n_pad;
  p.nd_row = static_cast<float *>(workspace);
  p.nls = p.nd_row + (size_t)num_heads * p.n_pad;
  p.parts = plan.parts;
  p.nkb_pre = plan.nkb_pre;
  p.nkb_win = plan.nkb_win;
  p.kpre = plan.kpre;
  if (plan.parts > 1) {
    p.part_dk = p.nls + (size_t)num_heads * p.n_pad;
    p.part_dv = p.part_dk + (size_t)plan.parts * num_heads * plan.kpre * 128;
  }
  p.ref_len = ref_len;
  p.window = window;
  p.heads = num_heads;
  p.prefix_mode = prefix_mode;
  p.scale = scale == 0.f ? 1.f / sqrtf((float)head_dim) : scale;
  p.scale_log2 = p.scale * kLog2e;
  const hipError_t e = launch_masked_bwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

size_t rswa_masked_bwd_varlen_workspace_size(int32_t total_tokens, int32_t num_heads) {
  if (total_tokens < 0 || num_heads < 1 || !packed_sizes_fit(total_tokens, num_heads)) return 0;
  const size_t n_pad = ((size_t)total_tokens + 31) / 32 * 32;
  return 2 * (size_t)num_heads * n_pad * sizeof(float);
}

rswa_status_t rswa_masked_attn_bwd_varlen(const void *q, const void *k, const void *v,
                                          const void *out, const void *dout, const float *lse,
                                          void *dq, void *dk, void *dv,
                                          const int32_t *cu_seqlens, const int32_t *ref_lens,
                                          int32_t num_seqs, int32_t total_tokens,
                                          int32_t max_seq_len, int32_t window, int32_t num_heads,
                                          int32_t head_dim, int32_t dtype, int32_t prefix_mode,
                                          float scale, void *workspace, size_t workspace_bytes,
                                          void *stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr ||
      lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || cu_seqlens == nullptr ||
      ref_lens == nullptr)
    return RSWA_ERR_NULL;
  if (num_seqs < 0 || total_tokens < 0 || max_seq_len < 0 || window < 1 || num_heads < 1)
    return RSWA_ERR_SHAPE;
  if (dtype != RSWA_BF16 || head_dim != 128) return RSWA_ERR_UNSUPPORTED;
  if (prefix_mode != RSWA_PREFIX_CAUSAL && prefix_mode != RSWA_PREFIX_FULL)
    return RSWA_ERR_UNSUPPORTED;
  if (!packed_sizes_fit(total_tokens, num_heads)) return RSWA_ERR_CAPACITY;
  if ((int64_t)num_seqs * num_heads * ((max_seq_len + 127) / 128) >= ((int64_t)1 << 31))
    return RSWA_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return RSWA_ERR_ALIGN;
  if (((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(cu_seqlens) |
        reinterpret_cast<uintptr_t>(ref_lens)) & 3u) != 0)
    return RSWA_ERR_ALIGN;
  if (!isfinite(scale) || scale < 0.f) return RSWA_ERR_SHAPE;  // see rswa_masked_attn
  if (num_seqs == 0 || total_tokens == 0 || max_seq_len == 0) return RSWA_OK;
  const size_t need = rswa_masked_bwd_varlen_workspace_size(total_tokens, num_heads);
  if (workspace == nullptr) return RSWA_ERR_NULL;
  if (!aligned16(workspace)) return RSWA_ERR_ALIGN;
  if (workspace_bytes < need) return RSWA_ERR_WORKSPACE;
  MaskedBwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.seq_len = total_tokens;
  p.n_pad = (int32_t)(need / (2 * (size_t)num_heads * sizeof(float)));
  p.nd_row = static_cast<float *>(workspace);
  p.nls = p.nd_row + (size_t)num_heads * p.n_pad;
  p.parts = 1;
  p.cu_seqlens = cu_seqlens;
  p.ref_lens = ref_lens;
  p.num_seqs = num_seqs;
  p.max_seq_len = max_seq_len;
  p.window = window;
  p.heads = num_heads;
  p.prefix_mode = prefix_mode;
  p.scale = scale == 0.f ? 1.f / sqrtf((float)head_dim) : scale;
  p.scale_log2 = p.scale * kLog2e;
  const hipError_t e = launch_masked_bwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

struct rswa_decode_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
  int32_t layers;
};

rswa_status_t rswa_decode_graph_create(const rswa_cache_t *caches, int32_t num_layers,
                                       const void *const *q, void *const *out,
                                       const void *const *k_new, const void *const *v_new,
                                       float scale, int32_t num_splits, void *workspace,
                                       size_t workspace_bytes, rswa_decode_graph_t **graph) {
  if (graph == nullptr) return RSWA_ERR_NULL;
  *graph = nullptr;
  if (caches == nullptr || q == nullptr || out == nullptr) return RSWA_ERR_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return RSWA_ERR_NULL;
  if (num_layers < 1) return RSWA_ERR_SHAPE;
  // Every layer is validated before anything is captured.
  for (int32_t l = 0; l < num_layers; ++l) {
    const rswa_cache_t *c = &caches[l];
    rswa_status_t st = check_cache(c);
    if (st != RSWA_OK) return st;
    if (q[l] == nullptr || out[l] == nullptr) return RSWA_ERR_NULL;
    if (k_new != nullptr && ((k_new[l] == nullptr) != (v_new[l] == nullptr))) return RSWA_ERR_NULL;
    if (!aligned16(q[l]) || !aligned16(out[l])) return RSWA_ERR_ALIGN;
    if (k_new != nullptr && k_new[l] != nullptr && (!aligned16(k_new[l]) || !aligned16(v_new[l])))
      return RSWA_ERR_ALIGN;
    if (!isfinite(scale) || num_splits < 0) return RSWA_ERR_SHAPE;
    if (workspace == nullptr || workspace_bytes < rswa_decode_workspace_size(c, num_splits))
      return RSWA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return RSWA_ERR_ALIGN;
  }
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return RSWA_ERR_HIP;
  if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(s);
    return RSWA_ERR_HIP;
  }
  rswa_status_t st = RSWA_OK;
  for (int32_t l = 0; l < num_layers && st == RSWA_OK; ++l)
    st = rswa_decode_attn(&caches[l], q[l], out[l], k_new != nullptr ? k_new[l] : nullptr,
                          v_new != nullptr ? v_new[l] : nullptr, scale, num_splits, workspace,
                          workspace_bytes, s);
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(s, &g);
  (void)hipStreamDestroy(s);
  if (st != RSWA_OK || ec != hipSuccess || g == nullptr) {
    if (g != nullptr) (void)hipGraphDestroy(g);
    return st != RSWA_OK ? st : RSWA_ERR_HIP;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return RSWA_ERR_HIP;
  }
  *graph = new rswa_decode_graph{g, exec, num_layers};
  return RSWA_OK;
}

rswa_status_t rswa_decode_graph_launch(const rswa_decode_graph_t *graph, void *stream) {
  if (graph == nullptr) return RSWA_ERR_NULL;
  return hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? RSWA_OK
                                                                                      : RSWA_ERR_HIP;
}

rswa_status_t rswa_decode_graph_destroy(rswa_decode_graph_t *graph) {
  if (graph == nullptr) return RSWA_OK;
  const bool ok = hipGraphExecDestroy(graph->exec) == hipSuccess && hipGraphDestroy(graph->graph) == hipSuccess;
  delete graph;
  return ok ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_probe_stream_read(const void *buf, size_t bytes, float *sink, int32_t workgroups,
                                     void *stream) {
  if (buf == nullptr || sink == nullptr) return RSWA_ERR_NULL;
  if (bytes % 16 != 0 || workgroups < 0) return RSWA_ERR_SHAPE;
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return RSWA_ERR_ALIGN;
  if (bytes == 0) return RSWA_OK;
  const hipError_t e = launch_probe_read(buf, bytes, sink, workgroups == 0 ? 1024 : workgroups,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_probe_mfma(float *sink, int32_t workgroups, int32_t iters, void *stream) {
  if (sink == nullptr) return RSWA_ERR_NULL;
  if (workgroups < 0 || iters < 1) return RSWA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return RSWA_ERR_ALIGN;
  const hipError_t e = launch_probe_mfma(sink, workgroups == 0 ? 512 : workgroups, iters,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_probe_cu(uint32_t *out, int32_t workgroups, int32_t iters, int32_t kind, void *stream) {
  if (out == nullptr) return RSWA_ERR_NULL;
  if (workgroups < 0 || iters < 1 || kind < RSWA_PROBE_LDS_B128 || kind > RSWA_PROBE_FMA) return RSWA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0) return RSWA_ERR_ALIGN;
  const hipError_t e = launch_probe_cu(out, workgroups == 0 ? 256 : workgroups, iters, kind,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RSWA_OK : RSWA_ERR_HIP;
}

rswa_status_t rswa_device_facts(int32_t device, int64_t *out, int32_t count) {
  if (out == nullptr) return RSWA_ERR_NULL;
  if (device < 0 || count < 1) return RSWA_ERR_SHAPE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return RSWA_ERR_HIP;
  const int64_t facts[RSWA_FACT_COUNT] = {
      prop.multiProcessorCount,          (int64_t)prop.maxSharedMemoryPerMultiProcessor,
      prop.l2CacheSize,                  prop.clockRate,
      prop.memoryClockRate,              prop.memoryBusWidth,
      (int64_t)prop.totalGlobalMem,      prop.warpSize};
  for (int i = 0; i < count && i < RSWA_FACT_COUNT; ++i) out[i] = facts[i];
  return RSWA_OK;
}

rswa_status_t rswa_check_device_error(const rswa_cache_t *cache, int32_t *flags, void *stream) {
  if (cache == nullptr || cache->error == nullptr || flags == nullptr) return RSWA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t word = 0;
  if (hipMemcpyAsync(&word, cache->error, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess)
    return RSWA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return RSWA_ERR_HIP;
  *flags = word;
  if (word != 0) {
    if (launch_clear_word(cache->error, s) != hipSuccess) return RSWA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return RSWA_ERR_HIP;
    return RSWA_ERR_STATE;
  }
  return RSWA_OK;
}

}  // extern "C"
