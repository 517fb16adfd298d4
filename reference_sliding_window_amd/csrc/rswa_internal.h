// Internal declarations shared by the host API and the kernel files of librswa.
// Not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rswa.h"

namespace rswa {

// Work split of one decode launch: every (sequence, head) is cut into `splits`
// chunks of `chunk` key slots, each chunk one workgroup; or, when flat_wgs > 0,
// the visible slots of all (sequence, head) pairs form one list cut into
// flat_wgs equal pieces, one per workgroup.
struct SplitPlan {
  int32_t splits;
  int32_t chunk;
  int32_t flat_wgs;
};

// Chooses the split plan from host-known sizes only (the per-sequence lengths
// live on the device). requested = 0 selects the library's choice.
SplitPlan plan_decode_splits(int32_t batch, int32_t heads, int32_t max_len, int32_t requested);

// Byte layout of the decode workspace. Partial states: [B*H][splits] for
// per-(sequence, head) chunks, [flat_wgs + B*H] for the flat list.
struct WorkspaceLayout {
  size_t part_o;     // float [units][d]: unnormalised partial outputs
  size_t part_ml;    // float [units][2]: running max (base 2) and sum
  size_t seq_state;  // int32 [B]: new step value for the merge pass, or -1
  size_t seq_pre;    // int64 [B + 1]: flat list, visible slots before sequence b
  size_t total;
};
WorkspaceLayout decode_workspace_layout(int32_t batch, int32_t heads, int32_t head_dim,
                                        const SplitPlan &plan);

struct DecodeParams {
  const void *q;
  void *out;
  const void *k_new;  // nullptr: attend only
  const void *v_new;
  void *k;
  void *v;
  const int64_t *seq_base;
  const int32_t *ref_len;
  int32_t *step;
  int32_t *error;
  float *part_o;
  float *part_ml;
  int32_t *seq_state;
  int64_t *seq_pre;  // flat list only
  // One launch (splits == 1 and, for a fused call, arrival counters given): the
  // split kernel writes out itself; the last of a sequence's H workgroups to
  // count itself in arrive[b] publishes step[b] and sets arrive[b] back to 0.
  int32_t *arrive;
  int32_t one_launch;
  int32_t batch, heads, window, max_ref_len;
  int32_t splits, chunk;
  int32_t flat_wgs;  // > 0: flat work list over this many workgroups
  float scale_log2;  // softmax scale * log2(e)
};

struct AppendParams {
  const void *k_new;
  const void *v_new;
  const uint8_t *active;
  void *k;
  void *v;
  const int64_t *seq_base;
  const int32_t *ref_len;
  int32_t *step;
  int32_t *error;
  int32_t batch, heads, window, max_ref_len;
};

struct InitParams {
  const void *k_ref;
  const void *v_ref;
  const int64_t *ref_base;
  void *k;
  void *v;
  const int64_t *seq_base;
  const int32_t *ref_len;
  int32_t *step;
  int32_t *error;
  int32_t *arrive;  // nullable
  int32_t batch, heads, window, max_ref_len;
};

struct MaskedParams {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  float *lse;  // nullable [H][seq_len], natural log of each row's softmax normaliser
  // Several samples per pack: cu_seqlens (device [num_seqs + 1]) and ref_lens
  // (device [num_seqs]); nullptr for one sequence of seq_len rows and ref_len.
  const int32_t *cu_seqlens;
  const int32_t *ref_lens;
  int32_t num_seqs, max_seq_len;
  int32_t seq_len, ref_len, window, heads, prefix_mode;  // seq_len: total rows of the pack
  float scale_log2;
  // Prefill hand-off (cache_k == nullptr: none). Sample b of the pack is cache
  // sequence b, ref_lens is the cache's ref_len[] and window the cache's n: the
  // reference rows and the last min(n, T0) output rows (T0 = rows - ref_len[b])
  // are also written into their slots, and step[b] = T0.
  void *cache_k;
  void *cache_v;
  const int64_t *seq_base;
  int32_t *step;
  int32_t *error;
  int32_t *arrive;  // nullable: the cache's decode arrival counters, reset with step
  int32_t max_ref_len;
};

struct MaskedBwdParams {
  const void *q;
  const void *k;
  const void *v;
  const void *out;
  const void *dout;
  const float *lse;  // [H][N], natural log
  void *dq;
  void *dk;
  void *dv;
  float *nd_row;   // workspace [H][n_pad]: -(dO_i . O_i), written by the dQ kernel
  float *nls;      // workspace [H][n_pad]: -lse_i / scale (raw score units), likewise
  float *part_dk;  // workspace [parts][H][kpre][d]: partial dK of the segment's key blocks
  float *part_dv;  // workspace [parts][H][kpre][d]
  int32_t seq_len, n_pad, ref_len, window, heads, prefix_mode;
  int32_t parts;    // runs each reference-segment key block's query walk is cut into
  int32_t nkb_pre;  // 128-key blocks starting below ref_len
  int32_t nkb_win;  // the remaining 128-key blocks
  int32_t kpre;     // 128 * nkb_pre
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  // Pack of independent samples (nullptr: one sequence of seq_len rows).
  // Sample s is rows [cu_seqlens[s], cu_seqlens[s + 1]) with reference length
  // ref_lens[s] (device arrays); seq_len is then the pack's total rows and
  // parts is 1.
  const int32_t *cu_seqlens;
  const int32_t *ref_lens;
  int32_t num_seqs;
  int32_t max_seq_len;
};

// Launchers (enqueue only; return the launch's hipError_t).
hipError_t launch_cache_init(const InitParams &p, int32_t dtype, int32_t head_dim, hipStream_t s);
hipError_t launch_append(const AppendParams &p, int32_t dtype, int32_t head_dim, hipStream_t s);
hipError_t launch_decode(const DecodeParams &p, int32_t dtype, int32_t head_dim, hipStream_t s);
hipError_t launch_masked(const MaskedParams &p, int32_t head_dim, hipStream_t s);
// Work split of the packed backward (host-known sizes only).
struct BwdPlan {
  int32_t parts, nkb_pre, nkb_win, n_pad, kpre;
  size_t bytes_rows;   // nd_row + nls
  size_t bytes_parts;  // part_dk + part_dv (0 when parts == 1)
};
BwdPlan plan_masked_bwd(int32_t seq_len, int32_t ref_len, int32_t heads, int32_t requested_parts);
hipError_t launch_masked_bwd(const MaskedBwdParams &p, hipStream_t s);
hipError_t launch_clear_word(int32_t *word, hipStream_t s);
hipError_t launch_probe_read(const void *buf, size_t bytes, float *sink, int32_t workgroups, hipStream_t s);
hipError_t launch_probe_mfma(float *sink, int32_t workgroups, int32_t iters, hipStream_t s);
hipError_t launch_probe_cu(uint32_t *out, int32_t workgroups, int32_t iters, int32_t kind, hipStream_t s);

}  // namespace rswa
